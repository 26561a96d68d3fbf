"""Every planted mistake in the oracle (PKVO_MUTANT=n in pkv_oracle.c) must fail at least one
pin: this shows the pins can tell a wrong oracle from the right one."""
import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    1: "RoPE: wrong sign on the first rotated half",
    2: "RoPE: frequency exponent i/D instead of 2i/D",
    3: "RMSNorm: eps dropped",
    4: "GQA: query head h reads KV head h % Hkv",
    5: "gather: slot off by one",
    6: "attention: scale dropped",
    7: "conversion: ties rounded away from zero",
    8: "RoPE: position off by one",
    9: "attention: one token short",
    10: "prefill append: positions off by one",
    11: "prefill attention: a query token does not see itself",
    12: "partial rotary: frequencies over head_dim instead of rope_dim",
    13: "V norm: eps dropped",
    14: "sliding window: one token too many",
    15: "RoPE at read: key positions off by one",
    16: "QK-norm: q and k weights swapped",
    17: "QK-norm: K norm skipped",
    18: "QK-norm: K rotated before it is normed",
    19: "norm / RoPE: an arithmetic NaN stored with its own sign and payload",
}


@pytest.mark.parametrize("n", sorted(MUTANTS), ids=lambda n: MUTANTS[n])
def test_mutant_is_caught(tmp_path, n):
    path = str(tmp_path / f"libpkv_oracle_m{n}.so")
    oracle.build(path, defines=(f"PKVO_MUTANT={n}",))
    lib = oracle.load(path)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {n} ({MUTANTS[n]}) passed every pin"
