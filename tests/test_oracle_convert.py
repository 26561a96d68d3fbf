"""Pins of the oracle's float -> fp16 / bf16 conversions and the exact decodes.

Sources: page "makarna/pkg/kvcache/paged_cache.go", float32ToFloat16Bits and
float32ToBFloat16Bits (the stored-bit rules). The oracle writes the rules as the IEEE
round-to-nearest-even definition on the value; these tests hold it to things it does not share:
hand-derived values from the page's bit rules, an exhaustive property + hardware check over all
2^32 inputs, numpy's float16 cast and torch's bfloat16 cast.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    rows = []
    with open(os.path.join(HERE, "golden", "convert_values.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            rows.append((int(parts[0], 16), int(parts[1], 16), int(parts[2], 16), parts[3]))
    return rows


@pytest.mark.parametrize("row", _golden(), ids=lambda r: f"{r[0]:08x}")
def test_golden_values(olib, row):
    bits, f16, b16, _tag = row
    x = np.array([bits], dtype=np.uint32).view(np.float32)
    assert int(oracle.encode(x, "f16", olib)[0]) == f16
    assert int(oracle.encode(x, "bf16", olib)[0]) == b16


def test_exhaustive_all_float_bit_patterns(olib, tmp_path):
    """All 2^32 inputs: nearest-even property and x86 F16C / AVX512-BF16 agreement."""
    exe = tmp_path / "conv_ex"
    subprocess.run(["gcc", "-O2", "-fopenmp", os.path.join(HERE, "native", "convert_exhaustive.c"),
                    oracle.LIB_PATH, f"-Wl,-rpath,{os.path.dirname(oracle.LIB_PATH)}", "-lm",
                    "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    lines = dict(l.split(" ", 1) for l in res.strip().splitlines())
    assert "bf16" in lines
    for fmt, rest in lines.items():
        if rest.startswith("skipped"):
            continue
        kv = dict(p.split("=") for p in rest.split())
        assert int(kv["checked"]) == 1 << 32, res
        assert int(kv["bad_property"]) == 0, res
        assert int(kv["bad_hw"]) == 0, res


def _sample_bits(n, seed):
    rng = np.random.default_rng(seed)
    u = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    # around every fp16/bf16 rounding boundary: all 2^16 upper halves with critical low halves
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    crit = np.array([0, 1, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x7FFF, 0x8000, 0x8001, 0xFFFF],
                    dtype=np.uint32)
    return np.concatenate([u, (hi[:, None] | crit[None, :]).ravel()])


def test_fp16_matches_numpy(olib):
    u = _sample_bits(1 << 22, 11)
    x = u.view(np.float32)
    keep = ~np.isnan(x)
    x = x[keep]
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle.encode(x, "f16", olib), ref)


def test_bf16_matches_torch(olib):
    u = _sample_bits(1 << 22, 12)
    x = u.view(np.float32)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.encode(x, "bf16", olib), ref)


def test_decode_all_codes(olib):
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f16 = oracle.decode(codes, "f16", olib)
    ref16 = codes.view(np.float16).astype(np.float32)
    nan = np.isnan(ref16)
    assert np.array_equal(np.isnan(f16), nan)
    np.testing.assert_array_equal(f16[~nan].view(np.uint32), ref16[~nan].view(np.uint32))
    b16 = oracle.decode(codes, "bf16", olib)
    refb = (codes.astype(np.uint32) << 16).view(np.float32)
    nan = np.isnan(refb)
    assert np.array_equal(np.isnan(b16), nan)
    np.testing.assert_array_equal(b16[~nan].view(np.uint32), refb[~nan].view(np.uint32))


def test_roundtrip_is_identity_on_codes(olib):
    """encode(decode(c)) == c for every non-NaN code: representable values are kept exactly."""
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for dt in ("f16", "bf16"):
        x = oracle.decode(codes, dt, olib)
        keep = ~np.isnan(x)
        np.testing.assert_array_equal(oracle.encode(x[keep], dt, olib), codes[keep])
