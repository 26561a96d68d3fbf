/*
 * pkv_oracle.c — plain, slow, single-threaded CPU oracle of the paged-KV decode step.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
 * leg load this library. The product path (paged_kv_cache_315_amd/) never links, imports
 * or calls it, and this file shares no code, header, table or constant with the HIP path.
 *
 * Arithmetic: IEEE double, evaluated in program order. Build with
 *   gcc -O2 -ffp-contract=off -fno-fast-math
 * so that no product and sum are fused and nothing is reassociated.
 *
 * Sources (web pages, cited by title and section):
 *   [MK-DEC]  makarna/pkg/model/arch/hybrid_decoder.go
 *             - runHybridAttentionBlock: QK-norm before RoPE; the attention scale is one over the
 *               square root of the head dimension, held as a float; the new tokens go in at the
 *               cache's current length, and attention covers that length plus the new tokens.
 *             - runHybridAttentionBlockBatch: one new token per sequence; its position is the
 *               number of tokens already cached and it attends to one more token than that;
 *               per-sequence block lists.
 *   [MK-KV]   makarna/pkg/kvcache/paged_cache.go
 *             - float32ToFloat16Bits / float32ToBFloat16Bits: the stored-bit rules.
 *             - GetBlockForPosition / GetBlockOffset: block = list[pos / BlockSize], slot = pos % BlockSize.
 *             - Append: inside its block, a token's row of (KV heads x head dim) values starts at
 *               its slot times the row length (token-major block rows); K and V are separate
 *               tensors per block.
 *             - viewsLockedAt: only the first kvLen tokens of the block list are valid.
 *   [GL-FWD]  soft3/glia/run/arch/decoder/forward.rs
 *             - forward_layer, QK-norm step: RMS normalisation per head vector with q_norm/k_norm.
 *             - forward_layer, RoPE step: full head_dim rotary for LlamaStyle layers.
 *             - forward_layer, CPU attention path: query head h reads KV head h divided by the
 *               group size; scores are scaled dot products, exponentials are taken after
 *               subtracting the maximum, normalised by their sum, and weight the value rows.
 *             - forward_layer, RoPE step: a per-layer rotary dimension (partial rotary);
 *               CPU path: per-head V normalisation in float (v_norm_per_head); the KV cache as a
 *               ring of cache_seq slots from which the last min(total, cache_seq) tokens are read.
 *
 * Readings where the pages are silent (each one is listed with its reason in the design notes):
 *   R-ROPE   rotate-half pairing (i, i + D/2), angle pos * theta^(-2i/D), all in double,
 *            one rounding of each rotated element to float.
 *   R-NORM   y = x / sqrt(mean(x^2) + eps) * w per head vector, double internals.
 *   R-BF16NAN  NaN inputs to the bf16 rule keep the sign and the 7 leading payload bits,
 *            forced non-zero (the fp16 rule's NaN treatment carried to bf16 width).
 *   R-PART   partial rotary (rope_dim < D): rotate-half pairs (i, i + rope_dim/2) inside the first
 *            rope_dim dims, angle pos * theta^(-2i/rope_dim); dims from rope_dim on unchanged.
 *   R-WIN    sliding window W: a query at attended length L sees positions max(0, L - W) .. L - 1
 *            (the last W tokens, the ring's read range without its storage reuse).
 *   R-READ   RoPE applied at read: the append with rope_dim = 0 rotates nothing (the pool holds the
 *            un-rotated, normed keys, q_out is the normed query); attention then rotates the
 *            query to position L - 1 and key t to position t, in double.
 *   R-NAN    a NaN that the norm / V-norm / RoPE arithmetic produces is the canonical quiet NaN
 *            0x7FC00000 (IEEE 754 leaves the sign and payload of such a NaN to the
 *            implementation); a NaN that reaches the converter untouched (V) keeps its bits.
 *
 * Parity status of each function is stated in its comment ("pinned by" / "parity unpinned").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PKVO_OK 0
#define PKVO_ERR_ARG 1
#define PKVO_ERR_RANGE 2

#define PKVO_F16 1
#define PKVO_BF16 2
#define PKVO_F32 3  /* float32 pool elements (no conversion) */

/* Planted mistakes for the tests that prove the pins bite (0 = the oracle as specified).
 * Each mutant is a plausible slip: a dropped term, a wrong sign or index, an off-by-one. */
#ifndef PKVO_MUTANT
#define PKVO_MUTANT 0
#endif
#define MUT(n) (PKVO_MUTANT == (n))

/* ------------------------------------------------------------------------------------------
 * Conversions float -> 16-bit codes.
 *
 * [MK-KV] float32ToFloat16Bits and float32ToBFloat16Bits fix the stored bits. For every
 * non-NaN input both rules give the IEEE-754 round-to-nearest, ties-to-even result (with
 * overflow to infinity at max + half an ulp), so the oracle writes that definition out
 * directly on the VALUE: count how many quanta of the target format's spacing the magnitude
 * holds, round that count with rint() (ties to even under the default rounding mode), and
 * assemble the code. Only the NaN branch is a bit rule and is taken from the page as stated.
 *
 * Pinned by: the exhaustive nearest/ties-to-even property over all 2^32 inputs, x86 F16C /
 * AVX512-BF16 hardware conversion on normal inputs, numpy's float16 cast, and hand-derived
 * values from the page's rules (tests/golden/convert_values.txt).
 * ------------------------------------------------------------------------------------------ */

/* Round the magnitude a >= 0 (finite) to a binary format with `prec` significand bits
 * (implicit bit included) and minimum normal exponent emin, maximum exponent emax.
 * Returns the code without sign: exponent field (biased by 1 - emin) << (prec-1) | fraction,
 * or the infinity code when the rounded value exceeds the largest finite one. */
static uint32_t round_magnitude(double a, int prec, int emin, int emax)
{
    const uint32_t frac_bits = (uint32_t)(prec - 1);
    const uint32_t inf_code = (uint32_t)(emax - emin + 2) << frac_bits;
    const double one_binade = ldexp(1.0, prec - 1); /* quanta count at the bottom of a binade */
    if (a == 0.0)
        return 0;
    int e2;
    (void)frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;      /* a in [2^E, 2^(E+1)) */
    if (E < emin)
        E = emin;        /* subnormal range: the quantum stays at 2^(emin - prec + 1) */
    /* number of quanta of size 2^(E - prec + 1); exact (a has at most 24 significant bits) */
    double q = MUT(7) ? round(ldexp(a, prec - 1 - E)) : rint(ldexp(a, prec - 1 - E));
    if (q >= 2.0 * one_binade) { /* rounding carried into the next binade */
        q = q / 2.0;
        E += 1;
    }
    if (E > emax)
        return inf_code;
    if (q < one_binade) /* subnormal (or zero): exponent field 0, fraction = quanta count */
        return (uint32_t)q;
    return ((uint32_t)(E - emin + 1) << frac_bits) | ((uint32_t)q - (uint32_t)one_binade);
}

/* [MK-KV] float32ToFloat16Bits. */
uint16_t pkvo_f32_to_f16(float x)
{
    uint32_t bits;
    memcpy(&bits, &x, 4);
    const uint16_t sign = (bits & 0x80000000u) ? 0x8000u : 0u;
    if (isnan(x)) {
        /* page rule: keep the sign, all-ones exponent, and the 10 leading payload bits,
         * forced to be non-zero so the code stays a NaN (no quieting). */
        uint16_t payload = (uint16_t)((bits & 0x007FFFFFu) >> 13);
        if (payload == 0)
            payload = 1;
        return (uint16_t)(sign | 0x7C00u | payload);
    }
    if (isinf(x))
        return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | round_magnitude(fabs((double)x), 11, -14, 15));
}

/* [MK-KV] float32ToBFloat16Bits for non-NaN inputs; R-BF16NAN for NaN inputs (the page's
 * rule, applied to a NaN, can round the payload into an infinity or wrap it to zero). */
uint16_t pkvo_f32_to_bf16(float x)
{
    uint32_t bits;
    memcpy(&bits, &x, 4);
    const uint16_t sign = (bits & 0x80000000u) ? 0x8000u : 0u;
    if (isnan(x)) {
        uint16_t payload = (uint16_t)((bits & 0x007FFFFFu) >> 16);
        if (payload == 0)
            payload = 1;
        return (uint16_t)(sign | 0x7F80u | payload);
    }
    if (isinf(x))
        return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | round_magnitude(fabs((double)x), 8, -126, 127));
}

/* Exact decode of a 16-bit code to float: value = significand * 2^exponent, built with
 * ldexp (every fp16 and bf16 value is a float). Pinned by numpy float16 -> float32 and by
 * bf16 bits << 16 reinterpretation in the tests. */
static float decode_code(uint16_t c, int prec, int emin, int emax)
{
    const int frac_bits = prec - 1;
    const int exp_bits = 15 - frac_bits;
    const uint32_t frac = c & ((1u << frac_bits) - 1u);
    const uint32_t ef = (c >> frac_bits) & ((1u << exp_bits) - 1u);
    const int neg = (c & 0x8000u) != 0;
    double v;
    if (ef == (1u << exp_bits) - 1u)
        v = frac ? NAN : INFINITY;
    else if (ef == 0)
        v = ldexp((double)frac, emin - frac_bits);
    else
        v = ldexp((double)((1u << frac_bits) | frac), (int)ef - 1 + emin - frac_bits);
    (void)emax;
    return (float)(neg ? -v : v);
}

float pkvo_f16_to_f32(uint16_t c) { return decode_code(c, 11, -14, 15); }
float pkvo_bf16_to_f32(uint16_t c) { return decode_code(c, 8, -126, 127); }

static uint16_t encode(float x, int dtype)
{
    return dtype == PKVO_F16 ? pkvo_f32_to_f16(x) : pkvo_f32_to_bf16(x);
}

static float decode(uint16_t c, int dtype)
{
    return dtype == PKVO_F16 ? pkvo_f16_to_f32(c) : pkvo_bf16_to_f32(c);
}

/* Pool elements: 16-bit codes, or (PKVO_F32) the float itself — [MK-KV] Append copies float32
 * rows into a float32 block unchanged, and [MK-DEC] dispatches float32 KV to its plain paged
 * kernel. A NaN from the norm / RoPE arithmetic is already canonical (R-NAN); a NaN input that
 * reaches the pool untouched keeps its bits, as it does through the 16-bit converters. */
static float pool_get(const void* pool, int64_t o, int dtype)
{
    if (dtype == PKVO_F32)
        return ((const float*)pool)[o];
    return decode(((const uint16_t*)pool)[o], dtype);
}

static void pool_put(void* pool, int64_t o, float x, int dtype)
{
    if (dtype == PKVO_F32)
        ((float*)pool)[o] = x;
    else
        ((uint16_t*)pool)[o] = encode(x, dtype);
}

/* Convert n floats to codes (array form for the tests). */
void pkvo_encode_array(const float* x, uint16_t* out, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = encode(x[i], dtype);
}

void pkvo_decode_array(const uint16_t* c, float* out, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = decode(c[i], dtype);
}

/* ------------------------------------------------------------------------------------------
 * Per-head QK RMS normalisation, reading R-NORM.
 * [MK-DEC] runHybridAttentionBlock applies QNorm / KNorm (RMSNorm with a weight and eps) to
 * the projected Q and K before RoPE; [GL-FWD] forward_layer reshapes Q to [num_heads, head_dim]
 * and K to [kv_heads, head_dim] and normalises each row with the q_norm / k_norm weight, and its
 * per-head V norm shows the form x / sqrt(mean(x^2) + eps).
 * Pinned by: constant-vector closed form, mean(y^2) identity with unit weight, an independent
 * numpy formula (tests/oracle_pins.py, pin_norm_*), and inside the append by an independent
 * numpy chain norm -> complex-form RoPE -> library cast with distinct q / k weights
 * (pin_append_qk_norm_chain); the canonical NaN of norm / RoPE results by pin_append_nan_rows.
 * ------------------------------------------------------------------------------------------ */
static float canonical_nan_if_nan(float v)
{
    if (isnan(v) && !MUT(19)) {
        const uint32_t qnan = 0x7FC00000u;
        memcpy(&v, &qnan, 4);
    }
    return v;
}

void pkvo_rmsnorm_head(const float* x, const float* w, float eps, int D, float* y)
{
    double ss = 0.0;
    for (int j = 0; j < D; ++j)
        ss += (double)x[j] * (double)x[j];
    const double r = 1.0 / sqrt(ss / (double)D + (MUT(3) ? 0.0 : (double)eps));
    for (int j = 0; j < D; ++j)
        y[j] = canonical_nan_if_nan((float)(((double)x[j] * r) * (double)w[j]));
}

/* ------------------------------------------------------------------------------------------
 * RoPE on one head vector, reading R-ROPE.
 * [MK-DEC] runHybridAttentionBlock rotates Q and K with the RoPE op (positions, head dim, base)
 * after the QK-norm (and only fuses it when HeadDim is even and at most 256); [GL-FWD]
 * forward_layer rotates the full head dimension for LlamaStyle layers.
 * Each rotated element that comes out NaN is stored as the canonical quiet NaN (R-NAN).
 * Pinned by: position 0 is the identity bit for bit, norm preservation, the relative-position
 * property, an independent complex-exponential formulation in numpy.
 * ------------------------------------------------------------------------------------------ */
/* Partial rotary (R-PART): the first rope_dim dims rotate as a rope_dim-sized head; the rest
 * are copied unchanged. rope_dim = D is the full rotation. */
void pkvo_rope_head_partial(const float* x, int D, int rope_dim, int pos, float theta, float* y)
{
    const int half = rope_dim / 2;
    const double span = MUT(12) ? (double)D : (double)rope_dim;
    for (int i = 0; i < half; ++i) {
        const double inv_freq = pow((double)theta, -((MUT(2) ? 1.0 : 2.0) * (double)i) / span);
        const double angle = (double)(pos + (MUT(8) ? 1 : 0)) * inv_freq;
        const double c = cos(angle);
        const double s = sin(angle);
        const double x0 = (double)x[i];
        const double x1 = (double)x[i + half];
        y[i] = canonical_nan_if_nan((float)(MUT(1) ? x0 * c + x1 * s : x0 * c - x1 * s));
        y[i + half] = canonical_nan_if_nan((float)(x1 * c + x0 * s));
    }
    for (int j = 2 * half; j < D; ++j)
        y[j] = x[j];
}

void pkvo_rope_head(const float* x, int D, int pos, float theta, float* y)
{
    pkvo_rope_head_partial(x, D, D, pos, theta, y);
}

/* ------------------------------------------------------------------------------------------
 * Per-head V normalisation. [GL-FWD] forward_layer, CPU path (v_norm_per_head): for each KV
 * head, the sum of squares is accumulated in float in index order, rms = sqrt(sum * (1/D) +
 * eps) in float, and every element is multiplied by the float reciprocal of rms. The page fixes
 * float arithmetic here, so the oracle keeps float (single rounding per operation, no fused
 * multiply-add).
 * Pinned by: the constant-vector closed form, the unit-mean-square property, and the
 * reduction to a plain copy when the rows already have unit mean square and eps = 0.
 * ------------------------------------------------------------------------------------------ */
void pkvo_vnorm_head(const float* v, int D, float eps, float* y)
{
    float sumsq = 0.0f;
    for (int j = 0; j < D; ++j) {
        const float sq = v[j] * v[j];
        sumsq = sumsq + sq;
    }
    const float inv_d = 1.0f / (float)D;
    const float rms = sqrtf(sumsq * inv_d + (MUT(13) ? 0.0f : eps));
    const float scale = 1.0f / rms;
    for (int j = 0; j < D; ++j)
        y[j] = canonical_nan_if_nan(v[j] * scale);
}

/* Pool element offset of (block, slot, kv head, dim) in a [num_blocks, bs, Hkv, D] pool
 * ([MK-KV] Append: a token's row of Hkv * D values starts at slot * (Hkv * D), head-minor). */
static int64_t pool_offset(int64_t blk, int slot, int g, int d, int bs, int Hkv, int D)
{
    return ((blk * bs + slot) * Hkv + g) * (int64_t)D + d;
}

/* One new token: the query heads are normed (optional) and rotated into q_out; the K heads are
 * normed, rotated, converted and stored, and the V heads converted and stored, into the pool row
 * (table_row[pos / bs], pos % bs). Returns PKVO_ERR_RANGE (storing nothing) if the position or
 * its block id is out of range. tmp / rot: scratch of D floats. */
static int append_token(const float* q_in, const float* k_in, const float* v_in, float* q_out,
                        void* k_pool, void* v_pool, const int32_t* table_row,
                        int max_blocks, int pos, const float* q_norm_w, const float* k_norm_w,
                        float eps, float theta, int rope_dim, int v_norm, int Hq, int Hkv, int D,
                        int bs, int64_t num_blocks, int dtype, float* tmp, float* rot)
{
    if (pos < 0 || pos / bs >= max_blocks)
        return PKVO_ERR_RANGE;
    const int64_t blk = table_row[pos / bs];
    const int slot = pos % bs;
    if (blk < 0 || blk >= num_blocks)
        return PKVO_ERR_RANGE;
    const float* qw = MUT(16) ? k_norm_w : q_norm_w;
    const float* kw = MUT(16) ? q_norm_w : k_norm_w;
    /* Q: optional norm, then RoPE; the float result is the output (not stored in the pool). */
    for (int h = 0; h < Hq; ++h) {
        const float* x = q_in + (int64_t)h * D;
        const float* src = x;
        if (qw) {
            pkvo_rmsnorm_head(x, qw, eps, D, tmp);
            src = tmp;
        }
        pkvo_rope_head_partial(src, D, rope_dim, pos, theta, q_out + (int64_t)h * D);
    }
    /* K: optional norm, RoPE, convert, store. V: convert, store. */
    for (int g = 0; g < Hkv; ++g) {
        const float* x = k_in + (int64_t)g * D;
        const float* src = x;
        if (MUT(18) && kw) {
            /* planted: rotated first, normed after */
            pkvo_rope_head_partial(x, D, rope_dim, pos, theta, tmp);
            pkvo_rmsnorm_head(tmp, kw, eps, D, rot);
        } else {
            if (kw && !MUT(17)) {
                pkvo_rmsnorm_head(x, kw, eps, D, tmp);
                src = tmp;
            }
            pkvo_rope_head_partial(src, D, rope_dim, pos, theta, rot);
        }
        const float* v = v_in + (int64_t)g * D;
        if (v_norm) {
            pkvo_vnorm_head(v, D, eps, tmp);
            v = tmp;
        }
        for (int d = 0; d < D; ++d) {
            const int64_t o = pool_offset(blk, slot, g, d, bs, Hkv, D);
            pool_put(k_pool, o, rot[d], dtype);
            pool_put(v_pool, o, v[d], dtype);
        }
    }
    return PKVO_OK;
}

/* ------------------------------------------------------------------------------------------
 * KV append for a batch of one new token per sequence.
 * [MK-DEC] runHybridAttentionBlockBatch: for each sequence the new K/V row is appended at
 * the sequence's current length (the number of tokens already cached), and RoPE uses that
 * position.
 * [MK-KV] Append: the block is list[pos / BlockSize], the slot pos % BlockSize, and the value is
 * converted f32 -> fp16 (CastF32ToF16 on the GPU path, float32ToFloat16Bits on the CPU path).
 *
 * Inputs (host): q_in [B,Hq,D], k_in / v_in [B,Hkv,D] f32; pools [num_blocks,bs,Hkv,D] codes;
 * tables [B,max_blocks]; positions [B]; q_norm_w / k_norm_w [D] (both NULL: no QK-norm).
 * Outputs: q_out [B,Hq,D] f32 (normed, rotated), the new rows of k_pool / v_pool.
 * Returns PKVO_ERR_RANGE (and writes nothing more) if a position or block id is out of range.
 * ------------------------------------------------------------------------------------------ */
int pkvo_kv_append_v(const float* q_in, const float* k_in, const float* v_in, float* q_out,
                     void* k_pool, void* v_pool, const int32_t* tables, int max_blocks,
                     const int32_t* positions, const float* q_norm_w, const float* k_norm_w,
                     float eps, float theta, int rope_dim, int v_norm, int B, int Hq, int Hkv,
                     int D, int bs, int64_t num_blocks, int dtype)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || (D & 1) || bs <= 0 || Hq % Hkv)
        return PKVO_ERR_ARG;
    if (rope_dim < 0 || rope_dim > D || (rope_dim & 1))
        return PKVO_ERR_ARG;
    if ((q_norm_w == NULL) != (k_norm_w == NULL))
        return PKVO_ERR_ARG;
    float* tmp = (float*)malloc(sizeof(float) * (size_t)D);
    float* rot = (float*)malloc(sizeof(float) * (size_t)D);
    if (!tmp || !rot) {
        free(tmp);
        free(rot);
        return PKVO_ERR_ARG;
    }
    int status = PKVO_OK;
    for (int b = 0; b < B && status == PKVO_OK; ++b)
        status = append_token(q_in + (int64_t)b * Hq * D, k_in + (int64_t)b * Hkv * D,
                              v_in + (int64_t)b * Hkv * D, q_out + (int64_t)b * Hq * D, k_pool,
                              v_pool, tables + (int64_t)b * max_blocks, max_blocks, positions[b],
                              q_norm_w, k_norm_w, eps, theta, rope_dim, v_norm, Hq, Hkv, D, bs,
                              num_blocks, dtype, tmp, rot);
    free(tmp);
    free(rot);
    return status;
}

int pkvo_kv_append(const float* q_in, const float* k_in, const float* v_in, float* q_out,
                   void* k_pool, void* v_pool, const int32_t* tables, int max_blocks,
                   const int32_t* positions, const float* q_norm_w, const float* k_norm_w,
                   float eps, float theta, int B, int Hq, int Hkv, int D, int bs,
                   int64_t num_blocks, int dtype)
{
    return pkvo_kv_append_v(q_in, k_in, v_in, q_out, k_pool, v_pool, tables, max_blocks,
                            positions, q_norm_w, k_norm_w, eps, theta, D, 0, B, Hq, Hkv, D, bs,
                            num_blocks, dtype);
}

/* ------------------------------------------------------------------------------------------
 * KV append of a chunk of new tokens per sequence (prefill, or several tokens at a time).
 * [MK-DEC] runHybridAttentionBlock: a block of seqLen tokens (token-major q [seqLen, Hq*D],
 * k / v [seqLen, Hkv*D]) goes into the cache at its current length startPos, token i at position
 * startPos + i, RoPE taking each token's own position; [MK-KV] Append fills the block list from
 * that position on, spanning as many blocks as needed.
 * Tokens of sequence b are q_in rows cu_seqlens[b] .. cu_seqlens[b+1]-1, at positions
 * start_pos[b] + i; they are processed in that order. With one token per sequence this is
 * pkvo_kv_append with positions = start_pos.
 * Pinned by: equality with pkvo_kv_append when every sequence has one token, equality of one call
 * with a chunk split over two calls, and the per-token rows stored where the table says.
 * ------------------------------------------------------------------------------------------ */
int pkvo_prefill_append_v(const float* q_in, const float* k_in, const float* v_in,
                          float* q_out, void* k_pool, void* v_pool, const int32_t* tables,
                          int max_blocks, const int32_t* cu_seqlens, const int32_t* start_pos,
                          const float* q_norm_w, const float* k_norm_w, float eps, float theta,
                          int rope_dim, int v_norm, int B, int Hq, int Hkv, int D, int bs,
                          int64_t num_blocks, int dtype)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || (D & 1) || bs <= 0 || Hq % Hkv)
        return PKVO_ERR_ARG;
    if (rope_dim < 0 || rope_dim > D || (rope_dim & 1))
        return PKVO_ERR_ARG;
    if ((q_norm_w == NULL) != (k_norm_w == NULL))
        return PKVO_ERR_ARG;
    for (int b = 0; b < B; ++b)
        if (cu_seqlens[b + 1] < cu_seqlens[b])
            return PKVO_ERR_ARG;
    float* tmp = (float*)malloc(sizeof(float) * (size_t)D);
    float* rot = (float*)malloc(sizeof(float) * (size_t)D);
    if (!tmp || !rot) {
        free(tmp);
        free(rot);
        return PKVO_ERR_ARG;
    }
    int status = PKVO_OK;
    for (int b = 0; b < B && status == PKVO_OK; ++b)
        for (int r = cu_seqlens[b]; r < cu_seqlens[b + 1] && status == PKVO_OK; ++r) {
            const int pos = start_pos[b] + (r - cu_seqlens[b]) + (MUT(10) ? 1 : 0);
            status = append_token(q_in + (int64_t)r * Hq * D, k_in + (int64_t)r * Hkv * D,
                                  v_in + (int64_t)r * Hkv * D, q_out + (int64_t)r * Hq * D,
                                  k_pool, v_pool, tables + (int64_t)b * max_blocks, max_blocks,
                                  pos, q_norm_w, k_norm_w, eps, theta, rope_dim, v_norm, Hq, Hkv,
                                  D, bs, num_blocks, dtype, tmp, rot);
        }
    free(tmp);
    free(rot);
    return status;
}

int pkvo_prefill_append(const float* q_in, const float* k_in, const float* v_in, float* q_out,
                        void* k_pool, void* v_pool, const int32_t* tables, int max_blocks,
                        const int32_t* cu_seqlens, const int32_t* start_pos,
                        const float* q_norm_w, const float* k_norm_w, float eps, float theta,
                        int B, int Hq, int Hkv, int D, int bs, int64_t num_blocks, int dtype)
{
    return pkvo_prefill_append_v(q_in, k_in, v_in, q_out, k_pool, v_pool, tables, max_blocks,
                                 cu_seqlens, start_pos, q_norm_w, k_norm_w, eps, theta, D, 0, B,
                                 Hq, Hkv, D, bs, num_blocks, dtype);
}

/* RoPE of one head vector in double, not rounded (R-ROPE angles, R-PART pairing): used when
 * the pool holds un-rotated keys and attention rotates query and keys itself (R-READ). */
static void rope_double(const double* x, int D, int rope_dim, int pos, double theta, double* y)
{
    const int half = rope_dim / 2;
    for (int i = 0; i < half; ++i) {
        const double inv_freq = pow(theta, -(2.0 * (double)i) / (double)rope_dim);
        const double angle = (double)pos * inv_freq;
        const double c = cos(angle);
        const double s = sin(angle);
        y[i] = x[i] * c - x[i + half] * s;
        y[i + half] = x[i + half] * c + x[i] * s;
    }
    for (int j = 2 * half; j < D; ++j)
        y[j] = x[j];
}

/* Attention of one query token (all Hq heads, q_row [Hq, D]) over the first L tokens of the
 * sequence whose block list is table_row; writes out_row [Hq, D]. kc / vc: scratch of
 * L * Hkv * D floats, e: scratch of L doubles. read_theta > 0 (R-READ): the query is rotated to
 * position L - 1 and key t to position t (first rope_dim dims, double) before the dot product. */
static int attend_row(const float* q_row, const void* k_pool, const void* v_pool,
                      const int32_t* table_row, int max_blocks, int L, int window, float scale,
                      float* out_row, int Hq, int Hkv, int D, int bs, int64_t num_blocks,
                      int dtype, float* kc, float* vc, double* e, double read_theta,
                      int rope_dim)
{
    const int G = Hq / Hkv;
    if (L < 1 || (L + bs - 1) / bs > max_blocks)
        return PKVO_ERR_RANGE;
    /* R-WIN: the query sees positions lo .. L-1; gathered as tokens 0 .. L-lo-1 */
    const int lo = window > 0 && L > window ? L - window - (MUT(14) ? 1 : 0) : 0;
    const int n = L - lo;
    /* gather: token t lives in block table_row[t / bs] at slot t % bs */
    for (int i = 0; i < n; ++i) {
        const int t = lo + i;
        const int64_t blk = table_row[t / bs];
        if (blk < 0 || blk >= num_blocks)
            return PKVO_ERR_RANGE;
        for (int g = 0; g < Hkv; ++g)
            for (int d = 0; d < D; ++d) {
                const int64_t o = pool_offset(blk, (t + (MUT(5) ? 1 : 0)) % bs, g, d, bs, Hkv, D);
                kc[((int64_t)i * Hkv + g) * D + d] = pool_get(k_pool, o, dtype);
                vc[((int64_t)i * Hkv + g) * D + d] = pool_get(v_pool, o, dtype);
            }
    }
    const int qpos = L - 1;
    L = n;
    double qd[256], qr[256], kd[256], kr[256];
    if (read_theta > 0.0 && (D > 256 || rope_dim < 2 || rope_dim > D))
        return PKVO_ERR_ARG;
    for (int h = 0; h < Hq; ++h) {
        const int g = MUT(4) ? h % Hkv : h / G;
        const float* qh = q_row + (int64_t)h * D;
        if (read_theta > 0.0) {
            for (int d = 0; d < D; ++d)
                qd[d] = (double)qh[d];
            rope_double(qd, D, rope_dim, qpos, read_theta, qr);
        }
        double m = -INFINITY;
        for (int t = 0; t < L; ++t) {
            const float* kt = kc + ((int64_t)t * Hkv + g) * D;
            double dot = 0.0;
            if (read_theta > 0.0) {
                for (int d = 0; d < D; ++d)
                    kd[d] = (double)kt[d];
                rope_double(kd, D, rope_dim, lo + t + (MUT(15) ? 1 : 0), read_theta, kr);
                for (int d = 0; d < D; ++d)
                    dot += qr[d] * kr[d];
            } else {
                for (int d = 0; d < D; ++d)
                    dot += (double)qh[d] * (double)kt[d];
            }
            e[t] = (MUT(6) ? 1.0 : (double)scale) * dot;
            if (e[t] > m) /* NaN never compares greater: ignored by the max */
                m = e[t];
        }
        double l = 0.0;
        for (int t = 0; t < L; ++t) {
            e[t] = exp(e[t] - m);
            l += e[t];
        }
        for (int d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int t = 0; t < L; ++t)
                acc += e[t] * (double)vc[((int64_t)t * Hkv + g) * D + d];
            out_row[(int64_t)h * D + d] = (float)(acc / l);
        }
    }
    return PKVO_OK;
}

/* Runs attend_row over n rows: row r reads q + r*Hq*D, the block list of sequence seq[r] and
 * L = lens[r] tokens, writes out + r*Hq*D (rows with row_mask[r] == 0 are skipped). */
static int attend_rows(const float* q, const void* k_pool, const void* v_pool,
                       const int32_t* tables, int max_blocks, const int* seq, const int* lens,
                       int window, float scale, float* out, int n, int Hq, int Hkv, int D, int bs,
                       int64_t num_blocks, int dtype, const uint8_t* row_mask, double read_theta,
                       int rope_dim)
{
    int Lmax = 1;
    for (int r = 0; r < n; ++r)
        if ((!row_mask || row_mask[r]) && lens[r] > Lmax)
            Lmax = lens[r];
    float* kc = (float*)malloc(sizeof(float) * (size_t)Lmax * Hkv * D);
    float* vc = (float*)malloc(sizeof(float) * (size_t)Lmax * Hkv * D);
    double* e = (double*)malloc(sizeof(double) * (size_t)Lmax);
    int status = (kc && vc && e) ? PKVO_OK : PKVO_ERR_ARG;
    for (int r = 0; r < n && status == PKVO_OK; ++r) {
        if (row_mask && !row_mask[r])
            continue;
        status = attend_row(q + (int64_t)r * Hq * D, k_pool, v_pool,
                            tables + (int64_t)seq[r] * max_blocks, max_blocks, lens[r], window,
                            scale,
                            out + (int64_t)r * Hq * D, Hq, Hkv, D, bs, num_blocks, dtype, kc, vc,
                            e, read_theta, rope_dim);
    }
    free(kc);
    free(vc);
    free(e);
    return status;
}

/* ------------------------------------------------------------------------------------------
 * Paged-attention decode for one query token per sequence.
 * [MK-DEC] runHybridAttentionBlockBatch passes q [B, Hq*D], per-sequence block lists, the attended lengths and
 * scale = 1/sqrt(HeadDim); [MK-KV] viewsLockedAt clips the last block to kvLen tokens;
 * [GL-FWD] forward_layer's CPU attention path fixes the arithmetic: the query head h reads KV head
 * h / (Hq/Hkv); s_t = (q . k_t) * scale; m = max s_t; e_t = exp(s_t - m); out = sum e_t v_t / sum e_t.
 * Steps as written here: gather the sequence's K and V into contiguous float arrays
 * [L, Hkv, D] (exact decode of the codes), then dense attention in double for every query head.
 * The max ignores NaN scores (as a float max fold does); a NaN score still makes sum e_t NaN.
 *
 * row_mask (may be NULL): compute only the sequences b with row_mask[b] != 0.
 * Pinned by: brute force against an independent numpy formulation, closed forms (L = 1,
 * K = 0, V[t] = t), block-permutation invariance, GQA = MHA with duplicated heads.
 * ------------------------------------------------------------------------------------------ */
int pkvo_paged_attn_decode_v(const float* q, const void* k_pool, const void* v_pool,
                             const int32_t* tables, int max_blocks, const int32_t* context_lens,
                             int window, float scale, float* out, int B, int Hq, int Hkv, int D,
                             int bs, int64_t num_blocks, int dtype, const uint8_t* row_mask)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || Hq % Hkv || window < 0)
        return PKVO_ERR_ARG;
    int* seq = (int*)malloc(sizeof(int) * (size_t)(B > 0 ? B : 1));
    int* lens = (int*)malloc(sizeof(int) * (size_t)(B > 0 ? B : 1));
    if (!seq || !lens) {
        free(seq);
        free(lens);
        return PKVO_ERR_ARG;
    }
    for (int b = 0; b < B; ++b) {
        seq[b] = b;
        lens[b] = context_lens[b] - (MUT(9) && context_lens[b] > 1 ? 1 : 0);
    }
    const int status = attend_rows(q, k_pool, v_pool, tables, max_blocks, seq, lens, window,
                                   scale, out, B, Hq, Hkv, D, bs, num_blocks, dtype, row_mask,
                                   0.0, D);
    free(seq);
    free(lens);
    return status;
}

/* ------------------------------------------------------------------------------------------
 * Decode over a pool of un-rotated keys, rotating at read (R-READ).
 * [MK-DEC] runHybridAttentionBlock / runHybridAttentionBlockBatch: when RoPE is fused into the
 * paged kernel the standalone RoPE of Q and K is skipped, the cache receives the un-rotated K,
 * and the kernel (given the RoPE base) applies RoPE itself. What it computes is therefore the
 * decode above with q rotated to its position (L - 1) and every key t rotated to position t:
 * s_t = scale * (R_{L-1} q) . (R_t k_t), the rotations of R-ROPE / R-PART in double.
 * Pinned by: agreement with the stored-rotated path on float-exact pools (a pool of rotated keys
 * that the codes hold exactly), the relative-position property (shifting every position leaves
 * the output unchanged), an independent numpy complex-exponential formulation, and a planted
 * off-by-one key position that those catch.
 * ------------------------------------------------------------------------------------------ */
int pkvo_paged_attn_decode_rope(const float* q, const void* k_pool, const void* v_pool,
                                const int32_t* tables, int max_blocks,
                                const int32_t* context_lens, int window, float theta,
                                int rope_dim, float scale, float* out, int B, int Hq, int Hkv,
                                int D, int bs, int64_t num_blocks, int dtype,
                                const uint8_t* row_mask)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || D > 256 || bs <= 0 || Hq % Hkv ||
        window < 0 || !(theta > 0.0f) || rope_dim < 2 || rope_dim > D || (rope_dim & 1))
        return PKVO_ERR_ARG;
    int* seq = (int*)malloc(sizeof(int) * (size_t)(B > 0 ? B : 1));
    int* lens = (int*)malloc(sizeof(int) * (size_t)(B > 0 ? B : 1));
    if (!seq || !lens) {
        free(seq);
        free(lens);
        return PKVO_ERR_ARG;
    }
    for (int b = 0; b < B; ++b) {
        seq[b] = b;
        lens[b] = context_lens[b];
    }
    const int status = attend_rows(q, k_pool, v_pool, tables, max_blocks, seq, lens, window,
                                   scale, out, B, Hq, Hkv, D, bs, num_blocks, dtype, row_mask,
                                   (double)theta, rope_dim);
    free(seq);
    free(lens);
    return status;
}

int pkvo_paged_attn_decode(const float* q, const void* k_pool, const void* v_pool,
                           const int32_t* tables, int max_blocks, const int32_t* context_lens,
                           float scale, float* out, int B, int Hq, int Hkv, int D, int bs,
                           int64_t num_blocks, int dtype, const uint8_t* row_mask)
{
    return pkvo_paged_attn_decode_v(q, k_pool, v_pool, tables, max_blocks, context_lens, 0,
                                    scale, out, B, Hq, Hkv, D, bs, num_blocks, dtype, row_mask);
}

/* ------------------------------------------------------------------------------------------
 * Paged attention of a chunk of query tokens per sequence, causal.
 * [MK-DEC] runHybridAttentionBlock: after a block of seqLen tokens is appended at startPos, the
 * attention covers kvLen = startPos + seqLen tokens and is causal from startPos: query token i
 * (position startPos + i) sees the cached tokens and the new tokens up to and including itself,
 * that is the first startPos + i + 1 tokens of the sequence. The arithmetic of each query token
 * is that of the decode above with that length.
 * q / out [N, Hq, D] token-major; tokens of sequence b are rows cu_seqlens[b] ..
 * cu_seqlens[b+1]-1 at positions start_pos[b] + i. row_mask (may be NULL) selects rows.
 * Pinned by: equality with pkvo_paged_attn_decode for one token per sequence, an independent
 * numpy formulation with an explicit causal mask, insensitivity of each row to the K/V of later
 * positions, and equality of one call with a chunk split over two calls.
 * ------------------------------------------------------------------------------------------ */
int pkvo_paged_attn_prefill_v(const float* q, const void* k_pool, const void* v_pool,
                              const int32_t* tables, int max_blocks, const int32_t* cu_seqlens,
                              const int32_t* start_pos, int window, float scale, float* out,
                              int B, int Hq, int Hkv, int D, int bs, int64_t num_blocks,
                              int dtype, const uint8_t* row_mask)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || Hq % Hkv || window < 0)
        return PKVO_ERR_ARG;
    const int n = B > 0 ? cu_seqlens[B] : 0;
    for (int b = 0; b < B; ++b)
        if (cu_seqlens[b + 1] < cu_seqlens[b])
            return PKVO_ERR_ARG;
    int* seq = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    int* lens = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    if (!seq || !lens) {
        free(seq);
        free(lens);
        return PKVO_ERR_ARG;
    }
    for (int b = 0; b < B; ++b)
        for (int r = cu_seqlens[b]; r < cu_seqlens[b + 1]; ++r) {
            seq[r] = b;
            /* query token i of the chunk attends positions 0 .. start_pos[b] + i */
            lens[r] = start_pos[b] + (r - cu_seqlens[b]) + (MUT(11) ? 0 : 1);
        }
    const int status = attend_rows(q, k_pool, v_pool, tables, max_blocks, seq, lens, window,
                                   scale, out, n, Hq, Hkv, D, bs, num_blocks, dtype, row_mask,
                                   0.0, D);
    free(seq);
    free(lens);
    return status;
}

int pkvo_paged_attn_prefill(const float* q, const void* k_pool, const void* v_pool,
                            const int32_t* tables, int max_blocks, const int32_t* cu_seqlens,
                            const int32_t* start_pos, float scale, float* out, int B, int Hq,
                            int Hkv, int D, int bs, int64_t num_blocks, int dtype,
                            const uint8_t* row_mask)
{
    return pkvo_paged_attn_prefill_v(q, k_pool, v_pool, tables, max_blocks, cu_seqlens,
                                     start_pos, 0, scale, out, B, Hq, Hkv, D, bs, num_blocks,
                                     dtype, row_mask);
}
