// kv_append.hip — new-token append of the paged-KV decode step (gfx950).
//
// One wave per head vector of the batch: B * (Hq + Hkv) vectors, Q heads first, then KV heads
// (a KV-head wave also stores the matching V row). Per vector:
//   optional RMS normalisation  y = x / sqrt(mean(x^2) + eps) * w
//     (page "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlock: QNorm/KNorm
//      before RoPE; page "soft3/glia/run/arch/decoder/forward.rs", forward_layer: per-head norm)
//   RoPE, rotate-half pairs (i, i + D/2) by pos * theta^(-2i/D)
//     (hybrid_decoder.go, runHybridAttentionBlock: HybridRoPE(positions, HeadDim, RopeTheta);
//      forward.rs, forward_layer: rope_dim = head_dim for LlamaStyle layers)
//   f32 -> 16-bit code, round to nearest even, and the store into row
//   (tables[b][pos / bs], pos % bs) of the [num_blocks, bs, Hkv, D] pool
//     (page "makarna/pkg/kvcache/paged_cache.go": float32ToFloat16Bits, float32ToBFloat16Bits,
//      GetBlockForPosition, GetBlockOffset, Append).
//
// Numerics, chosen so the stored bits are reproducible on any IEEE machine:
//   - the sum of squares is accumulated in double in index order, every product and sum
//     rounded separately (no contraction in this file);
//   - angle, cos, sin and both rotation terms are double; each result is rounded once to float;
//   - a NaN that comes out of this arithmetic is stored as the canonical quiet NaN 0x7FC00000
//     (IEEE 754 leaves its sign and payload to the implementation); V is converted untouched,
//     so its NaN payloads follow the conversion rule.
// The kernel is latency bound (a few hundred KiB per step), so it favours exactness over speed.
#include "pkv_internal.h"

#pragma clang fp contract(off)

namespace pkv {
namespace {

// f32 bits -> IEEE binary16 bits, round to nearest even. Normal results use the
// "add half-ulp minus one plus the kept lsb, then truncate" form on the re-biased word, so a
// carry out of the fraction bumps the exponent by itself; subnormal results shift the
// significand (with its implicit bit) into the 2^-24 grid and round on the dropped bits.
__device__ __forceinline__ uint16_t f32_to_f16_bits(uint32_t u) {
    const uint32_t sign = (u >> 16) & 0x8000u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) {  // NaN: sign, all-ones exponent, 10 leading payload bits, non-zero
        uint32_t pl = (a >> 13) & 0x3FFu;
        return (uint16_t)(sign | 0x7C00u | (pl ? pl : 1u));
    }
    if (a >= 0x477FF000u)   // >= 65520 (max + half ulp) and +-Inf: infinity
        return (uint16_t)(sign | 0x7C00u);
    if (a >= 0x38800000u) { // >= 2^-14: normal binary16
        const uint32_t r = a - 0x38000000u;  // exponent bias 127 -> 15
        return (uint16_t)(sign | ((r + 0x0FFFu + ((r >> 13) & 1u)) >> 13));
    }
    if (a <= 0x33000000u)   // <= 2^-25: rounds to zero (2^-25 itself is a tie to even 0)
        return (uint16_t)sign;
    const uint32_t e = a >> 23;                     // 102 .. 112
    const uint32_t m = (a & 0x007FFFFFu) | 0x00800000u;
    const uint32_t sh = 126u - e;                   // 14 .. 24
    uint32_t q = m >> sh;
    const uint32_t rem = m & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1u);
    q += (rem > half) | ((rem == half) & (q & 1u));
    return (uint16_t)(sign | q);  // q == 0x400 is the smallest normal, encoded correctly
}

// f32 bits -> bfloat16 bits, round to nearest even on the low half word (carries into the
// exponent and overflows to Inf by themselves); NaN keeps sign and 7 leading payload bits,
// forced non-zero.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(uint32_t u) {
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) {
        uint32_t pl = (u >> 16) & 0x7Fu;
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7F80u | (pl ? pl : 1u));
    }
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint16_t encode16(float x, bool bf16) {
    const uint32_t u = __float_as_uint(x);
    return bf16 ? f32_to_bf16_bits(u) : f32_to_f16_bits(u);
}

__device__ __forceinline__ float canonical_if_nan(float v) {
    return __builtin_isnan(v) ? __uint_as_float(0x7FC00000u) : v;
}

constexpr int kWaves = 4;
constexpr int kMaxD = 256;

__global__ __launch_bounds__(kWaves * 64) void kv_append_kernel(AppendArgs a) {
    __shared__ float xs[kWaves][kMaxD];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int per_seq = a.Hq + a.Hkv;
    const int64_t vec = (int64_t)blockIdx.x * kWaves + wave;
    const bool active = vec < (int64_t)a.B * per_seq;
    const int D = a.D;
    const int half = D >> 1;

    int b = 0, head = 0;
    bool is_q = false;
    const float* src = nullptr;
    if (active) {
        b = (int)(vec / per_seq);
        const int j = (int)(vec % per_seq);
        is_q = j < a.Hq;
        head = is_q ? j : j - a.Hq;
        src = is_q ? a.q_in + ((int64_t)b * a.Hq + head) * D
                   : a.k_in + ((int64_t)b * a.Hkv + head) * D;
        for (int d = lane; d < D; d += 64) xs[wave][d] = src[d];
    }
    __syncthreads();  // staged before q_out (which may alias q_in) is written
    if (!active) return;

    const float* x = xs[wave];
    const float* w = is_q ? a.q_norm_w : a.k_norm_w;
    double r = 1.0;
    if (w != nullptr) {
        double ss = 0.0;
        for (int d = 0; d < D; ++d) {
            const double xd = (double)x[d];
            ss = ss + xd * xd;
        }
        r = 1.0 / sqrt(ss / (double)D + (double)a.eps);
    }

    const int pos = a.positions[b];
    // destination row; an out-of-range position or block id skips the pool store
    int64_t row = -1;
    if (!is_q && pos >= 0 && pos / a.bs < a.max_blocks) {
        const int64_t blk = a.tables[(int64_t)b * a.max_blocks + pos / a.bs];
        if (blk >= 0 && blk < a.num_blocks)
            row = ((blk * a.bs + pos % a.bs) * a.Hkv + head) * (int64_t)D;
    }

    for (int i = lane; i < half; i += 64) {
        float x0 = x[i];
        float x1 = x[i + half];
        if (w != nullptr) {
            x0 = (float)(((double)x0 * r) * (double)w[i]);
            x1 = (float)(((double)x1 * r) * (double)w[i + half]);
        }
        const double inv_freq = pow((double)a.theta, -(2.0 * (double)i) / (double)D);
        const double angle = (double)pos * inv_freq;
        double s, c;
        sincos(angle, &s, &c);
        const double t0 = (double)x0 * c;
        const double t1 = (double)x1 * s;
        const double t2 = (double)x1 * c;
        const double t3 = (double)x0 * s;
        const float y0 = canonical_if_nan((float)(t0 - t1));
        const float y1 = canonical_if_nan((float)(t2 + t3));
        if (is_q) {
            float* qo = a.q_out + ((int64_t)b * a.Hq + head) * D;
            qo[i] = y0;
            qo[i + half] = y1;
        } else if (row >= 0) {
            a.k_pool[row + i] = encode16(y0, a.bf16);
            a.k_pool[row + i + half] = encode16(y1, a.bf16);
        }
    }
    if (!is_q && row >= 0) {
        const float* vsrc = a.v_in + ((int64_t)b * a.Hkv + head) * D;
        for (int d = lane; d < D; d += 64) a.v_pool[row + d] = encode16(vsrc[d], a.bf16);
    }
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
    const int64_t vecs = (int64_t)a.B * (a.Hq + a.Hkv);
    const int64_t grid = (vecs + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
