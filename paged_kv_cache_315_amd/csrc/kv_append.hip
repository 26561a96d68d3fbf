// kv_append.hip — new-token append of the paged-KV decode step (gfx950).
//
// One workgroup per row, its waves taking the row's Hq + Hkv head vectors in turn (a KV head also
// stores the matching V row). A row is one new token: sequence b at positions[b]
// (one token per sequence), or token i of sequence b's chunk at positions[b] + i (page
// "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlock: a block of tokens is
// appended at the cache's current length). Per vector:
//   optional RMS normalisation  y = x / sqrt(mean(x^2) + eps) * w
//     (page "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlock: QNorm/KNorm
//      before RoPE; page "soft3/glia/run/arch/decoder/forward.rs", forward_layer: per-head norm)
//   RoPE, rotate-half pairs (i, i + R/2) by pos * theta^(-2i/R) over the first R = rope_dim dims
//     (hybrid_decoder.go, runHybridAttentionBlock: the RoPE op takes positions, head dim and
//      base; forward.rs, forward_layer: the full head dimension rotates for LlamaStyle layers,
//      and a per-layer rotary dimension R < D gives partial rotary), the other dims only normed
//   optional per-head V normalisation in float (forward.rs, forward_layer CPU path,
//     v_norm_per_head): v * (1 / sqrt(sum(v^2) / D + eps)), one rounding per operation
//   f32 -> 16-bit code, round to nearest even, and the store into row
//   (tables[b][pos / bs], pos % bs) of the [num_blocks, bs, Hkv, D] pool
//     (page "makarna/pkg/kvcache/paged_cache.go": float32ToFloat16Bits, float32ToBFloat16Bits,
//      GetBlockForPosition, GetBlockOffset, Append).
//
// Numerics (helpers in pkv_device.h), chosen so the stored bits are reproducible on any IEEE
// machine:
//   - the sum of squares is accumulated in double in index order, every product and sum
//     rounded separately (no contraction in this file);
//   - angle, cos, sin and both rotation terms are double; each result is rounded once to float;
//   - a NaN that comes out of this arithmetic is stored as the canonical quiet NaN 0x7FC00000
//     (IEEE 754 leaves its sign and payload to the implementation); V is converted untouched,
//     so its NaN payloads follow the conversion rule.
// The kernel is latency bound (a few hundred KiB per step), so it favours exactness over speed.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kMaxD = 256;

// Stores one value into a pool: a 16-bit code, or the float itself for float32 pools (page
// "makarna/pkg/kvcache/paged_cache.go", Append: float32 rows are copied unchanged).
__device__ __forceinline__ void store_elem(uint16_t* pool, int64_t i, float y, const AppendArgs& a) {
    if (a.f32) reinterpret_cast<float*>(pool)[i] = y;
    else pool[i] = encode16(y, a.bf16);
}

// One workgroup per row (new token): the rotary cos / sin of the token's position are computed
// once into LDS and shared by its Hq + Hkv head vectors, which the 4 waves take in turn.
__global__ __launch_bounds__(kWaves * 64) void kv_append_kernel(AppendArgs a) {
    __shared__ float xs[kWaves][kMaxD];
    __shared__ double s_cs[kMaxD / 2][2];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x;
    const int D = a.D;

    int b, pos;
    if (a.cu_seqlens != nullptr) {
        // sequence of the row: the last b with cu_seqlens[b] <= row
        int lo = 0, hi = a.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu_seqlens[mid] <= row) lo = mid; else hi = mid - 1;
        }
        b = lo;
        pos = a.positions[b] + (row - a.cu_seqlens[b]);
    } else {
        b = row;
        pos = a.positions[b];
    }
    const int rhalf = a.rope_dim >> 1;   // rotary pairs (i, i + rhalf), i < rhalf
    for (int i = threadIdx.x; i < rhalf; i += kWaves * 64)
        rope_cs(pos, a.theta, i, a.rope_dim, s_cs[i][0], s_cs[i][1]);
    // destination pool row of the token (per KV head: + head * D); an out-of-range position or
    // block id skips the pool stores
    int64_t prow0 = -1;
    if (pos >= 0 && pos / a.bs < a.max_blocks) {
        const int64_t blk = a.tables[(int64_t)b * a.max_blocks + pos / a.bs];
        if (blk >= 0 && blk < a.num_blocks) prow0 = (blk * a.bs + pos % a.bs) * a.Hkv * (int64_t)D;
    }
    __syncthreads();  // cos / sin ready

    float* x = xs[wave];
    for (int j = wave; j < a.Hq + a.Hkv; j += kWaves) {
        const bool is_q = j < a.Hq;
        const int head = is_q ? j : j - a.Hq;
        const float* src = is_q ? a.q_in + ((int64_t)row * a.Hq + head) * D
                                : a.k_in + ((int64_t)row * a.Hkv + head) * D;
        for (int d = lane; d < D; d += 64) x[d] = src[d];
        wave_lds_sync();
        const float* w = is_q ? a.q_norm_w : a.k_norm_w;
        const double r = w != nullptr ? rms_inv(x, D, a.eps) : 1.0;
        const int64_t prow = is_q || prow0 < 0 ? -1 : prow0 + (int64_t)head * D;
        float* qo = a.q_out + ((int64_t)row * a.Hq + head) * D;
        for (int i = lane; i < rhalf; i += 64) {
            float x0 = x[i];
            float x1 = x[i + rhalf];
            if (w != nullptr) {
                x0 = norm_elem(x0, r, w[i]);
                x1 = norm_elem(x1, r, w[i + rhalf]);
            }
            float y0, y1;
            rope_rotate(x0, x1, s_cs[i][0], s_cs[i][1], y0, y1);
            if (is_q) {
                qo[i] = y0;
                qo[i + rhalf] = y1;
            } else if (prow >= 0) {
                store_elem(a.k_pool, prow + i, y0, a);
                store_elem(a.k_pool, prow + i + rhalf, y1, a);
            }
        }
        // partial rotary: the dims from rope_dim on are only normed
        for (int j = a.rope_dim + lane; j < D; j += 64) {
            const float y = w != nullptr ? norm_elem(x[j], r, w[j]) : x[j];
            if (is_q) qo[j] = y;
            else if (prow >= 0) store_elem(a.k_pool, prow + j, y, a);
        }
        if (prow >= 0) {
            const float* vsrc = a.v_in + ((int64_t)row * a.Hkv + head) * D;
            if (a.v_norm) {
                wave_lds_sync();
                for (int d = lane; d < D; d += 64) x[d] = vsrc[d];
                wave_lds_sync();
                const float sc = vnorm_scale(x, D, a.eps);
                for (int d = lane; d < D; d += 64)
                    store_elem(a.v_pool, prow + d, vnorm_elem(x[d], sc), a);
            } else {
                for (int d = lane; d < D; d += 64) store_elem(a.v_pool, prow + d, vsrc[d], a);
            }
        }
        wave_lds_sync();  // x is reused by the wave's next vector
    }
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)a.rows), dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
