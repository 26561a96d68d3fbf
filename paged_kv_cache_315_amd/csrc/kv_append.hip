// kv_append.hip — new-token append of the paged-KV decode step (gfx950).
//
// One wave per head vector: rows * (Hq + Hkv) vectors, Q heads first, then KV heads (a KV-head
// wave also stores the matching V row). A row is one new token: sequence b at positions[b]
// (one token per sequence), or token i of sequence b's chunk at positions[b] + i (page
// "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlock: a block of tokens is
// appended at the cache's current length). Per vector:
//   optional RMS normalisation  y = x / sqrt(mean(x^2) + eps) * w
//     (page "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlock: QNorm/KNorm
//      before RoPE; page "soft3/glia/run/arch/decoder/forward.rs", forward_layer: per-head norm)
//   RoPE, rotate-half pairs (i, i + D/2) by pos * theta^(-2i/D)
//     (hybrid_decoder.go, runHybridAttentionBlock: the RoPE op takes positions, head dim and
//      base; forward.rs, forward_layer: the full head dimension rotates for LlamaStyle layers)
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

__global__ __launch_bounds__(kWaves * 64) void kv_append_kernel(AppendArgs a) {
    __shared__ float xs[kWaves][kMaxD];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int per_row = a.Hq + a.Hkv;
    const int64_t vec = (int64_t)blockIdx.x * kWaves + wave;
    const bool active = vec < (int64_t)a.rows * per_row;
    const int D = a.D;
    const int half = D >> 1;

    int row = 0, b = 0, head = 0, pos = 0;
    bool is_q = false;
    const float* src = nullptr;
    if (active) {
        row = (int)(vec / per_row);
        const int j = (int)(vec % per_row);
        is_q = j < a.Hq;
        head = is_q ? j : j - a.Hq;
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
        src = is_q ? a.q_in + ((int64_t)row * a.Hq + head) * D
                   : a.k_in + ((int64_t)row * a.Hkv + head) * D;
        for (int d = lane; d < D; d += 64) xs[wave][d] = src[d];
    }
    __syncthreads();  // staged before q_out (which may alias q_in) is written
    if (!active) return;

    const float* x = xs[wave];
    const float* w = is_q ? a.q_norm_w : a.k_norm_w;
    const double r = w != nullptr ? rms_inv(x, D, a.eps) : 1.0;

    // destination pool row; an out-of-range position or block id skips the pool store
    int64_t prow = -1;
    if (!is_q && pos >= 0 && pos / a.bs < a.max_blocks) {
        const int64_t blk = a.tables[(int64_t)b * a.max_blocks + pos / a.bs];
        if (blk >= 0 && blk < a.num_blocks)
            prow = ((blk * a.bs + pos % a.bs) * a.Hkv + head) * (int64_t)D;
    }

    for (int i = lane; i < half; i += 64) {
        float x0 = x[i];
        float x1 = x[i + half];
        if (w != nullptr) {
            x0 = norm_elem(x0, r, w[i]);
            x1 = norm_elem(x1, r, w[i + half]);
        }
        double c, s;
        rope_cs(pos, a.theta, i, D, c, s);
        float y0, y1;
        rope_rotate(x0, x1, c, s, y0, y1);
        if (is_q) {
            float* qo = a.q_out + ((int64_t)row * a.Hq + head) * D;
            qo[i] = y0;
            qo[i + half] = y1;
        } else if (prow >= 0) {
            a.k_pool[prow + i] = encode16(y0, a.bf16);
            a.k_pool[prow + i + half] = encode16(y1, a.bf16);
        }
    }
    if (!is_q && prow >= 0) {
        const float* vsrc = a.v_in + ((int64_t)row * a.Hkv + head) * D;
        for (int d = lane; d < D; d += 64) a.v_pool[prow + d] = encode16(vsrc[d], a.bf16);
    }
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
    const int64_t vecs = (int64_t)a.rows * (a.Hq + a.Hkv);
    const int64_t grid = (vecs + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
