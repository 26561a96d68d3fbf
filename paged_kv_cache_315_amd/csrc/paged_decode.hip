// paged_decode.hip — paged-attention decode of the paged-KV decode step (gfx950).
//
// out[b][h] = softmax_t(scale * q[b][h] . K[t][g]) . V[t][g], g = h / G, t < context_lens[b],
// token t of sequence b at block tables[b][t / bs], slot t % bs of the
// [num_blocks, bs, Hkv, D] pools.
//   (page "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlockBatch: one query
//    row per sequence over per-sequence block lists, kvLens, scale = 1/sqrt(HeadDim);
//    page "soft3/glia/run/arch/decoder/forward.rs", forward_layer CPU attention path: kv head
//    h / (Hq / Hkv), max-subtracted exponentials normalised by their sum;
//    page "makarna/pkg/kvcache/paged_cache.go", viewsLockedAt: only the first kvLen tokens of
//    the block list are valid.)
//
// Work decomposition (split-K over the token axis):
//   grid (S, Hkv, B); workgroup (s, g, b) owns tokens [s*P, min((s+1)*P, L)) of sequence b and
//   the G query heads of KV head g, so every K/V row is read from HBM exactly once per step.
//   Its 4 waves take interleaved 16-token tiles. Inside a wave a K or V row of D codes is
//   spread over R = D/8 lanes (one 16-byte load each), so one dwordx4 load instruction moves
//   64/R consecutive token rows. Scores are reduced over the R lanes with DPP row operations
//   (every lane ends with the same sum), the online softmax keeps a running max m, sum l and
//   weighted V sum per head in float, with exp2 on log2(e)-prescaled scores.
//   The 4 waves merge through LDS; a sequence with one partition writes out directly, otherwise
//   the workgroup stores (m, l, acc) and the merge kernel combines the partitions:
//     M = max m_i, out = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i.
//
// Numerics: K/V codes decode exactly to float; dot products, exponentials and sums are float.
// Tokens outside [0, L) are never multiplied in (their rows are not loaded), so NaN padding in
// unused slots cannot leak into the result. A running max of -inf (no finite score yet) uses 0
// as the exponent base so exp2(-inf - (-inf)) never appears.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kTileTokens = 16;          // tokens per wave per iteration
constexpr float kLog2e = 1.4426950408889634f;

// ---- cross-lane helpers ------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over groups of R consecutive lanes; every lane of a group receives the same value (each
// step adds a lane to its partner under an involution, so both partners add the same pair).
template <int R>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(R == 4 || R == 8 || R == 16 || R == 32, "R");
    x += dpp_f<0xB1>(x);                      // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp_f<0x4E>(x);                      // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (R >= 8) x += dpp_f<0x141>(x);   // row_half_mirror: quad <-> quad in 8 lanes
    if constexpr (R >= 16) x += dpp_f<0x140>(x);  // row_mirror: half <-> half in 16 lanes
    if constexpr (R >= 32) x += __shfl_xor(x, 16);
    return x;
}

// Reduction across the 64/R groups of a wave (lanes l, l ^ R, l ^ 2R, ...).
template <int R>
__device__ __forceinline__ float cross_group_max(float x) {
#pragma unroll
    for (int off = R; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
template <int R>
__device__ __forceinline__ float cross_group_sum(float x) {
#pragma unroll
    for (int off = R; off < 64; off <<= 1) x += __shfl_xor(x, off);
    return x;
}

template <bool BF16>
__device__ __forceinline__ void decode8(const uint4 raw, float (&f)[8]) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (BF16) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        } else {
            f[2 * i] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w[i] & 0xFFFFu));
            f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w[i] >> 16));
        }
    }
}

// Attended length of a sequence: context_lens[b], capped by max_context_len and by the
// tokens its table row can address (so every table and pool index stays in range).
__device__ __forceinline__ int clamp_len(int L, const DecodeArgs& a) {
    const int64_t cap = min((int64_t)a.max_context_len, (int64_t)a.max_blocks * a.bs);
    return (int)min((int64_t)L, cap);
}

// ---- partition kernel --------------------------------------------------------------------
template <int D, int G, bool BF16>
__global__ __launch_bounds__(kWaves * 64) void paged_decode_part_kernel(DecodeArgs a) {
    constexpr int R = D / 8;                 // lanes per token row (8 codes per lane)
    constexpr int TPL = 64 / R;              // token rows per load instruction
    constexpr int U = kTileTokens / TPL;     // loads per tile
    static_assert(U >= 1 && U * TPL == kTileTokens, "tile");

    __shared__ float s_acc[kWaves][G][D];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];

    const int s = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int row = lane / R;
    const int col = lane % R;

    const int L = clamp_len(a.context_lens[b], a);
    const int t_begin = s * a.split_tokens;
    if (t_begin >= L) return;                // whole workgroup exits together
    const int t_end = min(L, t_begin + a.split_tokens);
    const int nsplit = (L + a.split_tokens - 1) / a.split_tokens;

    const int Hq = a.Hkv * G;
    const float qs = a.scale * kLog2e;
    float qr[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float4* qp = reinterpret_cast<const float4*>(
            a.q + ((int64_t)b * Hq + g * G + h) * D + col * 8);
        const float4 q0 = qp[0], q1 = qp[1];
        qr[h][0] = q0.x * qs; qr[h][1] = q0.y * qs; qr[h][2] = q0.z * qs; qr[h][3] = q0.w * qs;
        qr[h][4] = q1.x * qs; qr[h][5] = q1.y * qs; qr[h][6] = q1.z * qs; qr[h][7] = q1.w * qs;
    }

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
    }

    const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
    const int64_t nb_max = a.num_blocks - 1;
    const int64_t tok_stride = (int64_t)a.Hkv * D;   // codes between slots of a block

    for (int base = t_begin + wave * kTileTokens; base < t_end; base += kWaves * kTileTokens) {
        uint4 kraw[U], vraw[U];
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = base + u * TPL + row;
            valid[u] = t < t_end;
            if (valid[u]) {
                int64_t blk = trow[t / a.bs];
                blk = blk < 0 ? 0 : (blk > nb_max ? nb_max : blk);
                const int64_t off = (blk * a.bs + t % a.bs) * tok_stride + (int64_t)g * D + col * 8;
                kraw[u] = *reinterpret_cast<const uint4*>(a.k_pool + off);
                vraw[u] = *reinterpret_cast<const uint4*>(a.v_pool + off);
            } else {
                kraw[u] = make_uint4(0, 0, 0, 0);
                vraw[u] = make_uint4(0, 0, 0, 0);
            }
        }
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[8];
            decode8<BF16>(kraw[u], kf);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d0 = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) d0 = fmaf(qr[h][j], kf[j], d0);
                sc[u][h] = group_sum<R>(d0);
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (valid[u]) mx = fmaxf(mx, sc[u][h]);
            mx = cross_group_max<R>(mx);
            const float m_new = fmaxf(m[h], mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2f(m[h] - m_use);
            m[h] = m_new;
            l[h] *= alpha;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[h][j] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (valid[u]) {
                    const float p = exp2f(sc[u][h] - m_use);
                    l[h] += p;
                    float vf[8];
                    decode8<BF16>(vraw[u], vf);
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(p, vf[j], acc[h][j]);
                }
            }
        }
    }

    // combine the token-row groups of the wave, then the waves of the workgroup
#pragma unroll
    for (int h = 0; h < G; ++h) {
        l[h] = cross_group_sum<R>(l[h]);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] = cross_group_sum<R>(acc[h][j]);
    }
    if (row == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) s_acc[wave][h][col * 8 + j] = acc[h][j];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            s_m[wave][h] = m[h];
            s_l[wave][h] = l[h];
        }
    }
    __syncthreads();

    for (int i = threadIdx.x; i < G * D; i += kWaves * 64) {
        const int h = i / D;
        const int d = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float e = exp2f(s_m[w][h] - M_use);
            num = fmaf(e, s_acc[w][h][d], num);
            den = fmaf(e, s_l[w][h], den);
        }
        const int hq = g * G + h;
        if (nsplit == 1) {
            a.out[((int64_t)b * Hq + hq) * D + d] = num / den;
        } else {
            const int64_t pi = ((int64_t)b * Hq + hq) * a.S + s;
            a.part_acc[pi * D + d] = num;
            if (d == 0) {
                a.part_ml[pi * 2] = M;
                a.part_ml[pi * 2 + 1] = den;
            }
        }
    }
}

// ---- merge kernel: one wave per (b, query head) --------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void paged_decode_merge_kernel(DecodeArgs a) {
    constexpr int PER_LANE = (D + 63) / 64;
    const int Hq = a.Hkv * (a.Hq / a.Hkv);
    const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (pair >= (int64_t)a.B * Hq) return;
    const int b = (int)(pair / Hq);
    const int L = clamp_len(a.context_lens[b], a);
    const int nsplit = (L + a.split_tokens - 1) / a.split_tokens;
    if (nsplit <= 1) return;  // written by the partition kernel (or nothing to attend)
    const float* ml = a.part_ml + pair * a.S * 2;
    float M = -INFINITY;
    for (int i = 0; i < nsplit; ++i) M = fmaxf(M, ml[2 * i]);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    float num[PER_LANE];
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) num[k] = 0.f;
    float den = 0.f;
    const float* pa = a.part_acc + pair * a.S * D;
    for (int i = 0; i < nsplit; ++i) {
        const float e = exp2f(ml[2 * i] - M_use);
        den = fmaf(e, ml[2 * i + 1], den);
#pragma unroll
        for (int k = 0; k < PER_LANE; ++k) {
            const int d = lane + 64 * k;
            if (d < D) num[k] = fmaf(e, pa[(int64_t)i * D + d], num[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) {
        const int d = lane + 64 * k;
        if (d < D) a.out[pair * D + d] = num[k] / den;
    }
}

template <int D, int G, bool BF16>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    dim3 grid((unsigned)a.S, (unsigned)a.Hkv, (unsigned)a.B);
    hipLaunchKernelGGL((paged_decode_part_kernel<D, G, BF16>), grid, dim3(kWaves * 64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.S <= 1) return e;
    const int64_t pairs = (int64_t)a.B * a.Hq;
    hipLaunchKernelGGL((paged_decode_merge_kernel<D>), dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t dispatch_g(const DecodeArgs& a, hipStream_t stream) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_typed<D, 1, BF16>(a, stream);
        case 2: return launch_typed<D, 2, BF16>(a, stream);
        case 3: return launch_typed<D, 3, BF16>(a, stream);
        case 4: return launch_typed<D, 4, BF16>(a, stream);
        case 5: return launch_typed<D, 5, BF16>(a, stream);
        case 6: return launch_typed<D, 6, BF16>(a, stream);
        case 7: return launch_typed<D, 7, BF16>(a, stream);
        case 8: return launch_typed<D, 8, BF16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16>
hipError_t dispatch_d(const DecodeArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 32: return dispatch_g<32, BF16>(a, stream);
        case 64: return dispatch_g<64, BF16>(a, stream);
        case 128: return dispatch_g<128, BF16>(a, stream);
        case 256: return dispatch_g<256, BF16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
    return a.bf16 ? dispatch_d<true>(a, stream) : dispatch_d<false>(a, stream);
}

}  // namespace pkv
