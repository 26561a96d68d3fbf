// paged_decode.hip — paged-attention decode of the paged-KV decode step (gfx950), fixed
// partitions of the token axis.
//
// out[b][h] = softmax_t(scale * q[b][h] . K[t][g]) . V[t][g], g = h / G, t < context_lens[b],
// token t of sequence b at block tables[b][t / bs], slot t % bs of the
// [num_blocks, bs, Hkv, D] pools.
//   (page "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlockBatch: one query
//    row per sequence over per-sequence block lists and lengths, scale one over sqrt(head dim);
//    page "soft3/glia/run/arch/decoder/forward.rs", forward_layer CPU attention path: kv head
//    h / (Hq / Hkv), max-subtracted exponentials normalised by their sum;
//    page "makarna/pkg/kvcache/paged_cache.go", viewsLockedAt: only the first kvLen tokens of
//    the block list are valid.)
//
// Work decomposition (split-K over the token axis):
//   grid (Hkv, S, B); work item (g, s, b) owns tokens [s*P, min((s+1)*P, L)) of sequence b and
//   the G query heads of KV head g, so every K/V row is read from HBM once per step. The KV
//   head is the fastest item index and each XCD takes a block of consecutive items, so the
//   workgroups of one XCD stream whole [bs, Hkv, D] rows of blocks (all head slices). The 4 waves of a workgroup take interleaved
//   16-token tiles, computed as decode_tile.h describes (QK^T and PV on the matrix cores, the
//   online softmax in registers, an exact float path for tiles holding non-finite codes), each
//   wave keeping the next tile's K/V rows in flight.
//   The 4 waves merge through LDS. A sequence with one partition writes out directly; otherwise
//   each workgroup stores (m, l, acc), and the last workgroup of (b, g) to finish (counted with
//   an atomic in the workspace, which it resets to zero) merges the partitions:
//     M = max m_i, out = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i.
//
// Tokens outside [0, L) (and before a sliding window) are never multiplied in, so NaN padding
// in unused slots cannot leak into the result. A running max of -inf uses 0 as the exponent
// base so exp2(-inf - (-inf)) never appears.
#include "decode_tile.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

using namespace dev;

constexpr int kWaves = kDecodeWaves;
constexpr int kTile = 16;       // tokens per wave per iteration
constexpr int kTblCap = 1024;   // block ids staged in LDS per workgroup (bounds split_tokens)
constexpr int kGMax = 8;        // query heads per KV head

// Attended length of a sequence: context_lens[b], capped by max_context_len and by the
// tokens its table row can address (so every table and pool index stays in range).
__device__ __forceinline__ int clamp_len(int L, const DecodeArgs& a) {
    const int64_t cap = min((int64_t)a.max_context_len, (int64_t)a.max_blocks * a.bs);
    if (a.lens_are_positions) return (L >= 0 && L < cap) ? L + 1 : 0;
    return (int)min((int64_t)L, cap);
}

template <int D, bool BF16>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void paged_decode_kernel(DecodeArgs a) {
    using Tile = DecodeTile<D, BF16>;
    union WaveLds {
        typename Tile::Scratch scr;  // the exact path's tile while streaming
        float acc[kGMax][D];         // the wave's partial result after it
    };
    __shared__ __align__(16) WaveLds s_w[kWaves];
    __shared__ int32_t s_tbl[kTblCap];
    __shared__ __align__(16) float s_q[kGMax][D];
    __shared__ float s_m[kWaves][kGMax];
    __shared__ float s_l[kWaves][kGMax];
    __shared__ int s_def[kWaves][kDecodeDefCap];
    __shared__ int s_last;

    // work item (g, s, b) of this workgroup: consecutive items per XCD (xcd_range), so the
    // workgroups of one XCD read all KV heads of their sequences
    const int n_items = (int)(gridDim.x * gridDim.y * gridDim.z);
    const int lin = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    const int item = xcd_range(lin, n_items);
    const int g = item % (int)gridDim.x;
    const int s = (item / (int)gridDim.x) % (int)gridDim.y;
    const int b = item / (int)(gridDim.x * gridDim.y);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int G = a.Hq / a.Hkv;

    const int L = clamp_len(a.context_lens[b], a);
    const int P = a.split_tokens;
    const int vis_lo = window_lo(L, a.window);        // first key the query sees
    const int t_first = vis_lo / kTile * kTile;       // partitions start at its tile
    const int t_begin = t_first + s * P;
    if (t_begin >= L) return;           // whole workgroup exits together
    const int t_end = min(L, t_begin + P);
    const int nsplit = (L - t_first + P - 1) / P;
    const int Hq = a.Hq;

    // ---- block ids of this partition and the G query rows -> LDS (the host keeps
    // split_tokens within kTblCap ids)
    const BlockDiv bdiv = make_div((uint32_t)a.bs);
    const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
    const int first_blk = (int)bdiv.div((uint32_t)t_begin);
    const int n_blk = min((int)bdiv.div((uint32_t)(t_end - 1)) - first_blk + 1, kTblCap);
    const int64_t nb_max = a.num_blocks - 1;
    for (int i = threadIdx.x; i < n_blk; i += kWaves * 64) {
        const int64_t id = trow[first_blk + i];
        s_tbl[i] = (int32_t)(id < 0 ? 0 : (id > nb_max ? nb_max : id));
    }
    const float* qsrc = a.q + ((int64_t)b * Hq + g * G) * D;
    for (int i = threadIdx.x; i < G * D; i += kWaves * 64) s_q[i / D][i % D] = qsrc[i];
    __syncthreads();

    auto qf = [&](int h, int d0, float (&o)[8]) {
        const float4* src = reinterpret_cast<const float4*>(&s_q[h][d0]);
        const float4 x0 = src[0], x1 = src[1];
        o[0] = x0.x; o[1] = x0.y; o[2] = x0.z; o[3] = x0.w;
        o[4] = x1.x; o[5] = x1.y; o[6] = x1.z; o[7] = x1.w;
    };
    TileSource src;
    src.k_pool = a.k_pool;
    src.v_pool = a.v_pool;
    src.tbl = s_tbl;
    src.first_blk = first_blk;
    src.tbl_cap = kTblCap;
    src.bdiv = bdiv;
    src.bs = a.bs;
    src.tile_in_block = a.bs % kTile == 0;
    src.tok_stride = (int64_t)a.Hkv * D;
    src.head_off = (int64_t)g * D;
    // this wave's first tile is requested before the query operands are built (always: a
    // wave without tiles reads the range's last tile, in bounds, and drops it)
    const int first_base = t_begin + wave * kTile;
    const bool have_first = first_base < t_end;
    typename Tile::Regs first;
    Tile::load_tile(src, first_base, t_begin, t_end, first);
    const float qs = a.scale * kLog2e;
    typename Tile::Query qop;
    Tile::setup_query(qf, G, qs, qop);
    typename Tile::State st;
    Tile::init(st);
    Tile::stream(src, t_begin, t_end, vis_lo, qop, st, G, qs, qf, s_w[wave].scr, s_def[wave],
                 []() {}, first, have_first);

    // ---- combine within each wave, then across the waves
    Tile::flush(st, G, s_m[wave], s_l[wave], &s_w[wave].acc[0][0]);
    __syncthreads();

    // ---- combine the waves: this partition's (M, den, num) per (head, dim)
    // Partials and counters are shared between workgroups that may sit on different XCDs
    // (each with its own L2), so every access to them is an agent-scope atomic: those are
    // coherent device-wide without writing back or invalidating whole L2s, which a release /
    // acquire fence at agent scope would do for every workgroup.
    float* part_acc = a.part_acc;
    float* part_ml = a.part_ml;
    for (int i = threadIdx.x; i < G * D; i += kWaves * 64) {
        const int h = i / D;
        const int d = i % D;
        float Mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) Mx = fmaxf(Mx, s_m[w][h]);
        const float M_use = (Mx == -INFINITY) ? 0.f : Mx;
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float e = exp2f(s_m[w][h] - M_use);
            num = fmaf(e, s_w[w].acc[h][d], num);
            den = fmaf(e, s_l[w][h], den);
        }
        const int hq = g * G + h;
        if (nsplit == 1) {
            a.out[((int64_t)b * Hq + hq) * D + d] = num / den;
        } else {
            const int64_t pi = ((int64_t)b * Hq + hq) * a.S + s;
            store_shared(part_acc + pi * D + d, num);
            if (d == 0) {
                store_shared(part_ml + pi * 2, Mx);
                store_shared(part_ml + pi * 2 + 1, den);
            }
        }
    }
    if (nsplit == 1) return;

    // ---- the last partition of (b, g) to finish merges all of them
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
    __syncthreads();                // ... and so are every other thread's
    int* counter = a.counters + (int64_t)b * a.Hkv + g;
    if (threadIdx.x == 0) s_last = arrive(counter) == nsplit - 1;
    __syncthreads();
    if (!s_last) return;
    for (int i = threadIdx.x; i < G * D; i += kWaves * 64) {
        const int h = i / D;
        const int d = i % D;
        const int64_t p0 = ((int64_t)b * Hq + g * G + h) * a.S;
        float Mx = -INFINITY;
        for (int k0 = 0; k0 < nsplit; k0 += 8) {
            float mk[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                mk[k] = k0 + k < nsplit ? load_shared(part_ml + (p0 + k0 + k) * 2) : -INFINITY;
#pragma unroll
            for (int k = 0; k < 8; ++k) Mx = fmaxf(Mx, mk[k]);
        }
        const float M_use = (Mx == -INFINITY) ? 0.f : Mx;
        float num = 0.f, den = 0.f;
        for (int k0 = 0; k0 < nsplit; k0 += 8) {
            float mk[8], lk[8], ak[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const bool ok = k0 + k < nsplit;
                const int64_t pk = p0 + k0 + k;
                mk[k] = ok ? load_shared(part_ml + pk * 2) : -INFINITY;
                lk[k] = ok ? load_shared(part_ml + pk * 2 + 1) : 0.f;
                ak[k] = ok ? load_shared(part_acc + pk * D + d) : 0.f;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float e = exp2f(mk[k] - M_use);
                den = fmaf(e, lk[k], den);
                num = fmaf(e, ak[k], num);
            }
        }
        a.out[((int64_t)b * Hq + g * G + h) * D + d] = num / den;
    }
    if (threadIdx.x == 0) store_shared(counter, 0);  // ready for the next call
}

template <int D, bool BF16>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    if (a.Hq / a.Hkv > kGMax) return hipErrorInvalidValue;
    dim3 grid((unsigned)a.Hkv, (unsigned)a.S, (unsigned)a.B);
    hipLaunchKernelGGL((paged_decode_kernel<D, BF16>), grid, dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

template <bool BF16>
hipError_t dispatch_d(const DecodeArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 32: return launch_typed<32, BF16>(a, stream);
        case 64: return launch_typed<64, BF16>(a, stream);
        case 128: return launch_typed<128, BF16>(a, stream);
        case 256: return launch_typed<256, BF16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
    return a.bf16 ? dispatch_d<true>(a, stream) : dispatch_d<false>(a, stream);
}

}  // namespace pkv
