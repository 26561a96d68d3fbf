// decode_balanced.hip — paged-attention decode with a balanced schedule over the whole batch,
// optionally fused with the new-token append (gfx950).
//
// What it computes is the decode of paged_decode.hip (and, fused, the append of kv_append.hip):
//   out[b][h] = softmax_t(scale * q[b][h] . K[t][g]) . V[t][g], g = h / G, t < L_b,
// with K/V read through the block table of each sequence
//   (page "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlockBatch;
//    page "soft3/glia/run/arch/decoder/forward.rs", forward_layer CPU attention path;
//    page "makarna/pkg/kvcache/paged_cache.go", GetBlockForPosition / GetBlockOffset / Append).
//
// Schedule. The K/V rows of the batch form one list of 16-token tiles: segment (b, g) holds the
// ceil(L_b / 16) tiles of KV head g of sequence b, segments in (b, g) order, each preceded by
// kUnitCost empty positions that stand for what starting a unit costs. The grid has one
// workgroup per resident slot (normally two per compute unit) and workgroup w takes positions
// [w*T, (w+1)*T), T = ceil(total / grid): every workgroup has the same work (tiles streamed
// plus units started) whatever the mix of lengths, and all of them are resident from start to
// end. Inside a
// workgroup the 4 waves interleave the 16-token tiles of each unit (the part of one segment
// that falls in the range); a tile is computed as decode_tile.h describes (QK^T and PV on the
// matrix cores, online softmax in registers, an exact float path for tiles holding non-finite
// codes), with the next tile's K/V loads in flight. When the block size is a multiple of 16 a
// tile lies in one block: one block id per tile, read from LDS by the whole wave. A unit
// requests its query heads (and, fused, the new K row) together with its first chunk of block
// ids, and the angles per position of the rotary pairs are computed once per workgroup.
//
// Pieces. A segment that lies inside one range is finished there (out = acc / l). A segment cut
// by range boundaries leaves one piece (m, l, acc) per workgroup it touches; a workgroup holds at
// most two such pieces (its first and its last segment), in slots 2w and 2w+1 of the workspace.
// The last workgroup to finish a segment (an agent-scope atomic counter per segment, reset after
// use) merges its pieces:  M = max m_i, out = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i.
//
// Fused append (APPEND): L_b = positions[b] + 1. Every unit rotates the query heads of its
// segment itself (norm + RoPE in double, like kv_append.hip; cos/sin computed once per unit and
// shared by its heads), the unit holding the segment's first tile writes q_out, and the unit
// holding its last tile (the new token p = L_b - 1) rotates and converts the new K row, converts
// the V row and stores both into the pool row (tables[b][p / bs], p % bs) before it streams its
// tiles; a workgroup barrier (release / acquire at workgroup scope) orders those stores before
// its own loads of the row. No other workgroup reads that row, so one launch does the step.
//
// Layer variants (VAR): partial rotary, V normalisation and a sliding window are run-time fields
// of the arguments. kVarNone takes them as the plain layer's constants (rotary over the whole
// head, no V norm, no window), which keeps the plain step free of their registers; kVarWindow
// reads only the window; kVarFull reads all three.
#include "decode_tile.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

using namespace dev;

#ifdef PKV_TIMELINE
#define PKV_STAMP(k, v)                                                                       \
    do {                                                                                      \
        if (threadIdx.x == 0 && a.timeline != nullptr)                                        \
            a.timeline[(int64_t)blockIdx.x * kTimelineStamps + (k)] = (v);                    \
    } while (0)
#else
#define PKV_STAMP(k, v) \
    do {                \
    } while (0)
#endif

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 16;
constexpr int kTblCap = 1024;     // block ids staged in LDS per chunk of a unit
constexpr int kUnitCost = kBalancedUnitCost;
constexpr int kPerThread = (kMaxBalancedBatch + kThreads - 1) / kThreads;
constexpr int kGMax = 8;          // query heads per KV head
constexpr int kVarNone = 0, kVarWindow = 1, kVarFull = 2;

// Query rotation of one unit and, for the unit holding a segment's last tile, the new token's
// K/V row (norm + RoPE in double over the first rope_dim dims, optional V norm in float,
// round-to-nearest-even codes; see kv_append.hip), stored into the pool before the unit streams
// its tiles. Expects s_q to hold the raw query heads, s_kx / s_vx the new K / V rows and s_wq /
// s_wk the norm weights (all staged in LDS, so the rotation issues no global loads), and s_inv
// the angles per position of the rotary pairs; ends with a barrier, after which this
// workgroup's own loads of the new row see the stored codes.
template <int D, bool BF16, int VAR>
__device__ __forceinline__ void rotate_and_append(const BalancedArgs& a, int G, int b, int g, int pnew,
                                               int64_t blk_new, bool owns_new, bool seg_first,
                                               float* s_q,
                                               const float* s_kx, const float* s_vx,
                                               const float* s_wq, const float* s_wk,
                                               const double* s_inv, double* s_cs, double* s_r,
                                               float* s_vsc) {
    const int tid = threadIdx.x;
    const int Hkv = a.Hkv;
    const int Hq = Hkv * G;
    const int rope_dim = VAR == kVarFull ? a.rope_dim : D;
    const int rhalf = rope_dim >> 1;       // rotary pairs (i, i + rhalf), i < rhalf
    const int64_t tok_stride = (int64_t)Hkv * D;
    for (int i = tid; i < rhalf; i += kThreads)
        rope_cs_from(pnew, s_inv[i], s_cs[2 * i], s_cs[2 * i + 1]);
    const bool norm = a.q_norm_w != nullptr;
    const bool vnorm = VAR == kVarFull && a.v_norm && owns_new;
    // the norms read whole staged rows that other waves wrote: wait for every staging store
    // (the condition is the same in every thread of the workgroup)
    if (norm || vnorm) __syncthreads();
    if (norm) {
        if (tid < G) s_r[tid] = rms_inv(s_q + tid * D, D, a.eps);
        if (tid == G && owns_new) s_r[G] = rms_inv(s_kx, D, a.eps);
    }
    if (vnorm && tid == G + 1) *s_vsc = vnorm_scale(s_vx, D, a.eps);
    __syncthreads();
    float* qo = a.q_out + ((int64_t)b * Hq + g * G) * D;
    for (int idx = tid; idx < G * rhalf; idx += kThreads) {
        const int h = idx / rhalf;
        const int i = idx - h * rhalf;
        float x0 = s_q[h * D + i], x1 = s_q[h * D + i + rhalf];
        if (norm) {
            x0 = norm_elem(x0, s_r[h], s_wq[i]);
            x1 = norm_elem(x1, s_r[h], s_wq[i + rhalf]);
        }
        float y0, y1;
        rope_rotate(x0, x1, s_cs[2 * i], s_cs[2 * i + 1], y0, y1);
        s_q[h * D + i] = y0;
        s_q[h * D + i + rhalf] = y1;
        if (seg_first) {
            qo[h * D + i] = y0;
            qo[h * D + i + rhalf] = y1;
        }
    }
    // partial rotary: the dims from rope_dim on are only normed
    const int rest = D - rope_dim;
    if (rest > 0)
        for (int idx = tid; idx < G * rest; idx += kThreads) {
            const int h = idx / rest;
            const int j = rope_dim + (idx - h * rest);
            const float y = norm ? norm_elem(s_q[h * D + j], s_r[h], s_wq[j]) : s_q[h * D + j];
            s_q[h * D + j] = y;
            if (seg_first) qo[h * D + j] = y;
        }
    if (owns_new) {
        int64_t row = -1;
        if (blk_new >= 0 && blk_new < a.num_blocks)
            row = (blk_new * a.bs + pnew % a.bs) * tok_stride + (int64_t)g * D;
        for (int i = tid; i < rhalf; i += kThreads) {
            float x0 = s_kx[i], x1 = s_kx[i + rhalf];
            if (norm) {
                x0 = norm_elem(x0, s_r[G], s_wk[i]);
                x1 = norm_elem(x1, s_r[G], s_wk[i + rhalf]);
            }
            float y0, y1;
            rope_rotate(x0, x1, s_cs[2 * i], s_cs[2 * i + 1], y0, y1);
            if (row >= 0) {
                a.k_pool[row + i] = encode16(y0, BF16);
                a.k_pool[row + i + rhalf] = encode16(y1, BF16);
            }
        }
        if (row >= 0) {
            for (int j = rope_dim + tid; j < D; j += kThreads) {
                const float y = norm ? norm_elem(s_kx[j], s_r[G], s_wk[j]) : s_kx[j];
                a.k_pool[row + j] = encode16(y, BF16);
            }
            const float vsc = vnorm ? *s_vsc : 1.f;
            for (int i = tid; i < D; i += kThreads)
                a.v_pool[row + i] = encode16(vnorm ? vnorm_elem(s_vx[i], vsc) : s_vx[i], BF16);
        }
    }
    __syncthreads();
}

template <int D, bool BF16, bool APPEND, int VAR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void decode_balanced_kernel(BalancedArgs a) {
    using Tile = DecodeTile<D, BF16>;
    constexpr int HALF = D / 2;

    __shared__ int s_len[kMaxBalancedBatch];
    __shared__ int s_pre[kMaxBalancedBatch + 1];
    __shared__ int s_scan[kWaves];
    __shared__ int32_t s_tbl[kTblCap];
    __shared__ __align__(16) float s_q[kGMax][D];
    __shared__ float s_kx[APPEND ? D : 1];
    __shared__ float s_vx[APPEND ? D : 1];
    __shared__ float s_wq[APPEND ? D : 1];   // QK-norm weights
    __shared__ float s_wk[APPEND ? D : 1];
    __shared__ float s_vsc;
    __shared__ double s_inv[APPEND ? HALF : 1];  // theta^(-2i/rope_dim) of rotary pair i
    __shared__ double s_cs[APPEND ? HALF : 1][2];
    __shared__ double s_r[kGMax + 1];
    // per wave: the exact path's tile while streaming, the wave's partial result after it
    union WaveLds {
        typename Tile::Scratch scr;
        float acc[kGMax][D];
    };
    __shared__ __align__(16) WaveLds s_w[kWaves];
    __shared__ float s_m[kWaves][kGMax];
    __shared__ float s_l[kWaves][kGMax];
    __shared__ int s_def[kWaves][kDecodeDefCap];   // tiles a wave left for the exact path
    __shared__ int s_last;

    PKV_STAMP(0, wall_clock64());
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int q4 = lane >> 4;
    const int B = a.B;
    const int Hkv = a.Hkv;
    const int G = a.Hq / a.Hkv;
    const int Hq = a.Hq;
    const int W = VAR != kVarNone ? a.window : 0;
    // tiles of a sequence of L tokens: from the one holding its first visible key to the last
    auto ntiles = [=](int L) { return (L + kTile - 1) / kTile - window_lo(L, W) / kTile; };
    // positions a segment of nt tiles takes in the list: its start cost, then its tiles
    auto span = [=](int nt) { return nt > 0 ? nt + kUnitCost : 0; };

    // ---- 1. lengths and the tile prefix of every sequence (all heads) -> LDS
    const int64_t cap64 = (int64_t)a.max_blocks * a.bs;
    const int cap = (int)min(cap64, (int64_t)(APPEND ? 0x7FFFFFFF : a.max_context_len));
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int b = tid * kPerThread + k;
        if (b < B) {
            int L;
            if constexpr (APPEND) {
                const int p = a.lens[b];  // positions: out-of-range sequences get no work
                L = (p >= 0 && p < cap) ? p + 1 : 0;
            } else {
                L = max(0, min(a.lens[b], cap));
            }
            s_len[b] = L;
            cnt += span(ntiles(L));
        }
    }
    if constexpr (APPEND) {  // while the lengths arrive
        const int rope_dim = VAR == kVarFull ? a.rope_dim : D;
        for (int i = tid; i < (rope_dim >> 1); i += kThreads)
            s_inv[i] = rope_inv_freq(a.theta, i, rope_dim);
        if (a.q_norm_w != nullptr)
            for (int i = tid; i < D; i += kThreads) {
                s_wq[i] = a.q_norm_w[i];
                s_wk[i] = a.k_norm_w[i];
            }
    }
    // prefix of the tile counts: inclusive scan inside each wave, the wave totals through LDS
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
    }
    if (lane == 63) s_scan[wave] = incl;
    __syncthreads();
    PKV_STAMP(1, wall_clock64());
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_scan[w];
    {
        int run = (before + incl - cnt) * Hkv;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const int b = tid * kPerThread + k;
            if (b < B) {
                s_pre[b] = run;
                run += Hkv * span(ntiles(s_len[b]));
            }
        }
        if (tid == kThreads - 1) s_pre[B] = (before + incl) * Hkv;
    }
    __syncthreads();

    // ---- 2. this workgroup's tile range
    const int total = s_pre[B];
    const int T = (total + (int)gridDim.x - 1) / (int)gridDim.x;
    // range of this workgroup (profiling builds can deal the ranges out rotated)
#ifdef PKV_TIMELINE
    const int wr = xcd_range((int)((blockIdx.x + (unsigned)a.timeline_rot) % gridDim.x),
                             (int)gridDim.x);
#else
    const int wr = xcd_range((int)blockIdx.x, (int)gridDim.x);
#endif
    const int r0 = (int)min((int64_t)wr * T, (int64_t)total);
    const int r1 = min(total, r0 + T);
    PKV_STAMP(2, wall_clock64());
    PKV_STAMP(8, (uint64_t)(r1 > r0 ? r1 - r0 : 0));
    if (r0 >= r1) {  // whole workgroup together
        PKV_STAMP(6, wall_clock64());
        return;
    }
#ifdef PKV_TIMELINE
    int n_units = 0;
    bool first_tile = true;
#endif

    int b;
    {  // last sequence whose prefix is <= r0 (its segment list contains tile r0)
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_pre[mid] <= r0) lo = mid; else hi = mid - 1;
        }
        b = lo;
    }
    int g = (r0 - s_pre[b]) / span(ntiles(s_len[b]));

    const BlockDiv bdiv = make_div((uint32_t)a.bs);
    const bool tile_in_block = a.bs % kTile == 0;   // a 16-token tile never crosses a block
    const int64_t nb_max = a.num_blocks - 1;
    const int64_t tok_stride = (int64_t)Hkv * D;   // codes between consecutive slots
    const int chunk_tokens = ((kTblCap - 2) * a.bs) / 64 * 64;
    const float qs = a.scale * kLog2e;
    float* part_acc = a.part_acc;
    float* part_ml = a.part_ml;

    for (int x = r0; x < r1;) {
        // ---- one unit: tiles [x, u_end) of segment (b, g)
        const int L = s_len[b];
        const int vis_lo = window_lo(L, W);          // first key the query sees
        const int t0 = vis_lo / kTile * kTile;        // first token of the segment's first tile
        const int nb = ntiles(L);
        const int seg_start = s_pre[b] + g * span(nb) + kUnitCost;  // its first tile
        const int seg_end = seg_start + nb;
        if (x < seg_start) {  // the range starts in the segment's start cost
            x = seg_start;
            if (x >= r1) break;  // ... and ends there: nothing of this segment is ours
        }
        const int u_end = min(seg_end, r1);
        const int tok_lo = t0 + (x - seg_start) * kTile;
        const int tok_hi = min(t0 + (u_end - seg_start) * kTile, L);
        const bool seg_first = x == seg_start;
        const bool owns_new = APPEND && u_end == seg_end;
        const int pnew = L - 1;
        const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
        const int64_t head_off = (int64_t)g * D;

        // chunk of the block table staged in LDS (kTblCap ids cover chunk_tokens tokens)
        auto stage_table = [&](int c_lo, int c_hi) {
            const int first_blk = (int)bdiv.div((uint32_t)c_lo);
            const int n_blk = min((int)bdiv.div((uint32_t)(c_hi - 1)) - first_blk + 1, kTblCap);
            for (int i = tid; i < n_blk; i += kThreads) {
                const int64_t id = trow[first_blk + i];
                s_tbl[i] = (int32_t)(id < 0 ? 0 : (id > nb_max ? nb_max : id));
            }
        };

        // Q of this segment (rotated here when the append is fused) and the first table chunk,
        // requested together; then the MFMA operands.
        auto qf = [&](int h, int d0, float (&o)[8]) {
            const float4* src = reinterpret_cast<const float4*>(&s_q[h][d0]);
            const float4 x0 = src[0], x1 = src[1];
            o[0] = x0.x; o[1] = x0.y; o[2] = x0.z; o[3] = x0.w;
            o[4] = x1.x; o[5] = x1.y; o[6] = x1.z; o[7] = x1.w;
        };
        auto source = [&](int c_lo) {
            TileSource src;
            src.k_pool = a.k_pool;
            src.v_pool = a.v_pool;
            src.tbl = s_tbl;
            src.first_blk = (int)bdiv.div((uint32_t)c_lo);
            src.tbl_cap = kTblCap;
            src.bdiv = bdiv;
            src.bs = a.bs;
            src.tile_in_block = tile_in_block;
            src.tok_stride = tok_stride;
            src.head_off = head_off;
            return src;
        };
        // The first table chunk, the query rows (and, fused, the new K / V rows) are staged
        // together; then each wave's first tile is requested before the query work, so its
        // latency overlaps the rotation (not for the tile holding the new token, whose row the
        // rotation stores).
        const int c_hi0 = min(tok_hi, tok_lo + chunk_tokens);
        stage_table(tok_lo, c_hi0);
        {
            const float* qsrc = a.q + ((int64_t)b * Hq + g * G) * D;
            for (int i = tid; i < G * D; i += kThreads) s_q[i / D][i % D] = qsrc[i];
        }
        int64_t blk_new = -1;
        if constexpr (APPEND) {
            // the new row's block id, requested with the query
            if (owns_new) blk_new = (int64_t)a.tables[(int64_t)b * a.max_blocks + pnew / a.bs];
            if (owns_new) {
                const float* ksrc = a.k_in + ((int64_t)b * Hkv + g) * D;
                const float* vsrc = a.v_in + ((int64_t)b * Hkv + g) * D;
                for (int i = tid; i < D; i += kThreads) {
                    s_kx[i] = ksrc[i];
                    s_vx[i] = vsrc[i];
                }
            }
        }
        __syncthreads();
        const TileSource src0 = source(tok_lo);
        const int first_base = tok_lo + wave * kTile;
        const bool have_first = first_base < c_hi0 && !(owns_new && first_base + kTile > pnew);
        typename Tile::Regs first;  // requested in every wave (in bounds), used if have_first
        Tile::load_tile(src0, first_base, tok_lo, c_hi0, first);
        if constexpr (APPEND)
            rotate_and_append<D, BF16, VAR>(a, G, b, g, pnew, blk_new, owns_new, seg_first,
                                            &s_q[0][0], s_kx, s_vx, s_wq, s_wk, s_inv,
                                            &s_cs[0][0], s_r, &s_vsc);
        typename Tile::Query qop;
        Tile::setup_query(qf, G, qs, qop);
#ifdef PKV_TIMELINE
        if (n_units++ == 0) PKV_STAMP(3, wall_clock64());
#endif
        typename Tile::State st;
        Tile::init(st);

        for (int c_lo = tok_lo; c_lo < tok_hi; c_lo += chunk_tokens) {
            const int c_hi = min(tok_hi, c_lo + chunk_tokens);
            if (c_lo != tok_lo) {  // the first chunk was staged with the query
                __syncthreads();  // previous readers of s_tbl are done
                stage_table(c_lo, c_hi);
                __syncthreads();
            }
            Tile::stream(source(c_lo), c_lo, c_hi, vis_lo, qop, st, G, qs, qf, s_w[wave].scr,
                         s_def[wave],
                         [&]() {
#ifdef PKV_TIMELINE
                             if (first_tile) {
                                 PKV_STAMP(4, wall_clock64());
                                 first_tile = false;
                             }
#endif
                         },
                         first, have_first && c_lo == tok_lo);
        }

        // ---- combine within each wave, then across the waves
#ifdef PKV_TIMELINE
        if (u_end == r1) PKV_STAMP(5, wall_clock64());
#endif
        Tile::flush(st, G, s_m[wave], s_l[wave], &s_w[wave].acc[0][0]);
        __syncthreads();
        const bool full = seg_first && u_end == seg_end;
        const int slot = wr * 2 + (seg_start > r0 ? 1 : 0);
        for (int i = tid; i < G * D; i += kThreads) {
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
            if (full) {
                a.out[((int64_t)b * Hq + g * G + h) * D + d] = num / den;
            } else {
                store_shared(part_acc + ((int64_t)slot * G + h) * D + d, num);
                if (d == 0) {
                    store_shared(part_ml + ((int64_t)slot * G + h) * 2, Mx);
                    store_shared(part_ml + ((int64_t)slot * G + h) * 2 + 1, den);
                }
            }
        }
        if (!full) {
            const int w_a = seg_start / T;
            const int w_b = (seg_end - 1) / T;
            __builtin_amdgcn_s_waitcnt(0);  // this thread's piece stores are complete
            __syncthreads();                // ... and so are every other thread's
            int* counter = a.counters + (int64_t)b * Hkv + g;
            if (tid == 0) s_last = arrive(counter) == w_b - w_a;
            __syncthreads();
            if (s_last) {
                for (int i = tid; i < G * D; i += kThreads) {
                    const int h = i / D;
                    const int d = i % D;
                    float Mx = -INFINITY;
                    for (int w0 = w_a; w0 <= w_b; w0 += 8) {
                        float mk[8];
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            const int w = w0 + k;
                            const int sl = w * 2 + (w == w_a && seg_start != w_a * T ? 1 : 0);
                            mk[k] = w <= w_b ? load_shared(part_ml + ((int64_t)sl * G + h) * 2)
                                             : -INFINITY;
                        }
#pragma unroll
                        for (int k = 0; k < 8; ++k) Mx = fmaxf(Mx, mk[k]);
                    }
                    const float M_use = (Mx == -INFINITY) ? 0.f : Mx;
                    float num = 0.f, den = 0.f;
                    for (int w0 = w_a; w0 <= w_b; w0 += 8) {
                        float mk[8], lk[8], ak[8];
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            const int w = w0 + k;
                            const int sl = w * 2 + (w == w_a && seg_start != w_a * T ? 1 : 0);
                            const bool ok = w <= w_b;
                            mk[k] = ok ? load_shared(part_ml + ((int64_t)sl * G + h) * 2) : -INFINITY;
                            lk[k] = ok ? load_shared(part_ml + ((int64_t)sl * G + h) * 2 + 1) : 0.f;
                            ak[k] = ok ? load_shared(part_acc + ((int64_t)sl * G + h) * D + d) : 0.f;
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
                if (tid == 0) store_shared(counter, 0);  // ready for the next call
            }
        }
        __syncthreads();  // LDS (s_q, s_acc, s_m, s_l, s_tbl) is reused by the next unit

        x = u_end;
        if (x < r1) {
            if (++g == Hkv) {
                g = 0;
                do { ++b; } while (b < B - 1 && s_len[b] == 0);
            }
        }
    }
    PKV_STAMP(6, wall_clock64());
#ifdef PKV_TIMELINE
    PKV_STAMP(7, (uint64_t)n_units);
#endif
}

template <int D, bool BF16, bool APPEND>
hipError_t launch_typed(const BalancedArgs& a, hipStream_t stream) {
    if (a.Hq / a.Hkv > kGMax) return hipErrorInvalidValue;
    // the append's variant fields matter only when the append is fused
    const bool full = APPEND && (a.rope_dim != D || a.v_norm);
    auto kern = full            ? decode_balanced_kernel<D, BF16, APPEND, APPEND ? kVarFull : kVarWindow>
                : a.window != 0 ? decode_balanced_kernel<D, BF16, APPEND, kVarWindow>
                                : decode_balanced_kernel<D, BF16, APPEND, kVarNone>;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    int64_t cap = kMaxBalancedGrid;
    if (a.max_grid > 0) cap = std::min<int64_t>(cap, a.max_grid);
    const int grid = (int)std::min<int64_t>((int64_t)per_cu * a.num_cus, cap);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <bool BF16, bool APPEND>
hipError_t dispatch_d(const BalancedArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 32: return launch_typed<32, BF16, APPEND>(a, stream);
        case 64: return launch_typed<64, BF16, APPEND>(a, stream);
        case 128: return launch_typed<128, BF16, APPEND>(a, stream);
        case 256: return launch_typed<256, BF16, APPEND>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_balanced(const BalancedArgs& a, hipStream_t stream) {
    if (a.append) return a.bf16 ? dispatch_d<true, true>(a, stream) : dispatch_d<false, true>(a, stream);
    return a.bf16 ? dispatch_d<true, false>(a, stream) : dispatch_d<false, false>(a, stream);
}

}  // namespace pkv
