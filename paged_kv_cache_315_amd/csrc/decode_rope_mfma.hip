// decode_rope_mfma.hip — paged-attention decode over un-rotated keys (RoPE applied at read) and
// over float32 pools, with both products on the float32 matrix cores (gfx950).
//
// What it computes is what decode_rope.hip computes (page "makarna/pkg/model/arch/
// hybrid_decoder.go", runHybridAttentionBlock / runHybridAttentionBlockBatch: the RoPE-fused
// paged kernel rotates the cached un-rotated keys itself, and float32 KV goes to the plain paged
// kernel):
//   out[b][h] = softmax_t(scale * q[b][h] . (R_{t-p} K[t][g])) . V[t][g],  p = L_b - 1,
// R_x the rotate-half RoPE of the first rope_dim dims at position x (pair (i, i + rope_dim/2),
// angle x * theta^(-2i/rope_dim)); without rotation (float32 pools) R is the identity.
// (R_p q) . (R_t k) = q . (R_{t-p} k): the query is used as it is and each key is turned back by
// delta = p - t.
//
// Work decomposition: the balanced schedule of decode_balanced.hip (decode only) — one list of
// 16-token tiles over the batch, each (sequence, KV head) segment preceded by a start cost,
// equal ranges of it per resident workgroup, pieces of cut segments merged by the last
// workgroup to finish; inside a workgroup the 4 waves take 16-token tiles in turn (wave w: the
// tiles starting at c_lo + 16 w + 64 k of a run of tiles whose block ids are staged in LDS).
// A tile is two products on v_mfma_f32_16x16x4f32 (A 16x4: lane l holds A[l%16][l/16];
// B 4x16: lane l holds B[l/16][l%16]; C 16x16: lane l, register r holds C[4(l/16) + r][l%16]);
// below q4 = l/16, l16 = l%16.
//   S^T = K Q^T   rows = the 16 tokens, columns = query heads (G <= 8 of 16, the rest zero
//                 rows of Q). K-step s = 8 j + e uses, in lane (q4, l16), dim 8(q4 + 4j) + e:
//                 the A value is that dim of token l16's key (element e of the lane's loaded
//                 chunk j), the B value the same dim of query head l16. Every dim enters once;
//                 products and sums are float32 (no operand splitting, so non-finite codes give
//                 what float arithmetic gives). Lane (q4, l16) receives the scores of tokens
//                 4 q4 + r (r < 4) for head l16.
//   O^T += V^T P^T rows = dims, columns = heads, 4 tokens per product: product (b, m) takes, in
//                 lane (q4, l16), V[token 4 q4 + m][dim W l16 + b] (W = D/16) as the A value and
//                 the lane's own weight of token 4 q4 + m as the B value. The weights never
//                 leave the registers and V is used as loaded (W consecutive dims of 4 tokens
//                 per lane). Output block b, register r of lane (q4, l16): head l16, dim
//                 W(4 q4 + r) + b.
// Online softmax per head in exp2 units: tile maximum in the lane, then across the four lane
// groups with two permlane swaps; the exponent base of a head moves only when a score passes it
// by more than 8, so the accumulators are rescaled only then. Tokens outside [window start, L)
// get score -inf and zero V (their slots may hold anything, NaN included). The next tile's K/V
// loads are in flight while a tile is computed.
//
// Rotation at read. rope_dim is a multiple of 64, so the partner of the lane's first-half dim
// 8(q4 + 4j) + e is element e of its own chunk j + rope_dim/64:
//   first half  k'_i     = k_i c + k_{i+h} s,    second half  k'_{i+h} = k_{i+h} c - k_i s,
// with c, s = cos, sin(delta f_i). cos / sin of the 64 token offsets of a step are built once per
// workgroup (double precision at every 16th offset, one-token float steps between) and then
// advanced by 64 tokens per tile with the angle-difference formulas in float (about one ulp per
// step; a run of tiles is seeded afresh and has at most 4096 tokens, 64 steps).
#include "decode_tile.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTblCap = 1024;          // block ids staged in LDS per workgroup
constexpr int kStep = 16 * kWaves;     // tokens between a lane's consecutive tiles

enum ElemKind { kF16 = 0, kBF16 = 1, kF32 = 2 };

__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// N dwords of streamed pool data (N = 2, 4 or 8), non-temporal.
template <int N>
__device__ __forceinline__ void load_dw(const uint32_t* p, uint32_t (&w)[N]) {
    if constexpr (N == 2) {
        typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        w[0] = v[0];
        w[1] = v[1];
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const uint4 v = load_stream(reinterpret_cast<const uint16_t*>(p + i));
            w[i] = v.x;
            w[i + 1] = v.y;
            w[i + 2] = v.z;
            w[i + 3] = v.w;
        }
    }
}

// Elements held by N dwords as floats.
template <int EK, int N>
__device__ __forceinline__ void to_float(const uint32_t (&w)[N], float (&f)[EK == kF32 ? N : 2 * N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if constexpr (EK == kF32) {
            f[i] = __uint_as_float(w[i]);
        } else if constexpr (EK == kBF16) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        } else {
            f[2 * i] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w[i] & 0xFFFFu));
            f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w[i] >> 16));
        }
    }
}


// One wave's 16-token tile on the float32 matrix cores, and what a wave keeps between tiles.
template <int D, int EK, int NJR>
struct RTile {
    static constexpr int EPD = EK == kF32 ? 1 : 2;   // elements per dword
    static constexpr int NK = D / 32;                // key chunks of 8 dims per lane
    static constexpr int W = D / 16;                 // V dims per lane and token
    static constexpr int KDW = 8 / EPD;              // dwords per key chunk
    static constexpr int VDW = W / EPD;              // dwords per V piece
    static constexpr int HR = 32 * NJR;              // rotary pairs (rope_dim / 2)
    static constexpr int NR = NJR > 0 ? NJR : 1;
    static_assert((D == 64 || D == 128) && NJR >= 0 && 2 * NJR <= NK, "shape");

    struct Regs {
        uint32_t k[NK][KDW];   // token l16, dims 8(q4 + 4j) .. + 7
        uint32_t v[4][VDW];    // token 4 q4 + m, dims W l16 .. + W - 1
    };
    struct State {
        float m;               // exponent base of head l16 (log2 units)
        float l;               // this lane's part of the sum of weights of head l16
        f32x4 acc[W];          // block c, register r: head l16, dim W(4 q4 + r) + c
        float cs[NR][8];       // rotation of the lane's next key: cos / sin (delta f_i) of its
        float sn[NR][8];       //   first-half pairs i = 8(q4 + 4j) + e
    };
    // LDS a workgroup shares for the rotation
    struct RotLds {
        float2 seed[NJR > 0 ? kStep : 1][NJR > 0 ? HR : 1];   // cos / sin per offset, pair
        float2 step[NJR > 0 ? HR : 1];                          // cos / sin of 64 f_i
    };

    static __device__ __forceinline__ void init(State& st) {
        st.m = -INFINITY;
        st.l = 0.f;
#pragma unroll
        for (int c = 0; c < W; ++c) st.acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // The query operand in LDS (all threads of the workgroup; the caller meets at a barrier
    // before it is read): rows 0 .. G - 1 the G heads scaled by qs = scale * log2 e, rows
    // G .. 15 zero (written once per workgroup by zero_query_rows). Rows are D + 4 floats apart,
    // so the 16 lanes of a lane group (16 rows, 16 bytes each) hit distinct banks.
    static __device__ __forceinline__ void zero_query_rows(int G, float (*sq)[D + 4]) {
        for (int i = threadIdx.x + G * D; i < 16 * D; i += kThreads) sq[i / D][i % D] = 0.f;
    }

    // Rotation seeds of a run of tiles starting at token c_lo (all threads of the workgroup;
    // the caller meets at a barrier before the lanes read them): pair i, offsets o < 64 of a
    // step, cos / sin((pq - c_lo - o) f_i); double precision at every 16th offset, one-token
    // float steps between.
    static __device__ __forceinline__ void seeds(RotLds& r, float theta, int pq, int c_lo) {
        if constexpr (NJR > 0) {
            for (int idx = threadIdx.x; idx < HR * (kStep / 16); idx += kThreads) {
                const int i = idx % HR;
                const int part = idx / HR;
                const double f = rope_inv_freq(theta, i, 2 * HR);
                double sn, cs;
                sincos((double)(pq - c_lo - 16 * part) * f, &sn, &cs);
                float c = (float)cs, sv = (float)sn;
                sincos(f, &sn, &cs);
                const float c1 = (float)cs, s1 = (float)sn;
                if (part == 0) {
                    sincos((double)kStep * f, &sn, &cs);
                    r.step[i] = make_float2((float)cs, (float)sn);
                }
                for (int k = 0; k < 16; ++k) {
                    r.seed[16 * part + k][i] = make_float2(c, sv);
                    // delta -> delta - 1
                    const float nc = fmaf(c, c1, sv * s1);
                    const float ns = fmaf(sv, c1, -(c * s1));
                    c = nc;
                    sv = ns;
                }
            }
        }
    }

    // The lane's rotation at its first tile of the run (token c_lo + 16 wave + l16).
    static __device__ __forceinline__ void start_rotation(const RotLds& r, int wave, State& st) {
        if constexpr (NJR > 0) {
            const int lane = threadIdx.x & 63;
            const int l16 = lane & 15, q4 = lane >> 4;
            const int o = 16 * wave + l16;
#pragma unroll
            for (int j = 0; j < NJR; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float2 x = r.seed[o][8 * (q4 + 4 * j) + e];
                    st.cs[j][e] = x.x;
                    st.sn[j][e] = x.y;
                }
        }
    }

    // Loads of the tile at token tb (a multiple of 16) of a run ending at hi; rows past hi are
    // clamped into the run (and masked at use). row_off(t): element offset of token t's row of
    // this KV head; in_block: the 16 rows of a tile lie in one block.
    template <typename RowOff>
    static __device__ __forceinline__ void load(Regs& r, int tb, int hi, bool in_block,
                                                RowOff&& row_off, const uint32_t* kpool,
                                                const uint32_t* vpool, int64_t tok_stride) {
        const int lane = threadIdx.x & 63;
        const int l16 = lane & 15, q4 = lane >> 4;
        int64_t ko, vo[4];
        if (in_block) {
            const int64_t o0 = row_off(min(tb, (hi - 1) & ~15));
            ko = o0 + l16 * tok_stride;
#pragma unroll
            for (int m = 0; m < 4; ++m) vo[m] = o0 + (4 * q4 + m) * tok_stride;
        } else {
            ko = row_off(min(tb + l16, hi - 1));
#pragma unroll
            for (int m = 0; m < 4; ++m) vo[m] = row_off(min(tb + 4 * q4 + m, hi - 1));
        }
#pragma unroll
        for (int j = 0; j < NK; ++j) load_dw<KDW>(kpool + (ko + 8 * (q4 + 4 * j)) / EPD, r.k[j]);
#pragma unroll
        for (int m = 0; m < 4; ++m) load_dw<VDW>(vpool + (vo[m] + W * l16) / EPD, r.v[m]);
    }

    // One tile: tokens tb .. tb + 15, of which [lo, hi) are attended.
    static __device__ __forceinline__ void compute(const Regs& r, int tb, int lo, int hi,
                                                   const float (*sq)[D + 4], const RotLds& rl,
                                                   State& st) {
        const int lane = threadIdx.x & 63;
        const int l16 = lane & 15, q4 = lane >> 4;
        // keys as floats, turned back by delta = p - t when rotating
        float kf[NK][8];
#pragma unroll
        for (int j = 0; j < NK; ++j) to_float<EK, KDW>(r.k[j], kf[j]);
        if constexpr (NJR > 0) {
#pragma unroll
            for (int j = 0; j < NJR; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = kf[j][e], y = kf[j + NJR][e];
                    kf[j][e] = fmaf(x, st.cs[j][e], y * st.sn[j][e]);
                    kf[j + NJR][e] = fmaf(y, st.cs[j][e], -(x * st.sn[j][e]));
                }
        }
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
        // the query is read from LDS at every tile: an opaque column offset keeps the compiler
        // from hoisting the reads out of the tile loop into 32 more registers
        int qcol = 8 * q4;
        asm volatile("" : "+v"(qcol));
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const float4* qp = reinterpret_cast<const float4*>(&sq[l16][qcol + 32 * j]);
            const float4 x0 = qp[0], x1 = qp[1];
            const float qv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) sacc = mma4(kf[j][e], qv[e], sacc);
        }
        if constexpr (NJR > 0) {
            // delta -> delta - 64 for the lane's next tile: cos(a - b) = cos a cos b + sin a sin b,
            //                                               sin(a - b) = sin a cos b - cos a sin b
#pragma unroll
            for (int j = 0; j < NJR; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float2 sp = rl.step[8 * (q4 + 4 * j) + e];
                    const float nc = fmaf(st.cs[j][e], sp.x, st.sn[j][e] * sp.y);
                    const float ns = fmaf(st.sn[j][e], sp.x, -(st.cs[j][e] * sp.y));
                    st.cs[j][e] = nc;
                    st.sn[j][e] = ns;
                }
        }

        // online softmax over the lane's four tokens of head l16
        bool valid[4];
        float sc[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int t = tb + 4 * q4 + r4;
            valid[r4] = t >= lo && t < hi;
            sc[r4] = valid[r4] ? sacc[r4] : -INFINITY;
        }
        float tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        tmax = swap16_max(tmax);
        tmax = swap32_max(tmax);
        const bool grow = tmax > st.m + 8.f;   // -inf base: any finite score; NaN: never
        const float m_new = grow ? tmax : st.m;
        const float alpha = grow ? fast_exp2(st.m - m_new) : 1.f;
        st.m = m_new;
        const float mb = m_new == -INFINITY ? 0.f : m_new;
        float p[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) p[r4] = fast_exp2(sc[r4] - mb);
        st.l = fmaf(st.l, alpha, (p[0] + p[1]) + (p[2] + p[3]));
        if (__any(grow)) {
#pragma unroll
            for (int c = 0; c < W; ++c) st.acc[c] *= alpha;
        }

        // PV: 4 tokens per product, V as loaded (invalid tokens' rows zeroed)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float vf[W];
            to_float<EK, VDW>(r.v[m], vf);
#pragma unroll
            for (int c = 0; c < W; ++c) {
                const float x = valid[m] ? vf[c] : 0.f;
                st.acc[c] = mma4(x, p[m], st.acc[c]);
            }
        }
    }

    // The wave's tiles of the run [c_lo, hi) (tokens before lo masked), in pairs with no exit
    // between them (an odd count runs one masked tile more; an exit inside the pair made the
    // compiler copy the buffers).
    template <typename RowOff>
    static __device__ __forceinline__ void stream(int c_lo, int hi, int lo, int wave,
                                                  bool in_block, RowOff&& row_off,
                                                  const uint32_t* kpool, const uint32_t* vpool,
                                                  int64_t tok_stride, const float (*sq)[D + 4],
                                                  const RotLds& rl, State& st) {
        const int first = c_lo + 16 * wave;
        const int n_tiles = first < hi ? (hi - first + kStep - 1) / kStep : 0;
        const int n_pairs = (n_tiles + 1) >> 1;
        Regs ra, rb;
        int tb = first;
        load(ra, tb, hi, in_block, row_off, kpool, vpool, tok_stride);
        for (int it = 0; it < n_pairs; ++it) {
            load(rb, tb + kStep, hi, in_block, row_off, kpool, vpool, tok_stride);
            compute(ra, tb, lo, hi, sq, rl, st);
            load(ra, tb + 2 * kStep, hi, in_block, row_off, kpool, vpool, tok_stride);
            compute(rb, tb + kStep, lo, hi, sq, rl, st);
            tb += 2 * kStep;
        }
    }

    // The wave's state -> LDS: exponent bases and sums of weights per head, accumulators per
    // head and dim (the sums over the four lane groups first).
    static __device__ __forceinline__ void flush(State& st, int G, float* m_w, float* l_w,
                                                 float (*acc_w)[D]) {
        const int lane = threadIdx.x & 63;
        const int l16 = lane & 15, q4 = lane >> 4;
        float l = swap16_sum(st.l);
        l = swap32_sum(l);
        if (l16 < G) {
#pragma unroll
            for (int c = 0; c < W; ++c)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) acc_w[l16][W * (4 * q4 + r4) + c] = st.acc[c][r4];
            if (q4 == 0) {
                m_w[l16] = st.m;
                l_w[l16] = l;
            }
        }
    }
};

// Two waves per SIMD, except float32 pools rotated over 128 dims (their two tiles of float K/V
// in flight and 32 cos / sin pairs per lane need more than 256 registers).
#define PKV_RTILE_WAVES(EK, NJR) (EK == kF32 && NJR == 2 ? 1 : 2)

#ifndef PKV_F32_UNIT_COST
#define PKV_F32_UNIT_COST 6
#endif

// ---- balanced schedule (the decode_balanced.hip deal, decode only)
// The K/V rows of the batch form one list of 16-token tiles, segment (b, g) = KV head g of
// sequence b preceded by a start cost of empty positions; workgroup w takes positions
// [r T, (r + 1) T), r its range under the XCD-aware deal. A segment inside one range is finished
// there; a cut one leaves one piece per workgroup it touches (a workgroup holds at most two:
// slots 2r and 2r + 1), and the last workgroup to finish it merges the pieces.
constexpr int kPerThread = (kMaxBalancedBatch + kThreads - 1) / kThreads;

template <int D, int EK, int NJR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(PKV_RTILE_WAVES(EK, NJR))))
void decode_rope_balanced_kernel(BalancedArgs a) {
    using Tile = RTile<D, EK, NJR>;
    __shared__ int s_len[kMaxBalancedBatch];
    __shared__ int s_pre[kMaxBalancedBatch + 1];
    __shared__ int s_scan[kWaves];
    __shared__ int32_t s_tbl[kTblCap];
    __shared__ typename Tile::RotLds s_rot;
    __shared__ __align__(16) float s_q[16][D + 4];   // rows padded: conflict-free reads
    __shared__ float s_acc[kWaves][8][D];
    __shared__ float s_m[kWaves][8];
    __shared__ float s_l[kWaves][8];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int B = a.B;
    const int Hkv = a.Hkv;
    const int G = a.Hq / Hkv;
    const int Hq = a.Hq;
    const int W = a.window;
    auto ntiles = [=](int L) { return (L + 15) / 16 - window_lo(L, W) / 16; };
    // empty positions before each segment: the 16-bit decode's start cost, or 6 tiles over
    // float32 pools (on the llama3-8b lengths: 6 tiles 122.8 us, 15 tiles 125.0 us, 30 tiles
    // 132.9 us; rotating at read 15 tiles is best: 92.2 against 95.2 and 95.9 us); never more
    // than kBalancedUnitCost, which the host's size checks assume (PKV_F32_UNIT_COST overrides
    // the 6 in builds that sweep it)
    constexpr int kCost = EK == kF32 && NJR == 0 && kBalancedUnitCost > PKV_F32_UNIT_COST
                              ? PKV_F32_UNIT_COST
                              : kBalancedUnitCost;
    auto span = [=](int nt) { return nt > 0 ? nt + kCost : 0; };

    // ---- lengths and the tile prefix of every sequence (all heads) -> LDS
    const int cap = (int)min((int64_t)a.max_context_len, (int64_t)a.max_blocks * a.bs);
    // all of a thread's loads first (one round trip), then the counts
    int lv[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) lv[k] = a.lens[min(tid * kPerThread + k, B - 1)];
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int b = tid * kPerThread + k;
        if (b < B) {
            const int L = max(0, min(lv[k], cap));
            s_len[b] = L;
            cnt += span(ntiles(L));
        }
    }
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
    }
    if (lane == 63) s_scan[wave] = incl;
    __syncthreads();
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

    // ---- this workgroup's range of the list
    const int total = s_pre[B];
    const int T = (total + (int)gridDim.x - 1) / (int)gridDim.x;
    const int wr = xcd_range((int)blockIdx.x, (int)gridDim.x);
    const int r0 = (int)min((int64_t)wr * T, (int64_t)total);
    const int r1 = min(total, r0 + T);
    if (r0 >= r1) return;  // whole workgroup together

    int b;
    {  // last sequence whose prefix is <= r0 (its segment list contains position r0)
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_pre[mid] <= r0) lo = mid; else hi = mid - 1;
        }
        b = lo;
    }
    int g = (r0 - s_pre[b]) / span(ntiles(s_len[b]));

    const BlockDiv bdiv = make_div((uint32_t)a.bs);
    const bool in_block = a.bs % 16 == 0;
    const int64_t nb_max = a.num_blocks - 1;
    const int64_t tok_stride = (int64_t)Hkv * D;
    // a run of tiles stages at most kTblCap - 1 block ids and, when rotating, covers at most
    // 4096 tokens (the rotation is seeded in double precision at each run, then carried by at
    // most 64 float steps)
    int chunk_tokens = ((kTblCap - 2) * a.bs) / 64 * 64;
    if (NJR > 0) chunk_tokens = min(chunk_tokens, 4096);
    const float qs = a.scale * kLog2e;
    const uint32_t* kpool = reinterpret_cast<const uint32_t*>(a.k_pool);
    const uint32_t* vpool = reinterpret_cast<const uint32_t*>(a.v_pool);
    float* part_acc = a.part_acc;
    float* part_ml = a.part_ml;

    Tile::zero_query_rows(G, s_q);  // read after the first unit's barrier
    for (int x = r0; x < r1;) {
        // ---- one unit: tiles [x, u_end) of segment (b, g)
        const int L = s_len[b];
        const int vis_lo = window_lo(L, W);
        const int t0 = vis_lo / 16 * 16;
        const int nb = ntiles(L);
        const int seg_start = s_pre[b] + g * span(nb) + kCost;  // its first tile
        const int seg_end = seg_start + nb;
        if (x < seg_start) {  // the range starts in the segment's start cost
            x = seg_start;
            if (x >= r1) break;  // ... and ends there: nothing of this segment is ours
        }
        const int u_end = min(seg_end, r1);
        const int tok_lo = t0 + (x - seg_start) * 16;
        const int tok_hi = min(t0 + (u_end - seg_start) * 16, L);
        const bool seg_first = x == seg_start;
        const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
        const int64_t head_off = (int64_t)g * D;

        const float* qsrc = a.q + ((int64_t)b * Hq + g * G) * D;
        typename Tile::State st;
        Tile::init(st);
        for (int c_lo = tok_lo; c_lo < tok_hi; c_lo += chunk_tokens) {
            const int c_hi = min(tok_hi, c_lo + chunk_tokens);
            if (c_lo != tok_lo) __syncthreads();  // readers of s_tbl / s_rot are done
            // block ids of the run -> LDS (at most kTblCap - 1 of them)
            const int first_blk = (int)bdiv.div((uint32_t)c_lo);
            const int n_blk = min((int)bdiv.div((uint32_t)(c_hi - 1)) - first_blk + 1, kTblCap);
            // (with the query rows for the first run: one round trip for both)
            {
                float qv[8 * D / kThreads];
                batched_load<kThreads>(c_lo == tok_lo ? G * D : 0,
                                       [&](int i) { return qsrc[i]; }, qv);
                int32_t tv[kTblCap / kThreads];
                batched_load<kThreads>(n_blk, [&](int i) { return trow[first_blk + i]; }, tv);
                batched_store<kThreads>(c_lo == tok_lo ? G * D : 0, qv,
                                        [&](int i, float v) { s_q[i / D][i % D] = v * qs; });
                batched_store<kThreads>(n_blk, tv, [&](int i, int32_t id) {
                    s_tbl[i] = id < 0 ? 0 : (int32_t)min((int64_t)id, nb_max);
                });
            }
            Tile::seeds(s_rot, a.theta, L - 1, c_lo);
            __syncthreads();
            Tile::start_rotation(s_rot, wave, st);
            auto row_off = [&](int t) -> int64_t {
                const int j = (int)bdiv.div((uint32_t)t);
                const int64_t blk = s_tbl[min(j - first_blk, kTblCap - 1)];
                return (blk * a.bs + (t - j * a.bs)) * tok_stride + head_off;
            };
            Tile::stream(c_lo, c_hi, vis_lo, wave, in_block, row_off, kpool, vpool, tok_stride,
                         s_q, s_rot, st);
        }

        // ---- combine the waves; the output, or this workgroup's piece of the segment
        Tile::flush(st, G, s_m[wave], s_l[wave], s_acc[wave]);
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
                num = fmaf(e, s_acc[w][h][d], num);
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
            // the workgroups holding pieces of this segment: w_a .. w_b (ranges)
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
                    for (int w = w_a; w <= w_b; ++w) {
                        const int sl = w * 2 + (w == w_a && seg_start != w_a * T ? 1 : 0);
                        Mx = fmaxf(Mx, load_shared(part_ml + ((int64_t)sl * G + h) * 2));
                    }
                    const float M_use = (Mx == -INFINITY) ? 0.f : Mx;
                    float num = 0.f, den = 0.f;
                    for (int w = w_a; w <= w_b; ++w) {
                        const int sl = w * 2 + (w == w_a && seg_start != w_a * T ? 1 : 0);
                        const float e =
                            exp2f(load_shared(part_ml + ((int64_t)sl * G + h) * 2) - M_use);
                        den = fmaf(e, load_shared(part_ml + ((int64_t)sl * G + h) * 2 + 1), den);
                        num = fmaf(e, load_shared(part_acc + ((int64_t)sl * G + h) * D + d), num);
                    }
                    a.out[((int64_t)b * Hq + g * G + h) * D + d] = num / den;
                }
                if (tid == 0) store_shared(counter, 0);  // ready for the next call
            }
        }
        __syncthreads();  // LDS (s_tbl, s_rot, s_q, s_acc, s_m, s_l) is reused by the next unit

        x = u_end;
        if (x < r1) {
            if (++g == Hkv) {
                g = 0;
                do { ++b; } while (b < B - 1 && s_len[b] == 0);
            }
        }
    }
}

template <int D, int EK, int NJR>
hipError_t launch_balanced(const BalancedArgs& a, hipStream_t stream) {
    auto kern = decode_rope_balanced_kernel<D, EK, NJR>;
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

struct GoBalanced {
    const BalancedArgs& a;
    hipStream_t s;
    template <int D, int EK, int NJR>
    hipError_t operator()() const { return launch_balanced<D, EK, NJR>(a, s); }
};

// Instantiation for (head_dim, rotated chunk pairs): f<D, EK, NJR>() with rope_dim = 64 NJR.
template <int EK, typename F>
hipError_t dispatch(int D, int rope_dim, const F& f) {
    const int njr = rope_dim / 64;
    if (D == 64) {
        if (njr == 0) return f.template operator()<64, EK, 0>();
        if (njr == 1) return f.template operator()<64, EK, 1>();
    } else if (D == 128) {
        if (njr == 0) return f.template operator()<128, EK, 0>();
        if (njr == 1) return f.template operator()<128, EK, 1>();
        if (njr == 2) return f.template operator()<128, EK, 2>();
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool decode_rope_mfma_ok(int D, int G, int rope_dim) {
    return (D == 64 || D == 128) && G >= 1 && G <= 8 && rope_dim >= 0 && rope_dim % 64 == 0 &&
           rope_dim <= D;
}

hipError_t launch_decode_rope_balanced(const BalancedArgs& a, hipStream_t stream) {
    if (!decode_rope_mfma_ok(a.D, a.Hq / a.Hkv, a.rope_dim)) return hipErrorInvalidValue;
    const GoBalanced go{a, stream};
    if (a.f32) return dispatch<kF32>(a.D, a.rope_dim, go);
    return a.bf16 ? dispatch<kBF16>(a.D, a.rope_dim, go) : dispatch<kF16>(a.D, a.rope_dim, go);
}

}  // namespace pkv
