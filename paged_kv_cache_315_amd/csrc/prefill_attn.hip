// prefill_attn.hip — paged attention of a chunk of query tokens per sequence, causal (gfx950).
//
// out[r][h] = softmax_t(scale * q[r][h] . K[t][g]) . V[t][g], g = h / G, over the positions
// t <= p_r of the token's sequence, where query row r is token i of sequence b at position
// p_r = start_pos[b] + i (rows cu_seqlens[b] .. cu_seqlens[b+1]-1, token-major).
//   (page "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlock: a block of seqLen
//    tokens goes into the cache at startPos and the attention over startPos + seqLen tokens is
//    causal from startPos; the single-request kernel takes any seqLen;
//    page "makarna/pkg/kvcache/paged_cache.go", GetBlockForPosition / GetBlockOffset.)
//
// Work decomposition: a query tile is QT = 16 / G consecutive tokens of one sequence and the
// G query heads of one KV head, i.e. 16 rows (token, head) = the rows of one MFMA tile. Grid
// (Hkv, S, B * QTmax): workgroup (g, s, b*QTmax + qt) owns query tile qt of sequence b and
// keys [s*P, min((s+1)*P, L_tile)), L_tile = one past the last token's position. The 4 waves
// take interleaved 16-key tiles with the next tile's K/V loads in flight, as in the decode.
//
// Per 16-key tile and wave:
//   S = Q K^T on the matrix cores (v_mfma_f32_16x16x32, Q split into a 16-bit head and a 16-bit
//     remainder, scaled by scale*log2(e)), then the causal mask per row (key <= the row's
//     position) and the online softmax per row (DPP row max, exp2).
//   O += P V on the matrix cores (v_mfma_f32_16x16x16): P goes through LDS to the A layout and
//     is split into a 16-bit head and remainder (two MFMAs), V goes through LDS to the B layout
//     (keys along k). A tile holding a non-finite V code takes an exact vector-ALU product
//     instead (the split's zero remainder, or a masked key's zero weight, times Inf would
//     give NaN where float arithmetic gives Inf or nothing).
//   The waves merge through LDS; a tile with one partition writes out, otherwise the last of
//   its partitions merges the pieces (agent-scope atomics, as the decode does).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 16;
constexpr int kTblCap = 1024;

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;

template <bool BF16>
struct Mma16;
template <>
struct Mma16<true> {
    using vec = bf16x4;
    using elem = __bf16;
    static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mma16<false> {
    using vec = f16x4;
    using elem = _Float16;
    static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
    }
};

template <bool BF16>
__device__ __forceinline__ float code_to_float(uint16_t c) {
    if constexpr (BF16) return __uint_as_float((uint32_t)c << 16);
    else return (float)__builtin_bit_cast(_Float16, c);
}

// any of the 8 codes in w an Inf or NaN
template <bool BF16>
__device__ __forceinline__ bool any_nonfinite(const uint4 w) {
    constexpr uint32_t E = BF16 ? 0x7F807F80u : 0x7C007C00u;
    const uint32_t lo = BF16 ? 0x7F80u : 0x7C00u;
    const uint32_t hi = lo << 16;
    bool bad = false;
    const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t e = x[i] & E;
        bad |= (e & 0xFFFFu) == lo || (e & 0xFFFF0000u) == hi;
    }
    return bad;
}

template <int D, int G, bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void prefill_attn_kernel(PrefillArgs a) {
    using M = Mma<BF16>;
    using M16 = Mma16<BF16>;
    constexpr int NK = D / 32;          // QK^T k-steps (and K loads) per tile
    constexpr int NT = D / 16;          // PV output tiles of 16 dims
    constexpr int R = D / 8;            // lanes per V row (8 codes per lane)
    constexpr int TPL = 64 / R;         // V rows per load instruction
    constexpr int U = kTile / TPL;      // V loads per tile
    constexpr int QT = 16 / G;          // query tokens per tile
    constexpr int VS = D + 8;           // LDS row stride of a V tile, in codes (bank spread)
    constexpr int PS = 20;              // LDS row stride of a P tile, in floats
    static_assert(D % 32 == 0 && U * TPL == kTile, "tile shape");
    static_assert(G >= 1 && G <= 8, "GQA group");

    constexpr int kVBytes = kWaves * kTile * VS * 2;
    constexpr int kAccBytes = kWaves * 16 * D * 4;
    __shared__ __align__(16) char s_big[kVBytes > kAccBytes ? kVBytes : kAccBytes];
    __shared__ __align__(16) float s_p[kWaves][16][PS];
    __shared__ int32_t s_tbl[kTblCap];
    __shared__ float s_m[kWaves][16];
    __shared__ float s_l[kWaves][16];
    __shared__ int s_last;
    uint16_t (*s_v)[kTile][VS] = reinterpret_cast<uint16_t (*)[kTile][VS]>(s_big);
    float (*s_acc)[16][D] = reinterpret_cast<float (*)[16][D]>(s_big);

    const int g = blockIdx.x;
    const int s = blockIdx.y;
    const int b = blockIdx.z / a.QTmax;
    const int qt = blockIdx.z - b * a.QTmax;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15;          // key of the score layout / row of the A operands
    const int q4 = lane >> 4;           // lane group: k-slice of the operands, row quad of S / O
    const int vrow = lane / R;          // V load layout: key row within a load
    const int vcol = lane % R;          //                8-dim column
    const int Hq = a.Hkv * G;

    const int c0 = a.cu_seqlens[b];
    const int T = max(0, a.cu_seqlens[b + 1] - c0);
    const int tok0 = qt * QT;
    if (tok0 >= T) return;              // whole workgroup exits together
    const int ntok = min(QT, T - tok0);
    const int st = a.start_pos[b];
    const int64_t cap = min((int64_t)a.max_context_len, (int64_t)a.max_blocks * a.bs);
    // keys a row may see: positions 0 .. st + token (capped so every index stays in range)
    auto row_limit = [&](int t) -> int {
        return (int)max((int64_t)0, min((int64_t)st + tok0 + t + 1, cap));
    };
    // ... and the first of them (a sliding window hides the keys before it)
    auto row_lo = [&](int t) -> int { return window_lo(row_limit(t), a.window); };
    const int L_tile = row_limit(ntok - 1);
    const int t_first = row_lo(0) / kTile * kTile;   // partitions start at the tile holding it
    const int P = a.split_tokens;
    const int t_begin = t_first + s * P;
    if (t_begin >= L_tile) return;
    const int t_end = min(L_tile, t_begin + P);
    const int nsplit = (L_tile - t_first + P - 1) / P;

    // ---- block ids of this partition -> LDS
    const BlockDiv bdiv = make_div((uint32_t)a.bs);
    const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
    const int first_blk = (int)bdiv.div((uint32_t)t_begin);
    const int n_blk = min((int)bdiv.div((uint32_t)(t_end - 1)) - first_blk + 1, kTblCap);
    const int64_t nb_max = a.num_blocks - 1;
    for (int i = threadIdx.x; i < n_blk; i += kThreads) {
        const int64_t id = trow[first_blk + i];
        s_tbl[i] = (int32_t)(id < 0 ? 0 : (id > nb_max ? nb_max : id));
    }

    // ---- Q operand: row l16 = (token l16 / G, head l16 % G), zero where no valid token
    typename M::vec qhi[NK], qlo[NK];
    float score_fix = 1.f;
    {
        const int tq = l16 / G;
        const bool qok = l16 < QT * G && tq < ntok;
        const float* qrow = a.q + ((int64_t)(c0 + tok0 + min(tq, ntok - 1)) * Hq + g * G +
                                   l16 % G) * D + 8 * q4;
        const float qs = a.scale * kLog2e;
        float qv[NK][8];
        float qmax = 0.f;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const float4 x0 = *reinterpret_cast<const float4*>(qrow + 32 * i);
            const float4 x1 = *reinterpret_cast<const float4*>(qrow + 32 * i + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                qv[i][j] = qok ? xs[j] * qs : 0.f;
                qmax = fmaxf(qmax, fabsf(qv[i][j]));
            }
        }
        float qscale = 1.f;
        if constexpr (!BF16) {
            // fp16 operand: bring max |q| below 2^14 with an exact power-of-two scale
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, off));
            if (qmax >= 16384.f && qmax <= 3.0e38f) {
                const int e = ilogbf(qmax) - 13;
                qscale = ldexpf(1.f, -e);
                score_fix = ldexpf(1.f, e);
            }
        }
#pragma unroll
        for (int i = 0; i < NK; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = qv[i][j] * qscale;
                const typename M::elem hi = (typename M::elem)x;
                qhi[i][j] = hi;
                qlo[i][j] = (typename M::elem)(x - (float)hi);
            }
    }
    // the rows of the score / output layout this lane holds: 4 * q4 + r
    int lim[4], lo[4];   // the row sees keys lo .. lim-1
    bool rvalid[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * q4 + r;
        const int t = row / G;
        rvalid[r] = row < QT * G && t < ntok;
        lim[r] = rvalid[r] ? min(row_limit(t), t_end) : 0;
        lo[r] = rvalid[r] ? row_lo(t) : 0;
    }
    __syncthreads();  // s_tbl ready

    const int64_t tok_stride = (int64_t)a.Hkv * D;   // codes between consecutive slots
    const int64_t head_off = (int64_t)g * D;
    auto row_off = [&](int t) -> int64_t {
        const int j = (int)bdiv.div((uint32_t)t);
        const int64_t blk = s_tbl[min(j - first_blk, kTblCap - 1)];
        return (blk * a.bs + (t - j * a.bs)) * tok_stride + head_off;
    };
    // loads are unconditional (keys past the partition clamp to its last key, masked at use)
    auto load_tile = [&](int base, uint4 (&kr)[NK], uint4 (&vr)[U]) {
        const uint16_t* kp = a.k_pool + row_off(min(base + l16, t_end - 1)) + 8 * q4;
#pragma unroll
        for (int i = 0; i < NK; ++i) kr[i] = load_stream(kp + 32 * i);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tv = min(base + u * TPL + vrow, t_end - 1);
            vr[u] = load_stream(a.v_pool + row_off(tv) + 8 * vcol);
        }
    };

    float m[4], lsum[4];
    f32x4 acc[NT];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m[r] = -INFINITY;
        lsum[r] = 0.f;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute_tile = [&](int base, const uint4 (&kc)[NK], const uint4 (&vc)[U]) {
        // scores
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const typename M::vec kv = __builtin_bit_cast(typename M::vec, kc[i]);
            sacc = M::mma(qhi[i], kv, sacc);
            sacc = M::mma(qlo[i], kv, sacc);
        }
        const int key = base + l16;
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float sc = key < lim[r] && key >= lo[r] ? sacc[r] * score_fix : -INFINITY;
            const float tmax = row16_max(sc);
            const float m_new = fmaxf(m[r], tmax);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2f(m[r] - m_use);   // 1 unless the row's max grew
            p[r] = exp2f(sc - m_use);
            lsum[r] = fmaf(lsum[r], alpha, p[r]);
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[n][r] *= alpha;
            m[r] = m_new;
        }
        // P -> LDS [row][key]; V -> LDS [key][dim] (keys past the partition as zero codes)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_p[wave][4 * q4 + r][l16] = p[r];
        bool vbad = false;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kr = u * TPL + vrow;
            const uint4 raw = base + kr < t_end ? vc[u] : make_uint4(0, 0, 0, 0);
            vbad |= any_nonfinite<BF16>(raw);
            *reinterpret_cast<uint4*>(&s_v[wave][kr][8 * vcol]) = raw;
        }
        wave_lds_sync();
        if (!__any(vbad)) {
            // A = P rows l16, keys 4*q4 .. 4*q4+3, split into head and remainder
            const float4 pr = *reinterpret_cast<const float4*>(&s_p[wave][l16][4 * q4]);
            const float pf[4] = {pr.x, pr.y, pr.z, pr.w};
            typename M16::vec phi, plo;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const typename M16::elem h = (typename M16::elem)pf[j];
                phi[j] = h;
                plo[j] = (typename M16::elem)(pf[j] - (float)h);
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                // B = V keys 4*q4 .. 4*q4+3, dim 16*n + l16
                typename M16::vec vb;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    vb[j] = __builtin_bit_cast(typename M16::elem, s_v[wave][4 * q4 + j][16 * n + l16]);
                acc[n] = M16::mma(phi, vb, acc[n]);
                acc[n] = M16::mma(plo, vb, acc[n]);
            }
        } else {
            // exact float products for a tile with Inf / NaN values
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * q4 + r;
                for (int k = 0; k < kTile; ++k) {
                    if (base + k >= lim[r] || base + k < lo[r]) continue;
                    const float pk = s_p[wave][row][k];
#pragma unroll
                    for (int n = 0; n < NT; ++n)
                        acc[n][r] = fmaf(pk, code_to_float<BF16>(s_v[wave][k][16 * n + l16]),
                                         acc[n][r]);
                }
            }
        }
        wave_lds_sync();
    };

    // ---- stream the partition: two register buffers, the next tile in flight
    constexpr int kStride = kWaves * kTile;
    int base = t_begin + wave * kTile;
    {
        uint4 ka[NK], va[U], kb[NK], vb[U];
        load_tile(base, ka, va);
        while (base < t_end) {
            load_tile(base + kStride, kb, vb);
            compute_tile(base, ka, va);
            base += kStride;
            if (base >= t_end) break;
            load_tile(base + kStride, ka, va);
            compute_tile(base, kb, vb);
            base += kStride;
        }
    }

    // ---- combine the waves through LDS (s_acc reuses the V staging space)
#pragma unroll
    for (int r = 0; r < 4; ++r) lsum[r] = row16_sum(lsum[r]);
    __syncthreads();  // every wave is done with its V tiles
    if (l16 == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s_m[wave][4 * q4 + r] = m[r];
            s_l[wave][4 * q4 + r] = lsum[r];
        }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_acc[wave][4 * q4 + r][16 * n + l16] = acc[n][r];
    __syncthreads();

    const int64_t item = ((int64_t)b * a.QTmax + qt) * a.Hkv + g;
    for (int i = threadIdx.x; i < 16 * D; i += kThreads) {
        const int row = i / D;
        const int d = i % D;
        const int t = row / G;
        if (row >= QT * G || t >= ntok) continue;
        float Mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) Mx = fmaxf(Mx, s_m[w][row]);
        const float M_use = (Mx == -INFINITY) ? 0.f : Mx;
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float e = exp2f(s_m[w][row] - M_use);
            num = fmaf(e, s_acc[w][row][d], num);
            den = fmaf(e, s_l[w][row], den);
        }
        if (nsplit == 1) {
            a.out[((int64_t)(c0 + tok0 + t) * Hq + g * G + row % G) * D + d] = num / den;
        } else {
            const int64_t pi = (item * a.S + s) * 16 + row;
            store_shared(a.part_acc + pi * D + d, num);
            if (d == 0) {
                store_shared(a.part_ml + pi * 2, Mx);
                store_shared(a.part_ml + pi * 2 + 1, den);
            }
        }
    }
    if (nsplit == 1) return;

    // ---- the last partition of the tile to finish merges all of them
    __builtin_amdgcn_s_waitcnt(0);  // this thread's piece stores are complete
    __syncthreads();                // ... and so are every other thread's
    int* counter = a.counters + item;
    if (threadIdx.x == 0) s_last = fetch_add_shared(counter, 1) == nsplit - 1;
    __syncthreads();
    if (!s_last) return;
    for (int i = threadIdx.x; i < 16 * D; i += kThreads) {
        const int row = i / D;
        const int d = i % D;
        const int t = row / G;
        if (row >= QT * G || t >= ntok) continue;
        const int64_t p0 = item * a.S;
        float Mx = -INFINITY;
        for (int k0 = 0; k0 < nsplit; k0 += 8) {
            float mk[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                mk[k] = k0 + k < nsplit
                            ? load_shared(a.part_ml + ((p0 + k0 + k) * 16 + row) * 2)
                            : -INFINITY;
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
                const int64_t pk = (p0 + k0 + k) * 16 + row;
                mk[k] = ok ? load_shared(a.part_ml + pk * 2) : -INFINITY;
                lk[k] = ok ? load_shared(a.part_ml + pk * 2 + 1) : 0.f;
                ak[k] = ok ? load_shared(a.part_acc + pk * D + d) : 0.f;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float e = exp2f(mk[k] - M_use);
                den = fmaf(e, lk[k], den);
                num = fmaf(e, ak[k], num);
            }
        }
        a.out[((int64_t)(c0 + tok0 + t) * Hq + g * G + row % G) * D + d] = num / den;
    }
    if (threadIdx.x == 0) store_shared(counter, 0);  // ready for the next call
}

// Long chunks: a workgroup takes 4 consecutive query tiles of one sequence and KV head (wave w
// owns tile 4k + w and all of its keys), and the K/V rows of 64 keys at a time are loaded once
// into LDS (double-buffered: the next 64 keys' loads are in flight while these are used) for
// the 4 waves; V is stored transposed ([dim][key]) so a PV operand is one 8-byte read, and a
// 16-key group holding an Inf / NaN V code is flagged while it is stored. Each wave keeps its
// own rows' running max / sum / output and writes them at the end; a wave whose tokens all lie
// before a 16-key group skips its arithmetic. Grid (Hkv, ceil(QTmax / 4), B).
template <int D, int G, bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void prefill_attn_shared_kernel(PrefillArgs a) {
    using M = Mma<BF16>;
    using M16 = Mma16<BF16>;
    constexpr int NK = D / 32;
    constexpr int NT = D / 16;
    constexpr int QT = 16 / G;
    constexpr int KT = 64;              // keys per LDS stage
    constexpr int NSUB = KT / kTile;    // 16-key groups per stage
    constexpr int KS = D + 8;           // LDS row stride of K ([key][dim]), in codes
    constexpr int VS = KT + 4;          // LDS row stride of V^T ([dim][key]), in codes
    constexpr int PS = 20;
    constexpr int CH = KT * D / 8;      // 16-byte chunks of one stage of K (or V)
    constexpr int NKC = CH / kThreads;  // K chunks per thread
    constexpr int NV = CH / kThreads;   // V chunks (adjacent keys of one column) per thread
    constexpr int PER = NKC + NV;       // chunks of K and V per thread
    static_assert(CH % kThreads == 0 && (kThreads / (D / 8)) * NV == KT, "stage shape");
    static_assert(D % 32 == 0, "tile shape");
    static_assert(G >= 1 && G <= 8, "GQA group");

    __shared__ __align__(16) uint16_t s_k[2][KT][KS];
    __shared__ __align__(16) uint16_t s_vt[2][D][VS];
    __shared__ __align__(16) float s_p[kWaves][16][PS];
    __shared__ int32_t s_tbl[kTblCap];
    __shared__ int s_vbad[2][NSUB];     // stage base whose group holds a non-finite V code

    const int g = blockIdx.x;
    const int b = blockIdx.z;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15;
    const int q4 = lane >> 4;
    const int Hq = a.Hkv * G;

    const int c0 = a.cu_seqlens[b];
    const int T = max(0, a.cu_seqlens[b + 1] - c0);
    const int tok_wg = blockIdx.y * kWaves * QT;          // first token of the workgroup
    if (tok_wg >= T) return;
    const int st = a.start_pos[b];
    const int64_t cap = min((int64_t)a.max_context_len, (int64_t)a.max_blocks * a.bs);
    auto limit_of = [&](int tok) -> int {                 // keys token tok may see
        return (int)max((int64_t)0, min((int64_t)st + tok + 1, cap));
    };
    const int tok0 = tok_wg + wave * QT;                  // this wave's first token
    const int ntok = max(0, min(QT, T - tok0));           // 0: the wave has no tokens
    const int L_wg = limit_of(min(T, tok_wg + kWaves * QT) - 1);
    const int L_w = ntok > 0 ? limit_of(tok0 + ntok - 1) : 0;
    // first keys seen (a sliding window hides the ones before): workgroup (tile aligned), wave
    const int lo_wg = window_lo(limit_of(tok_wg), a.window) / kTile * kTile;
    const int lo_w = ntok > 0 ? window_lo(limit_of(tok0), a.window) : 0;
    if (threadIdx.x < 2 * NSUB) s_vbad[threadIdx.x / NSUB][threadIdx.x % NSUB] = -1;

    // ---- Q operand of this wave's tile
    typename M::vec qhi[NK], qlo[NK];
    float score_fix = 1.f;
    {
        const int tq = l16 / G;
        const bool qok = l16 < QT * G && tq < ntok;
        const int trow = c0 + min(tok0 + min(tq, max(ntok - 1, 0)), T - 1);
        const float* qrow = a.q + ((int64_t)trow * Hq + g * G + l16 % G) * D + 8 * q4;
        const float qs = a.scale * kLog2e;
        float qv[NK][8];
        float qmax = 0.f;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const float4 x0 = *reinterpret_cast<const float4*>(qrow + 32 * i);
            const float4 x1 = *reinterpret_cast<const float4*>(qrow + 32 * i + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                qv[i][j] = qok ? xs[j] * qs : 0.f;
                qmax = fmaxf(qmax, fabsf(qv[i][j]));
            }
        }
        float qscale = 1.f;
        if constexpr (!BF16) {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, off));
            if (qmax >= 16384.f && qmax <= 3.0e38f) {
                const int e = ilogbf(qmax) - 13;
                qscale = ldexpf(1.f, -e);
                score_fix = ldexpf(1.f, e);
            }
        }
#pragma unroll
        for (int i = 0; i < NK; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = qv[i][j] * qscale;
                const typename M::elem hi = (typename M::elem)x;
                qhi[i][j] = hi;
                qlo[i][j] = (typename M::elem)(x - (float)hi);
            }
    }
    int lim[4], lo[4];   // the row sees keys lo .. lim-1
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * q4 + r;
        const int t = row / G;
        const bool ok = row < QT * G && t < ntok;
        lim[r] = ok ? limit_of(tok0 + t) : 0;
        lo[r] = ok ? window_lo(lim[r], a.window) : 0;
    }

    float m[4], lsum[4];
    f32x4 acc[NT];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m[r] = -INFINITY;
        lsum[r] = 0.f;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const BlockDiv bdiv = make_div((uint32_t)a.bs);
    const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
    const int64_t nb_max = a.num_blocks - 1;
    const int64_t tok_stride = (int64_t)a.Hkv * D;
    const int64_t head_off = (int64_t)g * D;
    const int chunk_keys = (kTblCap - 2) * a.bs / KT * KT;

    for (int c_lo = lo_wg; c_lo < L_wg; c_lo += chunk_keys) {
        const int c_hi = min(L_wg, c_lo + chunk_keys);
        const int first_blk = (int)bdiv.div((uint32_t)c_lo);
        const int n_blk = min((int)bdiv.div((uint32_t)(c_hi - 1)) - first_blk + 1, kTblCap);
        __syncthreads();  // previous readers of s_tbl / s_k / s_vt are done
        for (int i = threadIdx.x; i < n_blk; i += kThreads) {
            const int64_t id = trow[first_blk + i];
            s_tbl[i] = (int32_t)(id < 0 ? 0 : (id > nb_max ? nb_max : id));
        }
        __syncthreads();
        auto row_off = [&](int t) -> int64_t {
            const int j = (int)bdiv.div((uint32_t)t);
            const int64_t blk = s_tbl[min(j - first_blk, kTblCap - 1)];
            return (blk * a.bs + (t - j * a.bs)) * tok_stride + head_off;
        };
        // the K and V rows of one stage, 16 bytes (8 dims of one key) per chunk. K: chunk
        // c = tid + k * kThreads (k < NKC) is key c / (D/8), column c % (D/8). V: a thread takes
        // NV adjacent keys of one column (key group tid / (D/8), column tid % (D/8)), so the
        // transposed store writes each dim's NV keys as one packed word instead of NV scattered
        // 16-bit stores. Keys past the chunk of ids clamp to its last key (zeroed when stored).
        auto load_kv = [&](int base, uint4 (&r)[PER]) {
#pragma unroll
            for (int k = 0; k < NKC; ++k) {
                const int c = threadIdx.x + k * kThreads;
                const int key = c / (D / 8);
                const int col = c % (D / 8);
                r[k] = load_stream(a.k_pool + row_off(min(base + key, c_hi - 1)) + 8 * col);
            }
            const int vcol = threadIdx.x % (D / 8);
            const int vkey0 = (threadIdx.x / (D / 8)) * NV;
#pragma unroll
            for (int j = 0; j < NV; ++j)
                r[NKC + j] = load_stream(a.v_pool + row_off(min(base + vkey0 + j, c_hi - 1)) +
                                         8 * vcol);
        };
        auto store_kv = [&](int base, const uint4 (&r)[PER], int buf) {
#pragma unroll
            for (int k = 0; k < NKC; ++k) {
                const int c = threadIdx.x + k * kThreads;
                const int key = c / (D / 8);
                const int col = c % (D / 8);
                const uint4 v = base + key < c_hi ? r[k] : make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4*>(&s_k[buf][key][8 * col]) = v;
            }
            const int vcol = threadIdx.x % (D / 8);
            const int vkey0 = (threadIdx.x / (D / 8)) * NV;
            uint16_t vv[NV][8];   // [key][dim] codes of this thread's keys
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const uint4 v = base + vkey0 + j < c_hi ? r[NKC + j] : make_uint4(0, 0, 0, 0);
                if (any_nonfinite<BF16>(v)) s_vbad[buf][(vkey0 + j) / kTile] = base;
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vv[j][2 * i] = (uint16_t)(w[i] & 0xFFFFu);
                    vv[j][2 * i + 1] = (uint16_t)(w[i] >> 16);
                }
            }
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                uint16_t* dst = &s_vt[buf][8 * vcol + d][vkey0];
                if constexpr (NV >= 4) {
#pragma unroll
                    for (int j = 0; j < NV; j += 4)
                        *reinterpret_cast<uint2*>(dst + j) = make_uint2(
                            (uint32_t)vv[j][d] | ((uint32_t)vv[j + 1][d] << 16),
                            (uint32_t)vv[j + 2][d] | ((uint32_t)vv[j + 3][d] << 16));
                } else if constexpr (NV == 2) {
                    *reinterpret_cast<uint32_t*>(dst) =
                        (uint32_t)vv[0][d] | ((uint32_t)vv[1][d] << 16);
                } else {
                    dst[0] = vv[0][d];
                }
            }
        };

        // one 16-key group (keys base .. base+15, LDS keys kk .. kk+15 of buffer buf)
        auto compute_group = [&](int base, int kk, int buf, bool vbad) {
            f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                const uint4 kw =
                    *reinterpret_cast<const uint4*>(&s_k[buf][kk + l16][32 * i + 8 * q4]);
                const typename M::vec kv = __builtin_bit_cast(typename M::vec, kw);
                sacc = M::mma(qhi[i], kv, sacc);
                sacc = M::mma(qlo[i], kv, sacc);
            }
            const int key = base + l16;
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float sc = key < lim[r] && key >= lo[r] ? sacc[r] * score_fix : -INFINITY;
                const float tmax = row16_max(sc);
                const float m_new = fmaxf(m[r], tmax);
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = exp2f(m[r] - m_use);
                p[r] = exp2f(sc - m_use);
                lsum[r] = fmaf(lsum[r], alpha, p[r]);
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[n][r] *= alpha;
                m[r] = m_new;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) s_p[wave][4 * q4 + r][l16] = p[r];
            wave_lds_sync();
            if (!vbad) {
                const float4 pr = *reinterpret_cast<const float4*>(&s_p[wave][l16][4 * q4]);
                const float pf[4] = {pr.x, pr.y, pr.z, pr.w};
                typename M16::vec phi, plo;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const typename M16::elem h = (typename M16::elem)pf[j];
                    phi[j] = h;
                    plo[j] = (typename M16::elem)(pf[j] - (float)h);
                }
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    // B = V keys kk + 4*q4 .. +3 of dim 16*n + l16: one 8-byte read of V^T
                    const uint2 vw =
                        *reinterpret_cast<const uint2*>(&s_vt[buf][16 * n + l16][kk + 4 * q4]);
                    const typename M16::vec vb = __builtin_bit_cast(typename M16::vec, vw);
                    acc[n] = M16::mma(phi, vb, acc[n]);
                    acc[n] = M16::mma(plo, vb, acc[n]);
                }
            } else {
                // exact float products for a group with Inf / NaN values
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * q4 + r;
                    for (int k = 0; k < kTile; ++k) {
                        if (base + k >= lim[r] || base + k < lo[r]) continue;
                        const float pk = s_p[wave][row][k];
#pragma unroll
                        for (int n = 0; n < NT; ++n)
                            acc[n][r] = fmaf(pk, code_to_float<BF16>(s_vt[buf][16 * n + l16][kk + k]),
                                             acc[n][r]);
                    }
                }
            }
            wave_lds_sync();
        };

        uint4 regs[PER];
        load_kv(c_lo, regs);
        store_kv(c_lo, regs, 0);
        __syncthreads();
        int buf = 0;
        for (int base = c_lo; base < c_hi; base += KT) {
            const bool more = base + KT < c_hi;
            if (more) load_kv(base + KT, regs);
#pragma unroll
            for (int sg = 0; sg < NSUB; ++sg) {
                const int gb = base + sg * kTile;
                if (gb < L_w && gb + kTile > lo_w)
                    compute_group(gb, sg * kTile, buf, s_vbad[buf][sg] == base);
            }
            if (more) store_kv(base + KT, regs, buf ^ 1);
            __syncthreads();
            buf ^= 1;
        }
    }

    // ---- this wave's rows: out = acc / l
#pragma unroll
    for (int r = 0; r < 4; ++r) lsum[r] = row16_sum(lsum[r]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * q4 + r;
        const int t = row / G;
        if (row < QT * G && t < ntok) {
            float* o = a.out + ((int64_t)(c0 + tok0 + t) * Hq + g * G + row % G) * D;
#pragma unroll
            for (int n = 0; n < NT; ++n) o[16 * n + l16] = acc[n][r] / lsum[r];
        }
    }
}

template <int D, int G, bool BF16>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
    if (a.shared_tiles) {
        dim3 grid((unsigned)a.Hkv, (unsigned)((a.QTmax + kWaves - 1) / kWaves), (unsigned)a.B);
        hipLaunchKernelGGL((prefill_attn_shared_kernel<D, G, BF16>), grid, dim3(kThreads), 0,
                           stream, a);
    } else {
        dim3 grid((unsigned)a.Hkv, (unsigned)a.S, (unsigned)((int64_t)a.B * a.QTmax));
        hipLaunchKernelGGL((prefill_attn_kernel<D, G, BF16>), grid, dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t dispatch_g(const PrefillArgs& a, hipStream_t stream) {
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
hipError_t dispatch_d(const PrefillArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 32: return dispatch_g<32, BF16>(a, stream);
        case 64: return dispatch_g<64, BF16>(a, stream);
        case 128: return dispatch_g<128, BF16>(a, stream);
        case 256: return dispatch_g<256, BF16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int prefill_tile_tokens(int G) { return G >= 1 && G <= 16 ? 16 / G : 1; }

hipError_t launch_prefill_attn(const PrefillArgs& a, hipStream_t stream) {
    return a.bf16 ? dispatch_d<true>(a, stream) : dispatch_d<false>(a, stream);
}

}  // namespace pkv
