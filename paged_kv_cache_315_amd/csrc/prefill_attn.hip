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
#include "decode_tile.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 16;
constexpr int kTblCap = 1024;

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
    if (threadIdx.x == 0) s_last = arrive(counter) == nsplit - 1;
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
// (ordinary cached loads: every query tile of the sequence reads them again) into LDS (double-buffered: the next 64 keys' loads are in flight while these are used) for
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
    constexpr int CH = KT * D / 8;      // 16-byte chunks of one stage of K (or V)
    constexpr int NKC = CH / kThreads;  // K chunks per thread
    constexpr int NV = CH / kThreads;   // V chunks (adjacent keys of one column) per thread
    constexpr int PER = NKC + NV;       // chunks of K and V per thread
    static_assert(CH % kThreads == 0 && (kThreads / (D / 8)) * NV == KT, "stage shape");
    static_assert(D % 32 == 0, "tile shape");
    static_assert(G >= 1 && G <= 8, "GQA group");

    __shared__ __align__(16) uint16_t s_k[2][KT][KS];
    __shared__ __align__(16) uint16_t s_vt[2][D][VS];
    // Position of key `key` in row `row` of the transposed V stage: groups of 4 keys are
    // permuted by row bits 4-6 (XOR of the group index with 0 .. 7). LDS serves 8-byte accesses
    // 16 lanes at a time over 32 banks: a store pass writes rows 8 dims apart (at 34 words per
    // row, two bank offsets without the permutation), a read pass reads 16 consecutive rows that
    // share bits 4-6; with it both fall on distinct banks.
    auto vt_key = [](int row, int key) -> int {
        return (((key >> 2) ^ ((row >> 4) & 7)) << 2) | (key & 3);
    };
    __shared__ int32_t s_tbl[kTblCap];
    __shared__ int s_vbad[2][NSUB];     // stage base whose group holds a non-finite V code

    const int g = blockIdx.x;
    const int b = blockIdx.z;
    const int qtg = blockIdx.y;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15;
    const int q4 = lane >> 4;
    const int Hq = a.Hkv * G;

    const int c0 = a.cu_seqlens[b];
    const int T = max(0, a.cu_seqlens[b + 1] - c0);
    const int tok_wg = qtg * kWaves * QT;                 // first token of the workgroup
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
    // this lane's query row: row l16 of the tile = token l16 / G, head l16 % G; it sees keys
    // lo_r .. lim_r - 1
    int lim_r = 0, lo_r = 0;
    {
        const int t = l16 / G;
        if (l16 < QT * G && t < ntok) {
            lim_r = limit_of(tok0 + t);
            lo_r = window_lo(lim_r, a.window);
        }
    }
    // keys every row of the wave sees (limits grow with the token): groups inside need no mask
    const int w_min_lim = ntok > 0 ? limit_of(tok0) : 0;
    const int w_max_lo = ntok > 0 ? window_lo(limit_of(tok0 + ntok - 1), a.window) : 0;
    float m = -INFINITY, lsum = 0.f;   // row l16's exponent base and this lane's part of its sum
    f32x4 acc[NT];                     // O^T: dims 16 n + 4 q4 + r of row l16
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
        // the K and V rows of one stage, 16 bytes (8 dims of one key) per chunk. K: chunk
        // c = tid + k * kThreads (k < NKC) is key c / (D/8), column c % (D/8). V: a thread takes
        // NV adjacent keys of one column (key group tid / (D/8), column tid % (D/8)), so the
        // transposed store writes each dim's keys as packed words. With the block size a
        // multiple of 16 every 16-key group of the stage lies in one block: its id is one
        // wave-uniform table read; otherwise each key's row is looked up. Keys past the chunk
        // of ids clamp to its last key (zeroed when stored).
        const bool grp_in_block = a.bs % kTile == 0;
        const int kkey0 = (int)threadIdx.x / (D / 8);          // K key of chunk k: kkey0 + k * KSTEP
        const int kcol = (int)threadIdx.x % (D / 8);
        constexpr int KSTEP = kThreads / (D / 8);              // keys between a thread's K chunks
        const int vkey0 = ((int)threadIdx.x / (D / 8)) * NV;
        auto load_kv = [&](int base, uint4 (&r)[PER]) {
            if (grp_in_block) {
                // block row of the 16-key group holding key `key` (group clamped into the chunk)
                auto grp_row = [&](int key) -> int64_t {
                    const int gk = min(base + key, c_hi - 1) / kTile * kTile;
                    const int j = (int)bdiv.div((uint32_t)gk);
                    const int64_t blk = s_tbl[min(j - first_blk, kTblCap - 1)];
                    return (blk * a.bs + (gk - j * a.bs)) * tok_stride + head_off;
                };
#pragma unroll
                for (int k = 0; k < NKC; ++k) {
                    const int key = kkey0 + k * KSTEP;
                    r[k] = load_cached(a.k_pool + grp_row(key) + (key % kTile) * tok_stride +
                                       8 * kcol);
                }
                const int64_t vrow = grp_row(vkey0);
#pragma unroll
                for (int j = 0; j < NV; ++j)
                    r[NKC + j] = load_cached(a.v_pool + vrow + ((vkey0 + j) % kTile) * tok_stride +
                                             8 * kcol);
            } else {
#pragma unroll
                for (int k = 0; k < NKC; ++k) {
                    const int key = kkey0 + k * KSTEP;
                    r[k] = load_cached(a.k_pool + row_off(min(base + key, c_hi - 1)) + 8 * kcol);
                }
#pragma unroll
                for (int j = 0; j < NV; ++j)
                    r[NKC + j] = load_cached(a.v_pool + row_off(min(base + vkey0 + j, c_hi - 1)) +
                                             8 * kcol);
            }
        };
        auto store_kv = [&](int base, uint4 (&r)[PER], int buf) {
            if (base + KT > c_hi) {   // the chunk's last stage: keys past its end stored as zero
#pragma unroll
                for (int k = 0; k < NKC; ++k)
                    if (base + kkey0 + k * KSTEP >= c_hi) r[k] = make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int j = 0; j < NV; ++j)
                    if (base + vkey0 + j >= c_hi) r[NKC + j] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int k = 0; k < NKC; ++k)
                *reinterpret_cast<uint4*>(&s_k[buf][kkey0 + k * KSTEP][8 * kcol]) = r[k];
            // V codes that may be Inf / NaN (IEEE-half view of code pairs: a * b + c stays
            // finite unless one is all-ones-exponent; for bf16 codes it also flags |x| >= 2^121,
            // which only sends a group down the exact path)
            {
                typedef __attribute__((ext_vector_type(2))) _Float16 h2;
                h2 chk = {(_Float16)0.f, (_Float16)0.f};
#pragma unroll
                for (int j = 0; j + 1 < NV; j += 2) {
                    const uint32_t x[4] = {r[NKC + j].x, r[NKC + j].y, r[NKC + j].z, r[NKC + j].w};
                    const uint32_t y[4] = {r[NKC + j + 1].x, r[NKC + j + 1].y, r[NKC + j + 1].z,
                                           r[NKC + j + 1].w};
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        chk = __builtin_elementwise_fma(__builtin_bit_cast(h2, x[w]),
                                                        __builtin_bit_cast(h2, y[w]), chk);
                }
                if constexpr (NV == 1) {
                    if (any_nonfinite<BF16>(r[NKC])) s_vbad[buf][vkey0 / kTile] = base;
                } else if (!__builtin_isfinite((float)chk[0]) || !__builtin_isfinite((float)chk[1])) {
                    s_vbad[buf][vkey0 / kTile] = base;
                }
            }
            // transposed V: dim 8 kcol + d of keys vkey0 .. vkey0 + NV - 1, two keys per word
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const int row = 8 * kcol + d;
                const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;
                auto word = [&](int j) -> uint32_t {
                    const uint4 v = r[NKC + j];
                    const int w = d >> 1;
                    return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
                };
                if constexpr (NV >= 4) {
#pragma unroll
                    for (int j = 0; j < NV; j += 4)
                        *reinterpret_cast<uint2*>(&s_vt[buf][row][vt_key(row, vkey0 + j)]) =
                            make_uint2(__builtin_amdgcn_perm(word(j + 1), word(j), sel),
                                       __builtin_amdgcn_perm(word(j + 3), word(j + 2), sel));
                } else if constexpr (NV == 2) {
                    *reinterpret_cast<uint32_t*>(&s_vt[buf][row][vt_key(row, vkey0)]) =
                        __builtin_amdgcn_perm(word(1), word(0), sel);
                } else {
                    s_vt[buf][row][vt_key(row, vkey0)] =
                        (uint16_t)((d & 1) ? word(0) >> 16 : word(0) & 0xFFFFu);
                }
            }
        };

        // one 32-key group (keys base .. base+31 = LDS keys kk .. kk+31 of buffer buf).
        // S^T = K Q^T: lane (q4, l16) gets keys base + 4 q4 + j (s0) and base + 16 + 4 q4 + j
        // (s1) of row l16, which is the B operand of O^T += V^T P^T (16x16x32, keys in the
        // order 4 q4 + j, 16 + 4 q4 + j), so P stays in registers; V^T is two 8-byte reads of
        // the transposed stage.
        auto compute_group = [&](int base, int kk, int buf, bool vbad) {
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                const typename M::vec k0v = __builtin_bit_cast(
                    typename M::vec,
                    *reinterpret_cast<const uint4*>(&s_k[buf][kk + l16][32 * i + 8 * q4]));
                const typename M::vec k1v = __builtin_bit_cast(
                    typename M::vec,
                    *reinterpret_cast<const uint4*>(&s_k[buf][kk + 16 + l16][32 * i + 8 * q4]));
                s0 = M::mma(k0v, qhi[i], s0);
                s0 = M::mma(k0v, qlo[i], s0);
                s1 = M::mma(k1v, qhi[i], s1);
                s1 = M::mma(k1v, qlo[i], s1);
            }
            float sc[8];
            if (base >= w_max_lo && base + 32 <= w_min_lim) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sc[j] = s0[j] * score_fix;
                    sc[4 + j] = s1[j] * score_fix;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int ka = base + 4 * q4 + j, kb = ka + 16;
                    sc[j] = ka < lim_r && ka >= lo_r ? s0[j] * score_fix : -INFINITY;
                    sc[4 + j] = kb < lim_r && kb >= lo_r ? s1[j] * score_fix : -INFINITY;
                }
            }
            float tmax = sc[0];
#pragma unroll
            for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, sc[j]);
            tmax = swap16_max(tmax);
            tmax = swap32_max(tmax);
            // the exponent base moves only when a score passes it by more than 8 (p <= 256)
            const bool grow = tmax > m + 8.f;
            const float m_new = grow ? tmax : m;
            const float alpha = grow ? fast_exp2(m - m_new) : 1.f;
            m = m_new;
            const float mb = m == -INFINITY ? 0.f : m;
            float p[8];
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                p[j] = fast_exp2(sc[j] - mb);
                psum += p[j];
            }
            lsum = fmaf(lsum, alpha, psum);
            if (__any(grow)) {
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[n] *= alpha;
            }
            if (!vbad) {
                typename M::vec phi, plo;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const typename M::elem h = (typename M::elem)p[j];
                    phi[j] = h;
                    plo[j] = (typename M::elem)(p[j] - (float)h);
                }
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const int row = 16 * n + l16;
                    const uint2 va =
                        *reinterpret_cast<const uint2*>(&s_vt[buf][row][vt_key(row, kk + 4 * q4)]);
                    const uint2 vb = *reinterpret_cast<const uint2*>(
                        &s_vt[buf][row][vt_key(row, kk + 16 + 4 * q4)]);
                    const typename M::vec vt =
                        __builtin_bit_cast(typename M::vec, make_uint4(va.x, va.y, vb.x, vb.y));
                    acc[n] = M::mma(vt, phi, acc[n]);
                    acc[n] = M::mma(vt, plo, acc[n]);
                }
            } else {
                // exact float products for a group with Inf / NaN values: the row's 32 weights
                // gathered from the four lanes holding them, keys outside its range skipped
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float pk = __shfl(p[j], l16 + 16 * qq);
                        const int k = j < 4 ? 4 * qq + j : 16 + 4 * qq + (j - 4);
                        const int key = base + k;
                        if (key < lim_r && key >= lo_r) {
#pragma unroll
                            for (int n = 0; n < NT; ++n)
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    acc[n][r] = fmaf(
                                        pk,
                                        code_to_float<BF16>(s_vt[buf][16 * n + 4 * q4 + r]
                                                                [vt_key(16 * n + 4 * q4 + r, kk + k)]),
                                        acc[n][r]);
                        }
                    }
            }
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
            for (int sg = 0; sg < KT / 32; ++sg) {
                const int gb = base + sg * 32;
                if (gb < L_w && gb + 32 > lo_w)
                    compute_group(gb, sg * 32, buf,
                                  s_vbad[buf][2 * sg] == base || s_vbad[buf][2 * sg + 1] == base);
            }
            if (more) store_kv(base + KT, regs, buf ^ 1);
            __syncthreads();
            buf ^= 1;
        }
    }

    // ---- this wave's rows: out = acc / l
    lsum = swap16_sum(lsum);
    lsum = swap32_sum(lsum);
    {
        const int t = l16 / G;
        if (l16 < QT * G && t < ntok) {
            float* o = a.out + ((int64_t)(c0 + tok0 + t) * Hq + g * G + l16 % G) * D;
#pragma unroll
            for (int n = 0; n < NT; ++n)
                *reinterpret_cast<float4*>(o + 16 * n + 4 * q4) =
                    make_float4(acc[n][0] / lsum, acc[n][1] / lsum, acc[n][2] / lsum,
                                acc[n][3] / lsum);
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
