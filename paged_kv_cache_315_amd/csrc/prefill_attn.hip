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
// Per 16-key tile and wave: the decode tile of decode_tile.h with its 16 rows taken as the
// (token, head) rows of the query tile and a key range per row (State::rlo / rhi: key <= the
// row's position, and the row's window start): scores as K Q^T on the matrix cores, so each lane
// holds four keys of one row, which is the B operand of O^T += V^T P^T — the weights stay in
// registers; the online softmax per row with a lazily moved exponent base; a tile holding a
// non-finite code (or a row-masked key meeting a non-finite value) is computed afterwards in
// float arithmetic, row ranges included.
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
    using Tile = DecodeTile<D, BF16, true>;
    constexpr int QT = 16 / G;          // query tokens per tile
    static_assert(G >= 1 && G <= 8, "GQA group");
    union WaveLds {
        typename Tile::Scratch scr;     // the exact path's tile while streaming
        float acc[16][D];               // the wave's partial result after it
    };
    __shared__ __align__(16) WaveLds s_w[kWaves];
    __shared__ int32_t s_tbl[kTblCap];
    __shared__ __align__(16) float s_q[16][D];
    __shared__ float s_m[kWaves][16];
    __shared__ float s_l[kWaves][16];
    __shared__ int s_def[kWaves][kDecodeDefCap];
    __shared__ int s_last;

    const int g = blockIdx.x;
    const int s = blockIdx.y;
    const int b = blockIdx.z / a.QTmax;
    const int qt = blockIdx.z - b * a.QTmax;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int l16 = threadIdx.x & 15;
    const int Hq = a.Hkv * G;

    const int c0 = a.cu_seqlens[b];
    const int T = max(0, a.cu_seqlens[b + 1] - c0);
    const int tok0 = qt * QT;
    if (tok0 >= T) return;              // whole workgroup exits together
    const int ntok = min(QT, T - tok0);
    const int R = ntok * G;             // valid rows: (token r / G, head r % G)
    const int st = a.start_pos[b];
    const int64_t cap = min((int64_t)a.max_context_len, (int64_t)a.max_blocks * a.bs);
    // keys a row may see: positions 0 .. st + token (capped so every index stays in range)
    auto row_limit = [&](int t) -> int {
        return (int)max((int64_t)0, min((int64_t)st + tok0 + t + 1, cap));
    };
    // ... and the first of them (a sliding window hides the keys before it)
    auto row_lo = [&](int t) -> int { return window_lo(row_limit(t), a.window); };
    const int L_tile = row_limit(ntok - 1);
    const int vis_lo = row_lo(0);                     // first key any row sees
    const int t_first = vis_lo / kTile * kTile;       // partitions start at the tile holding it
    const int P = a.split_tokens;
    const int t_begin = t_first + s * P;
    if (t_begin >= L_tile) return;
    const int t_end = min(L_tile, t_begin + P);
    const int nsplit = (L_tile - t_first + P - 1) / P;

    // ---- block ids of this partition and the tile's query rows -> LDS
    const BlockDiv bdiv = make_div((uint32_t)a.bs);
    const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
    const int first_blk = (int)bdiv.div((uint32_t)t_begin);
    const int n_blk = min((int)bdiv.div((uint32_t)(t_end - 1)) - first_blk + 1, kTblCap);
    const int64_t nb_max = a.num_blocks - 1;
    for (int i = threadIdx.x; i < n_blk; i += kThreads) {
        const int64_t id = trow[first_blk + i];
        s_tbl[i] = (int32_t)(id < 0 ? 0 : (id > nb_max ? nb_max : id));
    }
    for (int i = threadIdx.x; i < R * D; i += kThreads) {
        const int row = i / D;
        s_q[row][i % D] =
            a.q[((int64_t)(c0 + tok0 + row / G) * Hq + g * G + row % G) * D + i % D];
    }
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
    // this wave's first tile is requested before the query operands are built
    const int first_base = t_begin + wave * kTile;
    typename Tile::Regs first;
    Tile::load_tile(src, first_base, t_begin, t_end, first);
    const float qs = a.scale * kLog2e;
    typename Tile::Query qop;
    Tile::setup_query(qf, R, qs, qop);
    typename Tile::State stt;
    Tile::init(stt);
    // row l16's keys (limits and window starts grow with the token), and the keys all rows see
    stt.rlo = l16 < R ? row_lo(l16 / G) : 0;
    stt.rhi = l16 < R ? min(row_limit(l16 / G), t_end) : 0;
    stt.alo = row_lo(ntok - 1);
    stt.ahi = min(row_limit(0), t_end);
    Tile::stream(src, t_begin, t_end, vis_lo, qop, stt, R, qs, qf, s_w[wave].scr, s_def[wave],
                 []() {}, first, first_base < t_end);

    // ---- combine the waves through LDS
    Tile::flush(stt, R, s_m[wave], s_l[wave], &s_w[wave].acc[0][0]);
    __syncthreads();

    const int64_t item = ((int64_t)b * a.QTmax + qt) * a.Hkv + g;
    for (int i = threadIdx.x; i < R * D; i += kThreads) {
        const int row = i / D;
        const int d = i % D;
        const int t = row / G;
        float Mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) Mx = fmaxf(Mx, s_m[w][row]);
        const float M_use = (Mx == -INFINITY) ? 0.f : Mx;
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float e = exp2f(s_m[w][row] - M_use);
            num = fmaf(e, s_w[w].acc[row][d], num);
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
    for (int i = threadIdx.x; i < R * D; i += kThreads) {
        const int row = i / D;
        const int d = i % D;
        const int t = row / G;
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

// Chunks of at most one query tile per sequence (draft verification, short chunks): the
// balanced schedule of decode_balanced.hip over the same tile. Segment (b, g) = the keys the
// chunk of sequence b sees through KV head g, as 16-key tiles from the one holding its first
// token's first key to its last token's last, preceded by kPrefillUnitCost empty positions;
// workgroup w takes positions [r T, (r + 1) T) (r its range under the XCD-aware deal), with the
// chunk's (token, head) rows and their key ranges; a segment cut by ranges leaves one piece of
// 16 rows per workgroup (slots 2r, 2r + 1) and the last workgroup to finish merges them.
constexpr int kPerThread = (kMaxBalancedBatch + kThreads - 1) / kThreads;
// Empty positions before each segment in the list (the decode step's 15 tiles measured 89.2 us
// on 32 x 4 draft tokens over U{512..4096} cached, 6 tiles 84.2 us, 30 tiles 85.8 us; at most
// kBalancedUnitCost, which the host's size checks assume; PKV_PREFILL_UNIT_COST overrides it in
// builds that sweep it).
#ifndef PKV_PREFILL_UNIT_COST
#define PKV_PREFILL_UNIT_COST 6
#endif
constexpr int kPrefillUnitCost =
    kBalancedUnitCost < PKV_PREFILL_UNIT_COST ? kBalancedUnitCost : PKV_PREFILL_UNIT_COST;

template <int D, int G, bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void prefill_balanced_kernel(PrefillArgs a) {
    using Tile = DecodeTile<D, BF16, true>;
    union WaveLds {
        typename Tile::Scratch scr;     // the exact path's tile while streaming
        float acc[16][D];               // the wave's partial result after it
    };
    __shared__ __align__(16) WaveLds s_w[kWaves];
    __shared__ int s_pre[kMaxBalancedBatch + 1];  // list position of each sequence's segments
    __shared__ int s_c0[kMaxBalancedBatch + 1];   // cu_seqlens
    __shared__ int s_st[kMaxBalancedBatch];       // start positions
    __shared__ int s_scan[kWaves];
    __shared__ int32_t s_tbl[kTblCap];
    __shared__ __align__(16) float s_q[16][D];
    __shared__ float s_m[kWaves][16];
    __shared__ float s_l[kWaves][16];
    __shared__ int s_def[kWaves][kDecodeDefCap];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int B = a.B;
    const int Hkv = a.Hkv;
    const int Hq = a.Hq;
    const int W = a.window;
    const int64_t cap = min((int64_t)a.max_context_len, (int64_t)a.max_blocks * a.bs);
    // keys token t of a chunk starting at position st may see: 0 .. st + t (capped)
    auto limit = [&](int st, int t) -> int {
        return (int)max((int64_t)0, min((int64_t)st + t + 1, cap));
    };
    auto span = [=](int nt) { return nt > 0 ? nt + kPrefillUnitCost : 0; };

    // ---- each sequence's tile count and the tile prefix of every sequence (all heads) -> LDS;
    // all of a thread's loads first (one round trip)
    int cu[kPerThread + 1], sp[kPerThread], sn[kPerThread];
#pragma unroll
    for (int k = 0; k <= kPerThread; ++k) cu[k] = a.cu_seqlens[min(tid * kPerThread + k, B)];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) sp[k] = a.start_pos[min(tid * kPerThread + k, B - 1)];
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int b = tid * kPerThread + k;
        sn[k] = 0;
        if (b < B) {
            // tokens of the chunk (the plan guarantees at most one query tile: QT)
            const int Tb = min(16 / G, max(0, cu[k + 1] - cu[k]));
            int nt = 0;
            if (Tb > 0) {
                const int L = limit(sp[k], Tb - 1);
                const int vis = window_lo(limit(sp[k], 0), W);
                nt = L > vis ? (L + kTile - 1) / kTile - vis / kTile : 0;
            }
            s_c0[b] = cu[k];
            s_st[b] = sp[k];
            if (b == B - 1) s_c0[B] = cu[k + 1];
            sn[k] = nt;
            cnt += span(nt);
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
                run += Hkv * span(sn[k]);
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
    // tiles of sequence b's segment (one head), from its positions in the list
    auto seg_tiles = [&](int bb) {
        const int sp1 = (s_pre[bb + 1] - s_pre[bb]) / Hkv;
        return sp1 > 0 ? sp1 - kPrefillUnitCost : 0;
    };
    int g = (r0 - s_pre[b]) / span(seg_tiles(b));

    const BlockDiv bdiv = make_div((uint32_t)a.bs);
    const int64_t nb_max = a.num_blocks - 1;
    const int chunk_tokens = ((kTblCap - 2) * a.bs) / 64 * 64;
    const float qs = a.scale * kLog2e;
    auto qf = [&](int h, int d0, float (&o)[8]) {
        const float4* src = reinterpret_cast<const float4*>(&s_q[h][d0]);
        const float4 x0 = src[0], x1 = src[1];
        o[0] = x0.x; o[1] = x0.y; o[2] = x0.z; o[3] = x0.w;
        o[4] = x1.x; o[5] = x1.y; o[6] = x1.z; o[7] = x1.w;
    };

    for (int x = r0; x < r1;) {
        // ---- one unit: tiles [x, u_end) of segment (b, g)
        const int nb = seg_tiles(b);
        const int c0 = s_c0[b];
        const int Tb = min(16 / G, max(0, s_c0[b + 1] - c0));
        const int stp = s_st[b];
        const int L = limit(stp, Tb - 1);
        const int vis = window_lo(limit(stp, 0), W);   // first key any row sees
        const int t0 = vis / kTile * kTile;
        const int seg_start = s_pre[b] + g * span(nb) + kPrefillUnitCost;  // its first tile
        const int seg_end = seg_start + nb;
        if (x < seg_start) {  // the range starts in the segment's start cost
            x = seg_start;
            if (x >= r1) break;  // ... and ends there: nothing of this segment is ours
        }
        const int u_end = min(seg_end, r1);
        const int tok_lo = t0 + (x - seg_start) * kTile;
        const int tok_hi = min(t0 + (u_end - seg_start) * kTile, L);
        const bool seg_first = x == seg_start;
        const int R = Tb * G;                          // rows (token r / G, head r % G)
        const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;

        // the query rows and the first chunk of block ids, requested together
        float qv[16 * D / kThreads];
        batched_load<kThreads>(R * D, [&](int i) {
            const int row = i / D;
            return a.q[((int64_t)(c0 + row / G) * Hq + g * G + row % G) * D + i % D];
        }, qv);
        int32_t tv[kTblCap / kThreads];
        int n_blk = 0, first_blk = 0;
        auto load_table = [&](int c_lo, int c_hi) {
            first_blk = (int)bdiv.div((uint32_t)c_lo);
            n_blk = min((int)bdiv.div((uint32_t)(c_hi - 1)) - first_blk + 1, kTblCap);
            batched_load<kThreads>(n_blk, [&](int i) { return trow[first_blk + i]; }, tv);
        };
        auto store_table = [&]() {
            batched_store<kThreads>(n_blk, tv, [&](int i, int32_t id) {
                s_tbl[i] = id < 0 ? 0 : (int32_t)min((int64_t)id, nb_max);
            });
        };
        load_table(tok_lo, min(tok_hi, tok_lo + chunk_tokens));
        batched_store<kThreads>(R * D, qv, [&](int i, float v) { s_q[i / D][i % D] = v; });
        store_table();
        typename Tile::State stt;
        Tile::init(stt);
        // row l16's keys (limits and window starts grow with the token), and the keys all rows see
        stt.rlo = l16 < R ? window_lo(limit(stp, l16 / G), W) : 0;
        stt.rhi = l16 < R ? limit(stp, l16 / G) : 0;
        stt.alo = window_lo(limit(stp, Tb - 1), W);
        stt.ahi = limit(stp, 0);
        typename Tile::Query qop;
        typename Tile::Regs ra;   // each wave's first tile, requested before the query work
        for (int c_lo = tok_lo; c_lo < tok_hi; c_lo += chunk_tokens) {
            const int c_hi = min(tok_hi, c_lo + chunk_tokens);
            if (c_lo != tok_lo) {
                __syncthreads();  // readers of s_tbl are done
                load_table(c_lo, c_hi);
                store_table();
            }
            __syncthreads();  // s_tbl (and, for the first run, s_q)
            TileSource src;
            src.k_pool = a.k_pool;
            src.v_pool = a.v_pool;
            src.tbl = s_tbl;
            src.first_blk = first_blk;
            src.tbl_cap = kTblCap;
            src.bdiv = bdiv;
            src.bs = a.bs;
            src.tile_in_block = a.bs % kTile == 0;
            src.tok_stride = (int64_t)Hkv * D;
            src.head_off = (int64_t)g * D;
            const bool first = c_lo == tok_lo;
            if (first) {
                Tile::load_tile(src, c_lo + wave * kTile, c_lo, c_hi, ra);
                Tile::setup_query(qf, R, qs, qop);
            }
            Tile::stream(src, c_lo, c_hi, vis, qop, stt, R, qs, qf, s_w[wave].scr, s_def[wave],
                         []() {}, ra, first && c_lo + wave * kTile < c_hi);
        }

        // ---- combine the waves; the outputs, or this workgroup's piece of the segment
        Tile::flush(stt, R, s_m[wave], s_l[wave], &s_w[wave].acc[0][0]);
        __syncthreads();
        const bool full = seg_first && u_end == seg_end;
        const int slot = wr * 2 + (seg_start > r0 ? 1 : 0);
        for (int i = tid; i < R * D; i += kThreads) {
            const int row = i / D;
            const int d = i % D;
            float Mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) Mx = fmaxf(Mx, s_m[w][row]);
            const float M_use = (Mx == -INFINITY) ? 0.f : Mx;
            float num = 0.f, den = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float e = exp2f(s_m[w][row] - M_use);
                num = fmaf(e, s_w[w].acc[row][d], num);
                den = fmaf(e, s_l[w][row], den);
            }
            if (full) {
                a.out[((int64_t)(c0 + row / G) * Hq + g * G + row % G) * D + d] = num / den;
            } else {
                const int64_t pi = (int64_t)slot * 16 + row;
                store_shared(a.part_acc + pi * D + d, num);
                if (d == 0) {
                    store_shared(a.part_ml + pi * 2, Mx);
                    store_shared(a.part_ml + pi * 2 + 1, den);
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
                for (int i = tid; i < R * D; i += kThreads) {
                    const int row = i / D;
                    const int d = i % D;
                    float Mx = -INFINITY;
                    for (int w = w_a; w <= w_b; ++w) {
                        const int sl = w * 2 + (w == w_a && seg_start != w_a * T ? 1 : 0);
                        Mx = fmaxf(Mx, load_shared(a.part_ml + ((int64_t)sl * 16 + row) * 2));
                    }
                    const float M_use = (Mx == -INFINITY) ? 0.f : Mx;
                    float num = 0.f, den = 0.f;
                    for (int w = w_a; w <= w_b; ++w) {
                        const int sl = w * 2 + (w == w_a && seg_start != w_a * T ? 1 : 0);
                        const int64_t pk = (int64_t)sl * 16 + row;
                        const float e = exp2f(load_shared(a.part_ml + pk * 2) - M_use);
                        den = fmaf(e, load_shared(a.part_ml + pk * 2 + 1), den);
                        num = fmaf(e, load_shared(a.part_acc + pk * D + d), num);
                    }
                    a.out[((int64_t)(c0 + row / G) * Hq + g * G + row % G) * D + d] = num / den;
                }
                if (tid == 0) store_shared(counter, 0);  // ready for the next call
            }
        }
        __syncthreads();  // LDS (s_q, s_tbl, s_w, s_m, s_l) is reused by the next unit

        x = u_end;
        if (x < r1) {
            if (++g == Hkv) {
                g = 0;
                do { ++b; } while (b < B - 1 && s_pre[b + 1] == s_pre[b]);
            }
        }
    }
}

template <int D, int G, bool BF16>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
    if (a.balanced) {
        auto kern = prefill_balanced_kernel<D, G, BF16>;
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, 0) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        const int grid = (int)std::min<int64_t>(
            std::min<int64_t>((int64_t)per_cu * a.num_cus, a.max_grid), kMaxBalancedGrid);
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    } else if (a.shared_tiles) {
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
