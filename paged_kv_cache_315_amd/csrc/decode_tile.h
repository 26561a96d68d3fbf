// decode_tile.h — one wave's 16-token tile of paged-attention decode on the matrix cores
// (gfx950), shared by the balanced (decode_balanced.hip) and partitioned (paged_decode.hip)
// decode kernels.
//
// What a tile adds to the running softmax state of the G query heads of one KV head
// (page "soft3/glia/run/arch/decoder/forward.rs", forward_layer CPU attention path: scores
// q . k scaled, max-subtracted exponentials, weights times V, normalised by their sum; page
// "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlockBatch: the query heads of
// a group share one KV head):
//
//   scores  S^T[t][h] = sum_d K[t][d] * (q[h][d] * scale * log2 e): MFMA 16x16x32 with A = the
//           16 key rows (lane l: token l%16, dims 8*(l/16) + 32 i .. + 7, exactly the 16 bytes
//           the lane loaded) and B = Q^T (lane l: head l%16, the same dims). The query is split
//           into a 16-bit head and a 16-bit remainder, two MFMAs per k-step, so a score carries
//           ~2^-16 (bf16) / ~2^-22 (fp16) relative error. Lane (q4 = l/16, l16 = l%16) receives
//           the scores of tokens 4*q4 + r (r < 4) for head l16; heads >= G are zero rows of Q.
//   softmax per head: the tile maximum (in lane, then across the four lane groups with two
//           row swaps), p = exp2(s - m). The exponent base m of a head moves only when a score
//           passes it by more than 8, so p <= 256 (exact in the PV operands) and the
//           accumulators are rescaled only in those rare tiles.
//   PV      O^T[d][h] += sum_t V[t][d] * P^T[t][h]: MFMA 16x16x16 with B = P^T straight from the
//           score registers (the B layout is lane l: tokens 4*(l/16) + j of head l%16), P split
//           into a 16-bit head and remainder (two MFMAs, ~2^-16 relative), and A = V^T built
//           without a transpose: lane (q4, l16) loads tokens 4*q4 + j (j < 4) of the 8-dim
//           chunk l16, so element e of its four rows is row "dim 8*l16 + e" of A for tokens
//           4*q4 .. 4*q4 + 3 (one v_perm_b32 per pair of tokens). MFMA e of a chunk set covers
//           the dims {8*c + e}. Heads and dims of the output therefore sit as lane l16 = head,
//           rows 4*q4 + r = chunk, MFMA e = dim within the chunk.
//   exact path: a tile whose valid scores are not all finite (a key code holding Inf or NaN)
//           or whose V codes may hold Inf or NaN is left out of the streaming loop and computed
//           afterwards (reloaded) with float dot products and float multiply-adds; the online
//           softmax does not depend on the order of the tiles. In the matrix cores such a code meets zero operand parts
//           (the remainder of an exactly representable value, a zero weight) and 0 * Inf gives
//           NaN where float arithmetic gives +-Inf or a skipped token.
//
// Invalid tokens of a partial tile (outside [lo, hi)) get score -inf and zero V rows (their
// slots may hold anything, NaN included), so they contribute nothing.
#pragma once

#include "pkv_device.h"

namespace pkv {
namespace dev {

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

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

// x combined with the same register of lane l ^ 16 (rows 0<->1, 2<->3) / lane l ^ 32.
__device__ __forceinline__ float swap16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Exact value of one 16-bit code.
template <bool BF16>
__device__ __forceinline__ float code_to_float(uint32_t c) {
    if constexpr (BF16) return __uint_as_float(c << 16);
    else return (float)__builtin_bit_cast(_Float16, (unsigned short)c);
}

// Where the tiles of one chunk of a KV head's tokens live: the block ids of the chunk staged in
// LDS (tbl[j - first_blk] is the id of the sequence's block j), the pools and strides.
struct TileSource {
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    const int32_t* tbl;     // LDS, tbl_cap ids
    int first_blk;
    int tbl_cap;
    BlockDiv bdiv;          // division by the block size
    int bs;
    bool tile_in_block;     // bs % 16 == 0: a 16-token tile lies in one block
    int64_t tok_stride;     // codes between consecutive slots (Hkv * D)
    int64_t head_off;       // codes of the KV head inside a slot (g * D)
};

constexpr int kDecodeWaves = 4;     // waves per workgroup of the decode kernels
constexpr int kDecodeDefCap = 8;    // exact-path tiles a wave lists before it runs them

// ROWS: the 16 rows are (token, head) pairs of several query tokens, each row with its own key
// range [State::rlo, State::rhi) inside the tile-uniform one (chunked prefill); without it every
// row sees the same keys (decode).
template <int D, bool BF16, bool ROWS = false>
struct DecodeTile {
    static constexpr int NK = D / 32;              // K loads (and MFMA k-steps) per lane
    static constexpr int NC = D / 8;               // 8-dim chunks of a row
    static constexpr int NH = NC > 16 ? NC / 16 : 1;  // chunk sets of 16 lanes
    static constexpr int NV = 4 * NH;              // V loads per lane: 4 tokens per chunk set
    static constexpr int NQ = NC < 16 ? NC / 4 : 4;  // lane groups holding distinct chunks
    static_assert(D == 32 || D == 64 || D == 128 || D == 256, "head_dim");
    using M32 = Mma<BF16>;
    using M16 = Mma16<BF16>;
    using qvec = typename M32::vec;
    using pvec = typename M16::vec;

    struct Query {
        qvec hi[NK], lo[NK];
        float fix;  // scores are multiplied by it (power of two, fp16 range scale)
    };
    struct State {
        float m;            // exponent base of head l16 (log2 units)
        float l;            // this lane's part of the sum of weights of head l16
        f32x4 acc[NH][8];   // O^T rows 4*q4 + r (chunk), MFMA e (dim in chunk), head l16
        int rlo, rhi;       // ROWS: keys row l16 sees
        int alo, ahi;       // ROWS: keys every row sees (the same in every lane)
    };
    struct Regs {
        uint4 k[NK];        // token l16, dims 8*q4 + 32 i .. + 7
        uint4 v[NV];        // token 4*q4 + (u & 3), chunk (l16 % NC) + 16 (u >> 2)
    };
    // per-wave LDS of the exact path
    struct Scratch {
        uint4 k[16][NC];    // the tile's K rows (chunks of 8 codes)
        uint4 v[16][NC];    // the tile's V rows
        float s[16][17];    // weights [head][token]
    };

    static __device__ __forceinline__ int chunk_of(int l16, int set) { return (l16 % NC) + 16 * set; }

    // Lane offsets (in codes) inside a tile whose 16 rows lie tok_stride codes apart.
    static __device__ __forceinline__ uint32_t k_lane_off(int64_t tok_stride) {
        const int lane = threadIdx.x & 63;
        return (uint32_t)((lane & 15) * tok_stride + 8 * (lane >> 4));
    }
    static __device__ __forceinline__ uint32_t v_lane_off(int64_t tok_stride, int j) {
        const int lane = threadIdx.x & 63;
        return (uint32_t)((4 * (lane >> 4) + j) * tok_stride + 8 * ((lane & 15) % NC));
    }

    // The tile's rows start at k0 / v0 (row 0 of the tile, this KV head) and are tok_stride
    // codes apart (all 16 rows in one block).
    static __device__ __forceinline__ void load_block(const uint16_t* k0, const uint16_t* v0,
                                                      uint32_t koff, const uint32_t (&voff)[4],
                                                      Regs& r) {
#pragma unroll
        for (int i = 0; i < NK; ++i) r.k[i] = load_stream(k0 + koff + 32 * i);
#pragma unroll
        for (int s = 0; s < NH; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) r.v[4 * s + j] = load_stream(v0 + voff[j] + 128 * s);
    }

    // Rows anywhere: kp = this lane's K row (at dim 8*q4), vp[j] = row of token 4*q4 + j (at
    // dim 0 of the head).
    static __device__ __forceinline__ void load_rows(const uint16_t* kp, const uint16_t* const (&vp)[4],
                                                     Regs& r) {
        const int l16 = threadIdx.x & 15;
#pragma unroll
        for (int i = 0; i < NK; ++i) r.k[i] = load_stream(kp + 32 * i);
#pragma unroll
        for (int s = 0; s < NH; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) r.v[4 * s + j] = load_stream(vp[j] + 8 * chunk_of(l16, s));
    }

    // Query operand from the G rotated query rows (row h at q_rows + h * D), pre-scaled by
    // qs = scale * log2 e.
    template <typename QRow>
    static __device__ __forceinline__ void setup_query(QRow&& qrow, int G, float qs, Query& q) {
        const int lane = threadIdx.x & 63;
        const int l16 = lane & 15, q4 = lane >> 4;
        float qv[NK][8];
        float qmax = 0.f;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            if (l16 < G) {
                qrow(l16, 32 * i + 8 * q4, qv[i]);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) qv[i][j] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                qv[i][j] *= qs;
                qmax = fmaxf(qmax, fabsf(qv[i][j]));
            }
        }
        float qscale = 1.f;
        q.fix = 1.f;
        if constexpr (!BF16) {
            // fp16 operand: bring max |q| below 2^14 with an exact power-of-two scale
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, off));
            if (qmax >= 16384.f && qmax <= 3.0e38f) {
                const int e = ilogbf(qmax) - 13;
                qscale = ldexpf(1.f, -e);
                q.fix = ldexpf(1.f, e);
            }
        }
#pragma unroll
        for (int i = 0; i < NK; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = qv[i][j] * qscale;
                const typename M32::elem hi = (typename M32::elem)x;
                q.hi[i][j] = hi;
                q.lo[i][j] = (typename M32::elem)(x - (float)hi);
            }
    }

    static __device__ __forceinline__ void init(State& st) {
        st.m = -INFINITY;
        st.l = 0.f;
#pragma unroll
        for (int s = 0; s < NH; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) st.acc[s][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Online-softmax step over the four scores of head l16 held by this lane: new exponent
    // base, weights p, rescale of the running sum and (when some lane's base moved) of the
    // accumulators.
    static __device__ __forceinline__ void softmax(const float (&sc)[4], State& st, float (&p)[4]) {
        float tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        tmax = swap16_max(tmax);
        tmax = swap32_max(tmax);
        const bool grow = tmax > st.m + 8.f;   // -inf base: any finite score; NaN: never
        const float m_new = grow ? tmax : st.m;
        const float alpha = grow ? fast_exp2(st.m - m_new) : 1.f;
        st.m = m_new;
        const float mb = m_new == -INFINITY ? 0.f : m_new;   // all scores so far masked
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = fast_exp2(sc[r] - mb);
        st.l = fmaf(st.l, alpha, (p[0] + p[1]) + (p[2] + p[3]));
        if (__any(grow)) {
#pragma unroll
            for (int s = 0; s < NH; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) st.acc[s][e] *= alpha;
        }
    }

    // One tile: tokens base .. base + 15, of which [lo, hi) are attended. Returns true (the
    // same in every lane, state untouched) when the tile needs the exact path instead.
    static __device__ __forceinline__ bool compute(Regs& r, int base, int lo, int hi,
                                                   const Query& q, State& st) {
        const int lane = threadIdx.x & 63;
        const int l16 = lane & 15, q4 = lane >> 4;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const qvec kv = __builtin_bit_cast(qvec, r.k[i]);
            s = M32::mma(kv, q.hi[i], s);
            s = M32::mma(kv, q.lo[i], s);
        }
        bool full = base >= lo && base + 16 <= hi;   // the same in every lane
        if constexpr (ROWS) full = full && base >= st.alo && base + 16 <= st.ahi;
        if (!full) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = base + 4 * q4 + j;
                if (t < lo || t >= hi)
#pragma unroll
                    for (int w = 0; w < NH; ++w) r.v[4 * w + j] = make_uint4(0, 0, 0, 0);
            }
        }
        // V codes that may be Inf / NaN: IEEE-half view of the code pairs, (a * b + acc) stays
        // finite unless one of them has the all-ones exponent (for bf16 codes this also flags
        // |x| >= 2^121, and for fp16 products above 65504: those tiles take the exact path,
        // which is correct for any codes)
        f16x2 chk = {(_Float16)0.f, (_Float16)0.f};
#pragma unroll
        for (int u = 0; u < NV; u += 2) {
            const uint32_t a[4] = {r.v[u].x, r.v[u].y, r.v[u].z, r.v[u].w};
            const uint32_t b[4] = {r.v[u + 1].x, r.v[u + 1].y, r.v[u + 1].z, r.v[u + 1].w};
#pragma unroll
            for (int w = 0; w < 4; ++w)
                chk = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, a[w]),
                                                __builtin_bit_cast(f16x2, b[w]), chk);
        }
        bool bad = !__builtin_isfinite((float)chk[0]) || !__builtin_isfinite((float)chk[1]);
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = base + 4 * q4 + j;
            const bool ok = full || (t >= lo && t < hi && (!ROWS || (t >= st.rlo && t < st.rhi)));
            const float x = s[j] * q.fix;
            bad |= ok && !__builtin_isfinite(x);
            sc[j] = ok ? x : -INFINITY;
        }
        if (__any(bad)) return true;
        float p[4];
        softmax(sc, st, p);
        pvec phi, plo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const typename M16::elem h = (typename M16::elem)p[j];
            phi[j] = h;
            plo[j] = (typename M16::elem)(p[j] - (float)h);
        }
#pragma unroll
        for (int w = 0; w < NH; ++w) {
            const uint4* v = &r.v[4 * w];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int dw = e >> 1;
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                const uint32_t x0 = dw == 0 ? v[0].x : dw == 1 ? v[0].y : dw == 2 ? v[0].z : v[0].w;
                const uint32_t x1 = dw == 0 ? v[1].x : dw == 1 ? v[1].y : dw == 2 ? v[1].z : v[1].w;
                const uint32_t x2 = dw == 0 ? v[2].x : dw == 1 ? v[2].y : dw == 2 ? v[2].z : v[2].w;
                const uint32_t x3 = dw == 0 ? v[3].x : dw == 1 ? v[3].y : dw == 2 ? v[3].z : v[3].w;
                const uint32_t w01 = __builtin_amdgcn_perm(x1, x0, sel);
                const uint32_t w23 = __builtin_amdgcn_perm(x3, x2, sel);
                const pvec a = __builtin_bit_cast(pvec, make_uint2(w01, w23));
                st.acc[w][e] = M16::mma(a, phi, st.acc[w][e]);
                st.acc[w][e] = M16::mma(a, plo, st.acc[w][e]);
            }
        }
        return false;
    }

    // The tile in float arithmetic: scores as float dot products of the rotated query and the
    // decoded keys, weights times decoded V rows with float multiply-adds; invalid tokens are
    // skipped. The tile's K and V rows go through this wave's LDS so the registers of the tile
    // are free while it runs.
    // qf(h, d0, out[8]) gives the float query (rotated, unscaled) of head h, dims d0 .. d0 + 7;
    // scr is this wave's LDS for it.
    template <typename QF>
    static __device__ __forceinline__ void exact(const Regs& r, int base, int lo, int hi,
                                                 State& st, int G, float qs, QF&& qf, Scratch& scr) {
        const int lane = threadIdx.x & 63;
        const int l16 = lane & 15, q4 = lane >> 4;
        bool full = base >= lo && base + 16 <= hi;
        if constexpr (ROWS) full = full && base >= st.alo && base + 16 <= st.ahi;
#pragma unroll
        for (int i = 0; i < NK; ++i) scr.k[l16][4 * i + q4] = r.k[i];
#pragma unroll
        for (int w = 0; w < NH; ++w)
#pragma unroll
            for (int j = 0; j < 4; ++j) scr.v[4 * q4 + j][chunk_of(l16, w)] = r.v[4 * w + j];
        wave_lds_sync();
        // scores: lane (q4, l16) takes tokens 4*q4 + j of head l16 (heads >= G: -inf)
        const int hq = l16 < G ? l16 : 0;
        float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int c = 0; c < NC; ++c) {
            float qc[8];
            qf(hq, 8 * c, qc);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float kf[8];
                decode8<BF16>(scr.k[4 * q4 + j][c], kf);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[j] = fmaf(qc[e] * qs, kf[e], x[j]);
            }
        }
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = base + 4 * q4 + j;
            const bool ok = full || (t >= lo && t < hi && (!ROWS || (t >= st.rlo && t < st.rhi)));
            sc[j] = (ok && l16 < G) ? x[j] : -INFINITY;
        }
        float p[4];
        softmax(sc, st, p);
#pragma unroll
        for (int j = 0; j < 4; ++j) scr.s[l16][4 * q4 + j] = p[j];
        wave_lds_sync();
#pragma unroll 1
        for (int t = 0; t < 16; ++t) {
            const int tt = base + t;
            if (!(full || (tt >= lo && tt < hi))) continue;
            // a row that does not see this key has weight 0, which must not meet its values
            if (ROWS && !full && !(tt >= st.rlo && tt < st.rhi)) continue;
            const float pt = scr.s[l16][t];
#pragma unroll
            for (int w = 0; w < NH; ++w)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    float vf[8];
                    decode8<BF16>(scr.v[t][chunk_of(4 * q4 + rr, w)], vf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) st.acc[w][e][rr] = fmaf(pt, vf[e], st.acc[w][e][rr]);
                }
        }
        wave_lds_sync();
    }

    // Loads tile `base` (clamped to the chunk's last tile, so prefetches past the end stay in
    // range) of tokens [c_lo, c_hi). The loads are unconditional: a load behind a branch made
    // the compiler wait for the whole prefetch.
    static __device__ __forceinline__ void load_tile(const TileSource& src, int base, int c_lo,
                                                     int c_hi, Regs& r) {
        const int lane = threadIdx.x & 63;
        const int l16 = lane & 15, q4 = lane >> 4;
        const int bb = min(base, c_lo + (c_hi - 1 - c_lo) / 16 * 16);
        const uint16_t* kp;
        const uint16_t* vp[4];
        if (src.tile_in_block) {
            const int j = (int)src.bdiv.div((uint32_t)bb);
            const int blk =
                __builtin_amdgcn_readfirstlane(src.tbl[min(j - src.first_blk, src.tbl_cap - 1)]);
            const int64_t row0 =
                ((int64_t)blk * src.bs + (bb - j * src.bs)) * src.tok_stride + src.head_off;
            kp = src.k_pool + row0 + k_lane_off(src.tok_stride);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) vp[jj] = src.v_pool + row0 + (4 * q4 + jj) * src.tok_stride;
        } else {
            auto row_off = [&](int t) -> int64_t {
                const int j = (int)src.bdiv.div((uint32_t)t);
                const int64_t blk = src.tbl[min(j - src.first_blk, src.tbl_cap - 1)];
                return (blk * src.bs + (t - j * src.bs)) * src.tok_stride + src.head_off;
            };
            kp = src.k_pool + row_off(min(bb + l16, c_hi - 1)) + 8 * q4;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) vp[jj] = src.v_pool + row_off(min(bb + 4 * q4 + jj, c_hi - 1));
        }
        load_rows(kp, vp, r);
    }

    // The tiles of tokens [c_lo, c_hi) (c_lo a multiple of 16 apart from the range start),
    // tokens before lo not attended: wave w takes tiles c_lo + 16 (w + 4 k). Two register
    // buffers: the next tile's K/V rows load while one is computed (the loop is unrolled by two
    // so each buffer keeps its registers). Tiles that need the exact path are listed (def: this
    // wave's kDecodeDefCap ints of LDS) and run after the loop, reloaded. after_tile() is
    // called after each streamed tile.
    // ra: the first buffer; have_first: it already holds this wave's first tile (c_lo + 16
    // wave), requested by the caller.
    template <typename QF, typename After>
    static __device__ __forceinline__ void stream(const TileSource& src, int c_lo, int c_hi,
                                                  int lo, const Query& q, State& st, int G,
                                                  float qs, QF&& qf, Scratch& scr, int* def,
                                                  After&& after_tile, Regs& ra,
                                                  bool have_first) {
        constexpr int kStride = kDecodeWaves * 16;
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        const bool lane0 = (threadIdx.x & 63) == 0;
        int base = c_lo + wave * 16;
        Regs rb;
        if (!have_first) load_tile(src, base, c_lo, c_hi, ra);
        while (base < c_hi) {
            int ndef = 0;
            {
                while (true) {
                    load_tile(src, base + kStride, c_lo, c_hi, rb);
                    if (compute(ra, base, lo, c_hi, q, st)) {
                        if (lane0) def[ndef] = base;
                        ++ndef;
                    }
                    after_tile();
                    base += kStride;
                    if (base >= c_hi || ndef == kDecodeDefCap) break;
                    load_tile(src, base + kStride, c_lo, c_hi, ra);
                    if (compute(rb, base, lo, c_hi, q, st)) {
                        if (lane0) def[ndef] = base;
                        ++ndef;
                    }
                    after_tile();
                    base += kStride;
                    if (base >= c_hi || ndef == kDecodeDefCap) break;
                }
            }
            for (int i = 0; i < ndef; ++i) {
                wave_lds_sync();
                const int tb = def[i];
                Regs r;
                load_tile(src, tb, c_lo, c_hi, r);
                exact(r, tb, lo, c_hi, st, G, qs, qf, scr);
            }
            if (base < c_hi) load_tile(src, base, c_lo, c_hi, ra);  // after a full list
        }
    }

    // End of a unit: this wave's (m, l, acc) of heads h < G into LDS (m_w / l_w [h],
    // acc_w [h * D + d]).
    static __device__ __forceinline__ void flush(const State& st, int G, float* m_w, float* l_w,
                                                 float* acc_w) {
        const int lane = threadIdx.x & 63;
        const int l16 = lane & 15, q4 = lane >> 4;
        float l = swap16_sum(st.l);
        l = swap32_sum(l);
        if (l16 < G) {
            if (q4 == 0) {
                m_w[l16] = st.m;
                l_w[l16] = l;
            }
            if (q4 < NQ) {
#pragma unroll
                for (int w = 0; w < NH; ++w)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int c = 4 * q4 + rr + 16 * w;
                        float4* dst = reinterpret_cast<float4*>(acc_w + l16 * D + 8 * c);
                        dst[0] = make_float4(st.acc[w][0][rr], st.acc[w][1][rr], st.acc[w][2][rr],
                                             st.acc[w][3][rr]);
                        dst[1] = make_float4(st.acc[w][4][rr], st.acc[w][5][rr], st.acc[w][6][rr],
                                             st.acc[w][7][rr]);
                    }
            }
        }
    }
};

}  // namespace dev
}  // namespace pkv
