// paged_decode.hip — paged-attention decode of the paged-KV decode step (gfx950).
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
//   grid (Hkv, S, B); workgroup (g, s, b) owns tokens [s*P, min((s+1)*P, L)) of sequence b and
//   the G query heads of KV head g, so every K/V row is read from HBM once per step. The KV
//   head is the fastest grid index: the Hkv workgroups of one (b, s) run side by side and
//   together stream whole [bs, Hkv, D] blocks. The 4 waves of a workgroup take interleaved
//   16-token tiles; each wave keeps the K and V rows of its next two tiles (one for G > 4) in
//   flight while it computes the current one.
//
// Per 16-token tile and wave:
//   QK^T on the matrix cores: S[h][t] = sum_d Q[h][d] K[t][d] as D/32 MFMA 16x16x32 steps with
//     A = Q (16 rows: the G heads, zero-padded), B = K^T taken straight from the loaded rows
//     (lane l holds token l%16, 8 consecutive dims); Q is pre-scaled by scale*log2(e) and
//     split into a 16-bit high part and a 16-bit remainder, so two MFMAs per step give the
//     float product to ~2^-16 (bf16) / ~2^-22 (fp16) relative. For fp16 pools Q is also scaled
//     by a power of two into the fp16 range and the scores scaled back (exact).
//   Online softmax on the score layout (lane = token, 4 heads per lane): DPP row max, one exp2
//     per score, running max m / sum l per head; the P tile goes to LDS ([token][head]).
//   PV on the vector ALU: each V row is spread over D/8 lanes (16 bytes each, one dwordx4 load
//     moves 64/(D/8) rows); acc[h][8 dims] += p[h][t] * v[t][dims]; the running sums are
//     rescaled only in tiles where some head's max grew.
//   The 4 waves merge through LDS. A sequence with one partition writes out directly; otherwise
//   each workgroup stores (m, l, acc), and the last workgroup of (b, g) to finish (counted with
//   an atomic in the workspace, which it resets to zero) merges the partitions; partials and
//   counters are only touched with agent-scope atomic accesses, coherent across XCDs:
//     M = max m_i, out = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i.
//
// Numerics: K/V codes enter the MFMA unconverted and decode exactly on the PV side; exponentials
// and sums are float. Tokens outside [0, L) are never loaded or multiplied in, so NaN padding
// in unused slots cannot leak into the result. A running max of -inf uses 0 as the exponent
// base so exp2(-inf - (-inf)) never appears. One difference from a float dot product: a key
// holding +-Inf meets the zero remainder of an exactly representable q element in the MFMA,
// which gives NaN where float arithmetic would give an infinite score.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kTile = 16;       // tokens per wave per iteration
constexpr int kTblCap = 1024;   // block ids staged in LDS per workgroup (bounds split_tokens)

// Attended length of a sequence: context_lens[b], capped by max_context_len and by the
// tokens its table row can address (so every table and pool index stays in range).
__device__ __forceinline__ int clamp_len(int L, const DecodeArgs& a) {
    const int64_t cap = min((int64_t)a.max_context_len, (int64_t)a.max_blocks * a.bs);
    if (a.lens_are_positions) return (L >= 0 && L < cap) ? L + 1 : 0;
    return (int)min((int64_t)L, cap);
}

template <int D, int G, bool BF16>
__global__ __launch_bounds__(kWaves * 64) void paged_decode_kernel(DecodeArgs a) {
    using M = Mma<BF16>;
    constexpr int NK = D / 32;          // MFMA k-steps (and K loads) per tile
    constexpr int R = D / 8;            // lanes per V row (8 codes per lane)
    constexpr int TPL = 64 / R;         // V rows per load instruction
    constexpr int U = kTile / TPL;      // V loads per tile
    static_assert(D % 32 == 0 && U * TPL == kTile, "tile shape");
    static_assert(G >= 1 && G <= 8, "GQA group");

    __shared__ float s_p[kWaves][kTile][16];
    __shared__ float s_alpha[kWaves][16];
    __shared__ int32_t s_tbl[kTblCap];
    __shared__ float s_acc[kWaves][G][D];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];
    __shared__ int s_last;

    const int g = blockIdx.x;
    const int s = blockIdx.y;
    const int b = blockIdx.z;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15;          // token of the score layout / row of the Q operand
    const int q4 = lane >> 4;           // lane group: k-slice of the operands, head quad of S
    const int vrow = lane / R;          // V layout: token row within a load
    const int vcol = lane % R;          //           8-dim column

    const int L = clamp_len(a.context_lens[b], a);
    const int P = a.split_tokens;
    const int vis_lo = window_lo(L, a.window);        // first key the query sees
    const int t_first = vis_lo / kTile * kTile;       // partitions start at its tile
    const int t_begin = t_first + s * P;
    if (t_begin >= L) return;           // whole workgroup exits together
    const int t_end = min(L, t_begin + P);
    const int nsplit = (L - t_first + P - 1) / P;
    const int Hq = a.Hkv * G;

    // ---- block ids of this partition -> LDS (the host keeps split_tokens within kTblCap ids)
    const BlockDiv bdiv = make_div((uint32_t)a.bs);
    const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
    const int first_blk = (int)bdiv.div((uint32_t)t_begin);
    const int n_blk = min((int)bdiv.div((uint32_t)(t_end - 1)) - first_blk + 1, kTblCap);
    const int64_t nb_max = a.num_blocks - 1;
    for (int i = threadIdx.x; i < n_blk; i += kWaves * 64) {
        const int64_t id = trow[first_blk + i];
        s_tbl[i] = (int32_t)(id < 0 ? 0 : (id > nb_max ? nb_max : id));
    }

    // ---- Q operand: row l16 = head (zero beyond G), k-slice q4, pre-scaled, hi + remainder
    typename M::vec qhi[NK], qlo[NK];
    float score_fix = 1.f;
    {
        const float qs = a.scale * kLog2e;
        float qv[NK][8];
        float qmax = 0.f;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            if (l16 < G) {
                const float4* qp = reinterpret_cast<const float4*>(
                    a.q + ((int64_t)b * Hq + g * G + l16) * D + 32 * i + 8 * q4);
                const float4 x0 = qp[0], x1 = qp[1];
                qv[i][0] = x0.x; qv[i][1] = x0.y; qv[i][2] = x0.z; qv[i][3] = x0.w;
                qv[i][4] = x1.x; qv[i][5] = x1.y; qv[i][6] = x1.z; qv[i][7] = x1.w;
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
        for (int i = 0; i < NK; ++i) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = qv[i][j] * qscale;
                const typename M::elem hi = (typename M::elem)x;
                qhi[i][j] = hi;
                qlo[i][j] = (typename M::elem)(x - (float)hi);
            }
        }
    }
    __syncthreads();  // s_tbl ready

    const int64_t tok_stride = (int64_t)a.Hkv * D;   // codes between consecutive slots
    const int64_t head_off = (int64_t)g * D;
    // Loads are issued unconditionally (tokens past the partition end are clamped to its last
    // token and masked where they are used): a load behind a branch makes the compiler wait for
    // every outstanding load before it, which would drain the prefetch pipeline.
    auto row_off = [&](int t) -> int64_t {
        const int j = (int)bdiv.div((uint32_t)t);
        const int64_t blk = s_tbl[min(j - first_blk, kTblCap - 1)];
        return (blk * a.bs + (t - j * a.bs)) * tok_stride + head_off;
    };
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

    float m[4], lsum[4], acc[G][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m[r] = -INFINITY;
        lsum[r] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;

    // one 16-token tile: scores on the matrix cores, online softmax, P through LDS, PV on VALU
    auto compute_tile = [&](int base, const uint4 (&kc)[NK], const uint4 (&vc)[U]) {
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const typename M::vec kv = __builtin_bit_cast(typename M::vec, kc[i]);
            sacc = M::mma(qhi[i], kv, sacc);
            sacc = M::mma(qlo[i], kv, sacc);
        }
        const bool tok_ok = base + l16 < t_end && base + l16 >= vis_lo;
        float p[4], alpha[4];
        bool grew = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool ok = tok_ok && (4 * q4 + r) < G;
            const float sc = ok ? sacc[r] * score_fix : -INFINITY;
            const float tmax = row16_max(sc);
            const float m_new = fmaxf(m[r], tmax);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            alpha[r] = exp2f(m[r] - m_use);
            p[r] = exp2f(sc - m_use);
            lsum[r] = fmaf(lsum[r], alpha[r], p[r]);
            grew |= m_new != m[r];
            m[r] = m_new;
        }
        *reinterpret_cast<float4*>(&s_p[wave][l16][4 * q4]) = make_float4(p[0], p[1], p[2], p[3]);
        const bool rescale = __any(grew);
        if (rescale && l16 == 0)
            *reinterpret_cast<float4*>(&s_alpha[wave][4 * q4]) =
                make_float4(alpha[0], alpha[1], alpha[2], alpha[3]);
        wave_lds_sync();
        if (rescale) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float al = s_alpha[wave][h];
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[h][j] *= al;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tt = u * TPL + vrow;
            float pv[G];
#pragma unroll
            for (int h = 0; h < G; ++h) pv[h] = s_p[wave][tt][h];
            // rows past the end were clamped, rows before the window are not seen: drop them
            const bool v_ok = base + tt < t_end && base + tt >= vis_lo;
            const uint4 raw = v_ok ? vc[u] : make_uint4(0, 0, 0, 0);
            float vf[8];
            decode8<BF16>(raw, vf);
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(pv[h], vf[j], acc[h][j]);
        }
        wave_lds_sync();
    };

    // Register buffers for tiles in flight, loop unrolled so each buffer keeps its registers
    // (no copies between iterations): three buffers (two tiles ahead of the compute) while the
    // accumulators are small (G <= 4), two buffers (one ahead) otherwise to stay at two waves
    // per SIMD.
    constexpr int kStride = kWaves * kTile;
    int base = t_begin + wave * kTile;
    if constexpr (G <= 4) {
        uint4 ka[NK], va[U], kb[NK], vb[U], kcb[NK], vcb[U];
        load_tile(base, ka, va);
        load_tile(base + kStride, kb, vb);
        while (base < t_end) {
            load_tile(base + 2 * kStride, kcb, vcb);
            compute_tile(base, ka, va);
            base += kStride;
            if (base >= t_end) break;
            load_tile(base + 2 * kStride, ka, va);
            compute_tile(base, kb, vb);
            base += kStride;
            if (base >= t_end) break;
            load_tile(base + 2 * kStride, kb, vb);
            compute_tile(base, kcb, vcb);
            base += kStride;
        }
    } else {
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

    // ---- combine within the wave: l over the 16 token lanes, acc over the V row groups
#pragma unroll
    for (int r = 0; r < 4; ++r) lsum[r] = row16_sum(lsum[r]);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] = cross_group_sum<R>(acc[h][j]);
    if (l16 == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = 4 * q4 + r;
            if (h < G) {
                s_m[wave][h] = m[r];
                s_l[wave][h] = lsum[r];
            }
        }
    }
    if (vrow == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) s_acc[wave][h][vcol * 8 + j] = acc[h][j];
    }
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
            num = fmaf(e, s_acc[w][h][d], num);
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
    if (threadIdx.x == 0) s_last = fetch_add_shared(counter, 1) == nsplit - 1;
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

template <int D, int G, bool BF16>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    dim3 grid((unsigned)a.Hkv, (unsigned)a.S, (unsigned)a.B);
    hipLaunchKernelGGL((paged_decode_kernel<D, G, BF16>), grid, dim3(kWaves * 64), 0, stream, a);
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
