// decode_rope.hip — paged-attention decode over a pool of un-rotated keys, with RoPE applied at
// read (gfx950).
//
// What it computes (page "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlock and
// runHybridAttentionBlockBatch: when RoPE is fused into the paged kernel, the standalone rotation
// of Q and K is skipped, the cache receives un-rotated K and the kernel, given the RoPE base,
// rotates them itself):
//   out[b][h] = softmax_t(scale * (R_p q[b][h]) . (R_t K[t][g])) . V[t][g],  p = L_b - 1,
// with R_x the rotate-half RoPE of the first rope_dim dims at position x (angle
// x * theta^(-2i/rope_dim) for the pair (i, i + rope_dim/2)). Rotations are orthogonal and
// commute, so (R_p q) . (R_t k) = q . (R_{t-p} k): the query is used as it is and each key is
// turned back by delta = p - t, which only needs cos / sin of delta * f_i.
//
// Work decomposition: the partitioned schedule of paged_decode.hip — grid (Hkv, S, B), workgroup
// (g, s, b) owns P = split_tokens tokens of sequence b and the G query heads of KV head g, with
// the same workspace (partials + counters, last partition merges). Inside a workgroup every row
// of 8-dim columns is one token: lane column c holds dims 8c .. 8c+7 of the K and V rows
// (16-byte loads), 64 / (D/8) rows per wave, waves interleaved. A lane takes U rows per
// iteration (4, or 2 for float32 pools and groups above 4): their scores share one online-softmax
// update (the running sums are rescaled only when some lane's maximum grew), and the next U rows'
// K/V are in flight while these are computed.
//
// Rotation at read. rope_dim is a multiple of 16, so a column lies entirely in the first half of
// the rotated dims, entirely in the second half, or past rope_dim. A first-half lane gets its
// partner column (the dims rope_dim/2 further on) from the lane rope_dim/16 to its right with
// one cross-lane permute of the raw codes, a second-half lane from the lane as far to its left:
//   first half:  k'_i = k_i cos(delta f_i) + k_{i+h} sin(delta f_i)
//   second half: k'_{i+h} = k_{i+h} cos(delta f_i) - k_i sin(delta f_i).
// cos / sin of every pair are evaluated once per workgroup in double at the partition's first
// row, carried to the first rows of the lanes by one-token steps, and then advanced by the fixed
// row stride with the angle-difference formulas in float (error about one ulp per step; the host
// keeps partitions to at most 4096 tokens, a few hundred steps); the rest is float arithmetic:
// dot products reduced over the row's lanes (DPP), online softmax in exp2 units, PV on the
// vector ALU.
// Keys holding +-Inf are outside what this path reproduces (Inf times a zero sine is NaN here at
// other tokens than in a rotation by absolute positions).
//
// The same kernel serves float32 pools (page "makarna/pkg/model/arch/hybrid_decoder.go":
// float32 KV goes to the plain paged kernel): a lane then loads its 8 dims as two 16-byte
// pieces; with rope_dim = 0 no key is rotated and the kernel is a plain paged decode.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTblCap = 1024;   // block ids staged in LDS per workgroup (bounds split_tokens)

__device__ __forceinline__ int clamp_len(int L, const DecodeArgs& a) {
    const int64_t cap = min((int64_t)a.max_context_len, (int64_t)a.max_blocks * a.bs);
    return (int)min((int64_t)L, cap);
}

enum ElemKind { kF16 = 0, kBF16 = 1, kF32 = 2 };

// 8 consecutive pool elements of one row: one 16-byte piece of codes, or two of floats.
template <int EK>
struct Row8 {
    static constexpr int NW = EK == kF32 ? 2 : 1;
    uint4 w[NW];
};

template <int EK>
__device__ __forceinline__ Row8<EK> load_row8(const uint16_t* pool, int64_t off) {
    Row8<EK> r;
    if constexpr (EK == kF32) {
        const float* p = reinterpret_cast<const float*>(pool) + off;
        r.w[0] = load_stream(reinterpret_cast<const uint16_t*>(p));
        r.w[1] = load_stream(reinterpret_cast<const uint16_t*>(p + 4));
    } else {
        r.w[0] = load_stream(pool + off);
    }
    return r;
}

template <int EK>
__device__ __forceinline__ void decode_row8(const Row8<EK>& r, float (&f)[8]) {
    if constexpr (EK == kF32) {
        f[0] = __uint_as_float(r.w[0].x); f[1] = __uint_as_float(r.w[0].y);
        f[2] = __uint_as_float(r.w[0].z); f[3] = __uint_as_float(r.w[0].w);
        f[4] = __uint_as_float(r.w[1].x); f[5] = __uint_as_float(r.w[1].y);
        f[6] = __uint_as_float(r.w[1].z); f[7] = __uint_as_float(r.w[1].w);
    } else {
        decode8<EK == kBF16>(r.w[0], f);
    }
}

// Sum over the R consecutive lanes of a row (R = 4, 8, 16, 32); every lane of the row receives
// the total. DPP steps inside a row of 16 lanes (lane ^ 1, lane ^ 2, the other quad of the half
// row, the other half of the row), one cross-lane exchange for the second row of 32.
template <int R>
__device__ __forceinline__ float row_sum(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    if constexpr (R >= 8) x += dpp_f<0x141>(x);
    if constexpr (R >= 16) x += dpp_f<0x140>(x);
    if constexpr (R >= 32) x += __shfl_xor(x, 16);
    return x;
}

__device__ __forceinline__ uint4 permute_u4(uint4 x, int src_lane) {
    uint4 y;
    y.x = (uint32_t)__shfl((int)x.x, src_lane);
    y.y = (uint32_t)__shfl((int)x.y, src_lane);
    y.z = (uint32_t)__shfl((int)x.z, src_lane);
    y.w = (uint32_t)__shfl((int)x.w, src_lane);
    return y;
}

template <int D, int G, int EK, bool ROT>
__global__ __launch_bounds__(kThreads) void decode_rope_kernel(DecodeArgs a) {
    constexpr int R = D / 8;            // lanes per K/V row
    constexpr int RPW = 64 / R;         // rows per wave per step
    constexpr int STR = kWaves * RPW;   // tokens per step of the workgroup
    constexpr int U = (EK == kF32 || G > 4) ? 2 : 4;   // rows per lane per iteration
    static_assert(D % 32 == 0 && G >= 1 && G <= 8, "shape");

    __shared__ int32_t s_tbl[kTblCap];
    __shared__ float s_seed[STR * D / 2][2];   // cos / sin of the first row of each (row, pair)
    __shared__ float s_step[D / 2][2];         // cos / sin of STR f_i
    __shared__ float s_acc[kWaves][G][D];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];
    __shared__ int s_last;

    const int g = blockIdx.x;
    const int s = blockIdx.y;
    const int b = blockIdx.z;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int rg = lane / R;            // row of this lane within the wave's step
    const int d0 = 8 * (lane % R);      // first dim of this lane's column

    const int L = clamp_len(a.context_lens[b], a);
    const int P = a.split_tokens;
    const int vis_lo = window_lo(L, a.window);
    const int t_first = vis_lo / 16 * 16;
    const int t_begin = t_first + s * P;
    if (t_begin >= L) return;           // whole workgroup exits together
    const int t_end = min(L, t_begin + P);
    const int nsplit = (L - t_first + P - 1) / P;
    const int Hq = a.Hkv * G;
    const int pq = L - 1;               // position of the query

    // ---- block ids of this partition -> LDS (the host keeps split_tokens within kTblCap ids)
    const BlockDiv bdiv = make_div((uint32_t)a.bs);
    const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
    const int first_blk = (int)bdiv.div((uint32_t)t_begin);
    const int n_blk = min((int)bdiv.div((uint32_t)(t_end - 1)) - first_blk + 1, kTblCap);
    const int64_t nb_max = a.num_blocks - 1;
    for (int i = threadIdx.x; i < n_blk; i += kThreads) {
        const int64_t id = trow[first_blk + i];
        s_tbl[i] = (int32_t)(id < 0 ? 0 : (id > nb_max ? nb_max : id));
    }

    // ---- this lane's query dims, in exp2 units
    const float qs = a.scale * kLog2e;
    float qv[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float4* qp =
            reinterpret_cast<const float4*>(a.q + ((int64_t)b * Hq + g * G + h) * D + d0);
        const float4 x0 = qp[0], x1 = qp[1];
        qv[h][0] = x0.x * qs; qv[h][1] = x0.y * qs; qv[h][2] = x0.z * qs; qv[h][3] = x0.w * qs;
        qv[h][4] = x1.x * qs; qv[h][5] = x1.y * qs; qv[h][6] = x1.z * qs; qv[h][7] = x1.w * qs;
    }

    // ---- rotation role of the column, cos / sin at the first token and per step
    const int rhalf = a.rope_dim >> 1;
    const bool any_rot = ROT && a.rope_dim > 0;   // the host picks ROT = (rope_dim > 0)
    const bool first_half = d0 < rhalf;
    const bool rotated = ROT && d0 < a.rope_dim;
    const int src = first_half ? lane + rhalf / 8 : (rotated ? lane - rhalf / 8 : lane);
    const int pair0 = first_half ? d0 : d0 - rhalf;
    const float sgn = first_half ? 1.f : -1.f;
    const int t0 = t_begin + wave * RPW + rg;   // this lane's first token
    // Per rotary pair i (one thread each, double): the frequency f_i, cos / sin of
    // (pq - t_begin) f_i, of f_i and of STR f_i. The seeds of the STR first rows of the partition
    // follow by one-token steps in float (at most 63 steps), so each lane starts from the seed of
    // its own first row (t_begin + k, k = wave * RPW + rg) instead of evaluating 16 double-precision
    // sines and cosines itself.
    if (any_rot) {
        for (int i = threadIdx.x; i < rhalf; i += kThreads) {
            const double inv = pow((double)a.rope_theta, -2.0 * (double)i / a.rope_dim);
            double sn, cs;
            sincos((double)(pq - t_begin) * inv, &sn, &cs);
            float c = (float)cs, sv = (float)sn;
            sincos(inv, &sn, &cs);
            const float c1 = (float)cs, s1 = (float)sn;
            sincos((double)STR * inv, &sn, &cs);
            s_step[i][0] = (float)cs;
            s_step[i][1] = (float)sn;
            for (int k = 0; k < STR; ++k) {
                s_seed[k * rhalf + i][0] = c;
                s_seed[k * rhalf + i][1] = sv;
                const float nc = fmaf(c, c1, sv * s1);
                const float ns = fmaf(sv, c1, -(c * s1));
                c = nc;
                sv = ns;
            }
        }
    }
    __syncthreads();  // s_tbl, s_seed, s_step
    float cc[8], ss[8], stc[8], sts[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        cc[j] = 1.f;
        ss[j] = 0.f;
        stc[j] = 1.f;
        sts[j] = 0.f;
    }
    if (rotated) {
        const int k = wave * RPW + rg;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            cc[j] = s_seed[k * rhalf + pair0 + j][0];
            ss[j] = s_seed[k * rhalf + pair0 + j][1];
            stc[j] = s_step[pair0 + j][0];
            sts[j] = s_step[pair0 + j][1];
        }
    }

    float m[G], lsum[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        lsum[h] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
    }

    const int64_t tok_stride = (int64_t)a.Hkv * D;
    const int64_t col_off = (int64_t)g * D + d0;
    auto row_off = [&](int t) -> int64_t {
        const int j = (int)bdiv.div((uint32_t)t);
        const int64_t blk = s_tbl[min(j - first_blk, kTblCap - 1)];
        return (blk * a.bs + (t - j * a.bs)) * tok_stride + col_off;
    };

    // every lane runs the same number of steps (rows past the partition clamp to its last row
    // and are masked), so the cross-lane permutes and reductions see a converged wave
    // U rows per lane per iteration (rows t, t + STR, ..., t + (U-1) STR): their scores share one
    // softmax update, and the next iteration's U rows are in flight while these are computed
    // (two named register buffers, the loop unrolled by two, no divergent branch inside).
    auto load_rows = [&](Row8<EK> (&kr)[U], Row8<EK> (&vr)[U], int tt) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t o = row_off(min(tt + u * STR, t_end - 1));
            kr[u] = load_row8<EK>(a.k_pool, o);
            vr[u] = load_row8<EK>(a.v_pool, o);
        }
    };
    auto compute_rows = [&](const Row8<EK> (&kc)[U], const Row8<EK> (&vc)[U], int tt) {
        float sc[U][G];
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tu = tt + u * STR;
            valid[u] = tu < t_end && tu >= vis_lo;
            float kr[8];
            decode_row8<EK>(kc[u], kr);
            if constexpr (ROT) {
                Row8<EK> kp;
#pragma unroll
                for (int i = 0; i < Row8<EK>::NW; ++i) kp.w[i] = permute_u4(kc[u].w[i], src);
                float kpf[8];
                decode_row8<EK>(kp, kpf);
                // unrotated columns keep cos 1 / sin 0 and drop the partner term: exact, and
                // branch-free (a divergent branch here made the compiler drain the prefetch)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float kp_eff = rotated ? kpf[j] : 0.f;
                    kr[j] = fmaf(kr[j], cc[j], sgn * kp_eff * ss[j]);
                }
                // delta -> delta - STR: cos(a - b) = cos a cos b + sin a sin b,
                //                       sin(a - b) = sin a cos b - cos a sin b
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float nc = fmaf(cc[j], stc[j], ss[j] * sts[j]);
                    const float ns = fmaf(ss[j], stc[j], -(cc[j] * sts[j]));
                    cc[j] = nc;
                    ss[j] = ns;
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float dot = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) dot = fmaf(qv[h][j], kr[j], dot);
                dot = row_sum<R>(dot);
                sc[u][h] = valid[u] ? dot : -INFINITY;
            }
        }
        // one online-softmax update for the U rows
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mn = m[h];
#pragma unroll
            for (int u = 0; u < U; ++u) mn = fmaxf(mn, sc[u][h]);
            const float mu = mn == -INFINITY ? 0.f : mn;
            const float al = exp2f(m[h] - mu);
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                sc[u][h] = exp2f(sc[u][h] - mu);
                ps += sc[u][h];
            }
            lsum[h] = fmaf(lsum[h], al, ps);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[h][j] *= al;
            m[h] = mn;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[8];
            decode_row8<EK>(vc[u], vf);
#pragma unroll
            for (int j = 0; j < 8; ++j) vf[j] = valid[u] ? vf[j] : 0.f;  // poisoned slots
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(sc[u][h], vf[j], acc[h][j]);
        }
    };

    // iterations in pairs with no exit between them (an odd count runs one masked iteration
    // more): an exit inside the pair made the compiler merge the two buffers with copies, and a
    // load into a register a pending load still targets waits for every load in flight
    const int n_pairs = (t_end - t_begin + 2 * U * STR - 1) / (2 * U * STR);
    int t = t0;
    Row8<EK> ka[U], va[U], kb[U], vb[U];
    load_rows(ka, va, t);
    for (int it = 0; it < n_pairs; ++it) {
        load_rows(kb, vb, t + U * STR);
        compute_rows(ka, va, t);
        load_rows(ka, va, t + 2 * U * STR);
        compute_rows(kb, vb, t + U * STR);
        t += 2 * U * STR;
    }

    // ---- combine the rows of the wave (lanes of one column), then the waves through LDS
#pragma unroll
    for (int off = R; off < 64; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = __shfl_xor(m[h], off);
            const float lo = __shfl_xor(lsum[h], off);
            const float mx = fmaxf(m[h], mo);
            const float mu = mx == -INFINITY ? 0.f : mx;
            const float e = exp2f(m[h] - mu);
            const float eo = exp2f(mo - mu);
            lsum[h] = fmaf(lsum[h], e, lo * eo);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float ao = __shfl_xor(acc[h][j], off);
                acc[h][j] = fmaf(acc[h][j], e, ao * eo);
            }
            m[h] = mx;
        }
    }
    if (rg == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int j = 0; j < 8; ++j) s_acc[wave][h][d0 + j] = acc[h][j];
            if (lane == 0) {
                s_m[wave][h] = m[h];
                s_l[wave][h] = lsum[h];
            }
        }
    }
    __syncthreads();

    float* part_acc = a.part_acc;
    float* part_ml = a.part_ml;
    for (int i = threadIdx.x; i < G * D; i += kThreads) {
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

    // ---- the last partition of (b, g) to finish merges all of them (agent-scope atomics:
    // partials and counters are shared by workgroups on different XCDs)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int* counter = a.counters + (int64_t)b * a.Hkv + g;
    if (threadIdx.x == 0) s_last = arrive(counter) == nsplit - 1;
    __syncthreads();
    if (!s_last) return;
    for (int i = threadIdx.x; i < G * D; i += kThreads) {
        const int h = i / D;
        const int d = i % D;
        const int64_t p0 = ((int64_t)b * Hq + g * G + h) * a.S;
        float Mx = -INFINITY;
        for (int k = 0; k < nsplit; ++k) Mx = fmaxf(Mx, load_shared(part_ml + (p0 + k) * 2));
        const float M_use = (Mx == -INFINITY) ? 0.f : Mx;
        float num = 0.f, den = 0.f;
        for (int k = 0; k < nsplit; ++k) {
            const float e = exp2f(load_shared(part_ml + (p0 + k) * 2) - M_use);
            den = fmaf(e, load_shared(part_ml + (p0 + k) * 2 + 1), den);
            num = fmaf(e, load_shared(part_acc + (p0 + k) * D + d), num);
        }
        a.out[((int64_t)b * Hq + g * G + h) * D + d] = num / den;
    }
    if (threadIdx.x == 0) store_shared(counter, 0);  // ready for the next call
}

template <int D, int G, int EK>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    dim3 grid((unsigned)a.Hkv, (unsigned)a.S, (unsigned)a.B);
    // 16-bit pools come here only to be rotated at read (plain ones run the balanced kernel)
    if (EK != kF32 || a.rope_dim > 0)
        hipLaunchKernelGGL((decode_rope_kernel<D, G, EK, true>), grid, dim3(kThreads), 0, stream,
                           a);
    else
        hipLaunchKernelGGL((decode_rope_kernel<D, G, kF32, false>), grid, dim3(kThreads), 0,
                           stream, a);
    return hipGetLastError();
}

template <int D, int EK>
hipError_t dispatch_g(const DecodeArgs& a, hipStream_t stream) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_typed<D, 1, EK>(a, stream);
        case 2: return launch_typed<D, 2, EK>(a, stream);
        case 3: return launch_typed<D, 3, EK>(a, stream);
        case 4: return launch_typed<D, 4, EK>(a, stream);
        case 5: return launch_typed<D, 5, EK>(a, stream);
        case 6: return launch_typed<D, 6, EK>(a, stream);
        case 7: return launch_typed<D, 7, EK>(a, stream);
        case 8: return launch_typed<D, 8, EK>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int EK>
hipError_t dispatch_d(const DecodeArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 32: return dispatch_g<32, EK>(a, stream);
        case 64: return dispatch_g<64, EK>(a, stream);
        case 128: return dispatch_g<128, EK>(a, stream);
        case 256: return dispatch_g<256, EK>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_rope(const DecodeArgs& a, hipStream_t stream) {
    if (a.f32) return dispatch_d<kF32>(a, stream);
    return a.bf16 ? dispatch_d<kBF16>(a, stream) : dispatch_d<kF16>(a, stream);
}

}  // namespace pkv
