// pkv_device.h — device helpers shared by the HIP kernels of libpkv (internal, gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {
namespace dev {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;

// ---- f32 -> 16-bit codes (page "makarna/pkg/kvcache/paged_cache.go": float32ToFloat16Bits,
// float32ToBFloat16Bits; round to nearest even, overflow to infinity, NaN keeps sign and leading
// payload bits forced non-zero) -------------------------------------------------------------

// binary16: normal results use the "add half-ulp minus one plus the kept lsb, then truncate"
// form on the re-biased word, so a carry out of the fraction bumps the exponent by itself;
// subnormal results shift the significand (with its implicit bit) into the 2^-24 grid and round
// on the dropped bits.
__device__ __forceinline__ uint16_t f32_to_f16_bits(uint32_t u) {
    const uint32_t sign = (u >> 16) & 0x8000u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) {  // NaN
        const uint32_t pl = (a >> 13) & 0x3FFu;
        return (uint16_t)(sign | 0x7C00u | (pl ? pl : 1u));
    }
    if (a >= 0x477FF000u)   // >= 65520 (max + half ulp) and +-Inf
        return (uint16_t)(sign | 0x7C00u);
    if (a >= 0x38800000u) { // >= 2^-14: normal binary16
        const uint32_t r = a - 0x38000000u;  // exponent bias 127 -> 15
        return (uint16_t)(sign | ((r + 0x0FFFu + ((r >> 13) & 1u)) >> 13));
    }
    if (a <= 0x33000000u)   // <= 2^-25: zero (2^-25 itself is a tie to even 0)
        return (uint16_t)sign;
    const uint32_t e = a >> 23;                     // 102 .. 112
    const uint32_t m = (a & 0x007FFFFFu) | 0x00800000u;
    const uint32_t sh = 126u - e;                   // 14 .. 24
    uint32_t q = m >> sh;
    const uint32_t rem = m & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1u);
    q += (rem > half) | ((rem == half) & (q & 1u));
    return (uint16_t)(sign | q);  // q == 0x400 is the smallest normal, encoded correctly
}

// bfloat16: round to nearest even on the low half word (carries into the exponent and
// overflows to Inf by themselves); NaN keeps sign and 7 leading payload bits, forced non-zero.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(uint32_t u) {
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) {
        const uint32_t pl = (u >> 16) & 0x7Fu;
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7F80u | (pl ? pl : 1u));
    }
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint16_t encode16(float x, bool bf16) {
    const uint32_t u = __float_as_uint(x);
    return bf16 ? f32_to_bf16_bits(u) : f32_to_f16_bits(u);
}

__device__ __forceinline__ float canonical_if_nan(float v) {
    return __builtin_isnan(v) ? __uint_as_float(0x7FC00000u) : v;
}

// ---- per-head QK-RMSNorm and RoPE, in double with every product and sum rounded separately
// (pages "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlock: norm then RoPE;
// "soft3/glia/run/arch/decoder/forward.rs", forward_layer: per-head norm, full-dim RoPE) -------

// 1 / sqrt(mean(x^2) + eps) for a head vector, the squares summed in index order.
__device__ __forceinline__ double rms_inv(const float* x, int D, float eps) {
#pragma clang fp contract(off)
    double ss = 0.0;
    for (int d = 0; d < D; ++d) {
        const double xd = (double)x[d];
        ss = ss + xd * xd;
    }
    return 1.0 / sqrt(ss / (double)D + (double)eps);
}

__device__ __forceinline__ float norm_elem(float x, double r, float w) {
#pragma clang fp contract(off)
    return canonical_if_nan((float)(((double)x * r) * (double)w));
}

// Per-head V normalisation factor in float, in the order of page "soft3/glia/run/arch/decoder/
// forward.rs" forward_layer CPU path (v_norm_per_head): the squares summed in index order,
// rms = sqrt(sum * (1/D) + eps), factor = 1 / rms; every operation rounded once (no fused
// multiply-add; division and square root correctly rounded).
__device__ __forceinline__ float vnorm_scale(const float* v, int D, float eps) {
#pragma clang fp contract(off)
    float sumsq = 0.0f;
    for (int j = 0; j < D; ++j) {
        const float sq = v[j] * v[j];
        sumsq = sumsq + sq;
    }
    const float inv_d = 1.0f / (float)D;
    const float rms = __builtin_sqrtf(sumsq * inv_d + eps);
    return 1.0f / rms;
}

__device__ __forceinline__ float vnorm_elem(float v, float scale) {
#pragma clang fp contract(off)
    return canonical_if_nan(v * scale);
}

// theta^(-2i/D), the angle per position of rotary pair i (D = the rotated span: head_dim, or
// rope_dim for partial rotary).
__device__ __forceinline__ double rope_inv_freq(float theta, int i, int D) {
#pragma clang fp contract(off)
    return pow((double)theta, -(2.0 * (double)i) / (double)D);
}

// cos / sin of the angle pos * inv_freq (inv_freq from rope_inv_freq).
__device__ __forceinline__ void rope_cs_from(int pos, double inv_freq, double& c, double& s) {
#pragma clang fp contract(off)
    const double angle = (double)pos * inv_freq;
    sincos(angle, &s, &c);
}

// cos / sin of the angle pos * theta^(-2i/D) of rotary pair i.
__device__ __forceinline__ void rope_cs(int pos, float theta, int i, int D, double& c, double& s) {
    rope_cs_from(pos, rope_inv_freq(theta, i, D), c, s);
}

// Rotate the pair (x0, x1) = (x[i], x[i + D/2]); a NaN result becomes the canonical quiet NaN.
__device__ __forceinline__ void rope_rotate(float x0, float x1, double c, double s, float& y0,
                                            float& y1) {
#pragma clang fp contract(off)
    const double t0 = (double)x0 * c;
    const double t1 = (double)x1 * s;
    const double t2 = (double)x1 * c;
    const double t3 = (double)x0 * s;
    y0 = canonical_if_nan((float)(t0 - t1));
    y1 = canonical_if_nan((float)(t2 + t3));
}

// ---- matrix cores -----------------------------------------------------------------------
template <bool BF16>
struct Mma;
template <>
struct Mma<true> {
    using vec = bf16x8;
    using elem = __bf16;
    static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mma<false> {
    using vec = f16x8;
    using elem = _Float16;
    static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// ---- cross-lane helpers -------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Reductions over each row of 16 lanes; every lane of the row receives the same value (each
// step combines a lane with its partner under an involution: lane^1, lane^2, the other quad
// of the half row, the other half of the row).
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));
    x = fmaxf(x, dpp_f<0x4E>(x));
    x = fmaxf(x, dpp_f<0x141>(x));
    x = fmaxf(x, dpp_f<0x140>(x));
    return x;
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x141>(x);
    x += dpp_f<0x140>(x);
    return x;
}

// Sum across the 64/R lane groups of a wave (lanes l, l ^ R, l ^ 2R, ...).
template <int R>
__device__ __forceinline__ float cross_group_sum(float x) {
#pragma unroll
    for (int off = R; off < 64; off <<= 1) x += __shfl_xor(x, off);
    return x;
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroups are dealt to the 8 XCDs round robin (workgroup w runs on XCD w % 8, each XCD with
// its own L2). A block of consecutive work items per XCD keeps the work of one XCD spread over
// all KV heads, i.e. over all 256-byte head slices of the token rows and so over all of its L2
// channels: item = first item of XCD (w % 8) + w / 8. A permutation of [0, n).
__device__ __forceinline__ int xcd_range(int w, int n) {
    constexpr int kXcds = 8;
    const int x = w % kXcds;
    const int per = n / kXcds, rem = n % kXcds;
    return x * per + min(x, rem) + w / kXcds;
}

// 2^x with the hardware instruction alone (v_exp_f32, about 1 ulp): softmax weights whose value
// would be a float denormal (below 2^-126, i.e. scores more than 126 below the exponent base)
// come out as zero, which moves a weighted sum by less than 2^-126 of its largest term.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// First position a query at attended length L sees under a sliding window of W positions
// (0: no window).
__device__ __forceinline__ int window_lo(int L, int W) { return (W > 0 && L > W) ? L - W : 0; }

// Copy of n elements (n <= PER NT), element i -> st(i, ld(i)), by the NT threads of a
// workgroup, thread t taking i = t + k NT, in two halves: batched_load issues every load of a
// thread into registers, batched_store stores them. Copies whose loads are all issued before
// the first store wait for one memory round trip together, where a loop that stores each
// element as it arrives waits for one per element it takes. Lanes past n load element n - 1
// (in bounds) and store nothing. Every register of v is written (zero where nothing is
// loaded), so no value of an earlier copy stays live in it across the code between copies.
template <int NT, int PER, typename T, typename Ld>
__device__ __forceinline__ void batched_load(int n, Ld&& ld, T (&v)[PER]) {
#pragma unroll
    for (int k = 0; k < PER; ++k)
        v[k] = k * NT < n ? ld(min((int)threadIdx.x + k * NT, n - 1)) : T{};
}
template <int NT, int PER, typename T, typename St>
__device__ __forceinline__ void batched_store(int n, const T (&v)[PER], St&& st) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = (int)threadIdx.x + k * NT;
        if (i < n) st(i, v[k]);
    }
}

// ---- K/V codes ----------------------------------------------------------------------------
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

// 16-byte load of streamed K/V codes, marked non-temporal: every row is read once per call.
__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
    typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// 16-byte load of K/V codes that other workgroups read again (kept in the caches).
__device__ __forceinline__ uint4 load_cached(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// Unsigned division by the block size: shift for powers of two, otherwise a multiply-high
// with a precomputed magic number (round-up method with the add fix-up, exact for all u32).
struct BlockDiv {
    uint32_t magic, shift;
    bool pow2;
    __device__ __forceinline__ uint32_t div(uint32_t n) const {
        if (pow2) return n >> shift;
        const uint32_t t = __umulhi(n, magic);
        return (t + ((n - t) >> 1)) >> shift;
    }
};

__device__ __forceinline__ BlockDiv make_div(uint32_t d) {
    BlockDiv r;
    r.pow2 = (d & (d - 1)) == 0;
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;  // l = ceil(log2 d)
    if (r.pow2) {
        r.shift = l;
        r.magic = 0;
    } else {
        r.magic = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
        r.shift = l - 1;
    }
    return r;
}

// ---- values shared between workgroups -----------------------------------------------------
// Partial results and merge counters are written by one workgroup and read by another, which
// may sit on another XCD (each XCD has its own L2). Every access to them is an agent-scope
// atomic: on gfx950 those carry the sc1 cache policy, so a store is written through the XCD's
// L2 to the device-coherent memory side and counted complete (vmcnt) once it is there, a load
// misses the L2 and reads the memory side, and a read-modify-write is performed there. The
// protocol: every thread stores its pieces, waits for its stores (s_waitcnt vmcnt(0)), the
// workgroup meets at a barrier, then one thread counts the arrival (arrive, relaxed); the
// workgroup that brings the count to the total reads the pieces after the count returned. So the
// pieces are at the memory side before the count moves, and are read from there after it.
// Acquire / release order on the count would do the same through a whole-L2 write-back before
// and an invalidate after each count (measured: +46 % on the 32-sequence decode step).
__device__ __forceinline__ void store_shared(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_shared(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int arrive(int* counter) {
    return __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_shared(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dev
}  // namespace pkv
