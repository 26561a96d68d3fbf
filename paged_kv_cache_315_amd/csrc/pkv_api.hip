// pkv_api.hip — the extern "C" entry points of libpkv: argument checks, partition sizing,
// workspace carving and kernel launches on the caller's stream. Declared in include/pkv.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

thread_local char g_err[512] = "";

pkv_status fail(pkv_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

bool valid_dtype(pkv_dtype d) { return d == PKV_F16 || d == PKV_BF16; }

constexpr int kMaxGridDim = 65535;  // y / z grid limit used for Hkv and B
constexpr int kDefaultCUs = 256;
constexpr int kTblCap = 1024;  // block ids one decode workgroup stages (paged_decode.hip)

// Largest split_tokens whose partition spans at most kTblCap blocks (a partition starts at a
// multiple of 64 tokens, so it can straddle one extra block).
int64_t max_split_for(int block_size) { return (int64_t)(kTblCap - 2) * block_size; }

// Compute units of the current device, cached per device id.
int device_cus() {
    static std::mutex mu;
    static std::vector<int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kDefaultCUs;
    std::lock_guard<std::mutex> lk(mu);
    if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = kDefaultCUs;
        cache[dev] = cus;
    }
    return cache[dev];
}

// Tokens per partition: the largest multiple of 64 in [256, 4096] that still gives about
// eight workgroups per compute unit over the whole batch (B * Hkv * ceil(Lmax / P) >= 8 * CUs),
// so short batches split finely and long ones keep the partials small.
int choose_split(int B, int Hkv, int max_context_len, int block_size, int cus) {
    const int64_t target = 8LL * cus;
    const int cap = (int)std::min<int64_t>(4096, max_split_for(block_size) / 64 * 64);
    int best = std::min(256, cap);
    for (int p = cap; p >= 256; p -= 64) {
        const int64_t items = (int64_t)B * Hkv * ((max_context_len + p - 1) / p);
        if (items >= target) {
            best = p;
            break;
        }
    }
    return best;
}

// Workspace of the decode call: partial sums, partial (max, sum) pairs, merge counters.
struct WorkspaceLayout {
    size_t acc_off, ml_off, cnt_off, total;
};

WorkspaceLayout workspace_layout(int B, int Hq, int Hkv, int D, int64_t S) {
    WorkspaceLayout w{0, 0, 0, 0};
    if (S <= 1) return w;
    const size_t parts = (size_t)B * Hq * S;
    w.acc_off = 0;
    w.ml_off = parts * D * sizeof(float);
    w.cnt_off = w.ml_off + parts * 2 * sizeof(float);
    w.total = w.cnt_off + (size_t)B * Hkv * sizeof(int);
    return w;
}

bool decode_shape_supported(int Hq, int Hkv, int D) {
    const int G = Hq / Hkv;
    return (D == 32 || D == 64 || D == 128 || D == 256) && G >= 1 && G <= 8;
}

}  // namespace

extern "C" {

const char* pkv_version(void) { return "0.1.0"; }

const char* pkv_last_error(void) { return g_err; }

const char* pkv_status_string(pkv_status s) {
    switch (s) {
        case PKV_OK: return "PKV_OK";
        case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
        case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
        case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
        case PKV_ERR_HIP: return "PKV_ERR_HIP";
    }
    return "PKV_ERR_UNKNOWN";
}

pkv_status pkv_kv_append(const float* q_in, const float* k_in, const float* v_in, float* q_out,
                         void* k_pool, void* v_pool, const int32_t* block_tables,
                         int max_blocks_per_seq, const int32_t* positions, const float* q_norm_w,
                         const float* k_norm_w, float rms_eps, float rope_theta, int B,
                         int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                         int64_t num_blocks, pkv_dtype dtype, void* stream) {
    if (B < 0) return fail(PKV_ERR_INVALID_ARG, "kv_append: B = %d < 0", B);
    if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0 || max_blocks_per_seq <= 0)
        return fail(PKV_ERR_INVALID_ARG,
                    "kv_append: sizes must be positive (Hq=%d Hkv=%d D=%d bs=%d num_blocks=%lld "
                    "max_blocks_per_seq=%d)",
                    num_q_heads, num_kv_heads, head_dim, block_size, (long long)num_blocks,
                    max_blocks_per_seq);
    if (num_q_heads % num_kv_heads)
        return fail(PKV_ERR_INVALID_ARG, "kv_append: Hq=%d not a multiple of Hkv=%d", num_q_heads,
                    num_kv_heads);
    if (!(rope_theta > 0.f) || !isfinite(rope_theta))
        return fail(PKV_ERR_INVALID_ARG, "kv_append: rope_theta=%g must be finite and > 0",
                    (double)rope_theta);
    if ((q_norm_w == nullptr) != (k_norm_w == nullptr))
        return fail(PKV_ERR_INVALID_ARG, "kv_append: give both QK-norm weights or neither");
    if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID_ARG, "kv_append: unknown dtype %d", (int)dtype);
    if ((head_dim & 1) || head_dim > 256)
        return fail(PKV_ERR_UNSUPPORTED, "kv_append: head_dim=%d must be even and <= 256", head_dim);
    if (B == 0) return PKV_OK;
    if (!q_in || !k_in || !v_in || !q_out || !k_pool || !v_pool || !block_tables || !positions)
        return fail(PKV_ERR_INVALID_ARG, "kv_append: NULL pointer argument");

    pkv::AppendArgs a;
    a.q_in = q_in;
    a.k_in = k_in;
    a.v_in = v_in;
    a.q_out = q_out;
    a.k_pool = static_cast<uint16_t*>(k_pool);
    a.v_pool = static_cast<uint16_t*>(v_pool);
    a.tables = block_tables;
    a.positions = positions;
    a.q_norm_w = q_norm_w;
    a.k_norm_w = k_norm_w;
    a.max_blocks = max_blocks_per_seq;
    a.eps = rms_eps;
    a.theta = rope_theta;
    a.B = B;
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.D = head_dim;
    a.bs = block_size;
    a.num_blocks = num_blocks;
    a.bf16 = dtype == PKV_BF16;
    const hipError_t e = pkv::launch_kv_append(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "kv_append: launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

int pkv_decode_split_tokens(int B, int num_q_heads, int num_kv_heads, int head_dim,
                            int block_size, int max_context_len) {
    if (B <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_context_len <= 0)
        return 0;
    (void)num_q_heads;
    return choose_split(B, num_kv_heads, max_context_len, block_size, device_cus());
}

size_t pkv_decode_workspace_bytes(int B, int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int max_context_len, int split_tokens) {
    if (B <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_context_len <= 0)
        return 0;
    const int P = split_tokens > 0 ? split_tokens
                                   : pkv_decode_split_tokens(B, num_q_heads, num_kv_heads, head_dim,
                                                             block_size, max_context_len);
    if (P <= 0) return 0;
    const int64_t S = ((int64_t)max_context_len + P - 1) / P;
    return workspace_layout(B, num_q_heads, num_kv_heads, head_dim, S).total;
}

pkv_status pkv_paged_attn_decode(const float* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, int max_blocks_per_seq,
                                 const int32_t* context_lens, int max_context_len, float scale,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 int split_tokens, int B, int num_q_heads, int num_kv_heads,
                                 int head_dim, int block_size, int64_t num_blocks,
                                 pkv_dtype dtype, void* stream) {
    if (B < 0 || max_context_len < 0)
        return fail(PKV_ERR_INVALID_ARG, "decode: B=%d and max_context_len=%d must be >= 0", B,
                    max_context_len);
    if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0 || max_blocks_per_seq <= 0)
        return fail(PKV_ERR_INVALID_ARG,
                    "decode: sizes must be positive (Hq=%d Hkv=%d D=%d bs=%d num_blocks=%lld "
                    "max_blocks_per_seq=%d)",
                    num_q_heads, num_kv_heads, head_dim, block_size, (long long)num_blocks,
                    max_blocks_per_seq);
    if (num_q_heads % num_kv_heads)
        return fail(PKV_ERR_INVALID_ARG, "decode: Hq=%d not a multiple of Hkv=%d", num_q_heads,
                    num_kv_heads);
    if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID_ARG, "decode: unknown dtype %d", (int)dtype);
    if (split_tokens < 0 || split_tokens % 64 || split_tokens > max_split_for(block_size))
        return fail(PKV_ERR_INVALID_ARG,
                    "decode: split_tokens=%d must be 0 or a positive multiple of 64 of at most "
                    "%lld (= %d block ids per partition)",
                    split_tokens, (long long)max_split_for(block_size), kTblCap - 2);
    if (!decode_shape_supported(num_q_heads, num_kv_heads, head_dim))
        return fail(PKV_ERR_UNSUPPORTED,
                    "decode: head_dim=%d (need 32/64/128/256) or GQA group %d (need 1..8) not built",
                    head_dim, num_q_heads / num_kv_heads);
    if (B > kMaxGridDim || num_kv_heads > kMaxGridDim)
        return fail(PKV_ERR_UNSUPPORTED, "decode: B=%d or Hkv=%d above %d", B, num_kv_heads,
                    kMaxGridDim);
    if (B == 0 || max_context_len == 0) return PKV_OK;
    if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out)
        return fail(PKV_ERR_INVALID_ARG, "decode: NULL pointer argument");

    const int P = split_tokens > 0
                      ? split_tokens
                      : choose_split(B, num_kv_heads, max_context_len, block_size, device_cus());
    const int64_t S = ((int64_t)max_context_len + P - 1) / P;
    if (S > 0x7FFFFFFF) return fail(PKV_ERR_UNSUPPORTED, "decode: too many partitions");
    const WorkspaceLayout wl = workspace_layout(B, num_q_heads, num_kv_heads, head_dim, S);
    const size_t need = wl.total;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(PKV_ERR_WORKSPACE, "decode: workspace %zu bytes, need %zu", workspace_bytes, need);

    pkv::DecodeArgs a;
    a.q = q;
    a.k_pool = static_cast<const uint16_t*>(k_pool);
    a.v_pool = static_cast<const uint16_t*>(v_pool);
    a.tables = block_tables;
    a.context_lens = context_lens;
    a.out = out;
    char* ws = static_cast<char*>(workspace);
    a.part_acc = need ? reinterpret_cast<float*>(ws + wl.acc_off) : nullptr;
    a.part_ml = need ? reinterpret_cast<float*>(ws + wl.ml_off) : nullptr;
    a.counters = need ? reinterpret_cast<int*>(ws + wl.cnt_off) : nullptr;
    a.max_blocks = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.scale = scale;
    a.split_tokens = P;
    a.S = (int)S;
    a.B = B;
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.D = head_dim;
    a.bs = block_size;
    a.num_blocks = num_blocks;
    a.bf16 = dtype == PKV_BF16;
    const hipError_t e = pkv::launch_paged_decode(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode: launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

pkv_status pkv_validate_tables(const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* positions, const int32_t* context_lens, int B,
                               int block_size, int64_t num_blocks, int max_context_len) {
    if (B < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PKV_ERR_INVALID_ARG, "validate: bad sizes");
    const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
    for (int b = 0; b < B; ++b) {
        int64_t used_tokens = 0;
        if (positions) {
            const int p = positions[b];
            if (p < 0 || p >= cap)
                return fail(PKV_ERR_INVALID_ARG, "validate: positions[%d]=%d outside [0, %lld)", b, p,
                            (long long)cap);
            used_tokens = (int64_t)p + 1;
        }
        if (context_lens) {
            const int L = context_lens[b];
            if (L < 1 || L > max_context_len || L > cap)
                return fail(PKV_ERR_INVALID_ARG,
                            "validate: context_lens[%d]=%d outside [1, min(%d, %lld)]", b, L,
                            max_context_len, (long long)cap);
            if (L > used_tokens) used_tokens = L;
        }
        if (block_tables) {
            const int64_t nblk = (used_tokens + block_size - 1) / block_size;
            for (int64_t j = 0; j < nblk; ++j) {
                const int32_t id = block_tables[(int64_t)b * max_blocks_per_seq + j];
                if (id < 0 || id >= num_blocks)
                    return fail(PKV_ERR_INVALID_ARG, "validate: block_tables[%d][%lld]=%d outside [0, %lld)",
                                b, (long long)j, id, (long long)num_blocks);
            }
        }
    }
    if (block_tables && positions) {
        // no two sequences may append into the same (block, slot)
        std::vector<int64_t> dst((size_t)B);
        for (int b = 0; b < B; ++b) {
            const int p = positions[b];
            dst[b] = (int64_t)block_tables[(int64_t)b * max_blocks_per_seq + p / block_size] * block_size +
                     p % block_size;
        }
        std::vector<int64_t> sorted = dst;
        std::sort(sorted.begin(), sorted.end());
        for (size_t i = 1; i < sorted.size(); ++i)
            if (sorted[i] == sorted[i - 1])
                return fail(PKV_ERR_INVALID_ARG, "validate: two sequences append into block %lld slot %lld",
                            (long long)(sorted[i] / block_size), (long long)(sorted[i] % block_size));
    }
    return PKV_OK;
}

}  // extern "C"
