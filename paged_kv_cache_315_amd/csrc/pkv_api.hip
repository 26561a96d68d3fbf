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

}  // namespace

// The same thread-local message for the host block manager (block_manager.cpp).
namespace pkv {
pkv_status fail(pkv_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}
}  // namespace pkv

namespace {

bool valid_dtype(pkv_dtype d) { return d == PKV_F16 || d == PKV_BF16 || d == PKV_F32; }

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

// Workspace of the decode calls: the merge counters first (a fixed place whichever schedule a
// call uses, so they stay zero across calls of either kind), then the partial results.
struct WorkspaceLayout {
    size_t cnt_off, acc_off, ml_off, total;
    bool balanced;
    int64_t S;  // partitions per sequence (partitioned schedule)
};

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Whether rotation at read / float32 pools take the float32 matrix-core tile (when the caller
// leaves the schedule to the library) rather than the vector-ALU kernel: the tile pads the G
// query heads of a KV head to 16 columns. Measured on the llama3-8b lengths with 32 query heads
// (decode us, matrix-core tile / vector-ALU kernel): rotating at read, G = 4 92.0 / 125.1,
// G = 2 154.7 / 147.4, G = 1 283.7 / 212.0; float32 pools without rotation, G = 4 124.8 /
// 161.1, G = 2 224.9 / 245.8, G = 1 420.3 / 400.3.
bool rope_mfma_pays(int D, int G, int read_dim, bool f32) {
    if (!pkv::decode_rope_mfma_ok(D, G, read_dim)) return false;
    return G >= 3 || (f32 && read_dim == 0 && G == 2);
}

// Partition length of the vector-ALU rotation-at-read / float32 kernel when the caller leaves
// it to the library: choose_split's, at most 576 tokens (its many short partitions keep more
// rows in flight per compute unit; on the shapes above, 576 against choose_split's 4032:
// G = 1 rotating 212.0 / 237.5 us, float32 400.3 / 463.5 us).
constexpr int kValuSplitMax = 576;
int valu_split(int B, int Hkv, int max_context_len, int block_size, int cus) {
    return std::min(kValuSplitMax, choose_split(B, Hkv, max_context_len, block_size, cus));
}

// The balanced schedule needs the per-sequence tile prefix in LDS and int32 tile counts.
bool balanced_ok(int B, int Hkv, int64_t max_tokens) {
    // the tile list (tiles plus each segment's start cost) is indexed with 32-bit ints
    return B <= pkv::kMaxBalancedBatch &&
           (int64_t)B * Hkv * ((max_tokens + 15) / 16 + pkv::kBalancedUnitCost) < (1LL << 31);
}

WorkspaceLayout layout_for(int B, int Hq, int Hkv, int D, int64_t max_tokens, int split_tokens,
                           int block_size, bool balanced) {
    WorkspaceLayout w{0, 0, 0, 0, balanced, 1};
    const size_t cnt = align256((size_t)B * Hkv * sizeof(int));
    size_t parts;
    if (balanced) {
        parts = (size_t)pkv::kMaxBalancedGrid * 2 * (Hq / Hkv);
    } else {
        const int P = split_tokens;
        w.S = (max_tokens + P - 1) / P;
        if (w.S <= 1) return w;  // one partition per sequence: no partials, no counters
        parts = (size_t)B * Hq * w.S;
    }
    (void)block_size;
    w.cnt_off = 0;
    w.acc_off = cnt;
    w.ml_off = w.acc_off + align256(parts * D * sizeof(float));
    w.total = w.ml_off + align256(parts * 2 * sizeof(float));
    return w;
}

bool decode_shape_supported(int Hq, int Hkv, int D) {
    const int G = Hq / Hkv;
    return (D == 32 || D == 64 || D == 128 || D == 256) && G >= 1 && G <= 8;
}

// Size / shape checks shared by the calls; returns PKV_OK or sets the error text.
pkv_status check_common(const char* who, int B, int Hq, int Hkv, int D, int bs, int64_t nb,
                        int max_blocks, pkv_dtype dtype) {
    if (B < 0) return fail(PKV_ERR_INVALID_ARG, "%s: B = %d < 0", who, B);
    if (Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || nb <= 0 || max_blocks <= 0)
        return fail(PKV_ERR_INVALID_ARG,
                    "%s: sizes must be positive (Hq=%d Hkv=%d D=%d bs=%d num_blocks=%lld "
                    "max_blocks_per_seq=%d)",
                    who, Hq, Hkv, D, bs, (long long)nb, max_blocks);
    if (Hq % Hkv)
        return fail(PKV_ERR_INVALID_ARG, "%s: Hq=%d not a multiple of Hkv=%d", who, Hq, Hkv);
    if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID_ARG, "%s: unknown dtype %d", who, (int)dtype);
    return PKV_OK;
}

pkv_status check_rope(const char* who, float theta, const float* qn, const float* kn, int D) {
    if (!(theta > 0.f) || !isfinite(theta))
        return fail(PKV_ERR_INVALID_ARG, "%s: rope_theta=%g must be finite and > 0", who,
                    (double)theta);
    if ((qn == nullptr) != (kn == nullptr))
        return fail(PKV_ERR_INVALID_ARG, "%s: give both QK-norm weights or neither", who);
    if ((D & 1) || D > 256)
        return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim=%d must be even and <= 256", who, D);
    return PKV_OK;
}

// Layer options with the defaults filled in (rope_dim = D, no V norm, no window, rotation
// applied by the append).
struct Variant {
    int rope_dim;
    bool v_norm;
    int window;
    bool rope_read;
    float read_theta;
};

pkv_status resolve_variant(const char* who, const pkv_variant* v, int D, Variant& out) {
    out = Variant{D, false, 0, false, 0.f};
    if (v == nullptr) return PKV_OK;
    if (v->rope_dim < 0 || v->rope_dim > D || (v->rope_dim & 1))
        return fail(PKV_ERR_INVALID_ARG, "%s: rope_dim=%d must be 0 or even in [2, head_dim=%d]",
                    who, v->rope_dim, D);
    if (v->window < 0) return fail(PKV_ERR_INVALID_ARG, "%s: window=%d < 0", who, v->window);
    out.rope_dim = v->rope_dim ? v->rope_dim : D;
    out.v_norm = v->v_norm != 0;
    out.window = v->window;
    out.rope_read = v->rope_on_read != 0;
    out.read_theta = v->read_theta;
    return PKV_OK;
}

pkv_status check_decode_shape(const char* who, int B, int Hq, int Hkv, int D) {
    if (!decode_shape_supported(Hq, Hkv, D))
        return fail(PKV_ERR_UNSUPPORTED,
                    "%s: head_dim=%d (need 32/64/128/256) or GQA group %d (need 1..8) not built",
                    who, D, Hq / Hkv);
    if (B > kMaxGridDim || Hkv > kMaxGridDim)
        return fail(PKV_ERR_UNSUPPORTED, "%s: B=%d or Hkv=%d above %d", who, B, Hkv, kMaxGridDim);
    return PKV_OK;
}

}  // namespace

// Chunked prefill attention: query tiles per sequence, keys per partition and partitions.
struct PrefillPlan {
    int QTmax, P, S;
    bool shared;   // 4 query tiles per workgroup sharing each K/V tile (no key split)
    bool balanced; // one query tile per sequence: the balanced schedule
    int max_grid;  // balanced: workgroups the pieces are sized for
    size_t cnt_off, acc_off, ml_off, total;
};

PrefillPlan prefill_plan(int B, int Hq, int Hkv, int D, int bs, int max_chunk, int max_ctx,
                         int cus) {
    PrefillPlan p{};
    const int QT = pkv::prefill_tile_tokens(Hq / Hkv);
    p.QTmax = (max_chunk + QT - 1) / QT;
    const int64_t items = (int64_t)B * p.QTmax * Hkv;
    // long chunks: workgroups of 4 query tiles sharing the K/V tiles, when there are enough of
    // them to fill the device twice over
    if (p.QTmax >= 4 && (int64_t)B * ((p.QTmax + 3) / 4) * Hkv >= 2LL * cus) {
        p.shared = true;
        p.S = 1;
        p.P = 0;
        return p;
    }
    // at most one query tile per sequence (draft verification, short chunks): the balanced
    // schedule, pieces for two workgroups per compute unit
    if (p.QTmax == 1 && B <= pkv::kMaxBalancedBatch &&
        (int64_t)B * Hkv * ((max_ctx + 15) / 16 + pkv::kBalancedUnitCost) < (1LL << 31)) {
        p.balanced = true;
        p.S = 1;
        p.P = 0;
        p.max_grid = std::min(pkv::kMaxBalancedGrid, 2 * cus);
        const size_t parts = (size_t)p.max_grid * 2 * 16;
        p.cnt_off = 0;
        p.acc_off = align256((size_t)B * Hkv * sizeof(int));
        p.ml_off = p.acc_off + align256(parts * D * sizeof(float));
        p.total = p.ml_off + align256(parts * 2 * sizeof(float));
        return p;
    }
    // split the keys only as far as needed to give every compute unit a few workgroups
    const int64_t target = 4LL * cus;
    int64_t S = items >= target ? 1 : (target + items - 1) / items;
    S = std::min<int64_t>(S, std::max<int64_t>(1, ((int64_t)max_ctx + 255) / 256));
    const int64_t cap = max_split_for(bs) / 64 * 64;
    int64_t P = ((max_ctx + S - 1) / S + 63) / 64 * 64;
    P = std::max<int64_t>(64, std::min<int64_t>(P, cap));
    p.P = (int)P;
    p.S = (int)((max_ctx + P - 1) / P);
    if (p.S > 1) {
        const size_t parts = (size_t)items * p.S * 16;
        p.cnt_off = 0;
        p.acc_off = align256((size_t)items * sizeof(int));
        p.ml_off = p.acc_off + align256(parts * D * sizeof(float));
        p.total = p.ml_off + align256(parts * 2 * sizeof(float));
    }
    return p;
}

#ifdef PKV_TIMELINE
namespace pkv {
namespace {
uint64_t* g_timeline = nullptr;
int g_timeline_rot = 0;
}
uint64_t* timeline_buffer() { return g_timeline; }
int timeline_rotation() { return g_timeline_rot; }
}  // namespace pkv

// Profiling builds only (not part of include/pkv.h): the balanced decode kernel writes
// kTimelineStamps stamps per workgroup into buf (device, at least 2048 * 8 uint64), or nothing
// when buf is NULL; workgroup w takes tile range (w + rot) % grid.
extern "C" void pkv_timeline_set(void* buf, int rot) {
    pkv::g_timeline = static_cast<uint64_t*>(buf);
    pkv::g_timeline_rot = rot;
}
#endif

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
                         int64_t num_blocks, pkv_dtype dtype, const pkv_variant* variant,
                         void* stream) {
    pkv_status st = check_common("kv_append", B, num_q_heads, num_kv_heads, head_dim, block_size,
                                 num_blocks, max_blocks_per_seq, dtype);
    if (st != PKV_OK) return st;
    st = check_rope("kv_append", rope_theta, q_norm_w, k_norm_w, head_dim);
    if (st != PKV_OK) return st;
    Variant var;
    st = resolve_variant("kv_append", variant, head_dim, var);
    if (st != PKV_OK) return st;
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
    a.cu_seqlens = nullptr;
    a.rows = B;
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
    a.rope_dim = var.rope_read ? 0 : var.rope_dim;  // rotation at read: the pool keeps un-rotated K
    a.v_norm = var.v_norm;
    a.bf16 = dtype == PKV_BF16;
    a.f32 = dtype == PKV_F32;
    const hipError_t e = pkv::launch_kv_append(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "kv_append: launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

int pkv_decode_split_tokens(int B, int num_q_heads, int num_kv_heads, int head_dim,
                            int block_size, int max_context_len) {
    if (B <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_context_len <= 0)
        return 0;
    return choose_split(B, num_kv_heads, max_context_len, block_size, device_cus());
}

size_t pkv_decode_workspace_bytes(int B, int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int max_context_len, int split_tokens) {
    if (B <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_context_len <= 0 || split_tokens < 0 || num_q_heads % num_kv_heads)
        return 0;
    const bool bal = split_tokens == 0 && balanced_ok(B, num_kv_heads, max_context_len);
    int P = split_tokens;
    if (!bal && P == 0) P = pkv_decode_split_tokens(B, num_q_heads, num_kv_heads, head_dim,
                                                    block_size, max_context_len);
    return layout_for(B, num_q_heads, num_kv_heads, head_dim, max_context_len, P, block_size, bal)
        .total;
}

size_t pkv_decode_step_workspace_bytes(int B, int num_q_heads, int num_kv_heads, int head_dim,
                                       int block_size, int max_blocks_per_seq) {
    if (B <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks_per_seq <= 0 || num_q_heads % num_kv_heads)
        return 0;
    const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
    const int max_ctx = (int)std::min<int64_t>(cap, 0x7FFFFFFF);
    return pkv_decode_workspace_bytes(B, num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_ctx, 0);
}

namespace {

// Runs the decode on the schedule `wl` describes (q already rotated).
pkv_status run_decode(const float* q, const void* k_pool, const void* v_pool,
                      const int32_t* tables, int max_blocks, const int32_t* context_lens,
                      int max_context_len, float scale, float* out, void* workspace,
                      const WorkspaceLayout& wl, int P, int B, int Hq, int Hkv, int D, int bs,
                      int64_t nb, pkv_dtype dtype, int window, hipStream_t stream,
                      bool lens_are_positions = false) {
    char* ws = static_cast<char*>(workspace);
    const bool has_ws = wl.total > 0;
    hipError_t e;
    if (wl.balanced) {
        pkv::BalancedArgs a{};
        a.q = q;
        a.k_pool = static_cast<uint16_t*>(const_cast<void*>(k_pool));
        a.v_pool = static_cast<uint16_t*>(const_cast<void*>(v_pool));
        a.tables = tables;
        a.lens = context_lens;
        a.out = out;
        a.part_acc = reinterpret_cast<float*>(ws + wl.acc_off);
        a.part_ml = reinterpret_cast<float*>(ws + wl.ml_off);
        a.counters = reinterpret_cast<int*>(ws + wl.cnt_off);
        a.max_blocks = max_blocks;
        a.max_context_len = max_context_len;
        a.scale = scale;
        a.B = B;
        a.Hq = Hq;
        a.Hkv = Hkv;
        a.D = D;
        a.bs = bs;
        a.num_blocks = nb;
        a.num_cus = device_cus();
        a.rope_dim = D;
        a.window = window;
        a.bf16 = dtype == PKV_BF16;
        a.append = false;
#ifdef PKV_TIMELINE
        a.timeline = pkv::timeline_buffer();
        a.timeline_rot = pkv::timeline_rotation();
#endif
        e = pkv::launch_decode_balanced(a, stream);
    } else {
        pkv::DecodeArgs a;
        a.q = q;
        a.k_pool = static_cast<const uint16_t*>(k_pool);
        a.v_pool = static_cast<const uint16_t*>(v_pool);
        a.tables = tables;
        a.context_lens = context_lens;
        a.out = out;
        a.part_acc = has_ws ? reinterpret_cast<float*>(ws + wl.acc_off) : nullptr;
        a.part_ml = has_ws ? reinterpret_cast<float*>(ws + wl.ml_off) : nullptr;
        a.counters = has_ws ? reinterpret_cast<int*>(ws + wl.cnt_off) : nullptr;
        a.max_blocks = max_blocks;
        a.max_context_len = max_context_len;
        a.scale = scale;
        a.split_tokens = P;
        a.S = (int)wl.S;
        a.B = B;
        a.Hq = Hq;
        a.Hkv = Hkv;
        a.D = D;
        a.bs = bs;
        a.num_blocks = nb;
        a.window = window;
        a.bf16 = dtype == PKV_BF16;
        a.lens_are_positions = lens_are_positions;
        e = pkv::launch_paged_decode(a, stream);
    }
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode: launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

}  // namespace

pkv_status pkv_paged_attn_decode(const float* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, int max_blocks_per_seq,
                                 const int32_t* context_lens, int max_context_len, float scale,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 int split_tokens, int B, int num_q_heads, int num_kv_heads,
                                 int head_dim, int block_size, int64_t num_blocks,
                                 pkv_dtype dtype, const pkv_variant* variant, void* stream) {
    pkv_status st = check_common("decode", B, num_q_heads, num_kv_heads, head_dim, block_size,
                                 num_blocks, max_blocks_per_seq, dtype);
    if (st != PKV_OK) return st;
    Variant var;
    st = resolve_variant("decode", variant, head_dim, var);
    if (st != PKV_OK) return st;
    if (max_context_len < 0)
        return fail(PKV_ERR_INVALID_ARG, "decode: max_context_len=%d must be >= 0", max_context_len);
    if (split_tokens < 0 || split_tokens % 64 || split_tokens > max_split_for(block_size))
        return fail(PKV_ERR_INVALID_ARG,
                    "decode: split_tokens=%d must be 0 or a positive multiple of 64 of at most "
                    "%lld (= %d block ids per partition)",
                    split_tokens, (long long)max_split_for(block_size), kTblCap - 2);
    st = check_decode_shape("decode", B, num_q_heads, num_kv_heads, head_dim);
    if (st != PKV_OK) return st;
    if (var.rope_read) {
        if (!(var.read_theta > 0.f) || !isfinite(var.read_theta))
            return fail(PKV_ERR_INVALID_ARG, "decode: read_theta=%g must be finite and > 0",
                        (double)var.read_theta);
        if (var.rope_dim % 16)
            return fail(PKV_ERR_UNSUPPORTED,
                        "decode: rope_on_read needs rope_dim a multiple of 16 (got %d)",
                        var.rope_dim);
    }
    if (B == 0 || max_context_len == 0) return PKV_OK;
    if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out)
        return fail(PKV_ERR_INVALID_ARG, "decode: NULL pointer argument");
    if (var.rope_read || dtype == PKV_F32) {
        const int read_dim = var.rope_read ? var.rope_dim : 0;
        if (split_tokens == 0 && balanced_ok(B, num_kv_heads, max_context_len) &&
            rope_mfma_pays(head_dim, num_q_heads / num_kv_heads, read_dim, dtype == PKV_F32)) {
            // the float32 matrix-core tile on the balanced schedule (the workspace of the
            // 16-bit decode: pkv_decode_workspace_bytes with split_tokens = 0)
            const WorkspaceLayout wl = layout_for(B, num_q_heads, num_kv_heads, head_dim,
                                                  max_context_len, 0, block_size, true);
            if (workspace == nullptr || workspace_bytes < wl.total)
                return fail(PKV_ERR_WORKSPACE, "decode: workspace %zu bytes, need %zu",
                            workspace_bytes, wl.total);
            char* ws = static_cast<char*>(workspace);
            pkv::BalancedArgs a{};
            a.q = q;
            a.k_pool = static_cast<uint16_t*>(const_cast<void*>(k_pool));
            a.v_pool = static_cast<uint16_t*>(const_cast<void*>(v_pool));
            a.tables = block_tables;
            a.lens = context_lens;
            a.out = out;
            a.part_acc = reinterpret_cast<float*>(ws + wl.acc_off);
            a.part_ml = reinterpret_cast<float*>(ws + wl.ml_off);
            a.counters = reinterpret_cast<int*>(ws + wl.cnt_off);
            a.max_blocks = max_blocks_per_seq;
            a.max_context_len = max_context_len;
            a.scale = scale;
            a.theta = var.read_theta;
            a.B = B;
            a.Hq = num_q_heads;
            a.Hkv = num_kv_heads;
            a.D = head_dim;
            a.bs = block_size;
            a.num_blocks = num_blocks;
            a.num_cus = device_cus();
            a.rope_dim = read_dim;
            a.window = var.window;
            a.bf16 = dtype == PKV_BF16;
            a.f32 = dtype == PKV_F32;
            const hipError_t e = pkv::launch_decode_rope_balanced(a, static_cast<hipStream_t>(stream));
            if (e != hipSuccess)
                return fail(PKV_ERR_HIP, "decode: launch failed: %s", hipGetErrorString(e));
            return PKV_OK;
        }
        // otherwise the partitioned schedule of decode_rope.hip (the matrix-core tile where it
        // serves the shape, else the vector-ALU kernel)
        if (split_tokens > 4096)
            return fail(PKV_ERR_INVALID_ARG,
                        "decode: split_tokens=%d above 4096 for rope_on_read / float32 pools (the "
                        "rotation is carried across a partition in float steps)", split_tokens);
        const int P = split_tokens > 0 ? split_tokens
                                       : valu_split(B, num_kv_heads, max_context_len,
                                                    block_size, device_cus());
        if (((int64_t)max_context_len + P - 1) / P > 0x7FFFFFFF)
            return fail(PKV_ERR_UNSUPPORTED, "decode: too many partitions");
        const WorkspaceLayout wl = layout_for(B, num_q_heads, num_kv_heads, head_dim,
                                              max_context_len, P, block_size, false);
        if (wl.total > 0 && (workspace == nullptr || workspace_bytes < wl.total))
            return fail(PKV_ERR_WORKSPACE, "decode: workspace %zu bytes, need %zu",
                        workspace_bytes, wl.total);
        char* ws = static_cast<char*>(workspace);
        const bool has_ws = wl.total > 0;
        pkv::DecodeArgs a{};
        a.q = q;
        a.k_pool = static_cast<const uint16_t*>(k_pool);
        a.v_pool = static_cast<const uint16_t*>(v_pool);
        a.tables = block_tables;
        a.context_lens = context_lens;
        a.out = out;
        a.part_acc = has_ws ? reinterpret_cast<float*>(ws + wl.acc_off) : nullptr;
        a.part_ml = has_ws ? reinterpret_cast<float*>(ws + wl.ml_off) : nullptr;
        a.counters = has_ws ? reinterpret_cast<int*>(ws + wl.cnt_off) : nullptr;
        a.max_blocks = max_blocks_per_seq;
        a.max_context_len = max_context_len;
        a.scale = scale;
        a.split_tokens = P;
        a.S = (int)wl.S;
        a.B = B;
        a.Hq = num_q_heads;
        a.Hkv = num_kv_heads;
        a.D = head_dim;
        a.bs = block_size;
        a.num_blocks = num_blocks;
        a.window = var.window;
        a.bf16 = dtype == PKV_BF16;
        a.lens_are_positions = false;
        a.rope_theta = var.read_theta;
        a.rope_dim = var.rope_read ? var.rope_dim : 0;
        a.f32 = dtype == PKV_F32;
        const hipError_t e = pkv::launch_decode_rope(a, static_cast<hipStream_t>(stream));
        if (e != hipSuccess)
            return fail(PKV_ERR_HIP, "decode: launch failed: %s", hipGetErrorString(e));
        return PKV_OK;
    }

    const bool bal = split_tokens == 0 && balanced_ok(B, num_kv_heads, max_context_len);
    const int P = bal ? 0
                      : (split_tokens > 0 ? split_tokens
                                          : choose_split(B, num_kv_heads, max_context_len,
                                                         block_size, device_cus()));
    if (!bal && ((int64_t)max_context_len + P - 1) / P > 0x7FFFFFFF)
        return fail(PKV_ERR_UNSUPPORTED, "decode: too many partitions");
    const WorkspaceLayout wl = layout_for(B, num_q_heads, num_kv_heads, head_dim,
                                          max_context_len, P, block_size, bal);
    if (wl.total > 0 && (workspace == nullptr || workspace_bytes < wl.total))
        return fail(PKV_ERR_WORKSPACE, "decode: workspace %zu bytes, need %zu", workspace_bytes,
                    wl.total);
    return run_decode(q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                      max_context_len, scale, out, workspace, wl, P, B, num_q_heads, num_kv_heads,
                      head_dim, block_size, num_blocks, dtype, var.window,
                      static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---- scratch of the decode step that allocates nothing (pkv_decode_step_noalloc) ------------
// Device memory of this library, one copy per GPU, held until the process ends: the merge
// counters (B * Hkv ints) and the partial pieces of the balanced schedule (two per workgroup).
// In host code `scratch` names a host-side stand-in, not a device address; kernels get the
// address hipGetSymbolAddress returns for the current device (scratch_device_ptr).
static constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

__global__ void zero_ints_kernel(int* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept.
pkv_status scratch_device_ptr(char** out) {
    static std::mutex mu;
    static std::vector<void*> cache;
    int dev = -1;
    const hipError_t ge = hipGetDevice(&dev);
    if (ge != hipSuccess || dev < 0)
        return fail(PKV_ERR_HIP, "decode_step_noalloc: hipGetDevice failed: %s",
                    hipGetErrorString(ge));
    std::lock_guard<std::mutex> lk(mu);
    if ((int)cache.size() <= dev) cache.resize(dev + 1, nullptr);
    if (cache[dev] == nullptr) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(PKV_ERR_HIP, "decode_step_noalloc: hipGetSymbolAddress failed: %s",
                        hipGetErrorString(e));
        cache[dev] = ptr;
    }
    *out = static_cast<char*>(cache[dev]);
    return PKV_OK;
}

// The decode step with the caller's workspace (noalloc false) or with the library's scratch
// array (noalloc true: balanced schedule only, counters cleared by a fill kernel first, pieces
// for as many workgroups as the array holds).
pkv_status decode_step_impl(const float* q_in, const float* k_in, const float* v_in,
                            float* q_out, void* k_pool, void* v_pool,
                            const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* positions, const float* q_norm_w,
                            const float* k_norm_w, float rms_eps, float rope_theta, float scale,
                            float* out, void* workspace, size_t workspace_bytes, int B,
                            int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                            int64_t num_blocks, pkv_dtype dtype, const pkv_variant* variant,
                            void* stream, bool noalloc) {
    const char* who = noalloc ? "decode_step_noalloc" : "decode_step";
    pkv_status st = check_common(who, B, num_q_heads, num_kv_heads, head_dim,
                                 block_size, num_blocks, max_blocks_per_seq, dtype);
    if (st != PKV_OK) return st;
    st = check_rope(who, rope_theta, q_norm_w, k_norm_w, head_dim);
    if (st != PKV_OK) return st;
    Variant var;
    st = resolve_variant(who, variant, head_dim, var);
    if (st != PKV_OK) return st;
    if (var.rope_read || dtype == PKV_F32)
        return fail(PKV_ERR_UNSUPPORTED,
                    "%s: rope_on_read and float32 pools are served by pkv_kv_append + "
                    "pkv_paged_attn_decode", who);
    st = check_decode_shape(who, B, num_q_heads, num_kv_heads, head_dim);
    if (st != PKV_OK) return st;
    if (B == 0) return PKV_OK;
    if (!q_in || !k_in || !v_in || !q_out || !k_pool || !v_pool || !block_tables || !positions ||
        !out)
        return fail(PKV_ERR_INVALID_ARG, "%s: NULL pointer argument", who);
    if (q_out == q_in)
        return fail(PKV_ERR_INVALID_ARG,
                    "%s: q_out must not alias q_in (workgroups of one sequence read "
                    "q_in while another writes q_out)", who);
    const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
    const int max_ctx = (int)std::min<int64_t>(cap, 0x7FFFFFFF);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bal = balanced_ok(B, num_kv_heads, max_ctx);
    const int P = bal ? 0 : choose_split(B, num_kv_heads, max_ctx, block_size, device_cus());
    WorkspaceLayout wl;
    int max_grid = 0;
    if (noalloc) {
        if (!bal)
            return fail(PKV_ERR_UNSUPPORTED,
                        "decode_step_noalloc: %d sequences (max_blocks_per_seq %d): only batches "
                        "of at most %d sequences run without a workspace; use pkv_decode_step",
                        B, max_blocks_per_seq, pkv::kMaxBalancedBatch);
        // counters, then the pieces of as many workgroups as the array holds (at most the
        // balanced schedule's cap; at least one per compute unit)
        const int G = num_q_heads / num_kv_heads;
        const size_t cnt = align256((size_t)B * num_kv_heads * sizeof(int));
        const size_t per_wg = (size_t)2 * G * head_dim * sizeof(float) + (size_t)2 * G * 2 * sizeof(float);
        const size_t room = cnt + 512 < kScratchBytes ? kScratchBytes - cnt - 512 : 0;
        max_grid = (int)std::min<size_t>(room / per_wg, (size_t)pkv::kMaxBalancedGrid);
        const int cus = device_cus();
        if (max_grid < cus)
            return fail(PKV_ERR_WORKSPACE,
                        "decode_step_noalloc: B=%d, Hkv=%d, G=%d, head_dim=%d needs more than the "
                        "library's %zu-byte scratch (counters %zu bytes, pieces for %d workgroups); "
                        "use pkv_decode_step with a workspace",
                        B, num_kv_heads, G, head_dim, kScratchBytes, cnt, cus);
        wl.balanced = true;
        wl.S = 1;
        wl.cnt_off = 0;
        wl.acc_off = cnt;
        wl.ml_off = wl.acc_off + align256((size_t)max_grid * 2 * G * head_dim * sizeof(float));
        wl.total = wl.ml_off + align256((size_t)max_grid * 2 * G * 2 * sizeof(float));
        char* base = nullptr;
        st = scratch_device_ptr(&base);
        if (st != PKV_OK) return st;
        workspace = base;
        workspace_bytes = kScratchBytes;
        // the counters must start at zero: a fill kernel (not a memset) on the call's stream
        const int n_cnt = B * num_kv_heads;
        hipLaunchKernelGGL(zero_ints_kernel, dim3((unsigned)((n_cnt + 255) / 256)), dim3(256), 0,
                           s, reinterpret_cast<int*>(base + wl.cnt_off), n_cnt);
        const hipError_t ze = hipGetLastError();
        if (ze != hipSuccess)
            return fail(PKV_ERR_HIP, "decode_step_noalloc: launch failed: %s",
                        hipGetErrorString(ze));
    } else {
        wl = layout_for(B, num_q_heads, num_kv_heads, head_dim, max_ctx, P, block_size, bal);
        if (wl.total > 0 && (workspace == nullptr || workspace_bytes < wl.total))
            return fail(PKV_ERR_WORKSPACE, "decode_step: workspace %zu bytes, need %zu",
                        workspace_bytes, wl.total);
    }
    if (!bal) {
        // batches too large for the balanced schedule: the append kernel, then the partitioned
        // decode reading positions + 1 as the attended lengths
        st = pkv_kv_append(q_in, k_in, v_in, q_out, k_pool, v_pool, block_tables,
                           max_blocks_per_seq, positions, q_norm_w, k_norm_w, rms_eps, rope_theta,
                           B, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype,
                           variant, stream);
        if (st != PKV_OK) return st;
        return run_decode(q_out, k_pool, v_pool, block_tables, max_blocks_per_seq, positions,
                          max_ctx, scale, out, workspace, wl, P, B, num_q_heads, num_kv_heads,
                          head_dim, block_size, num_blocks, dtype, var.window, s, true);
    }
    char* ws = static_cast<char*>(workspace);
    pkv::BalancedArgs a{};
    a.q = q_in;
    a.k_in = k_in;
    a.v_in = v_in;
    a.q_out = q_out;
    a.k_pool = static_cast<uint16_t*>(k_pool);
    a.v_pool = static_cast<uint16_t*>(v_pool);
    a.tables = block_tables;
    a.lens = positions;
    a.q_norm_w = q_norm_w;
    a.k_norm_w = k_norm_w;
    a.out = out;
    a.part_acc = reinterpret_cast<float*>(ws + wl.acc_off);
    a.part_ml = reinterpret_cast<float*>(ws + wl.ml_off);
    a.counters = reinterpret_cast<int*>(ws + wl.cnt_off);
    a.max_blocks = max_blocks_per_seq;
    a.max_context_len = max_ctx;
    a.scale = scale;
    a.eps = rms_eps;
    a.theta = rope_theta;
    a.B = B;
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.D = head_dim;
    a.bs = block_size;
    a.num_blocks = num_blocks;
    a.num_cus = device_cus();
    a.max_grid = max_grid;
    a.rope_dim = var.rope_dim;
    a.v_norm = var.v_norm;
    a.window = var.window;
    a.bf16 = dtype == PKV_BF16;
    a.append = true;
#ifdef PKV_TIMELINE
    a.timeline = pkv::timeline_buffer();
    a.timeline_rot = pkv::timeline_rotation();
#endif
    const hipError_t e = pkv::launch_decode_balanced(a, s);
    if (e != hipSuccess)
        return fail(PKV_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_decode_step(const float* q_in, const float* k_in, const float* v_in, float* q_out,
                           void* k_pool, void* v_pool, const int32_t* block_tables,
                           int max_blocks_per_seq, const int32_t* positions,
                           const float* q_norm_w, const float* k_norm_w, float rms_eps,
                           float rope_theta, float scale, float* out, void* workspace,
                           size_t workspace_bytes, int B, int num_q_heads, int num_kv_heads,
                           int head_dim, int block_size, int64_t num_blocks, pkv_dtype dtype,
                           const pkv_variant* variant, void* stream) {
    return decode_step_impl(q_in, k_in, v_in, q_out, k_pool, v_pool, block_tables,
                            max_blocks_per_seq, positions, q_norm_w, k_norm_w, rms_eps,
                            rope_theta, scale, out, workspace, workspace_bytes, B, num_q_heads,
                            num_kv_heads, head_dim, block_size, num_blocks, dtype, variant, stream,
                            false);
}

pkv_status pkv_decode_step_noalloc(const float* q_in, const float* k_in, const float* v_in,
                                   float* q_out, void* k_pool, void* v_pool,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* positions, const float* q_norm_w,
                                   const float* k_norm_w, float rms_eps, float rope_theta,
                                   float scale, float* out, int B, int num_q_heads,
                                   int num_kv_heads, int head_dim, int block_size,
                                   int64_t num_blocks, pkv_dtype dtype,
                                   const pkv_variant* variant, void* stream) {
    return decode_step_impl(q_in, k_in, v_in, q_out, k_pool, v_pool, block_tables,
                            max_blocks_per_seq, positions, q_norm_w, k_norm_w, rms_eps,
                            rope_theta, scale, out, nullptr, 0, B, num_q_heads, num_kv_heads,
                            head_dim, block_size, num_blocks, dtype, variant, stream, true);
}

size_t pkv_decode_step_noalloc_scratch_bytes(void) { return kScratchBytes; }

pkv_status pkv_prefill_append(const float* q_in, const float* k_in, const float* v_in,
                              float* q_out, void* k_pool, void* v_pool,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* cu_seqlens, const int32_t* start_pos,
                              const float* q_norm_w, const float* k_norm_w, float rms_eps,
                              float rope_theta, int B, int num_tokens, int num_q_heads,
                              int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                              pkv_dtype dtype, const pkv_variant* variant, void* stream) {
    pkv_status st = check_common("prefill_append", B, num_q_heads, num_kv_heads, head_dim,
                                 block_size, num_blocks, max_blocks_per_seq, dtype);
    if (st != PKV_OK) return st;
    st = check_rope("prefill_append", rope_theta, q_norm_w, k_norm_w, head_dim);
    if (st != PKV_OK) return st;
    Variant var;
    st = resolve_variant("prefill_append", variant, head_dim, var);
    if (st != PKV_OK) return st;
    if (num_tokens < 0)
        return fail(PKV_ERR_INVALID_ARG, "prefill_append: num_tokens = %d < 0", num_tokens);
    if (B == 0 || num_tokens == 0) return PKV_OK;
    if (!q_in || !k_in || !v_in || !q_out || !k_pool || !v_pool || !block_tables ||
        !cu_seqlens || !start_pos)
        return fail(PKV_ERR_INVALID_ARG, "prefill_append: NULL pointer argument");
    pkv::AppendArgs a;
    a.q_in = q_in;
    a.k_in = k_in;
    a.v_in = v_in;
    a.q_out = q_out;
    a.k_pool = static_cast<uint16_t*>(k_pool);
    a.v_pool = static_cast<uint16_t*>(v_pool);
    a.tables = block_tables;
    a.positions = start_pos;
    a.cu_seqlens = cu_seqlens;
    a.rows = num_tokens;
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
    a.rope_dim = var.rope_read ? 0 : var.rope_dim;  // rotation at read: the pool keeps un-rotated K
    a.v_norm = var.v_norm;
    a.bf16 = dtype == PKV_BF16;
    a.f32 = dtype == PKV_F32;
    const hipError_t e = pkv::launch_kv_append(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(PKV_ERR_HIP, "prefill_append: launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

size_t pkv_prefill_workspace_bytes(int B, int num_q_heads, int num_kv_heads, int head_dim,
                                   int block_size, int max_chunk, int max_context_len) {
    if (B <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_chunk <= 0 || max_context_len <= 0 || num_q_heads % num_kv_heads)
        return 0;
    return prefill_plan(B, num_q_heads, num_kv_heads, head_dim, block_size, max_chunk,
                        max_context_len, device_cus())
        .total;
}

pkv_status pkv_paged_attn_prefill(const float* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, int max_blocks_per_seq,
                                  const int32_t* cu_seqlens, const int32_t* start_pos,
                                  int max_chunk, int max_context_len, float scale, float* out,
                                  void* workspace, size_t workspace_bytes, int B, int num_tokens,
                                  int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                  int64_t num_blocks, pkv_dtype dtype,
                                  const pkv_variant* variant, void* stream) {
    pkv_status st = check_common("prefill", B, num_q_heads, num_kv_heads, head_dim, block_size,
                                 num_blocks, max_blocks_per_seq, dtype);
    if (st != PKV_OK) return st;
    Variant var;
    st = resolve_variant("prefill", variant, head_dim, var);
    if (st != PKV_OK) return st;
    if (var.rope_read || dtype == PKV_F32)
        return fail(PKV_ERR_UNSUPPORTED,
                    "prefill: rope_on_read and float32 pools are not built for chunked prefill");
    st = check_decode_shape("prefill", B, num_q_heads, num_kv_heads, head_dim);
    if (st != PKV_OK) return st;
    if (num_tokens < 0 || max_chunk < 0 || max_context_len < 0)
        return fail(PKV_ERR_INVALID_ARG,
                    "prefill: num_tokens=%d, max_chunk=%d, max_context_len=%d must be >= 0",
                    num_tokens, max_chunk, max_context_len);
    if (B == 0 || num_tokens == 0 || max_chunk == 0 || max_context_len == 0) return PKV_OK;
    if (!q || !k_pool || !v_pool || !block_tables || !cu_seqlens || !start_pos || !out)
        return fail(PKV_ERR_INVALID_ARG, "prefill: NULL pointer argument");
    const PrefillPlan plan = prefill_plan(B, num_q_heads, num_kv_heads, head_dim, block_size,
                                          max_chunk, max_context_len, device_cus());
    if ((int64_t)B * plan.QTmax > kMaxGridDim || (int64_t)plan.S > kMaxGridDim)
        return fail(PKV_ERR_UNSUPPORTED, "prefill: %d sequences of up to %d tokens: grid too large",
                    B, max_chunk);
    if (plan.total > 0 && (workspace == nullptr || workspace_bytes < plan.total))
        return fail(PKV_ERR_WORKSPACE, "prefill: workspace %zu bytes, need %zu", workspace_bytes,
                    plan.total);
    char* ws = static_cast<char*>(workspace);
    pkv::PrefillArgs a{};
    a.q = q;
    a.k_pool = static_cast<const uint16_t*>(k_pool);
    a.v_pool = static_cast<const uint16_t*>(v_pool);
    a.tables = block_tables;
    a.cu_seqlens = cu_seqlens;
    a.start_pos = start_pos;
    a.out = out;
    a.part_acc = plan.total ? reinterpret_cast<float*>(ws + plan.acc_off) : nullptr;
    a.part_ml = plan.total ? reinterpret_cast<float*>(ws + plan.ml_off) : nullptr;
    a.counters = plan.total ? reinterpret_cast<int*>(ws + plan.cnt_off) : nullptr;
    a.max_blocks = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.scale = scale;
    a.split_tokens = plan.P;
    a.S = plan.S;
    a.QTmax = plan.QTmax;
    a.B = B;
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.D = head_dim;
    a.bs = block_size;
    a.num_blocks = num_blocks;
    a.window = var.window;
    a.bf16 = dtype == PKV_BF16;
    a.shared_tiles = plan.shared;
    a.balanced = plan.balanced;
    a.max_grid = plan.max_grid;
    a.num_cus = device_cus();
    const hipError_t e = pkv::launch_prefill_attn(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(PKV_ERR_HIP, "prefill: launch failed: %s", hipGetErrorString(e));
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
