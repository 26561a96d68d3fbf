/*
 * pkv.h — C ABI of the paged-KV decode step on AMD Instinct MI355X (gfx950).
 *
 * One decoder layer's decode step over a paged KV cache is two calls on one HIP stream:
 *
 *   pkv_kv_append          new token of every sequence: optional per-head QK-RMSNorm, RoPE,
 *                          f32 -> fp16/bf16 round-to-nearest-even, scatter of its K and V rows
 *                          into the block pools;
 *   pkv_paged_attn_decode  softmax(scale * q . K^T) . V over each sequence's block list, with
 *                          grouped-query heads sharing one KV head, split over the token axis
 *                          and merged.
 *
 * Sources (web pages, by title and section):
 *   makarna/pkg/model/arch/hybrid_decoder.go — runHybridAttentionBlock (QK-norm before RoPE,
 *     scale = 1/sqrt(HeadDim), fused-RoPE limits: even HeadDim <= 256) and
 *     runHybridAttentionBlockBatch (one query row per sequence, per-sequence block lists,
 *     the attended length is the cached length plus one, the query position is the cached
 *     length, and the longest length is passed for grid sizing).
 *   makarna/pkg/kvcache/paged_cache.go — float32ToFloat16Bits / float32ToBFloat16Bits (stored
 *     bits), GetBlockForPosition / GetBlockOffset (block = list[pos / BlockSize],
 *     slot = pos % BlockSize), Append (a token's row of kvDim = kv_heads * head_dim elements at
 *     offset slot * kvDim inside its block; K and V in separate tensors), viewsLockedAt (only
 *     the first kvLen tokens are valid).
 *   soft3/glia/run/arch/decoder/forward.rs — forward_layer: per-head QK-norm, RoPE over the
 *     full head_dim, CPU attention (kv head = h / (Hq / Hkv), max-subtracted softmax).
 *
 * Conventions shared by every call:
 *   - Pointers marked (device) are HIP device pointers owned by the caller; the library never
 *     allocates, frees or synchronises. Work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream) and the call returns as soon as it is enqueued.
 *   - Pools: k_pool and v_pool are two arrays of 16-bit codes (or float32 values, PKV_F32)
 *     shaped [num_blocks, block_size, num_kv_heads, head_dim], row-major: element (blk, slot, g, d)
 *     is at ((blk * block_size + slot) * num_kv_heads + g) * head_dim + d. Offsets are 64-bit.
 *   - block_tables: int32 [B, max_blocks_per_seq], row-major; row b lists the physical block
 *     ids of sequence b in logical order. Entries past a sequence's length are never read.
 *   - Device-array CONTENTS are preconditions, not checked on the hot path (checking needs a
 *     synchronisation): block ids in [0, num_blocks), positions[b] in
 *     [0, max_blocks_per_seq * block_size), context_lens[b] in [1, max_context_len], and no
 *     two sequences appending into the same (block, slot). Kernels clamp every index into its
 *     array, so a violated precondition gives wrong values, never an out-of-bounds access.
 *     pkv_validate_tables checks the contents on host copies.
 *   - Non-finite data is not an error: NaN and Inf propagate through the arithmetic.
 *   - Every call returns a pkv_status; on failure nothing was enqueued and pkv_last_error()
 *     returns a description (thread-local, valid until the thread's next failing call).
 *   - The functions are stateless and thread-safe.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, Hq % Hkv != 0, theta <= 0 ... */
    PKV_ERR_UNSUPPORTED = 2, /* shape the kernels are not built for (see each call) */
    PKV_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than pkv_decode_workspace_bytes */
    PKV_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} pkv_status;

typedef enum {
    PKV_F16 = 1,  /* IEEE binary16 */
    PKV_BF16 = 2, /* bfloat16 */
    PKV_F32 = 3   /* float32 elements, stored unchanged (page "makarna/pkg/kvcache/paged_cache.go",
                     Append copies float32 rows as they are; page "makarna/pkg/model/arch/
                     hybrid_decoder.go" sends float32 KV to its plain paged kernel). Taken by
                     pkv_kv_append, pkv_prefill_append and pkv_paged_attn_decode (which then runs
                     the kernels of the rotation-at-read path, rotating only with
                     rope_on_read); pkv_decode_step and pkv_paged_attn_prefill return
                     UNSUPPORTED for it. */
} pkv_dtype;

/*
 * pkv_variant — layer options of the glia decoder family (page
 * "soft3/glia/run/arch/decoder/forward.rs", forward_layer) and makarna's RoPE-in-attention
 * kernels (page "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlock), taken by
 * the append, decode and prefill calls. Passing NULL is the same as all fields zero: full
 * rotary applied by the append, no V normalisation, no window (the Llama-style layer every call
 * describes below).
 *
 * rope_dim  rotary dimension: 0 means head_dim; otherwise an even number in [2, head_dim].
 *           The pairs (i, i + rope_dim/2), i < rope_dim/2, are rotated by the angle
 *           p * rope_theta^(-2i/rope_dim) (partial rotary: a rope_dim-sized head inside the
 *           first rope_dim dims); dims rope_dim .. head_dim-1 pass through (after the optional
 *           QK-norm) unrotated. Used by the append calls (and pkv_decode_step), and by
 *           pkv_paged_attn_decode when rope_on_read is set.
 * v_norm    non-zero: every new V head vector v is stored as v * (1 / sqrt(sum(v^2) / D +
 *           rms_eps)) with float arithmetic: the sum of squares accumulated in index order, one
 *           rounding per operation (no fused multiply-add), no weight. Used by the append calls.
 * window    0 for full attention, else W > 0: a query at position p (attended length L = p + 1)
 *           sees the positions max(0, L - W) .. L - 1 only — the last W tokens, the range the
 *           page's ring cache of W slots reads (here the pool keeps every token; only the
 *           attended range shrinks). Used by the attention calls (and pkv_decode_step).
 * rope_on_read  non-zero: RoPE moves from the append to the attention, as in makarna's fused
 *           RoPE paged kernels. The append calls then rotate nothing (q_out is the normed query,
 *           the pool keeps normed, un-rotated keys); pkv_paged_attn_decode rotates the query to
 *           position L - 1 and key t to position t (the pairing and angles above, base
 *           read_theta) before the dot products, in float with cos / sin evaluated in double.
 *           Needs rope_dim (after the default) a multiple of 16 for the decode (UNSUPPORTED
 *           otherwise); pkv_decode_step and pkv_paged_attn_prefill return UNSUPPORTED with it.
 *           Keys holding +-Inf are outside what the rotated-at-read decode reproduces.
 * read_theta  RoPE base of the rotation at read (finite, > 0); used by pkv_paged_attn_decode
 *           when rope_on_read is set (the append calls take rope_theta as an argument).
 * A NaN that the norm, V-norm or RoPE arithmetic produces is stored as 0x7FC00000 (the
 * canonical quiet NaN) before conversion; a NaN that reaches the converter untouched keeps its
 * bits as described under pkv_kv_append.
 * Errors (INVALID_ARG): rope_dim odd, negative or above head_dim; window < 0; read_theta not
 * finite and > 0 when the decode rotates at read.
 */
typedef struct {
    int rope_dim;
    int v_norm;
    int window;
    int rope_on_read;
    float read_theta;
} pkv_variant;

/*
 * pkv_kv_append — write the new token of each of B sequences into the cache.
 *
 * For each sequence b, with p = positions[b] (the number of tokens already cached, which is
 * both the write slot and the RoPE position, as in the makarna batch path):
 *   1. if q_norm_w and k_norm_w are given: every head vector x of q and of k becomes
 *      x / sqrt(mean(x^2) + rms_eps) * w (w = q_norm_w for q heads, k_norm_w for k heads);
 *   2. RoPE: for i < D/2 the pair (x[i], x[i + D/2]) is rotated by the angle
 *      p * rope_theta^(-2i/D); the angle, cos, sin and the rotation are evaluated in double
 *      and each result is rounded once to float;
 *   3. q_out[b] = the rotated q (float);
 *   4. the rotated k and the input v are converted to 16-bit codes (round to nearest, ties to
 *      even, overflow to infinity; a NaN keeps its sign and leading payload bits, forced
 *      non-zero) and stored at block block_tables[b][p / block_size], slot p % block_size,
 *      for every KV head. No other pool element is written.
 *
 * q_in   (device) float [B, num_q_heads, head_dim]
 * k_in   (device) float [B, num_kv_heads, head_dim]
 * v_in   (device) float [B, num_kv_heads, head_dim]
 * q_out  (device) float [B, num_q_heads, head_dim]; may equal q_in (updated in place)
 * k_pool, v_pool (device) 16-bit codes, layout above; written at one row per sequence
 * block_tables (device) int32 [B, max_blocks_per_seq]
 * positions    (device) int32 [B]
 * q_norm_w, k_norm_w (device) float [head_dim] each, or both NULL for no QK-norm
 * rms_eps      used only with the norm weights
 * rope_theta   RoPE base, > 0
 * variant      (host) NULL, or rope_dim / v_norm as described under pkv_variant (window is not
 *              used here)
 * Errors: INVALID_ARG for a NULL required pointer, B < 0, a non-positive size, Hq % Hkv != 0,
 *   rope_theta <= 0 or not finite, exactly one norm weight NULL, an unknown dtype, an invalid
 *   variant;
 *   UNSUPPORTED for an odd head_dim or head_dim > 256 (the limits of the fused RoPE path).
 *   B == 0 is a no-op.
 */
pkv_status pkv_kv_append(const float* q_in, const float* k_in, const float* v_in, float* q_out,
                         void* k_pool, void* v_pool, const int32_t* block_tables,
                         int max_blocks_per_seq, const int32_t* positions, const float* q_norm_w,
                         const float* k_norm_w, float rms_eps, float rope_theta, int B,
                         int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                         int64_t num_blocks, pkv_dtype dtype, const pkv_variant* variant,
                         void* stream);

/*
 * pkv_paged_attn_decode — one query token per sequence against its paged K/V.
 *
 * For each sequence b with L = context_lens[b] tokens and each query head h (KV head
 * g = h / (num_q_heads / num_kv_heads)):
 *   s_t = scale * (q[b][h] . K[t][g]) for t < L, where token t of sequence b lives in block
 *         block_tables[b][t / block_size] at slot t % block_size;
 *   out[b][h] = sum_t exp(s_t - max s) V[t][g] / sum_t exp(s_t - max s).
 * Arithmetic is float (fp16/bf16 codes decode exactly; q . k runs on the matrix cores with q
 * split into a 16-bit high part and a 16-bit remainder, accurate to about 2^-16 relative);
 * each piece of the token axis keeps a running max / sum / weighted V (online softmax), and the
 * last piece of each (sequence, KV head) to finish merges the pieces with their max-rescaled
 * weights. With split_tokens == 0 (and B <= 2048) the pieces come from a balanced schedule:
 * the K/V tiles of the whole batch are cut into equal contiguous ranges, one per resident
 * workgroup. With split_tokens > 0 every sequence is cut into partitions of split_tokens
 * tokens, one workgroup each.
 *
 * q            (device) float [B, num_q_heads, head_dim] (q_out of pkv_kv_append)
 * k_pool, v_pool (device) 16-bit codes, layout above; read only
 * block_tables (device) int32 [B, max_blocks_per_seq]
 * context_lens (device) int32 [B]; tokens attended (= positions + 1 after an append)
 * max_context_len  host int >= every context_lens[b]; sizes the grid (tokens beyond it are
 *                  not attended)
 * scale        host float; the pages pass 1/sqrt(head_dim)
 * out          (device) float [B, num_q_heads, head_dim]
 * workspace    (device) scratch of at least pkv_decode_workspace_bytes(...) bytes, or NULL when
 *              that size is 0. It must be ZERO-FILLED before its first use: its last
 *              B * num_kv_heads ints count finished partitions, and every call leaves them zero
 *              again (the rest needs no initialisation). Calls that run concurrently (on
 *              different streams) need separate workspaces.
 * split_tokens 0 for the balanced schedule, or tokens per partition: a positive multiple of
 *              64 of at most 1022 * block_size (a partition stages its block ids in LDS).
 *              With rope_on_read (variant) or float32 pools: head_dim 64 or 128 with the
 *              rotated dims (rope_dim, when rotating at read) a multiple of 64 and at least 3
 *              query heads per KV head (2 for float32 pools without rotation) run a float32
 *              matrix-core kernel on the same schedules and workspace as 16-bit pools when
 *              split_tokens is 0; other shapes, and every positive split_tokens, run the
 *              partitioned vector-ALU kernel, where 0 means the smaller of
 *              pkv_decode_split_tokens(...)'s choice and 576 (size the workspace with that
 *              value).
 *              Either way split_tokens is at most 4096 (the rotation is carried across a
 *              partition in float steps).
 * variant      (host) NULL, or a window as described under pkv_variant: then only the keys
 *              max(0, L - window) .. L - 1 are attended (the partitions and tiles start at the
 *              16-token tile that holds the first of them; the rest of the context is not read)
 * Errors: INVALID_ARG as for pkv_kv_append, plus max_context_len < 0, split_tokens not 0 or a
 *   positive multiple of 64 up to 1022 * block_size; UNSUPPORTED for head_dim not in {32, 64, 128, 256} or a GQA group
 *   num_q_heads / num_kv_heads above 8; WORKSPACE when the workspace is too small.
 *   B == 0 or max_context_len == 0 is a no-op.
 */
pkv_status pkv_paged_attn_decode(const float* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, int max_blocks_per_seq,
                                 const int32_t* context_lens, int max_context_len, float scale,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 int split_tokens, int B, int num_q_heads, int num_kv_heads,
                                 int head_dim, int block_size, int64_t num_blocks,
                                 pkv_dtype dtype, const pkv_variant* variant, void* stream);

/*
 * pkv_decode_step — pkv_kv_append followed by pkv_paged_attn_decode, in one kernel launch.
 *
 * For each sequence b with p = positions[b]: the new token is appended exactly as
 * pkv_kv_append does (stored bits identical), q_out[b] receives the rotated query, and
 * out[b] = attention of q_out[b] over the L = p + 1 tokens now in the cache, exactly as
 * pkv_paged_attn_decode with context_lens[b] = p + 1 computes it.
 *
 * Schedule: the K/V tiles of the whole batch are cut into equal contiguous ranges, one per
 * resident workgroup; each workgroup rotates the query heads it needs itself, and the one that
 * holds a sequence's last tile writes that KV head's new row before streaming it. Batches above
 * 2048 sequences run the append kernel and the partitioned decode instead.
 *
 * Arguments as for pkv_kv_append and pkv_paged_attn_decode (variant: all three fields apply);
 * q_out must not alias q_in.
 * workspace: at least pkv_decode_step_workspace_bytes(...) bytes, zero-filled before first use
 * (counters the call leaves zero again). A sequence whose position is outside
 * [0, max_blocks_per_seq * block_size) is skipped (its q_out and out rows are not written).
 * Errors: the union of those of pkv_kv_append and pkv_paged_attn_decode; INVALID_ARG when
 * q_out == q_in.
 */
pkv_status pkv_decode_step(const float* q_in, const float* k_in, const float* v_in, float* q_out,
                           void* k_pool, void* v_pool, const int32_t* block_tables,
                           int max_blocks_per_seq, const int32_t* positions,
                           const float* q_norm_w, const float* k_norm_w, float rms_eps,
                           float rope_theta, float scale, float* out, void* workspace,
                           size_t workspace_bytes, int B, int num_q_heads, int num_kv_heads,
                           int head_dim, int block_size, int64_t num_blocks, pkv_dtype dtype,
                           const pkv_variant* variant, void* stream);

/*
 * pkv_decode_step_noalloc — pkv_decode_step without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). It allocates and frees nothing, and calls no allocating routine.
 *
 * The merge counters and partial pieces live in a 16 MiB array the library holds on each GPU
 * it runs on, from the first call on that GPU until the process ends
 * (pkv_decode_step_noalloc_scratch_bytes()). The first call on a GPU looks up the array's
 * device address (hipGetSymbolAddress) with that GPU current; every call clears the counters
 * with a small fill kernel on `stream` before the step's kernel. Every call on one GPU uses the
 * same array, so calls that overlap in time on one GPU (different streams or threads) race and
 * give wrong results; calls in one stream are ordered and safe.
 *
 * Arguments and results: as pkv_decode_step, without workspace / workspace_bytes.
 * Limits: batches of at most 2048 sequences (UNSUPPORTED otherwise: pkv_decode_step's
 * workspace path serves them); the counters (B * num_kv_heads ints) plus the pieces of at least
 * one workgroup per compute unit (2 * G * (head_dim + 2) floats each) must fit in the array
 * (WORKSPACE otherwise, e.g. B = 2048 with num_kv_heads above ~2000). Other errors as
 * pkv_decode_step; PKV_ERR_HIP if the array's address cannot be found.
 */
pkv_status pkv_decode_step_noalloc(const float* q_in, const float* k_in, const float* v_in,
                                   float* q_out, void* k_pool, void* v_pool,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* positions, const float* q_norm_w,
                                   const float* k_norm_w, float rms_eps, float rope_theta,
                                   float scale, float* out, int B, int num_q_heads,
                                   int num_kv_heads, int head_dim, int block_size,
                                   int64_t num_blocks, pkv_dtype dtype,
                                   const pkv_variant* variant, void* stream);

/* Bytes of the per-GPU array pkv_decode_step_noalloc works in (16 MiB). Host only. */
size_t pkv_decode_step_noalloc_scratch_bytes(void);

/* Workspace bytes pkv_decode_step needs. Host only. */
size_t pkv_decode_step_workspace_bytes(int B, int num_q_heads, int num_kv_heads, int head_dim,
                                       int block_size, int max_blocks_per_seq);

/* Tokens per partition of the partitioned schedule when pkv_paged_attn_decode has to choose
 * one itself (split_tokens == 0 with more than 2048 sequences). Host only; depends on the shape
 * and on the current device's compute-unit count. Returns 0 on invalid arguments. */
int pkv_decode_split_tokens(int B, int num_q_heads, int num_kv_heads, int head_dim,
                            int block_size, int max_context_len);

/* Workspace bytes pkv_paged_attn_decode needs for these arguments (split_tokens as passed to
 * it). Layout: B * num_kv_heads int counters (rounded up to 256 bytes), then the partial
 * results: for the balanced schedule 4096 pieces of G * (head_dim + 2) floats
 * (G = num_q_heads / num_kv_heads); for the partitioned one B * num_q_heads * S * (head_dim + 2)
 * floats with S = ceil(max_context_len / split_tokens), or nothing at all when S <= 1. Each
 * part is rounded up to 256 bytes. Host only. */
size_t pkv_decode_workspace_bytes(int B, int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int max_context_len, int split_tokens);

/*
 * pkv_prefill_append — append a chunk of new tokens per sequence (prefill, or several tokens
 * at a time).
 *
 * Page "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlock: a block of seqLen
 * tokens (token-major q [seqLen, Hq*D], k / v [seqLen, Hkv*D]) goes into the cache at its
 * current length startPos, token i at position startPos + i, RoPE at each token's own position;
 * page "makarna/pkg/kvcache/paged_cache.go", Append: the rows fill the block list from there on.
 * Token rows of sequence b are cu_seqlens[b] .. cu_seqlens[b+1]-1; token i of them is treated
 * exactly as pkv_kv_append treats sequence b's new token at position start_pos[b] + i (same
 * norm, RoPE, codes and pool row); with one token per sequence the two calls store identical bits.
 *
 * q_in, q_out (device) float [num_tokens, num_q_heads, head_dim]; q_out may equal q_in
 * k_in, v_in   (device) float [num_tokens, num_kv_heads, head_dim]
 * cu_seqlens   (device) int32 [B + 1], non-decreasing, cu_seqlens[0] = 0,
 *              cu_seqlens[B] = num_tokens
 * start_pos    (device) int32 [B]: tokens already cached = position of the chunk's first token
 * Other arguments (variant: rope_dim, v_norm) as for pkv_kv_append. A token whose position or
 * block id is out of range is not stored (its q_out row is still written). Chunks of different
 * sequences must not share a pool slot. Errors: as pkv_kv_append, plus num_tokens < 0. B == 0
 * or num_tokens == 0 is a no-op.
 */
pkv_status pkv_prefill_append(const float* q_in, const float* k_in, const float* v_in,
                              float* q_out, void* k_pool, void* v_pool,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* cu_seqlens, const int32_t* start_pos,
                              const float* q_norm_w, const float* k_norm_w, float rms_eps,
                              float rope_theta, int B, int num_tokens, int num_q_heads,
                              int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                              pkv_dtype dtype, const pkv_variant* variant, void* stream);

/*
 * pkv_paged_attn_prefill — causal paged attention of a chunk of query tokens per sequence.
 *
 * Page "makarna/pkg/model/arch/hybrid_decoder.go", runHybridAttentionBlock: after a block of
 * tokens is appended at startPos the attention covers startPos + seqLen tokens and is causal
 * from startPos. Query row r = token i of sequence b (rows as in pkv_prefill_append), at
 * position p = start_pos[b] + i, attends the first p + 1 tokens of sequence b's block list:
 * out[r][h] is what pkv_paged_attn_decode computes for that row with context length p + 1.
 * q . k and P . V run on the matrix cores with the query and the weights split into a 16-bit
 * high part and a 16-bit remainder (about 2^-16 relative); a key tile holding an Inf or NaN
 * value is multiplied out in float instead.
 *
 * q, out       (device) float [num_tokens, num_q_heads, head_dim] (q rotated: pkv_prefill_append)
 * cu_seqlens, start_pos  (device) as for pkv_prefill_append
 * max_chunk    host int >= every chunk length (sizes the grid)
 * max_context_len  host int >= every start_pos[b] + chunk length (keys beyond it are not
 *              attended)
 * workspace    (device) at least pkv_prefill_workspace_bytes(...) bytes (NULL when that is 0),
 *              ZERO-FILLED before its first use: its first ints are counters every call leaves
 *              zero. Concurrent calls need separate workspaces.
 * With a window W (variant) the row at position p attends max(0, p + 1 - W) .. p only.
 * Other arguments as for pkv_paged_attn_decode. Errors: as pkv_paged_attn_decode, plus
 *   num_tokens, max_chunk or max_context_len < 0; UNSUPPORTED when B * ceil(max_chunk / (16 /
 *   G)) exceeds 65535. A zero size is a no-op.
 */
pkv_status pkv_paged_attn_prefill(const float* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, int max_blocks_per_seq,
                                  const int32_t* cu_seqlens, const int32_t* start_pos,
                                  int max_chunk, int max_context_len, float scale, float* out,
                                  void* workspace, size_t workspace_bytes, int B, int num_tokens,
                                  int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                  int64_t num_blocks, pkv_dtype dtype, const pkv_variant* variant,
                                  void* stream);

/* Workspace bytes pkv_paged_attn_prefill needs: 0 when one partition covers every query
 * tile's keys, otherwise counters and partial results of the partitions. Host only; depends on
 * the current device's compute-unit count. */
size_t pkv_prefill_workspace_bytes(int B, int num_q_heads, int num_kv_heads, int head_dim,
                                   int block_size, int max_chunk, int max_context_len);

/* Debug check of the device-array preconditions on HOST copies of the arrays (any may be
 * NULL to skip it): every block id a sequence uses is in [0, num_blocks); positions[b] in
 * [0, max_blocks_per_seq * block_size); context_lens[b] in [1, max_context_len] and covered
 * by the table row; no two sequences append into the same (block, slot). Returns PKV_OK or
 * PKV_ERR_INVALID_ARG with the first violation in pkv_last_error(). */
pkv_status pkv_validate_tables(const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* positions, const int32_t* context_lens, int B,
                               int block_size, int64_t num_blocks, int max_context_len);

/* Static name of a status code. */
const char* pkv_status_string(pkv_status status);

/* Description of the calling thread's last failure ("" if none). */
const char* pkv_last_error(void);

/* Library version, "major.minor.patch". */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
