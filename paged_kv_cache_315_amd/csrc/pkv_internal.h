// Internal declarations shared by the HIP translation units of libpkv (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct AppendArgs {
    const float* q_in;      // [rows, Hq, D]
    const float* k_in;      // [rows, Hkv, D]
    const float* v_in;
    float* q_out;
    uint16_t* k_pool;
    uint16_t* v_pool;
    const int32_t* tables;
    // one token per sequence (cu_seqlens == nullptr): row b is sequence b at positions[b];
    // chunks: rows cu_seqlens[b] .. cu_seqlens[b+1]-1 are sequence b at positions[b] + i
    const int32_t* positions;
    const int32_t* cu_seqlens;
    int rows;
    const float* q_norm_w;  // nullptr: no QK-norm
    const float* k_norm_w;
    int max_blocks;
    float eps;
    float theta;
    int B, Hq, Hkv, D, bs;
    int64_t num_blocks;
    int rope_dim;           // rotated dims (even, <= D)
    bool v_norm;            // V rows normalised per KV head before they are stored
    bool bf16;
    bool f32;               // float32 pools: the values are stored as they are
};

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);

// Causal paged attention of chunks of query tokens (prefill_attn.hip).
struct PrefillArgs {
    const float* q;            // [N, Hq, D] rotated queries, token-major
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    const int32_t* tables;
    const int32_t* cu_seqlens;  // [B + 1]
    const int32_t* start_pos;   // [B]
    float* out;                 // [N, Hq, D]
    float* part_acc;            // [B * QTmax * Hkv, S, 16, D]
    float* part_ml;             // [B * QTmax * Hkv, S, 16, 2]
    int* counters;              // [B * QTmax * Hkv], zero between calls
    int max_blocks;
    int max_context_len;        // keys beyond it are not attended
    float scale;
    int split_tokens;           // keys per partition
    int S;                      // partitions per query tile
    int QTmax;                  // query tiles per sequence = ceil(max_chunk / QT)
    int B, Hq, Hkv, D, bs;
    int64_t num_blocks;
    int window;                 // sliding window (0: every token)
    bool bf16;
    bool shared_tiles;          // 4 query tiles per workgroup sharing each K/V tile (S == 1)
    bool balanced;              // one query tile per sequence on the balanced schedule: pieces
                                // [max_grid * 2, 16, D] / [max_grid * 2, 16, 2], counters [B, Hkv]
    int max_grid;               // balanced: workgroups (two piece slots each)
    int num_cus;                // balanced: compute units of the device
};

// Query tokens per tile (16 MFMA rows of G heads each).
int prefill_tile_tokens(int G);
hipError_t launch_prefill_attn(const PrefillArgs& a, hipStream_t stream);

struct DecodeArgs {
    const float* q;
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    const int32_t* tables;
    const int32_t* context_lens;
    float* out;
    float* part_acc;  // [B, Hq, S, D]
    float* part_ml;   // [B, Hq, S, 2]
    int* counters;    // [B, Hkv] finished partitions per (sequence, KV head); zero between calls
    int max_blocks;
    int max_context_len;
    float scale;
    int split_tokens;
    int S;            // partitions per sequence = ceil(max_context_len / split_tokens)
    int B, Hq, Hkv, D, bs;
    int64_t num_blocks;
    int window;               // sliding window (0: every token)
    bool bf16;
    bool lens_are_positions;  // context_lens holds positions: L = p + 1 (fused-step fallback)
    float rope_theta;         // decode_rope.hip only: RoPE base of the rotation at read
    int rope_dim;             // decode_rope.hip only: rotated dims, a multiple of 16 (0: none)
    bool f32;                 // decode_rope.hip only: float32 pools
};

// Launches the decode kernel (partitions + in-kernel merge by the last partition).
hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream);

// Decode over un-rotated keys, rotating query and keys at read (decode_rope.hip); the same
// partitions, workspace layout and merge as launch_paged_decode.
hipError_t launch_decode_rope(const DecodeArgs& a, hipStream_t stream);

// Shapes the float32 matrix-core tile of decode_rope_mfma.hip serves: head_dim 64 / 128, rotated
// dims at read a multiple of 64 (0: no rotation).
bool decode_rope_mfma_ok(int D, int G, int rope_dim);

// Balanced schedule (decode_balanced.hip): one resident workgroup per slot, equal tile ranges.
constexpr int kMaxBalancedBatch = 2048;  // sequences whose tile prefix fits in LDS
constexpr int kMaxBalancedGrid = 2048;   // workgroups; each owns two partial-piece slots
// What starting a unit costs a workgroup (staging its block ids and query, the rotation, the
// first tile's latency, the merge), in 16-token tiles: in the balanced tile list every segment
// is preceded by this many empty positions, so the ranges of workgroups that start more units
// hold fewer tiles. Measured on MI355X: a unit's start takes about 8 us and a 16-token tile of
// one KV head streams in about 0.58 us per workgroup, i.e. about 14 tiles.
#ifndef PKV_UNIT_COST
#define PKV_UNIT_COST 15
#endif
constexpr int kBalancedUnitCost = PKV_UNIT_COST;

struct BalancedArgs {
    const float* q;         // append: q_in (rotated in-kernel); decode: rotated q
    const float* k_in;      // append only
    const float* v_in;      // append only
    float* q_out;           // append only (must not alias q)
    uint16_t* k_pool;
    uint16_t* v_pool;
    const int32_t* tables;
    const int32_t* lens;    // append: positions (L = p + 1); decode: context_lens
    const float* q_norm_w;  // append only, nullptr: no QK-norm
    const float* k_norm_w;
    float* out;
    float* part_acc;        // [kMaxBalancedGrid * 2, G, D]
    float* part_ml;         // [kMaxBalancedGrid * 2, G, 2]
    int* counters;          // [B, Hkv], zero between calls
    int max_blocks;
    int max_context_len;    // decode only
    float scale;
    float eps;
    float theta;
    int B, Hq, Hkv, D, bs;
    int64_t num_blocks;
    int num_cus;
    int max_grid;           // cap on the workgroups (piece slots: 2 per workgroup); 0: none
    uint64_t* timeline;     // builds with PKV_TIMELINE: kTimelineStamps stamps per workgroup
    int timeline_rot;       // builds with PKV_TIMELINE: workgroup w takes range (w + rot) % grid
    int rope_dim;           // append only: rotated dims (even, <= D)
    int window;             // sliding window (0: every token)
    bool v_norm;            // append only: V rows normalised per KV head
    bool bf16;
    bool append;
    bool f32;               // decode_rope_mfma.hip: float32 pools
};

hipError_t launch_decode_balanced(const BalancedArgs& a, hipStream_t stream);

// The balanced schedule over the float32 matrix-core tile of decode_rope_mfma.hip (decode only:
// rotation at read with base `theta` over `rope_dim` dims, 0 = none; float32 or 16-bit pools),
// for the shapes decode_rope_mfma_ok accepts.
hipError_t launch_decode_rope_balanced(const BalancedArgs& a, hipStream_t stream);

// Profiling builds (-DPKV_TIMELINE): per workgroup of the balanced kernel, real-time counter
// stamps (100 MHz) at entry, lengths loaded, tile range known, first unit's query ready, wave
// 0's first tile done, last unit's streaming done, exit; then the number of units and tiles.
constexpr int kTimelineStamps = 10;
#ifdef PKV_TIMELINE
uint64_t* timeline_buffer();  // set by pkv_timeline_set (pkv_api.hip); nullptr: off
int timeline_rotation();
#endif

}  // namespace pkv
