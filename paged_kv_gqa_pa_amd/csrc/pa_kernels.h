// Internal launch interface between the C ABI (pa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Device-side precondition checks (a debug build, -DPA_DEVICE_CHECKS=1): a
// kernel that meets a violated precondition sets its bit in the status word
// whose address the launch passes (`check_status`) and goes on with the
// clamped value it uses anyway; release builds compile the checks out.
#ifndef PA_DEVICE_CHECKS
#define PA_DEVICE_CHECKS 0
#endif

namespace pa {

enum DType : int { kF32 = 0, kBF16 = 1, kI8 = 2 };

// Status bits (the same values as the PA_CHECK_* constants of pa.h).
constexpr unsigned kCheckTableEntry = 1u;     // a block-table entry read lies outside [0, num_blocks)
constexpr unsigned kCheckContextTable = 2u;   // context_lens[b] < 0 or > max_blocks_per_seq * 16
constexpr unsigned kCheckContextMax = 4u;     // context_lens[b] > max_context_len (pieces not launched)
constexpr unsigned kCheckSlot = 8u;           // a cache slot >= num_blocks * 16
constexpr unsigned kCheckQueryStart = 16u;    // query_start decreasing, past total, or above max tokens

constexpr int kBlockSizeHost = 16;  // tokens per cache block
constexpr int kMaxSplitTokens = 4096;  // a piece's table entries: kTabRegs per lane
constexpr int kTabRegs = kMaxSplitTokens / (kBlockSizeHost * 64);

struct CacheArgs {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const int64_t* slot_mapping;
  int num_tokens;
  int kv_heads;
  int num_blocks;
  int row_bytes;  // head_dim * element size
  unsigned* check_status;  // device checks (debug builds), else nullptr
};

struct QuantCacheArgs {
  const void* key;      // [num_tokens, kv_heads, head_dim], in_dtype
  const void* value;
  int8_t* k_cache;      // [kv_heads, num_blocks, 16, head_dim]
  int8_t* v_cache;
  float* k_scale;       // [kv_heads, num_blocks]
  float* v_scale;
  const int64_t* slot_mapping;
  int num_tokens;
  int kv_heads;
  int num_blocks;
  int head_dim;
  int in_dtype;
  unsigned* check_status;  // device checks (debug builds), else nullptr
};

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* part_o;    // [rows, max_pieces, head_dim]  (rows = num_seqs * T * q_heads)
  float* part_lse;  // [rows, max_pieces], log2 domain
  // Append mode only: the new token's K/V per sequence [num_seqs, kv_heads,
  // head_dim] and its cache slot [num_seqs].  With an int8 cache the rows are
  // new_dtype values (kF32 or kBF16), the slot's block is requantized and
  // k_scale / v_scale are written.
  const void* new_k;
  const void* new_v;
  const int64_t* slot_mapping;
  int new_dtype;
  // Variable-length verify only: sequence b's query tokens are packed rows
  // query_start[b] .. query_start[b+1]-1 of q and out ([total, q_heads,
  // head_dim]); nullptr for a fixed T per sequence.
  const int32_t* query_start;
  // Work plan (pa_plan): the order in which the (sequence, piece) units are
  // started, with copies of their lengths and block-table entries; nullptr =
  // natural order.
  const int32_t* plan;
  int total_query_tokens;
  int num_seqs;
  int num_query_tokens;  // T (1 for decode); the largest T_b for variable length
  int q_heads;
  int kv_heads;
  int head_dim;
  int num_blocks;
  int max_blocks_per_seq;
  int split_tokens;
  int max_pieces;
  float scale;
  int q_dtype;
  int kv_dtype;
  unsigned* check_status;  // device checks (debug builds), else nullptr
};


struct MergeArgs {
  void* out;
  const float* part_o;
  const float* part_lse;
  const int32_t* context_lens;
  const int32_t* query_start;  // variable-length verify (rows packed by token), else nullptr
  int num_seqs;
  int q_heads;
  int num_rows;
  int rows_per_seq;
  int max_pieces;
  int split_tokens;
  int max_len_clamp;  // max_blocks_per_seq * block_size
  int head_dim;
  int out_dtype;
};

// Work plans.  A plan is kPlanHeader ints (kPlanMagic, num_seqs, max_pieces,
// split_tokens, max_blocks_per_seq, snake_units, snake_rounds, the rest 0)
// and then one row per unit
// (sequence, piece) in the order the units are to be started: sequence,
// piece, context length, the piece's tile count (-1: the piece does not
// exist), then the piece's split_tokens / 16 block-table entries (0 past its
// tiles), padded to a multiple of 4 ints.
constexpr int kPlanHeader = 16;
constexpr int kPlanRowHead = 4;
constexpr int kPlanMagic = 0x50414E31;
constexpr int kMaxPlanUnits = 8192;  // units (num_seqs * max_pieces) one plan orders
__host__ __device__ inline int plan_stride(int split_tokens) {
  return kPlanRowHead + ((split_tokens / kBlockSizeHost + 3) & ~3);
}

struct PlanArgs {
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t* plan;
  int num_seqs;
  int max_blocks_per_seq;
  int max_pieces;
  int split_tokens;
  // The first snake_rounds rounds of snake_units units each (the workgroups
  // resident at once, one per CU per round) alternate longest-first and
  // shortest-first, so each CU holds a long and a short unit; 0 = plain
  // longest-first order.
  int snake_units;
  int snake_rounds;
};

// Workgroups of one attention kernel resident per CU (occupancy query).
int decode_pass1_resident(int q_dtype, int kv_dtype, int head_dim, int G);
int rows_pass1_resident(int kv_dtype, int head_dim, int rows);

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream);

// Prefill work plans.  kPlanHeader ints (kPrefillPlanMagic, num_seqs, row
// tiles per sequence, query rows per tile, total_query_tokens,
// max_query_tokens, max_blocks_per_seq, group size, the rest 0), then one row
// of kPrefillPlanRow ints per (sequence, row tile) unit, longest first:
// sequence, tile, first packed query token, query count, context length, the
// positions the tile's last row sees (-1: no rows), 0, 0.
constexpr int kPrefillPlanMagic = 0x50414E32;
constexpr int kPrefillPlanRow = 8;
constexpr int kPrefillBuckets = 256;

struct PrefillPlanArgs {
  const int32_t* context_lens;
  const int32_t* query_start;
  int32_t* plan;
  int num_seqs;
  int tiles;
  int rows_per_tile;
  int group;
  int total_query_tokens;
  int max_query_tokens;
  int max_blocks_per_seq;
};
hipError_t launch_prefill_plan(const PrefillPlanArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
// Chunked prefill (matrix cores): DecodeArgs with query_start set, no pieces.
hipError_t launch_prefill(const DecodeArgs& a, hipStream_t stream);
bool prefill_supported(int q_dtype, int kv_dtype, int head_dim);
int prefill_rows_per_workgroup();
hipError_t launch_reshape_and_cache(const CacheArgs& a, hipStream_t stream);
hipError_t launch_reshape_and_cache_quant(const QuantCacheArgs& a, hipStream_t stream);
hipError_t launch_decode_pass1(const DecodeArgs& a, bool append, hipStream_t stream);
// Matrix-core kernel for R = T * G <= 16 * kMaxRowTiles query rows per
// (sequence, KV head), in row tiles of 16: verify calls, and decode over an
// int8 cache or with bf16 groups of 4 or more query heads.
constexpr int kMaxRowTiles = 3;
hipError_t launch_rows_pass1(const DecodeArgs& a, hipStream_t stream);
bool decode_group_supported(int G);
bool rows_supported(int q_dtype, int kv_dtype, int head_dim, int G, int T);

}  // namespace pa
