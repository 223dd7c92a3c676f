// Work plan: the order in which an attention call's (sequence, piece) units
// are started, longest first.
//
// Every unit's arithmetic is fixed by the unit alone (its sequence, its piece
// of a fixed length), so the order changes no bit of any result; it only
// changes how evenly the chip is loaded.  In the natural order a long unit
// started late ends the launch alone; started first, it overlaps the short
// ones.  The decode step of "From 183 ms to 19 ms per decode step" (section
// "Four changes, one profile at a time", change 4) hands every layer of a step
// the same block tables and lengths, so one plan serves all of a step's
// layers.
//
// One workgroup orders the units with a counting sort on their tile counts
// (at most split_tokens / 16 + 2 distinct keys): a histogram, offsets in
// descending key order, then each unit takes the next place of its key
// (units of equal length land in any order).  Where the attention kernel
// keeps several workgroups per CU, all of them started at once, the first
// rounds snake: a CU's second workgroup gets a short unit opposite its first
// workgroup's long one, which evens the work per CU (a plain longest-first
// order pairs the c-th longest with the (c + CUs)-th longest).  Each unit's
// row receives its sequence, piece, length, tile count and a copy of the
// piece's block-table entries, so that an attention workgroup learns its unit
// and the piece's physical blocks in one round trip.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int s_key[kMaxPlanUnits];
  __shared__ int s_pos[kMaxPlanUnits];
  __shared__ int s_cnt[kMaxSplitTokens / kBlockSize + 2];
  const int N = a.num_seqs;
  const int U = a.max_pieces * N;
  const int sb = a.split_tokens / kBlockSize;
  const int max_len = a.max_blocks_per_seq * kBlockSize;
  const int tid = threadIdx.x;

  for (int i = tid; i < sb + 2; i += kPlanThreads) s_cnt[i] = 0;
  __syncthreads();
  // Key of unit v = (piece v / N, sequence v % N): its tile count, 0 for the
  // single piece of an empty context (it still writes a zero row), -1 for a
  // piece past the sequence's context (no work).
  for (int v = tid; v < U; v += kPlanThreads) {
    const int piece = v / N, b = v - piece * N;
    const int L = min(max(a.context_lens[b], 0), max_len);
    const int np = min(L > 0 ? cdiv(L, a.split_tokens) : 1, a.max_pieces);
    const int key = piece < np ? min(max(cdiv(L, kBlockSize) - piece * sb, 0), sb) : -1;
    s_key[v] = key;
    atomicAdd(&s_cnt[key + 1], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int k = sb + 1; k >= 0; --k) {
      const int c = s_cnt[k];
      s_cnt[k] = run;
      run += c;
    }
  }
  __syncthreads();
  // Rounds of resident workgroups: round r of snake_units units lands one
  // workgroup per CU, and round r + 1 the second workgroup of the same CUs in
  // the same CU order, so odd rounds are reversed (shortest first) to pair
  // each CU's long unit with a short one.
  const int S = a.snake_units;
  for (int v = tid; v < U; v += kPlanThreads) {
    int p = atomicAdd(&s_cnt[s_key[v] + 1], 1);
    if (S > 0) {
      const int r = p / S;
      if (r < a.snake_rounds && (r & 1)) {
        const int lo = r * S, n = min(S, U - lo);
        p = lo + (n - 1 - (p - lo));
      }
    }
    s_pos[v] = p;
  }
  __syncthreads();

  const int stride = plan_stride(a.split_tokens);
  int32_t* rows = a.plan + kPlanHeader;
  for (int v = tid; v < U; v += kPlanThreads) {
    const int piece = v / N, b = v - piece * N;
    int32_t* row = rows + size_t(s_pos[v]) * stride;
    row[0] = b;
    row[1] = piece;
    row[2] = min(max(a.context_lens[b], 0), max_len);
    row[3] = s_key[v];
  }
  // The piece's table entries, one per thread: entry i of unit v.
  const long entries = long(U) * sb;
  for (long idx = tid; idx < entries; idx += kPlanThreads) {
    const int v = int(idx / sb), i = int(idx - long(v) * sb);
    const int piece = v / N, b = v - piece * N;
    const int32_t* bt = a.block_tables + size_t(b) * a.max_blocks_per_seq;
    rows[size_t(s_pos[v]) * stride + kPlanRowHead + i] = i < s_key[v] ? bt[piece * sb + i] : 0;
  }
  if (tid < kPlanHeader) {
    int h = 0;
    switch (tid) {
      case 0: h = kPlanMagic; break;
      case 1: h = N; break;
      case 2: h = a.max_pieces; break;
      case 3: h = a.split_tokens; break;
      case 4: h = a.max_blocks_per_seq; break;
      case 5: h = a.snake_units; break;
      case 6: h = a.snake_rounds; break;
      default: h = 0;
    }
    a.plan[tid] = h;
  }
}

// The prefill work plan: the (sequence, row tile) units of a pa_prefill call
// sorted by the positions each tile's last row sees (the length of its loop
// over the cache), longest first, in kPrefillBuckets buckets of equal width.
// Causal chunks on top of prior contexts of different lengths give tiles
// that differ many times over in work; started in the natural order, the
// longest end the launch alone.
__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(PrefillPlanArgs a) {
  __shared__ int s_key[kMaxPlanUnits];
  __shared__ int s_pos[kMaxPlanUnits];
  __shared__ int s_cnt[kPrefillBuckets];
  const int N = a.num_seqs;
  const int U = N * a.tiles;
  const int max_len = a.max_blocks_per_seq * kBlockSize;
  const int width = max(1, cdiv(max_len + 1, kPrefillBuckets - 1));
  const int tid = threadIdx.x;
  for (int i = tid; i < kPrefillBuckets; i += kPlanThreads) s_cnt[i] = 0;
  __syncthreads();
  for (int u = tid; u < U; u += kPlanThreads) {
    const int b = u / a.tiles, t = u - b * a.tiles;
    const int L = min(a.context_lens[b], max_len);
    const int s0 = a.query_start[b], s1 = a.query_start[b + 1];
    const int q0 = min(max(s0, 0), a.total_query_tokens);
    const int T = min(max(s1 - s0, 0), min(a.max_query_tokens, a.total_query_tokens - q0));
    const int R = T * a.group, row0 = t * a.rows_per_tile;
    int key = -1;
    if (row0 < R) {
      const int tl = (min(row0 + a.rows_per_tile, R) - 1) / a.group;
      key = min(max(L - T + tl + 1, 0), max(L, 0));
    }
    const int bucket = key < 0 ? 0 : 1 + min(key / width, kPrefillBuckets - 2);
    s_key[u] = bucket;
    atomicAdd(&s_cnt[bucket], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int k = kPrefillBuckets - 1; k >= 0; --k) {
      const int c = s_cnt[k];
      s_cnt[k] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int u = tid; u < U; u += kPlanThreads) s_pos[u] = atomicAdd(&s_cnt[s_key[u]], 1);
  __syncthreads();
  for (int u = tid; u < U; u += kPlanThreads) {
    const int b = u / a.tiles, t = u - b * a.tiles;
    const int L = min(a.context_lens[b], max_len);
    const int s0 = a.query_start[b], s1 = a.query_start[b + 1];
    const int q0 = min(max(s0, 0), a.total_query_tokens);
    const int T = min(max(s1 - s0, 0), min(a.max_query_tokens, a.total_query_tokens - q0));
    const int R = T * a.group, row0 = t * a.rows_per_tile;
    int key = -1;
    if (row0 < R) {
      const int tl = (min(row0 + a.rows_per_tile, R) - 1) / a.group;
      key = min(max(L - T + tl + 1, 0), max(L, 0));
    }
    int32_t* row = a.plan + kPlanHeader + size_t(s_pos[u]) * kPrefillPlanRow;
    row[0] = b;
    row[1] = t;
    row[2] = q0;
    row[3] = T;
    row[4] = L;
    row[5] = key;
    row[6] = 0;
    row[7] = 0;
  }
  if (tid < kPlanHeader) {
    int h = 0;
    switch (tid) {
      case 0: h = kPrefillPlanMagic; break;
      case 1: h = N; break;
      case 2: h = a.tiles; break;
      case 3: h = a.rows_per_tile; break;
      case 4: h = a.total_query_tokens; break;
      case 5: h = a.max_query_tokens; break;
      case 6: h = a.max_blocks_per_seq; break;
      case 7: h = a.group; break;
      default: h = 0;
    }
    a.plan[tid] = h;
  }
}

}  // namespace

hipError_t launch_prefill_plan(const PrefillPlanArgs& a, hipStream_t stream) {
  prefill_plan_kernel<<<1, kPlanThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream) {
  plan_kernel<<<1, kPlanThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pa
