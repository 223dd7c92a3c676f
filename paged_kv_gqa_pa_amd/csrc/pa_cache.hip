// Cache write: place each new token's K and V rows into their cache slots.
//
// Slot s of KV head g is row (g * num_blocks * 16 + s) of the head-major cache
// viewed as [kv_heads * num_blocks * 16, head_dim] -- one index over the
// (block, offset) slots of a head, as in "From 183 ms to 19 ms per decode
// step", "Four changes", changes 2 and 4.  One thread moves one 16-byte chunk
// of a row for both K and V; consecutive threads cover consecutive chunks of a
// row, so reads and writes are coalesced per row.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheArgs a) {
  const int chunks = a.row_bytes / 16;
  const int total = a.num_tokens * a.kv_heads * chunks;  // < 2^31, checked by the host
  const int stride = gridDim.x * blockDim.x;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int ch = i % chunks;
    const int rest = i / chunks;
    const int g = rest % a.kv_heads;
    const int tok = rest / a.kv_heads;
    // The slot and the data are loaded together (one memory round trip).
    const size_t src = (size_t(tok) * a.kv_heads + g) * a.row_bytes + size_t(ch) * 16;
    const u32x4 k = load16(reinterpret_cast<const char*>(a.key) + src);
    const u32x4 v = load16(reinterpret_cast<const char*>(a.value) + src);
    const int64_t slot = a.slot_mapping[tok];
    if (ch == 0 && g == 0) check(slot < int64_t(a.num_blocks) * kBlockSize, kCheckSlot, a.check_status);
    if (slot < 0 || slot >= int64_t(a.num_blocks) * kBlockSize) continue;
    const size_t dst = (size_t(g) * a.num_blocks * kBlockSize + size_t(slot)) * a.row_bytes +
                       size_t(ch) * 16;
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.k_cache) + dst) = k;
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.v_cache) + dst) = v;
  }
}

// Requantizing write into an int8 cache ("A Rust inference server for Qwen2
// on Apple Silicon", "Day 4 measurements -- int8 KV", "Partial blocks"): a
// write dequantizes the block's 16 slots (code * scale), overwrites the
// incoming row, recomputes the block scale as max|x| / 127 (1 for an all-zero
// block) and requantizes the block, rint half to even, clipped to +-127.
// Tokens aimed at one block are applied in index order.
//
// One workgroup of four waves per (token, KV head, tensor); wave w holds rows
// 4w .. 4w + 3 of the block, lane l row 4w + l / 16 and D / 16 consecutive
// dims from (l % 16) * D / 16, so a requantization is 8 (D = 128) or 4 values
// per lane and the block maximum is one wave reduction plus an exchange of
// four values through LDS.  The workgroup of the first token aimed at a block
// owns that block for the whole call: it applies its own row, then every
// later token's row aimed at the same block, in order, keeping the
// dequantized block in registers.  Workgroups of later tokens for an owned
// block return at once, so each block has one writer.  Every step is an fp32
// operation with IEEE rounding (a true division, rint half to even), so the
// codes do not depend on the order of the lanes.  Every wave of a workgroup
// reads the same slots and takes the same branches, so the barriers are
// reached by all four or by none.
template <int N> struct WordsT;
template <> struct WordsT<1> { typedef uint32_t type; };
template <> struct WordsT<2> { typedef u32x2 type; };
template <> struct WordsT<4> { typedef u32x4 type; };
template <> struct WordsT<8> { typedef uint32_t type __attribute__((ext_vector_type(8))); };

template <int D, typename IN>
__global__ __launch_bounds__(256) void requant_write_kernel(QuantCacheArgs a) {
  constexpr int PER = D / 16;                        // values per lane
  constexpr int NIN = PER * int(sizeof(IN)) / 4;     // input words per lane
  typedef typename WordsT<PER / 4>::type CodeW;      // this lane's codes
  typedef typename WordsT<NIN>::type InW;            // this lane's part of a row
  constexpr int SCAN = 8;                            // slot chunks of 64 per load batch
  __shared__ float s_max[2][4];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int tensor = blockIdx.x & 1;                 // 0: K, 1: V
  const int pair = blockIdx.x >> 1;
  const int tok = pair / a.kv_heads;
  const int g = pair - tok * a.kv_heads;
  const int64_t nslots = int64_t(a.num_blocks) * kBlockSize;
  const int row = 4 * wave + (lane >> 4);
  const int d0 = (lane & 15) * PER;
  const IN* src = reinterpret_cast<const IN*>(tensor == 0 ? a.key : a.value);
  auto row_part = [&](int t) {
    return *reinterpret_cast<const InW*>(src + (size_t(t) * a.kv_heads + g) * D + d0);
  };
  // Requested before the slot is known: it does not depend on it.
  const InW nr = row_part(tok);
  auto in_block = [&](int64_t s, int64_t blk) { return s >= 0 && s < nslots && s / kBlockSize == blk; };

  // The chunk of 64 slots holding this token; earlier chunks in batches.
  const int cbase = tok & ~63;
  const int jc = cbase + lane;
  const int64_t sc = jc < a.num_tokens ? a.slot_mapping[jc] : -1;
  const int64_t slot = uint32_t(__builtin_amdgcn_readlane(int(sc), tok - cbase)) |
                       (int64_t(__builtin_amdgcn_readlane(int(sc >> 32), tok - cbase)) << 32);
  if (threadIdx.x == 0 && tensor == 0) check(slot < nslots, kCheckSlot, a.check_status);
  if (slot < 0 || slot >= nslots) return;
  const int64_t blk = slot / kBlockSize;
  if (__builtin_amdgcn_ballot_w64(jc < tok && in_block(sc, blk)) != 0) return;
  for (int base = 0; base < cbase; base += 64 * SCAN) {
    int64_t sj[SCAN];
#pragma unroll
    for (int u = 0; u < SCAN; ++u) {
      const int j = base + 64 * u + lane;
      sj[u] = j < cbase ? a.slot_mapping[j] : -1;
    }
    bool hit = false;
#pragma unroll
    for (int u = 0; u < SCAN; ++u) hit |= in_block(sj[u], blk);
    if (__builtin_amdgcn_ballot_w64(hit) != 0) return;
  }

  int8_t* codes = (tensor == 0 ? a.k_cache : a.v_cache) +
                  (size_t(g) * a.num_blocks + size_t(blk)) * kBlockSize * D + row * D + d0;
  float* scale_p = (tensor == 0 ? a.k_scale : a.v_scale) + size_t(g) * a.num_blocks + blk;

  // Dequantize this lane's part of the block.
  float x[PER];
  {
    const float s = *scale_p;
    const CodeW w = *reinterpret_cast<const CodeW*>(codes);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      uint32_t word;
      if constexpr (PER == 4) word = w; else word = w[e / 4];
      x[e] = float(int8_t((word >> (8 * (e % 4))) & 0xFFu)) * s;
    }
  }
  float scale = 0.0f;
  int8_t q[PER];
  int parity = 0;
  auto requant = [&]() {
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < PER; ++e) m = fmaxf(m, fabsf(x[e]));
    m = stride_max<1>(m);
    if (lane == 0) s_max[parity][wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(s_max[parity][0], s_max[parity][1]), fmaxf(s_max[parity][2], s_max[parity][3]));
    parity ^= 1;   // the next write goes to the other pair, so no second barrier is needed
    scale = m > 0.0f ? m / 127.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float c = fminf(fmaxf(__builtin_rintf(x[e] / scale), -127.0f), 127.0f);
      q[e] = int8_t(c);
      x[e] = c * scale;   // the next write dequantizes these codes at this scale
    }
  };
  auto put_row = [&](const InW& v) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if constexpr (sizeof(IN) == 2) {
        const uint32_t w = v[e / 2];
        x[e] = (e & 1) ? bf16_hi(w) : bf16_lo(w);
      } else {
        x[e] = __uint_as_float(v[e]);
      }
    }
  };
  if (row == int(slot % kBlockSize)) put_row(nr);
  requant();
  // Later tokens aimed at the same block, in index order.
  auto later = [&](int base, int64_t sj, bool valid) {
    uint64_t hits = __builtin_amdgcn_ballot_w64(valid && in_block(sj, blk));
    while (hits != 0) {
      const int k = __builtin_ctzll(hits);
      hits &= hits - 1;
      const int sk = __builtin_amdgcn_readlane(int(sj), k);  // sj < nslots < 2^31 here
      if (row == sk % kBlockSize) put_row(row_part(base + k));
      requant();
    }
  };
  later(cbase, sc, jc > tok);
  for (int base = cbase + 64; base < a.num_tokens; base += 64 * SCAN) {
    int64_t sj[SCAN];
#pragma unroll
    for (int u = 0; u < SCAN; ++u) {
      const int j = base + 64 * u + lane;
      sj[u] = j < a.num_tokens ? a.slot_mapping[j] : -1;
    }
#pragma unroll
    for (int u = 0; u < SCAN; ++u) later(base + 64 * u, sj[u], base + 64 * u + lane < a.num_tokens);
  }
  CodeW w;
#pragma unroll
  for (int k = 0; k < PER / 4; ++k) {
    const uint32_t word = uint32_t(uint8_t(q[4 * k])) | (uint32_t(uint8_t(q[4 * k + 1])) << 8) |
                          (uint32_t(uint8_t(q[4 * k + 2])) << 16) |
                          (uint32_t(uint8_t(q[4 * k + 3])) << 24);
    if constexpr (PER == 4) w = word; else w[k] = word;
  }
  *reinterpret_cast<CodeW*>(codes) = w;
  if (threadIdx.x == 0) *scale_p = scale;
}

}  // namespace

hipError_t launch_reshape_and_cache_quant(const QuantCacheArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const unsigned grid = unsigned(2L * a.num_tokens * a.kv_heads);
  if (a.head_dim == 128) {
    if (a.in_dtype == kBF16) requant_write_kernel<128, bf16_t><<<grid, 256, 0, stream>>>(a);
    else requant_write_kernel<128, float><<<grid, 256, 0, stream>>>(a);
  } else {
    if (a.in_dtype == kBF16) requant_write_kernel<64, bf16_t><<<grid, 256, 0, stream>>>(a);
    else requant_write_kernel<64, float><<<grid, 256, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const CacheArgs& a, hipStream_t stream) {
  const long total = long(a.num_tokens) * a.kv_heads * (a.row_bytes / 16);
  if (total == 0) return hipSuccess;
  const long want = (total + 255) / 256;
  const int blocks = int(want < 8192 ? want : 8192);
  reshape_and_cache_kernel<<<blocks, 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pa
