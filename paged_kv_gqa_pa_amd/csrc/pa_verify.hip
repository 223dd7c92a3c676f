// Multi-token (speculative verify) paged attention on the matrix cores.
//
// A verify step checks k+1 guessed tokens per sequence in one pass, with a
// causal mask among the new tokens ("From 183 ms to 19 ms per decode step",
// section "Then speculative decoding got slower": query tokens times group
// heads on the rows of one matrix product, on the tensor cores).  For one
// (sequence, KV head) the T query tokens of the G heads of the group form
// R = T*G <= 16 query rows, so each 16-token cache tile is one dense 16x16
// block of scores:
//
//   S^T[key, row] = sum_d K[key, d] * Q[row, d]      v_mfma_f32_16x16x32_bf16
//       A = K tile (key = lane % 16, 8 contiguous dims per lane: a 16-byte
//       load straight from the cache), B = the query rows (loaded once).
//   online softmax per row (fp32 running max and sum, rescaled per tile)
//   O[row, d] += sum_key P[row, key] * V[key, d]     v_mfma_f32_16x16x16_bf16
//       A = P: the score accumulator already holds, per lane, 4 keys of one
//       row -- exactly the A layout of the 16x16x16 product, so P needs no
//       shuffle.  B needs 4 keys of one dim per lane: the V tile goes through
//       LDS (row pitch padded so the transposed reads hit distinct banks).
//
// Row t*G + i is query token t of head g*G + i; token t sees positions
// 0 .. L - T + t.  Pieces, workspace partials and the merge pass are shared
// with decode (rows_per_seq = T * q_heads).
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 16;  // query rows of one matrix tile

template <int D, int NW>
__global__ __launch_bounds__(NW * kWave) void verify_pass1(DecodeArgs a) {
  constexpr int KCH = D / 32;            // 32-dim chunks of the score product
  constexpr int VLD = D / 32;            // 1 KiB wave loads per V tile (16 * D * 2 bytes)
  constexpr int OT = D / 16;             // 16-dim output tiles
  constexpr int PITCH = D + 4;           // LDS row pitch in bf16 elements
  constexpr int TILE_BYTES = kBlockSize * D * 2;

  const int pairs = a.num_seqs * a.kv_heads;
  const int piece = blockIdx.x / pairs;
  const int pair = blockIdx.x - piece * pairs;
  const int b = pair / a.kv_heads;
  const int g = pair - b * a.kv_heads;
  const int T = a.num_query_tokens;
  const int Hq = a.q_heads;
  const int G = Hq / a.kv_heads;
  const int R = T * G;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;     // key row of the K operand / query row of S and P
  const int grp = lane >> 4;   // which 8 dims (scores) or 4 keys (P, O rows)
  const int split_blocks = a.split_tokens / kBlockSize;
  const int blk_begin = piece * split_blocks;

  // Length-independent loads first: the piece's table entries and the query rows.
  const int32_t* bt = a.block_tables + size_t(b) * a.max_blocks_per_seq;
  const int tab = blk_begin + lane < a.max_blocks_per_seq ? bt[blk_begin + lane] : 0;
  const int t_row = n / G;
  const int h_row = g * G + (n - t_row * G);
  bf16x8 qb[KCH];
  {
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(a.q) +
                       ((size_t(b) * T + t_row) * Hq + h_row) * D + 8 * grp;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      u32x4 w = n < R ? load16(qp + 32 * j) : u32x4{0u, 0u, 0u, 0u};
      qb[j] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int L = min(a.context_lens[b], a.max_blocks_per_seq * kBlockSize);
  const int n_pieces = min(L > 0 ? cdiv(L, a.split_tokens) : 1, a.max_pieces);
  if (piece >= n_pieces) return;
  const int blk_end = min(cdiv(L, kBlockSize), blk_begin + split_blocks);
  // Last position row n may see (rows past R see nothing).
  const int last_vis = n < R ? L - T + t_row : -1;

  const size_t head_blocks = size_t(g) * a.num_blocks;
  const char* kbase = reinterpret_cast<const char*>(a.k_cache);
  const char* vbase = reinterpret_cast<const char*>(a.v_cache);
  const float sc = a.scale * kLog2e;

  __shared__ uint16_t s_v[NW][kBlockSize][PITCH];
  __shared__ float s_m[NW][kRows], s_l[NW][kRows];
  __shared__ float s_o[NW][kRows][D];

  float m = kNegInf;   // running max of row n (log2 units)
  float lsum = 0.0f;   // this lane's share of row n's running sum
  f32x4 o[OT];
#pragma unroll
  for (int c = 0; c < OT; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto fetch = [&](int blk, u32x4 (&kt)[KCH], u32x4 (&vt)[VLD]) {
    const int phys = min(max(__builtin_amdgcn_readlane(tab, blk - blk_begin), 0), a.num_blocks - 1);
    const size_t tile = (head_blocks + size_t(phys)) * TILE_BYTES;
#pragma unroll
    for (int j = 0; j < KCH; ++j)
      kt[j] = load16_stream(kbase + tile + n * (2 * D) + 64 * j + 16 * grp);
#pragma unroll
    for (int i = 0; i < VLD; ++i) vt[i] = load16_stream(vbase + tile + i * 1024 + lane * 16);
  };

  auto process = [&](int blk, u32x4 (&kt)[KCH], u32x4 (&vt)[VLD]) {
    // Stage V (zeros past the context: a zero weight must meet a finite value).
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int byte = i * 1024 + lane * 16;
      const int key = byte / (2 * D);
      const int d0 = (byte % (2 * D)) / 2;
      const bool valid = blk * kBlockSize + key < L;
      uint2* dst = reinterpret_cast<uint2*>(&s_v[wave][key][d0]);
      dst[0] = valid ? uint2{vt[i][0], vt[i][1]} : uint2{0u, 0u};
      dst[1] = valid ? uint2{vt[i][2], vt[i][3]} : uint2{0u, 0u};
    }
    // Scores of keys 4*grp .. 4*grp+3 for row n.
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KCH; ++j)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kt[j]), qb[j], s, 0,
                                                  0, 0);
    float tmax = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = blk * kBlockSize + 4 * grp + e;
      s[e] = pos <= last_vis ? s[e] * sc : kNegInf;
      tmax = fmaxf(tmax, s[e]);
    }
    tmax = max_xor32(max_xor16(tmax));   // over the 16 keys of the tile
    const float mnew = fmaxf(m, tmax);
    const float mref = mnew == kNegInf ? 0.0f : mnew;
    const float alpha = fast_exp2(m - mref);
    m = mnew;
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = fast_exp2(s[e] - mref);
    lsum = __builtin_fmaf(lsum, alpha, (p[0] + p[1]) + (p[2] + p[3]));
    // P as the A operand (row n, keys 4*grp ..), rounded to bf16.
    s16x4 pa;
#pragma unroll
    for (int e = 0; e < 4; ++e) pa[e] = short(f32_to_bf16(p[e]));
    // O rows 4*grp + e take the rescale factor of that row.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ar = __shfl(alpha, 4 * grp + e);
#pragma unroll
      for (int c = 0; c < OT; ++c) o[c][e] *= ar;
    }
    // V of keys 4*grp .. 4*grp+3 at dim 16*c + n: the transposed read.
#pragma unroll
    for (int c = 0; c < OT; ++c) {
      s16x4 vb;
#pragma unroll
      for (int e = 0; e < 4; ++e) vb[e] = short(s_v[wave][4 * grp + e][16 * c + n]);
      o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, o[c], 0, 0, 0);
    }
  };

  const int first = blk_begin + wave;
  const int n_my = first < blk_end ? cdiv(blk_end - first, NW) : 0;
  if (n_my > 0) {
    const int last = n_my - 1;
    u32x4 k0[KCH], v0[VLD], k1[KCH], v1[VLD];
    fetch(first, k0, v0);
    int j = 0;
    for (; j + 1 <= last; j += 2) {
      fetch(first + (j + 1) * NW, k1, v1);
      process(first + j * NW, k0, v0);
      fetch(first + min(j + 2, last) * NW, k0, v0);
      process(first + (j + 1) * NW, k1, v1);
    }
    if (j == last) process(first + j * NW, k0, v0);
  }

  // Row totals (all four lane groups share each row's max), then the waves
  // are merged through LDS.
  const float lrow = add_xor32(add_xor16(lsum));
  if (grp == 0) {
    s_m[wave][n] = m;
    s_l[wave][n] = lrow;
  }
#pragma unroll
  for (int c = 0; c < OT; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_o[wave][4 * grp + e][16 * c + n] = o[c][e];
  __syncthreads();

  for (int t = threadIdx.x; t < R * D; t += NW * kWave) {
    const int row = t / D, d = t % D;
    float M = s_m[0][row];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][row]);
    float lt = 0.0f, ot = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = s_m[w][row] == kNegInf ? 0.0f : fast_exp2(s_m[w][row] - M);
      lt = __builtin_fmaf(s_l[w][row], f, lt);
      ot = __builtin_fmaf(s_o[w][row][d], f, ot);
    }
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const int tq = row / G;
    const size_t orow = (size_t(b) * T + tq) * Hq + size_t(g) * G + (row - tq * G);
    if (n_pieces == 1) {
      reinterpret_cast<bf16_t*>(a.out)[orow * D + d].bits = f32_to_bf16(ot * inv);
    } else {
      const size_t prow = orow * a.max_pieces + piece;
      a.part_o[prow * D + d] = ot * inv;
      if (d == 0) a.part_lse[prow] = lt > 0.0f ? M + __log2f(lt) : kNegInf;
    }
  }
}

}  // namespace

bool verify_supported(int q_dtype, int kv_dtype, int head_dim, int G, int T) {
  return q_dtype == kBF16 && kv_dtype == kBF16 && (head_dim == 64 || head_dim == 128) &&
         G >= 1 && T >= 1 && long(G) * T <= kRows;
}

hipError_t launch_verify_pass1(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NW = 4;
  const long wgs = long(a.max_pieces) * a.num_seqs * a.kv_heads;
  if (a.head_dim == 128)
    verify_pass1<128, NW><<<dim3(unsigned(wgs)), NW * kWave, 0, stream>>>(a);
  else
    verify_pass1<64, NW><<<dim3(unsigned(wgs)), NW * kWave, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pa
