// Paged attention on the matrix cores for several query rows per
// (sequence, KV head): the T query tokens of a speculative verify step times
// the G heads of a group ("From 183 ms to 19 ms per decode step", section
// "Then speculative decoding got slower": query tokens times group heads as the
// rows of one matrix product), and the G heads of an int8-cache decode step,
// whose per-key work would otherwise bind on the vector ALUs.
//
// The R = T*G <= 16 rows of one (sequence, KV head) make each 16-token cache
// tile a dense 16x16 block of scores.  Per tile:
//
//   K and V tiles arrive as contiguous 1 KiB wave loads and are staged in the
//   wave's LDS (whole 128-byte lines per load; loading the product layouts
//   straight from the cache touches half lines and was measurably slower).
//   S^T[key, row] = sum_d K[key, d] Q[row, d]     16x16x32 products; A = key n's
//       8 dims per lane read from LDS, B = the query rows, loaded once.
//   online softmax per row: fp32 reference maximum with delayed rescaling.
//   O[row, d] += sum_key P[row, key] V[key, d]    16x16x16 products; A = P, which
//       the score accumulator already holds in the A layout; B = four keys of
//       one dim per lane.  bf16: transposed reads from LDS.  int8: each lane
//       reads 4 dims of one key and a product with the identity hands it 4 keys
//       of one dim instead (the result layout of a product is the B layout of
//       the next), the values passing through exactly.
//
// bf16 caches run all products in bf16 (P rounded to bf16).  int8 caches run
// the score products in fp16: a code c becomes the exact fp16 number c + 1152
// (byte permute under a constant high byte) and the scores lose the K bias as
// -1152 * sum_d q[row, d]; the transposing product removes the V bias by
// starting its accumulator at -1152, and P.V runs in bf16 (the codes are
// exact bf16 numbers) with P carrying the tile's V scale.
//
// Row t*G + i is query token t of head g*G + i; token t sees positions
// 0 .. L - T + t.  Pieces, workspace partials and the merge pass are shared
// with the vector-ALU decode kernel (rows_per_seq = T * q_heads).
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"
#include "pa_mfma.h"

namespace pa {
namespace {

template <typename KV, int D, int NW, int NS, int RT, bool AP = false>
__global__ __launch_bounds__(NW * kWave) void rows_pass1(DecodeArgs a) {
  constexpr bool kInt8 = __is_same(KV, i8_t);
  constexpr int ROWB = D * int(sizeof(KV));  // bytes per key row
  constexpr int NL = ROWB / 64;              // 1 KiB wave loads per tile (16 rows)
  constexpr int NQ = D / 32;                 // score products per tile
  constexpr int NT = D / 16;                 // output blocks of 16 dims
  constexpr int TILE_BYTES = kBlockSize * ROWB;
  // Per-wave LDS: a ring of two staged (K, V) tile pairs, written by the load
  // units directly (no registers), reused for the wave's O rows after its
  // loop.  Within a staged K tile (and an int8 V tile), 16-byte chunk k of key
  // row r sits at position k ^ ((r / RPB) mod CPR) of its row (RPB rows share
  // one 256-byte bank period), so that the operand reads below hit distinct
  // banks.  A bf16 V tile is swizzled for the LDS transpose reads that hand
  // out its B operand (vswz, pa_mfma.h).
  constexpr int CPR = ROWB / 16;             // 16-byte chunks per key row
  constexpr int RPB = ROWB >= 256 ? 1 : 256 / ROWB;
  constexpr int SLOT = 2 * TILE_BYTES;       // one (K, V) tile pair
  constexpr int OHALF = kRows / 2 * D * 4;   // O rows of one half of a row tile
  constexpr int WBYTES = SLOT > OHALF ? SLOT : OHALF;
  using M = MOps<KV>;

  const int lane = threadIdx.x & (kWave - 1);
  // The work unit (natural order or a work plan) and the piece's table
  // entries, requested before anything that depends on them.
  PieceTable<kTabRegs> tab;
  const WorkItem it = work_item(a, tab, lane);
  const int b = it.b, piece = it.piece, g = it.g;
  const int Hq = a.q_heads;
  const int G = Hq / a.kv_heads;
  // Sequence b's query tokens: T of them from packed token q0 (fixed T: b * T),
  // or its own count T_b from the offsets (clamped to the buffer and to T).
  int T = a.num_query_tokens;
  int q0 = b * T;
  if (a.query_start) {
    const int s0 = a.query_start[b], s1 = a.query_start[b + 1];
    if (threadIdx.x == 0)
      check(s0 >= 0 && s1 >= s0 && s1 <= a.total_query_tokens && s1 - s0 <= T, kCheckQueryStart,
            a.check_status);
    q0 = min(max(s0, 0), a.total_query_tokens);
    T = min(max(s1 - s0, 0), min(T, a.total_query_tokens - q0));
    if (T == 0) return;
  }
  const int R = T * G;   // at most 16 * RT (the launch picks RT)
  const int L = it.L;
  // Decode with append (AP).  bf16 cache: lane k < CPR of every wave holds
  // 16-byte chunk k of the new token's K and V rows (position L - 1).  int8
  // cache: the new rows are bf16 or fp32 values (new_dtype); the lane that
  // owns chunk k of row (L - 1) % 16 in the requantization below (chunk
  // index 16-row-major, lane = index % 64) holds dims 16k .. 16k + 15 of
  // both, as raw words.  Every wave also reads the token's slot.
  constexpr bool append = AP;
  u32x4 nk = {0u, 0u, 0u, 0u}, nv = {0u, 0u, 0u, 0u};
  u32x4 nq[2][4] = {};   // int8 append: [K, V][16-byte words] (bf16: 2 words, fp32: 4)
  int64_t new_slot = -1;
  if constexpr (append && !kInt8) {
    if (lane < CPR) {
      const size_t off = (size_t(b) * a.kv_heads + g) * ROWB + 16 * size_t(lane);
      nk = load16(reinterpret_cast<const char*>(a.new_k) + off);
      nv = load16(reinterpret_cast<const char*>(a.new_v) + off);
    }
  }
  if constexpr (append && kInt8) {
    const int ch = lane - (L > 0 ? ((L - 1) % kBlockSize) * CPR % kWave : 0);
    if (L > 0 && ch >= 0 && ch < CPR) {
      const int words = a.new_dtype == kF32 ? 4 : 2;
      const size_t off = ((size_t(b) * a.kv_heads + g) * D + 16 * size_t(ch)) * words;   // bytes per value = words
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (w < words) {
          nq[0][w] = load16(reinterpret_cast<const char*>(a.new_k) + off + 16 * w);
          nq[1][w] = load16(reinterpret_cast<const char*>(a.new_v) + off + 16 * w);
        }
      }
    }
  }
  if constexpr (append) new_slot = a.slot_mapping[b];

  const int wave = readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;     // key row of an operand read / query row of S, P
  const int grp = lane >> 4;   // 8-dim group of a score product / key quad of S, P, O
  const int split_blocks = a.split_tokens / kBlockSize;
  const int blk_begin = piece * split_blocks;

  // Row tile i holds rows 16i .. 16i + 15.  Query rows as the B operand of
  // score product c: lane (row n of tile i, group grp) holds
  // q[16i + n][32c + 8grp .. +7] (fp16 for an int8 cache).
  u32x4 qb[RT][NQ];
  float qsum[RT];     // row n's sum of (fp16) q over all dims (int8 K bias)
  int last_vis[RT];   // last position row n may see (rows past R see nothing)
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int row = kRows * i + n;
    const bool row_ok = row < R;
    const int t_row = row / G;
    const int h_row = g * G + (row - t_row * G);
    last_vis[i] = row_ok ? L - T + t_row : -1;
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(a.q) +
                       ((size_t(q0) + t_row) * Hq + h_row) * D + 8 * grp;
    float qpart = 0.0f;
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      const u32x4 w = row_ok ? load16(qp + 32 * c) : u32x4{0u, 0u, 0u, 0u};
      if constexpr (kInt8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f16x2 hp = to_f16x2(bf16_lo(w[e]), bf16_hi(w[e]));
          qb[i][c][e] = __builtin_bit_cast(uint32_t, hp);
          qpart += float(hp[0]) + float(hp[1]);
        }
      } else {
        qb[i][c] = w;
      }
    }
    qsum[i] = kInt8 ? add_xor32(add_xor16(qpart)) : 0.0f;
  }

  const int n_pieces = min(L > 0 ? cdiv(L, a.split_tokens) : 1, a.max_pieces);
  if (piece < 0 || piece >= n_pieces) return;
  const int blk_end = min(cdiv(L, kBlockSize), blk_begin + split_blocks);
  // The tile holding position L - 1 takes that row from the input (below); the
  // last piece's wave 0 also writes it into the cache slot after its tile
  // loop (slots < 0 are skipped, slots past the pool ignored).  Only this
  // workgroup uses the position, so no other reader waits on the write.
  const int blk_new = append && L > 0 ? (L - 1) / kBlockSize : -1;

  const size_t head_blocks = size_t(g) * a.num_blocks;
  const char* kbase = reinterpret_cast<const char*>(a.k_cache);
  const char* vbase = reinterpret_cast<const char*>(a.v_cache);
  const float sc = a.scale * kLog2e;

  // The two ring slots are separate LDS objects, so the compiler's wait for a
  // slot's direct-to-LDS loads does not also wait for the other slot's.
  __shared__ __attribute__((aligned(16))) char s_ring0[NW * WBYTES];
  __shared__ __attribute__((aligned(16))) char s_ring1[NW * WBYTES];
  __shared__ __attribute__((aligned(16))) char s_ring2[NS > 2 ? NW * WBYTES : 16];
  __shared__ __attribute__((aligned(16))) char s_ring3[NS > 3 ? NW * WBYTES : 16];
  // Each wave's row maxima and sums: in its slot-1 region behind its O rows
  // when there is room (keeps a bf16, D = 128 workgroup within 64 KiB).
  constexpr bool kMLInRing = WBYTES - OHALF >= 2 * kRows * 4;
  __shared__ float s_ml_own[kMLInRing ? 1 : NW][2][kRows];
  auto ml_of = [&](int w) {
    return kMLInRing ? reinterpret_cast<float*>(s_ring1 + w * WBYTES + OHALF) : &s_ml_own[w][0][0];
  };
  char* const s_w0 = s_ring0 + wave * WBYTES;
  char* const s_w1 = s_ring1 + wave * WBYTES;
  // slot is a compile-time constant at every call (the tile loop is unrolled
  // over the ring)
  auto kbuf = [&](int slot) {
    return slot == 0 ? s_w0 : slot == 1 ? s_w1 : slot == 2 ? s_ring2 + wave * WBYTES
                                                            : s_ring3 + wave * WBYTES;
  };
  auto vbuf = [&](int slot) { return kbuf(slot) + TILE_BYTES; };
  // Byte offset inside a staged tile of chunk k of key row r.
  auto sw = [](int r, int k) { return r * ROWB + 16 * (k ^ ((r / RPB) & (CPR - 1))); };

  // Identity as the B operand of the int8 V transposes: lane l holds I[4*grp + j][n].
  u32x2 ident;
  {
    uint32_t e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = 4 * grp + j == n ? M::kOne : 0u;
    ident = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
  }
  const f32x4 vinit = {M::kVInit, M::kVInit, M::kVInit, M::kVInit};

  float m[RT], lsum[RT];   // reference maximum of row n of tile i (log2 units); this
                           // lane's share of its sum
  f32x4 o[RT][NT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    m[i] = kNegInf;
    lsum[i] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) o[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Tiles are loaded straight into the wave's LDS ring: load c of a tile
  // fills 1 KiB of LDS, lane i writing 16 bytes at i * 16; the lane fetches
  // the cache chunk that belongs at that position, so every load still reads
  // whole 128-byte lines of the tile.  A fetch with live == false reads
  // nothing (zero-record buffer resource), so the loop keeps one instruction
  // stream and one set of wait counts.
  int src_off[NL], src_off_v[NL];
  constexpr bool kSwizzleV = kInt8;
#pragma unroll
  for (int c = 0; c < NL; ++c) {
    const int slot = 64 * c + lane;          // destination 16-byte slot
    const int r = slot / CPR, p = slot % CPR;
    src_off[c] = r * ROWB + 16 * (p ^ ((r / RPB) & (CPR - 1)));
    // bf16 V rows: the layout of the transposed operand reads
    src_off_v[c] = kSwizzleV ? src_off[c] : r * ROWB + 16 * (p ^ vswz<ROWB>(r));
  }
  auto fetch = [&](int blk, bool live, int slot, float& ks, float& vs) {
    const int entry = tab.at(blk - blk_begin);
    if (lane == 0) check(!live || (entry >= 0 && entry < a.num_blocks), kCheckTableEntry, a.check_status);
    const int phys = min(max(entry, 0), a.num_blocks - 1);
    const size_t tile = (head_blocks + size_t(phys)) * TILE_BYTES;
    const int bytes = live ? TILE_BYTES : 0;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + tile, bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + tile, bytes);
#pragma unroll
    for (int c = 0; c < NL; ++c)
      buffer_load16_to_lds(kr, kbuf(slot) + 1024 * c, src_off[c]);
#pragma unroll
    for (int c = 0; c < NL; ++c)
      buffer_load16_to_lds(vr, vbuf(slot) + 1024 * c, src_off_v[c]);
    if constexpr (kInt8) {
      ks = a.k_scale[head_blocks + phys];
      vs = a.v_scale[head_blocks + phys];
    } else {
      ks = 1.0f;
      vs = 1.0f;
    }
  };
  // Loads a fetch issues (tile chunks, then the two int8 scales).
  constexpr int kFetchLoads = 2 * NL + (kInt8 ? 2 : 0);

  // int8 append: the staged block holding position L - 1 is requantized in
  // place, as pa_reshape_and_cache_quant does it ("A Rust inference server
  // for Qwen2 on Apple Silicon", "Day 4 measurements -- int8 KV", "Partial
  // blocks"): its 16 rows dequantized (code * old scale), row (L - 1) % 16
  // replaced by the new values, the new scale max|x| / 127 (1 for an all-zero
  // block), every value turned back into rint(x / scale) clipped to +-127 --
  // the same fp32 operations, so the same codes and scale.  Lane l owns the
  // 16-byte chunks l, l + 64, .. of the block (16-row-major); it keeps its
  // new codes for the store after the tile loop.  Returns the new scale.
  constexpr int NCH = kBlockSize * CPR / kWave;   // chunks per lane
  u32x4 rq[2][NCH > 0 ? NCH : 1] = {};
  auto requant = [&](char* t, const u32x4 (&nrow)[4], float s_old, u32x4 (&codes)[NCH > 0 ? NCH : 1]) {
    const int rn = (L - 1) % kBlockSize;
    const bool f32_in = a.new_dtype == kF32;
    float x[NCH][16];
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int idx = lane + kWave * k, row = idx / CPR, ch = idx % CPR;
      const u32x4 w = *reinterpret_cast<const u32x4*>(t + sw(row, ch));
#pragma unroll
      for (int e = 0; e < 16; ++e)
        x[k][e] = float(int8_t((w[e / 4] >> (8 * (e % 4))) & 0xFFu)) * s_old;
      if (row == rn) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float nb = (e & 1) ? bf16_hi(nrow[e / 8][(e / 2) % 4]) : bf16_lo(nrow[e / 8][(e / 2) % 4]);
          x[k][e] = f32_in ? __uint_as_float(nrow[e / 4][e % 4]) : nb;
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(x[k][e]));
    }
    m = stride_max<1>(m);
    const float s_new = m > 0.0f ? m / 127.0f : 1.0f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int idx = lane + kWave * k, row = idx / CPR, ch = idx % CPR;
      uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float c = fminf(fmaxf(__builtin_rintf(x[k][e] / s_new), -127.0f), 127.0f);
        wd[e / 4] |= uint32_t(uint8_t(int8_t(c))) << (8 * (e % 4));
      }
      codes[k] = u32x4{wd[0], wd[1], wd[2], wd[3]};
      *reinterpret_cast<u32x4*>(t + sw(row, ch)) = codes[k];
    }
    return s_new;
  };
  float rq_scale[2] = {1.0f, 1.0f};

  // Delayed rescaling: m is a reference maximum; weights are exp2(s - m), and
  // O and the sum are rescaled only when a row's tile maximum exceeds its
  // reference by more than kSlack (log2 units), so weights stay below 2^kSlack
  // and the rescale almost never runs.  The final division by the sum makes
  // the result independent of the reference.
  constexpr float kSlack = 8.0f;
  // PENDING: loads issued after this tile's fetch that may still be in flight.
  auto process = [&](auto pending_tag, int blk, int slot, float ks, float vs) {
    constexpr int PENDING = decltype(pending_tag)::value;
    // The tile's LDS writes are counted with the vector-memory loads.
    __builtin_amdgcn_s_waitcnt((PENDING & 15) | ((PENDING >> 4) << 14) | (7 << 4) | (15 << 8));
    __asm__ __volatile__("" ::: "memory");
    char* const sk = kbuf(slot);
    char* const sv = vbuf(slot);
    // bf16 key rows past the context may hold anything, even NaN: their V rows
    // are cleared (a zero weight must meet a finite value); their scores are
    // replaced, not multiplied, below.
    if constexpr (!kInt8) {
      if ((blk + 1) * kBlockSize > L) {
#pragma unroll
        for (int c = 0; c < NL; ++c) {
          const int key = (64 * c + lane) / CPR;
          if (blk * kBlockSize + key >= L)
            *reinterpret_cast<u32x4*>(sv + 1024 * c + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        }
      }
      // Append: the staged row of position L - 1 is replaced by the input row,
      // chunk k at its swizzled place in the K and in the V tile.
      if (append && blk == blk_new && lane < CPR) {
        const int r = (L - 1) % kBlockSize;
        *reinterpret_cast<u32x4*>(sk + r * ROWB + 16 * (lane ^ ((r / RPB) & (CPR - 1)))) = nk;
        *reinterpret_cast<u32x4*>(sv + r * ROWB + 16 * (lane ^ vswz<ROWB>(r))) = nv;
      }
    }
    if constexpr (kInt8 && append) {
      if (blk == blk_new) {
        ks = rq_scale[0] = requant(sk, nq[0], ks, rq[0]);
        vs = rq_scale[1] = requant(sv, nq[1], vs, rq[1]);
      }
    }
    // Scores of keys 4*grp .. 4*grp+3 for row n of each row tile: product c
    // takes key n's dims 32c + 8grp .. +7 as the A operand (read once for all
    // row tiles).  Row tiles past R hold no rows (uniform per workgroup).
    f32x4 s[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) s[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      u32x4 kop;
      if constexpr (kInt8) {
        const int k = (32 * c + 8 * grp) / 16;
        const uint2 w = *reinterpret_cast<const uint2*>(sk + sw(n, k) + 8 * (grp & 1));
        kop = codes8_f16(w.x, w.y);
      } else {
        kop = *reinterpret_cast<const u32x4*>(sk + sw(n, 4 * c + grp));
      }
#pragma unroll
      for (int i = 0; i < RT; ++i)
        if (i == 0 || kRows * i < R) s[i] = M::qk(kop, qb[i][c], s[i]);
    }
    const float ssc = sc * ks;
    u32x2 pa[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      if (i > 0 && kRows * i >= R) {
        pa[i] = u32x2{0u, 0u};
        continue;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pos = blk * kBlockSize + 4 * grp + j;
        const float x = (kInt8 ? s[i][j] - kI8Bias * qsum[i] : s[i][j]) * ssc;
        s[i][j] = pos <= last_vis[i] ? x : kNegInf;
      }
      // The rescale test on this lane's own four scores: some lane passes
      // m + kSlack exactly when the row (16 keys of the tile) does, so the
      // row maximum (two lane exchanges) is taken on the rare path only.
      const float lmax = nmax(nmax3(s[i][0], s[i][1], s[i][2]), s[i][3]);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(lmax > m[i] + kSlack) != 0, 0)) {   // rare
        const float tmax = nmax_xor32(nmax_xor16(lmax));
        const float mnew = fmaxf(m[i], tmax);
        const float alpha = mnew == kNegInf ? 1.0f : fast_exp2(m[i] - mnew);
        m[i] = mnew;
        lsum[i] *= alpha;
        // O rows 4*grp + j take the factor of that row (held by lane 4*grp + j).
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float ar = __shfl(alpha, 4 * grp + j);
#pragma unroll
          for (int t = 0; t < NT; ++t) o[i][t][j] *= ar;
        }
      }
      const float mref = m[i] == kNegInf ? 0.0f : m[i];
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = fast_exp2(s[i][j] - mref);
      // P as the A operand (row n, keys 4*grp ..), bf16; an int8 tile's V scale
      // rides on it.
      pa[i] = u32x2{pack_bf16_round(p[0] * vs, p[1] * vs), pack_bf16_round(p[2] * vs, p[3] * vs)};
      // The row sum adds the weights as rounded for the P.V product (an int8
      // tile's divided by its V scale again), so numerator and denominator use
      // one set of weights.
      if constexpr (kInt8)
        lsum[i] = __builtin_fmaf(add_bf16_pair(pa[i][0], add_bf16_pair(pa[i][1], 0.0f)),
                                 __builtin_amdgcn_rcpf(vs), lsum[i]);
      else
        lsum[i] = add_bf16_pair(pa[i][0], add_bf16_pair(pa[i][1], lsum[i]));
    }
    // V of keys 4*grp .. 4*grp+3 at dim 16t + n (the B operand), read once for
    // all row tiles.  bf16: the NT transposed reads in one batch.
    u32x2 vbt[NT];
    if constexpr (!kInt8) {
      uint32_t va[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) va[t] = v_tr_addr<ROWB>(sv, t, lane);
      lds_read_tr<NT>(va, vbt);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      u32x2 vb;
      if constexpr (kInt8) {
        // key n's codes of dims 16t + 4grp .. +3, turned by the identity product
        const uint32_t u = *reinterpret_cast<const uint32_t*>(sv + sw(n, t) + 4 * grp) ^ 0x80808080u;
        const f32x4 tv = M::mm16(u32x2{f16pair_lo(u), f16pair_hi(u)}, ident, vinit);
        vb = u32x2{pack_bf16_exact(tv[0], tv[1]), pack_bf16_exact(tv[2], tv[3])};
      } else {
        vb = vbt[t];   // four keys of one dim
      }
#pragma unroll
      for (int i = 0; i < RT; ++i)
        if (i == 0 || kRows * i < R) o[i][t] = pv16(pa[i], vb, o[i][t]);
    }
    // This slot is loaded again next: its reads must be done first.
    __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));
  };

  // Each wave takes every NW-th tile of the piece through a ring of NS LDS
  // slots: tile j is used from slot j % NS while tiles j+1 .. j+NS-1 load.
  // Every step issues exactly one fetch (past the wave's last tile it reads
  // nothing), so the loads issued after a tile's own are always NS - 1
  // fetches' worth and one wait count serves every step.
  using Pend = std::integral_constant<int, (NS - 1) * kFetchLoads>;
  const int first = blk_begin + wave;
  const int n_my = first < blk_end ? cdiv(blk_end - first, NW) : 0;
  if (n_my > 0) {
    const int last = n_my - 1;
    auto tile = [&](int j) { return first + min(j, last) * NW; };
    float ks[NS], vs[NS];
#pragma unroll
    for (int v = 0; v < NS - 1; ++v) fetch(tile(v), v <= last, v, ks[v], vs[v]);
    for (int j = 0; j <= last; j += NS) {
#pragma unroll
      for (int v = 0; v < NS; ++v) {
        const int nf = (v + NS - 1) % NS;   // slot of tile j + v + NS - 1 (constant once unrolled)
        fetch(tile(j + v + NS - 1), j + v + NS - 1 <= last, nf, ks[nf], vs[nf]);
        if (j + v <= last) process(Pend{}, first + (j + v) * NW, v, ks[v], vs[v]);
      }
    }
  }
  // The last prefetch (reading nothing) may still be writing its LDS slot:
  // wait for it before the slots are reused below.
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
  __asm__ __volatile__("" ::: "memory");

  if constexpr (append && kInt8) {
    // The wave that requantized the block stores its codes and the two
    // scales at the slot's block (slots < 0 skipped, slots past the pool
    // ignored).
    if (piece == n_pieces - 1 && blk_new >= 0 && wave == (blk_new - blk_begin) % NW) {
      if (threadIdx.x % kWave == 0)
        check(new_slot < int64_t(a.num_blocks) * kBlockSize, kCheckSlot, a.check_status);
      if (new_slot >= 0 && new_slot < int64_t(a.num_blocks) * kBlockSize) {
        const size_t blk_off = (size_t(g) * a.num_blocks + size_t(new_slot / kBlockSize)) * TILE_BYTES;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
          const int idx = lane + kWave * k, row = idx / CPR, ch = idx % CPR;
          const size_t off = blk_off + size_t(row) * ROWB + 16 * size_t(ch);
          *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(const_cast<void*>(a.k_cache)) + off) = rq[0][k];
          *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(const_cast<void*>(a.v_cache)) + off) = rq[1][k];
        }
        if (lane == 0) {
          const size_t sidx = size_t(g) * a.num_blocks + size_t(new_slot / kBlockSize);
          const_cast<float*>(a.k_scale)[sidx] = rq_scale[0];
          const_cast<float*>(a.v_scale)[sidx] = rq_scale[1];
        }
      }
    }
  }
  if constexpr (append && !kInt8) {
    // (after the loop: issued before it, the store held wave 0's first tile
    // loads back until the new row had arrived)
    if (piece == n_pieces - 1) {
      if (threadIdx.x == 0)
        check(new_slot < int64_t(a.num_blocks) * kBlockSize, kCheckSlot, a.check_status);
      if (wave == 0 && lane < CPR && new_slot >= 0 &&
          new_slot < int64_t(a.num_blocks) * kBlockSize) {
        const size_t dst =
            (size_t(g) * a.num_blocks * kBlockSize + size_t(new_slot)) * ROWB + 16 * lane;
        *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(const_cast<void*>(a.k_cache)) + dst) = nk;
        *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(const_cast<void*>(a.v_cache)) + dst) = nv;
      }
    }
  }

  // Per row tile: row totals (the four key quads of each row), the wave's O
  // rows to its own LDS region (its staging buffers are no longer read); then
  // one thread per row turns the waves' maxima and sums into one weight per
  // wave (exp2(m_w - M) / total) and the row's output index, and every output
  // element is a weighted sum of the waves' values, read in one batch.  A
  // barrier before the next tile reuses the regions.
  __shared__ float s_coef[NW][kRows];
  __shared__ float s_lse[kRows];
  __shared__ long long s_orow[kRows];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    if (i > 0 && kRows * i >= R) break;   // uniform per workgroup
    if (i > 0) __syncthreads();
    const float lrow = add_xor32(add_xor16(lsum[i]));
    if (grp == 0) {
      ml_of(wave)[n] = m[i];
      ml_of(wave)[kRows + n] = lrow;
    }
    // O rows 0-7 of the tile go to the wave's slot-0 region, rows 8-15 to its
    // slot-1 region.
    float* const s_ow = reinterpret_cast<float*>(grp < 2 ? s_w0 : s_w1);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) s_ow[(4 * (grp & 1) + j) * D + 16 * t + n] = o[i][t][j];
    __syncthreads();

    const int rows_here = min(R - kRows * i, kRows);
    // Row weights: lane w of each group of NW lanes in the first waves takes
    // wave w's maximum and sum of row rl (rows past R included, they hold
    // -inf and 0); the group reduces them with DPP.
    static_assert(NW <= 16 && (NW & (NW - 1)) == 0, "weights use groups of NW lanes in one DPP row");
    if (threadIdx.x < kRows * NW) {
      const int rl = threadIdx.x / NW, w = threadIdx.x % NW;
      const float mw = ml_of(w)[rl], lw = ml_of(w)[kRows + rl];
      const float mx = group_max<NW>(mw);
      const float f = mw == kNegInf ? 0.0f : fast_exp2(mw - mx);
      const float lt = group_sum<NW>(lw * f);
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      s_coef[w][rl] = f * inv;
      if (w == 0 && rl < rows_here) {
        s_lse[rl] = lt > 0.0f ? mx + __log2f(lt) : kNegInf;
        const int row = kRows * i + rl;
        const int tq = row / G;
        s_orow[rl] = (long long)((size_t(q0) + tq) * Hq + size_t(g) * G + (row - tq * G));
      }
    }
    __syncthreads();

    // Two output elements per thread per pass, their LDS reads issued
    // together (a row index past the tile is clamped for the read and not
    // stored).
    for (int t0 = threadIdx.x; t0 < rows_here * D; t0 += 2 * NW * kWave) {
      float ot[2];
      int rls[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = t0 + u * NW * kWave;
        const int rl = min(t / D, kRows - 1), d = t % D;
        rls[u] = t < rows_here * D ? rl : -1;
        const int half = rl < kRows / 2 ? 0 : 1;
        const int off = (rl % (kRows / 2)) * D + d;
        float ow[NW], cw[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          cw[w] = s_coef[w][rl];
          ow[w] = reinterpret_cast<const float*>((half ? s_ring1 : s_ring0) + w * WBYTES)[off];
        }
        float x = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) x = __builtin_fmaf(ow[w], cw[w], x);
        ot[u] = x;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int rl = rls[u];
        if (rl < 0) continue;
        const int d = (t0 + u * NW * kWave) % D;
        const size_t orow = size_t(s_orow[rl]);
        if (n_pieces == 1) {
          reinterpret_cast<bf16_t*>(a.out)[orow * D + d].bits = f32_to_bf16(ot[u]);
        } else {
          const size_t prow = orow * a.max_pieces + piece;
          a.part_o[prow * D + d] = ot[u];
          if (d == 0) a.part_lse[prow] = s_lse[rl];
        }
      }
    }
  }
}

// LDS ring slots per wave: two (with eight waves a bf16 ring fills 128 KiB).
// int8 tiles are half the size, but three and four slots were measured slower
// on the long-context workload, in one process on the same caches (29.8 and
// 30.3 us against 28.6 us per call; also with the refill issued before the
// tile's arithmetic): more tiles in flight per wave only add contention.
#ifndef PA_ROWS_SLOTS_INT8
#define PA_ROWS_SLOTS_INT8 2
#endif
template <typename KV> struct RowsSlots : std::integral_constant<int, 2> {};
#ifndef PA_ROWS_WAVES
#define PA_ROWS_WAVES 8
#endif
template <> struct RowsSlots<i8_t> : std::integral_constant<int, PA_ROWS_SLOTS_INT8> {};

// Row tiles per (sequence, KV head) for rows = T * G query rows.
__host__ __device__ constexpr int row_tiles(long rows) { return int((rows + kRows - 1) / kRows); }

template <typename KV, int RT>
hipError_t launch_rows_rt(const DecodeArgs& a, hipStream_t stream) {
  // Eight waves per (piece, sequence, KV head): a long piece's tiles spread
  // over more waves, and with one such workgroup per CU (its LDS ring takes
  // 128 KiB for bf16, D = 128) later workgroups fill CUs as early ones finish.
  // Measured against four waves: verify 35.2 -> 33.4 us, Qwen2-shaped decode
  // 9.5 -> 9.2 us, long-context int8 equal at twice the piece length.
  constexpr int NW = PA_ROWS_WAVES;
  const long wgs = long(a.max_pieces) * a.num_seqs * a.kv_heads;
  if (a.new_k) {
    // Decode with append: one query token per sequence, groups of at most 16
    // heads (one row tile); the host refuses other shapes.
    if constexpr (RT == 1) {
      if (a.head_dim == 128)
        rows_pass1<KV, 128, NW, RowsSlots<KV>::value, 1, true><<<dim3(unsigned(wgs)), NW * kWave, 0, stream>>>(a);
      else
        rows_pass1<KV, 64, NW, RowsSlots<KV>::value, 1, true><<<dim3(unsigned(wgs)), NW * kWave, 0, stream>>>(a);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (a.head_dim == 128)
    rows_pass1<KV, 128, NW, RowsSlots<KV>::value, RT><<<dim3(unsigned(wgs)), NW * kWave, 0, stream>>>(a);
  else
    rows_pass1<KV, 64, NW, RowsSlots<KV>::value, RT><<<dim3(unsigned(wgs)), NW * kWave, 0, stream>>>(a);
  return hipGetLastError();
}

template <typename KV>
hipError_t launch_rows_t(const DecodeArgs& a, hipStream_t stream) {
  switch (row_tiles(long(a.num_query_tokens) * (a.q_heads / a.kv_heads))) {
    case 1: return launch_rows_rt<KV, 1>(a, stream);
    case 2: return launch_rows_rt<KV, 2>(a, stream);
    case 3: return launch_rows_rt<KV, 3>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename KV, int D, int RT>
int resident_rt() {
  int n = 0;
  constexpr int NW = PA_ROWS_WAVES;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &n, rows_pass1<KV, D, NW, RowsSlots<KV>::value, RT>, NW * kWave, 0);
  return e == hipSuccess && n > 0 ? n : 1;
}
template <typename KV, int D>
int resident_d(int rt) {
  return rt <= 1 ? resident_rt<KV, D, 1>() : rt == 2 ? resident_rt<KV, D, 2>() : resident_rt<KV, D, 3>();
}

}  // namespace

bool rows_supported(int q_dtype, int kv_dtype, int head_dim, int G, int T) {
  return q_dtype == kBF16 && (kv_dtype == kBF16 || kv_dtype == kI8) &&
         (head_dim == 64 || head_dim == 128) && G >= 1 && T >= 1 &&
         long(G) * T <= long(kRows) * kMaxRowTiles;
}

int rows_pass1_resident(int kv_dtype, int head_dim, int rows) {
  const int rt = row_tiles(rows);
  if (kv_dtype == kI8) return head_dim == 64 ? resident_d<i8_t, 64>(rt) : resident_d<i8_t, 128>(rt);
  return head_dim == 64 ? resident_d<bf16_t, 64>(rt) : resident_d<bf16_t, 128>(rt);
}

hipError_t launch_rows_pass1(const DecodeArgs& a, hipStream_t stream) {
  return a.kv_dtype == kI8 ? launch_rows_t<i8_t>(a, stream) : launch_rows_t<bf16_t>(a, stream);
}

}  // namespace pa
