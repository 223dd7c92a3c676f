// Paged grouped-query decode attention for gfx950.
//
// Pass 1: one workgroup per (piece of context, KV head, sequence).  It walks
// the sequence's block table over its piece, reads each 16-token K and V tile
// in place from the head-major cache with coalesced 16-byte loads (one
// wave-wide load covers 1 KiB of a tile), scores every query head of the
// group against each key read once, and keeps an fp32 online softmax (running
// maximum and sum, rescaled tile by tile) -- the kernel of "From 183 ms to 19
// ms per decode step", section "Four changes, one profile at a time", change 3.
//
// Lane layout for one wave-wide load: LPK consecutive lanes hold one key row
// (16 bytes each), so a load holds KPL = 64 / LPK key rows and a tile takes
// LPB = 16 / KPL loads.  A key's score for one head is a sum over its LPK
// lanes (DPP butterflies inside 16-lane rows).  Each lane keeps its own
// running sum and accumulator for the key rows it sees (one per load), so the
// per-tile work needs no cross-row exchange; the reference maximum is one per
// wave (raised rarely, see below), so at the end the rows of a wave add up
// as they are, and then the waves are merged.
//
// With a single piece the workgroup writes the output row directly.  With
// several pieces it writes a normalised partial output and its log2-sum-exp
// to the workspace, and a merge pass combines the pieces of each row.  (A
// merge inside this kernel by the last workgroup to arrive was measured: the
// arrival counter, the write-through of the partials and their reads put
// several microseconds on the tail, more than the second launch costs.)
// Piece length is fixed per call (never derived from the lengths in the
// batch), so each sequence's arithmetic depends on its own length only.
//
// This kernel serves fp32 and bf16 caches.  Over an int8 cache the per-key
// conversions and products bind on the vector ALUs; that case runs on the
// matrix cores (pa_verify.hip).
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"

#ifndef PA_PPL2_MAX_G
#define PA_PPL2_MAX_G 4
#endif


namespace pa {
namespace {

// Lane layout of a 16-token tile.  A lane's load unit is a 16-byte piece.  A
// lane holds PPL pieces of one key row (E = PPL * EPL elements): piece p
// covers dims p*D/PPL + c*EPL .. +EPL, with c = lane % LPK.  LPK lanes share
// a key row, a wave-wide load covers KPL rows, and load i reads piece i % PPL
// of key rows (i / PPL) * KPL + lane / LPK.  Every wave-wide load covers whole
// spans of 128 bytes or more of each row it touches.
template <typename KV, int D, int G>
struct Geo {
  static constexpr int PB = 16;                       // bytes per piece
  static constexpr int EPL = PB / int(sizeof(KV));    // elements per piece
  // Two pieces per lane halve the reduction steps per score but double the
  // per-lane accumulator; worth it for small bf16 groups only.
  static constexpr int PPL = (__is_same(KV, bf16_t) && G <= PA_PPL2_MAX_G) ? 2 : 1;  // pieces per lane
  static constexpr int E = PPL * EPL;                 // elements per lane per key row
  static constexpr int LPK = D / E;                   // lanes per key row
  static constexpr int KPL = kWave / LPK;             // key rows per wave-wide load
  static constexpr int ROWB = D * int(sizeof(KV));    // bytes per key row
  static constexpr int LPB = kBlockSize * ROWB / (kWave * PB);  // wave-wide loads per tile
  static constexpr int KR = LPB / PPL;                // key rows per lane per tile
  static constexpr int TILE_BYTES = kBlockSize * ROWB;
  static_assert(LPK >= 1 && LPK <= kWave && KR * KPL == kBlockSize, "unsupported geometry");
  // Byte offset of load i for this lane (r = lane / LPK, c = lane % LPK).
  __device__ static int offset(int i, int r, int c) {
    return (i / PPL) * (KPL * ROWB) + r * ROWB + (i % PPL) * (ROWB / PPL) + c * PB;
  }
};

// ---------------------------------------------------------------------------
// Query registers and per-load dot products for each (q, cache) dtype pair.
// ---------------------------------------------------------------------------
template <typename Q, typename KV, int D, int G> struct QRegs;

// fp32 q, fp32 cache.
template <int D, int G> struct QRegs<float, float, D, G> {
  float q[G][4];
  __device__ void load(const float* qrow, int c) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      u32x4 w = load16(qrow + size_t(h) * D + c * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) q[h][e] = __uint_as_float(w[e]);
    }
  }
  __device__ float dot_row(int h, const u32x4* k) const {
    float s = q[h][0] * __uint_as_float(k[0][0]);
#pragma unroll
    for (int e = 1; e < 4; ++e) s = __builtin_fmaf(q[h][e], __uint_as_float(k[0][e]), s);
    return s;
  }
};

// bf16 q, bf16 cache: packed bf16 dot products into fp32, PPL 16-byte pieces
// per lane.
template <int D, int G> struct QRegs<bf16_t, bf16_t, D, G> {
  static constexpr int PPL = Geo<bf16_t, D, G>::PPL;
  uint32_t q[G][PPL][4];
  __device__ void load(const bf16_t* qrow, int c) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int p = 0; p < PPL; ++p) {
        u32x4 w = load16(qrow + size_t(h) * D + p * (D / PPL) + c * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) q[h][p][e] = w[e];
      }
  }
  __device__ float dot_row(int h, const u32x4* k) const {
    float s = 0.0f;
#pragma unroll
    for (int p = 0; p < PPL; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // Copy the element out first: a bit cast applied directly to an
        // element of a vector value reads element 0 with this compiler.
        const uint32_t kw = k[p][e];
        const uint32_t qw = q[h][p][e];
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw),
                                            __builtin_bit_cast(bf16x2, kw), s, false);
      }
    return s;
  }
};

// V tile values of one load, widened to fp32.
template <typename KV> struct VWiden;
template <> struct VWiden<float> {
  static constexpr int EPL = 4;
  __device__ static void run(u32x4 v, float (&o)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __uint_as_float(v[e]);
  }
};
template <> struct VWiden<bf16_t> {
  static constexpr int EPL = 8;
  __device__ static void run(u32x4 v, float (&o)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = bf16_lo(v[e]);
      o[2 * e + 1] = bf16_hi(v[e]);
    }
  }
};
template <typename T> __device__ __forceinline__ void store_out(T* p, float v);
template <> __device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_out<bf16_t>(bf16_t* p, float v) {
  p->bits = f32_to_bf16(v);
}

// ---------------------------------------------------------------------------
// Pass 1
// ---------------------------------------------------------------------------
// With 8 waves per workgroup, keep two workgroups per CU (4 waves per SIMD,
// at most 128 VGPRs); with 4 the register budget is left to the compiler.
template <typename Q, typename KV, int D, int G, int NW, int RING, bool APPEND>
__global__ __launch_bounds__(NW * kWave, NW >= 8 ? (NW * 2) / 4 : 1) void decode_pass1(DecodeArgs a) {
  using GE = Geo<KV, D, G>;
  constexpr int EPL = GE::EPL, PPL = GE::PPL, E = GE::E, LPK = GE::LPK, KPL = GE::KPL;
  constexpr int LPB = GE::LPB, KR = GE::KR;
  // bf16 V: products over key pairs (below); needs an even count of key rows per lane.
  constexpr bool kPairPV = __is_same(KV, bf16_t) && KR % 2 == 0;
  using P = u32x4;

  // 1-D grid, piece-major: ids 0 .. N*Hkv-1 are piece 0 of every (sequence,
  // KV head), then piece 1, ...  Consecutive ids go to different XCDs, so the
  // always-present first pieces spread evenly over the chip, and all pieces of
  // one (sequence, head) land on the same XCD whenever N*Hkv is a multiple of 8.
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPK;   // key row inside a load
  const int c = lane % LPK;   // which 16-byte column of each piece

  // The work unit (natural order or a work plan) and the piece's table
  // entries (spread over the lanes; a tile's physical block is then read
  // with readlane), then this group's query rows: in the natural order the
  // length, the table row and q arrive in one round trip.
  PieceTable<kTabRegs> tab;
  const WorkItem it = work_item(a, tab, lane);
  const int b = it.b, piece = it.piece, g = it.g;
  const int split_blocks = a.split_tokens / kBlockSize;
  const int blk_begin = piece * split_blocks;
  const Q* qrow = reinterpret_cast<const Q*>(a.q) + (size_t(b) * a.q_heads + size_t(g) * G) * D;
  QRegs<Q, KV, D, G> qr;
  qr.load(qrow, c);

  // Append mode: this lane's pieces of the new token's K and V (position
  // L - 1), and its slot.  Requested after the first tiles' loads (below):
  // requested before them, every wait for a tile also waited for these rows
  // (20.47 -> 20.21 us per batch-64 launch, same process).
  P nk[PPL], nv[PPL];
  int64_t slot = -1;
  auto load_new = [&]() {
    if constexpr (APPEND) {
      const size_t row = (size_t(b) * a.kv_heads + g) * GE::ROWB;
#pragma unroll
      for (int p = 0; p < PPL; ++p) {
        const size_t off = row + size_t(p) * (GE::ROWB / PPL) + size_t(c) * GE::PB;
        nk[p] = *reinterpret_cast<const P*>(reinterpret_cast<const char*>(a.new_k) + off);
        nv[p] = *reinterpret_cast<const P*>(reinterpret_cast<const char*>(a.new_v) + off);
      }
      slot = a.slot_mapping[b];
    }
  };

  // Lengths beyond the table are clamped so that no access leaves the
  // buffers (the result of such a call is unspecified).
  const int L = it.L;
  const int n_pieces = min(L > 0 ? cdiv(L, a.split_tokens) : 1, a.max_pieces);
  if (piece < 0 || piece >= n_pieces) return;

  const int blk_end = min(cdiv(L, kBlockSize), blk_begin + split_blocks);
  const size_t head_blocks = size_t(g) * a.num_blocks;
  const char* kbase = reinterpret_cast<const char*>(a.k_cache);
  const char* vbase = reinterpret_cast<const char*>(a.v_cache);
  const float sc_log2 = a.scale * kLog2e;

  float m[G], l[G], acc[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;
  }

  // Out-of-range table entries are clamped into the pool (unspecified
  // result, but no access outside the cache).
  int lane_off[LPB];
#pragma unroll
  for (int i = 0; i < LPB; ++i) lane_off[i] = GE::offset(i, r, c);
  // A fetch with live == false (past the wave's last tile) keeps the
  // instruction stream, and so the wait counts, identical but reads nothing:
  // its buffer resource has zero records.
  auto fetch = [&](int blk, bool live, P (&kt)[LPB], P (&vt)[LPB]) {
    const int entry = tab.at(blk - blk_begin);
    if (lane == 0) check(!live || (entry >= 0 && entry < a.num_blocks), kCheckTableEntry, a.check_status);
    const int phys = min(max(entry, 0), a.num_blocks - 1);
    const size_t tile = (head_blocks + size_t(phys)) * GE::TILE_BYTES;
    const int bytes = live ? GE::TILE_BYTES : 0;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + tile, bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + tile, bytes);
#pragma unroll
    for (int i = 0; i < LPB; ++i) kt[i] = buffer_load16_stream(kr, lane_off[i]);
#pragma unroll
    for (int i = 0; i < LPB; ++i) vt[i] = buffer_load16_stream(vr, lane_off[i]);
  };

  // Reduce one tile.  MASK (only for a sequence's last, partial block) drops
  // positions >= L and zeroes their V rows: rows past the context may hold
  // anything, even NaN, and a zero weight must meet a finite value.
  //
  // Delayed rescaling: m is a reference maximum, not necessarily the running
  // one, and the same in every lane of the wave.  Weights are exp2(s - m); the
  // accumulator is rescaled only when some score of the wave exceeds the
  // reference by more than kSlack (log2 units), and then the reference becomes
  // the wave's maximum, so weights stay below 2^kSlack in fp32 and the rescale
  // (one multiply per accumulator element) almost never runs.  The final
  // normalisation by the running sum makes the result independent of m.
  constexpr float kSlack = 8.0f;
  auto process = [&](auto mask_tag, int blk, P (&kt)[LPB], P (&vt)[LPB]) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if constexpr (MASK && APPEND) {
      // Position L - 1 is the token being appended: take its row from the input.
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        const bool is_new = blk * kBlockSize + k * KPL + r == L - 1;
#pragma unroll
        for (int p = 0; p < PPL; ++p)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            kt[k * PPL + p][w] = is_new ? nk[p][w] : kt[k * PPL + p][w];
            vt[k * PPL + p][w] = is_new ? nv[p][w] : vt[k * PPL + p][w];
          }
      }
    }
    float s[G][KR];
#pragma unroll
    for (int k = 0; k < KR; ++k)
#pragma unroll
      for (int h = 0; h < G; ++h) s[h][k] = qr.dot_row(h, &kt[k * PPL]);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int k = 0; k < KR; ++k) s[h][k] = group_sum<LPK>(s[h][k]) * sc_log2;
    if constexpr (MASK) {
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        const bool valid = blk * kBlockSize + k * KPL + r < L;
#pragma unroll
        for (int h = 0; h < G; ++h) s[h][k] = valid ? s[h][k] : kNegInf;
#pragma unroll
        for (int p = 0; p < PPL; ++p)
#pragma unroll
          for (int w = 0; w < 4; ++w) vt[k * PPL + p][w] = valid ? vt[k * PPL + p][w] : 0u;
      }
    }
    // One comparison per head: the lane's largest score against its reference.
    float smax[G];
    bool grow = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      smax[h] = s[h][0];
#pragma unroll
      for (int k = 1; k < KR; ++k) smax[h] = fmaxf(smax[h], s[h][k]);
      grow |= smax[h] > m[h] + kSlack;
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) != 0, 0)) {  // wave-uniform, rare
#pragma unroll
      for (int h = 0; h < G; ++h) {
        // over the wave's key rows: one reference per wave
        const float mnew = fmaxf(m[h], stride_max<LPK>(smax[h]));
        const float alpha = m[h] == kNegInf ? 0.0f : fast_exp2(m[h] - mnew);
        m[h] = mnew;
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
      }
    }
    if constexpr (kPairPV) {
      // bf16 cache: the lane's key rows in pairs, each dimension's two values
      // in one word, so that one packed product adds both rows' terms.  The
      // weights are rounded to bf16 for this product (as on the matrix
      // cores), and the running sum adds the rounded weights: numerator and
      // denominator use one set of weights.
      uint32_t vp[KR / 2][E];
#pragma unroll
      for (int k2 = 0; k2 < KR / 2; ++k2)
#pragma unroll
        for (int p = 0; p < PPL; ++p)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t lo = vt[(2 * k2) * PPL + p][w], hi = vt[(2 * k2 + 1) * PPL + p][w];
            vp[k2][p * EPL + 2 * w] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
            vp[k2][p * EPL + 2 * w + 1] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
          }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mref = m[h] == kNegInf ? 0.0f : m[h];
        float pw[KR];
#pragma unroll
        for (int k = 0; k < KR; ++k) pw[k] = fast_exp2(s[h][k] - mref);
        bf16x2 pp[KR / 2];
        const bf16x2 ones = {__bf16(1.0f), __bf16(1.0f)};
        float lh = l[h];
#pragma unroll
        for (int k2 = 0; k2 < KR / 2; ++k2) {
          pp[k2] = pack_bf16x2(pw[2 * k2], pw[2 * k2 + 1]);
          lh = __builtin_amdgcn_fdot2_f32_bf16(pp[k2], ones, lh, false);
        }
        l[h] = lh;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float x = acc[h][e];
#pragma unroll
          for (int k2 = 0; k2 < KR / 2; ++k2)
            x = __builtin_amdgcn_fdot2_f32_bf16(pp[k2], __builtin_bit_cast(bf16x2, vp[k2][e]), x,
                                                false);
          acc[h][e] = x;
        }
      }
      return;
    }
    float vf[KR][E];
#pragma unroll
    for (int k = 0; k < KR; ++k)
#pragma unroll
      for (int p = 0; p < PPL; ++p) {
        float tmp[EPL];
        VWiden<KV>::run(vt[k * PPL + p], tmp);
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[k][p * EPL + e] = tmp[e];
      }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      // A row that has seen no position yet keeps m = -inf and weight 0.
      const float mref = m[h] == kNegInf ? 0.0f : m[h];
      float pw[KR];
      float psum = 0.0f;
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        pw[k] = fast_exp2(s[h][k] - mref);
        psum += pw[k];
      }
      l[h] += psum;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float x = acc[h][e];
#pragma unroll
        for (int k = 0; k < KR; ++k) x = __builtin_fmaf(pw[k], vf[k][e], x);
        acc[h][e] = x;
      }
    }
  };

  // Each wave takes every NW-th tile of the piece.  Tiles go through a ring
  // of RING register buffers: while tile j is reduced, tiles j+1 .. j+RING-1
  // are in flight.  The loop is unrolled over the ring so buffer indices are
  // compile-time constants.  Fetches inside the loop are unconditional (past
  // the wave's last tile they read nothing, see fetch), so every path has the
  // same loads outstanding and each wait covers exactly the tile about to be
  // reduced.  The sequence's masked last tile (and, in append mode, the tile
  // holding position L - 1) is reduced after the loop.
  using Plain = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  const int first = blk_begin + wave;
  const int n_my = first < blk_end ? cdiv(blk_end - first, NW) : 0;
  if (n_my > 0) {
    const int last = n_my - 1;
    const int last_blk = first + last * NW;
    const bool last_masked = (last_blk + 1) * kBlockSize > L ||
                             (APPEND && last_blk == cdiv(L, kBlockSize) - 1);
    const int n_plain = last_masked ? last : n_my;
    auto tile = [&](int j) { return first + min(j, last) * NW; };
    P kb[RING][LPB], vb[RING][LPB];
#pragma unroll
    for (int v = 0; v < RING - 1; ++v) fetch(tile(v), v <= last, kb[v], vb[v]);
    load_new();
    int j = 0;
    for (; j + RING - 1 < n_plain; j += RING) {
#pragma unroll
      for (int v = 0; v < RING; ++v) {
        const int nb = (v + RING - 1) % RING;  // constant once unrolled
        fetch(tile(j + v + RING - 1), j + v + RING - 1 <= last, kb[nb], vb[nb]);
        process(Plain{}, tile(j + v), kb[v], vb[v]);
      }
    }
    // Fewer than RING plain tiles remain, then possibly the masked one; tiles
    // up to j + RING - 2 are already in flight.
#pragma unroll
    for (int v = 0; v < RING; ++v) {
      if (j + v <= last) {
        if (v == RING - 1) fetch(tile(j + v), true, kb[v], vb[v]);
        if (j + v < n_plain)
          process(Plain{}, tile(j + v), kb[v], vb[v]);
        else
          process(Masked{}, tile(j + v), kb[v], vb[v]);
      }
    }
  } else {
    load_new();   // no tiles here; wave 0 may still write the new row
  }

  if constexpr (APPEND) {
    // The last piece writes the new row into the cache (one key row: the
    // first LPK lanes of wave 0, PPL pieces each).  Only this workgroup uses
    // position L - 1, and it took that row from registers, not the cache, so
    // the store waits until the tile loop is done: issued before the loop it
    // held wave 0's first tile loads back until the new row had arrived.
    // (Issued inside the loop, or as a streaming or write-through store, it
    // measured no faster, or slower: the ~0.7 us this store adds to a
    // batch-64 launch is the memory side's cost of 2048 scattered lines.)
    if (piece == n_pieces - 1 && threadIdx.x == 0)
      check(slot < int64_t(a.num_blocks) * kBlockSize, kCheckSlot, a.check_status);
    if (piece == n_pieces - 1 && wave == 0 && r == 0 && slot >= 0 &&
        slot < int64_t(a.num_blocks) * kBlockSize) {
      const size_t dst = (size_t(g) * a.num_blocks * kBlockSize + size_t(slot)) * GE::ROWB;
#pragma unroll
      for (int p = 0; p < PPL; ++p) {
        const size_t off = dst + size_t(p) * (GE::ROWB / PPL) + size_t(c) * GE::PB;
        *reinterpret_cast<P*>(reinterpret_cast<char*>(const_cast<void*>(a.k_cache)) + off) = nk[p];
        *reinterpret_cast<P*>(reinterpret_cast<char*>(const_cast<void*>(a.v_cache)) + off) = nv[p];
      }
    }
  }

  // Merge the key rows of this wave (lanes c, c + LPK, c + 2 LPK, ...): they
  // share the wave's reference maximum, so the sums add as they are and the
  // accumulators are reduce-scattered over lane ^ 32 and lane ^ 16 (each swap
  // step halves the values a lane holds); the row groups left inside a
  // 16-lane row are summed with the other waves through LDS.  (A reference per
  // lane, brought to the wave's maximum here, put one more reduction, an exp2
  // and a multiply per accumulator value on the launch's last workgroup:
  // 0.15 us per launch on the batch-64 workload, same process and caches.)
  constexpr int V = G * E;                                   // accumulator values per lane
  constexpr int X32 = LPK <= 32 ? 2 : 1, X16 = LPK <= 16 ? 2 : 1;
  constexpr int KEEP = V / (X32 * X16);                      // values a lane keeps
  constexpr int RG = LPK < 16 ? 16 / LPK : 1;                // row groups left per lane row
  float red[V];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = stride_sum<LPK>(l[h]);
#pragma unroll
    for (int e = 0; e < E; ++e) red[h * E + e] = acc[h][e];
  }
  if constexpr (X32 == 2) {
    // Lanes 0-31 keep the reduced first half of the values, lanes 32-63 the second.
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(red[i]),
                                                      __float_as_uint(red[i + V / 2]), false, false);
      red[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  }
  if constexpr (X16 == 2) {
    // Even 16-lane rows keep the first half of what is left, odd rows the second.
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(red[i]),
                                                      __float_as_uint(red[i + V / 4]), false, false);
      red[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  }

  // Merge the waves through LDS.
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_acc[NW][RG][G][D];
  {
    const int kbase = ((X32 == 2 ? (lane >> 5) * X16 : 0) + (X16 == 2 ? (lane >> 4) & 1 : 0)) * KEEP;
    const int rg = RG > 1 ? (lane & 15) / LPK : 0;
#pragma unroll
    for (int i = 0; i < KEEP; ++i) {
      const int v = kbase + i;
      const int h = v / E, e = v - h * E;
      s_acc[wave][rg][h][(e / EPL) * (D / PPL) + c * EPL + e % EPL] = red[i];
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  const int Hq = a.q_heads;
  for (int t = threadIdx.x; t < G * D; t += NW * kWave) {
    const int h = t / D, d = t % D;
    // Every LDS value this output needs, read in one batch.
    float mw[NW], lw[NW], xw[NW][RG];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = s_m[w][h];
      lw[w] = s_l[w][h];
#pragma unroll
      for (int j = 0; j < RG; ++j) xw[w][j] = s_acc[w][j][h][d];
    }
    float M = mw[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, mw[w]);
    float lsum = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = mw[w] == kNegInf ? 0.0f : fast_exp2(mw[w] - M);
      lsum = __builtin_fmaf(lw[w], f, lsum);
      float x = xw[w][0];
#pragma unroll
      for (int j = 1; j < RG; ++j) x += xw[w][j];
      o = __builtin_fmaf(x, f, o);
    }
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    const size_t row = size_t(b) * Hq + size_t(g) * G + h;
    if (n_pieces == 1) {
      store_out(reinterpret_cast<Q*>(a.out) + row * D + d, o * inv);
    } else {
      const size_t prow = row * a.max_pieces + piece;
      a.part_o[prow * D + d] = o * inv;
      if (d == 0) a.part_lse[prow] = lsum > 0.0f ? M + __log2f(lsum) : kNegInf;
    }
  }
}

// ---------------------------------------------------------------------------
// Merge pass (only launched when a call has more than one piece): one wave per
// output row merges that row's pieces in piece order with the log2-sum-exp
// weights.  Rows of single-piece sequences were written by pass 1.
// rows_per_seq is q_heads for decode and T * q_heads for verify.
// ---------------------------------------------------------------------------
template <typename O, int D, int CH>
__global__ __launch_bounds__(256) void merge_pieces(MergeArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.num_rows) return;
  const int lane = threadIdx.x & 63;
  const float* lse = a.part_lse + size_t(row) * a.max_pieces;
  const float* po = a.part_o + size_t(row) * a.max_pieces * D;
  // Pieces are taken CH at a time with every load of the chunk in flight at
  // once: lane u reads piece s0 + u's log2-sum-exp, every lane reads its dims
  // of all CH partial outputs.  The first chunk is requested together with the
  // context length (the partial buffers hold max_pieces slots per row, so the
  // reads stay in bounds whatever the length); slots past the row's piece
  // count are read but never used.  Chunks combine in piece order with a
  // running maximum.
  constexpr int PER = D / 64;
  const int first = min(CH, a.max_pieces);
  float lse0 = lane < first ? lse[lane] : kNegInf;
  float ov0[CH][PER];
#pragma unroll
  for (int u = 0; u < CH; ++u)
#pragma unroll
    for (int j = 0; j < PER; ++j) ov0[u][j] = po[size_t(min(u, first - 1)) * D + j * 64 + lane];
  int b;
  if (a.query_start) {
    // packed rows: the sequence holding token tok is the number of sequence
    // starts 1..num_seqs at or below it
    const int tok = row / a.q_heads;
    int cnt = 0;
    for (int s0 = 1; s0 <= a.num_seqs; s0 += 64) {
      const int s = s0 + lane;
      cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(s <= a.num_seqs && a.query_start[s] <= tok));
    }
    b = min(cnt, a.num_seqs - 1);
  } else {
    b = row / a.rows_per_seq;
  }
  const int L = min(a.context_lens[b], a.max_len_clamp);
  const int n_pieces = min(L > 0 ? cdiv(L, a.split_tokens) : 1, a.max_pieces);
  if (n_pieces <= 1) return;
  float M = kNegInf, wsum = 0.0f;
  float o[PER] = {};
  auto combine = [&](int cnt, float my_lse, const float (&ov)[CH][PER]) {
    my_lse = lane < cnt ? my_lse : kNegInf;
    const float cm = fmaxf(M, stride_max<1>(my_lse));
    if (cm == kNegInf) return;
    const float f = M == kNegInf ? 0.0f : fast_exp2(M - cm);
    M = cm;
    wsum *= f;
#pragma unroll
    for (int j = 0; j < PER; ++j) o[j] *= f;
    const float w_lane = my_lse == kNegInf ? 0.0f : fast_exp2(my_lse - M);
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      // slots past cnt may hold anything (even NaN): selected away, not weighted by 0
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), u));
      const bool use = u < cnt;
      wsum += use ? w : 0.0f;
#pragma unroll
      for (int j = 0; j < PER; ++j) o[j] = use ? __builtin_fmaf(w, ov[u][j], o[j]) : o[j];
    }
  };
  combine(min(CH, n_pieces), lse0, ov0);
  for (int s0 = CH; s0 < n_pieces; s0 += CH) {
    const int cnt = min(CH, n_pieces - s0);
    const float my_lse = lane < cnt ? lse[s0 + lane] : kNegInf;
    float ov[CH][PER];
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int j = 0; j < PER; ++j) ov[u][j] = po[size_t(s0 + min(u, cnt - 1)) * D + j * 64 + lane];
    combine(cnt, my_lse, ov);
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    store_out(reinterpret_cast<O*>(a.out) + size_t(row) * D + j * 64 + lane, o[j] * inv);
}

#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif


// Register ring depth per shape: three tile buffers for bf16 groups of up to
// two query heads (measured in one process on the same caches, batch-64
// workload: 19.75 -> 19.56 us per launch; the 235 VGPRs still leave two
// workgroups per CU), two elsewhere (a third buffer costs occupancy there).
template <typename KV, int G>
struct RingDepth : std::integral_constant<int, (__is_same(KV, bf16_t) && G <= 2) ? 3 : 2> {};
#ifdef PA_RING
#define PA_RING_OF(KV, G) PA_RING
#else
#define PA_RING_OF(KV, G) RingDepth<KV, G>::value
#endif

template <typename Q, typename KV, int D, int G>
hipError_t launch_decode_t(const DecodeArgs& a, bool append, hipStream_t stream) {
  constexpr int NW = PA_DECODE_WAVES;      // waves per workgroup
  constexpr int kRing = PA_RING_OF(KV, G); // tile buffers per wave
  const long wgs = long(a.max_pieces) * a.num_seqs * a.kv_heads;
  if (append) {
    decode_pass1<Q, KV, D, G, NW, kRing, true><<<dim3(unsigned(wgs)), NW * kWave, 0, stream>>>(a);
    return hipGetLastError();
  }
  decode_pass1<Q, KV, D, G, NW, kRing, false><<<dim3(unsigned(wgs)), NW * kWave, 0, stream>>>(a);
  return hipGetLastError();
}

template <typename Q, typename KV, int D>
hipError_t dispatch_group(const DecodeArgs& a, int G, bool ap, hipStream_t stream) {
  switch (G) {
    case 1: return launch_decode_t<Q, KV, D, 1>(a, ap, stream);
    case 2: return launch_decode_t<Q, KV, D, 2>(a, ap, stream);
    case 3: return launch_decode_t<Q, KV, D, 3>(a, ap, stream);
    case 4: return launch_decode_t<Q, KV, D, 4>(a, ap, stream);
    case 5: return launch_decode_t<Q, KV, D, 5>(a, ap, stream);
    case 6: return launch_decode_t<Q, KV, D, 6>(a, ap, stream);
    case 7: return launch_decode_t<Q, KV, D, 7>(a, ap, stream);
    case 8: return launch_decode_t<Q, KV, D, 8>(a, ap, stream);
    case 16: return launch_decode_t<Q, KV, D, 16>(a, ap, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename Q, typename KV>
hipError_t dispatch_dim(const DecodeArgs& a, int G, bool ap, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return dispatch_group<Q, KV, 64>(a, G, ap, stream);
    case 128: return dispatch_group<Q, KV, 128>(a, G, ap, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace


bool decode_group_supported(int G) { return (G >= 1 && G <= 8) || G == 16; }

namespace {
template <typename Q, typename KV, int D, int G>
int resident_t() {
  int n = 0;
  constexpr int NW = PA_DECODE_WAVES;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, decode_pass1<Q, KV, D, G, NW, PA_RING_OF(KV, G), false>, NW * kWave, 0) != hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}
template <typename Q, typename KV, int D>
int resident_group(int G) {
  switch (G) {
    case 1: return resident_t<Q, KV, D, 1>();
    case 2: return resident_t<Q, KV, D, 2>();
    case 3: return resident_t<Q, KV, D, 3>();
    case 4: return resident_t<Q, KV, D, 4>();
    case 5: return resident_t<Q, KV, D, 5>();
    case 6: return resident_t<Q, KV, D, 6>();
    case 7: return resident_t<Q, KV, D, 7>();
    case 8: return resident_t<Q, KV, D, 8>();
    case 16: return resident_t<Q, KV, D, 16>();
    default: return 1;
  }
}
}  // namespace

int decode_pass1_resident(int q_dtype, int kv_dtype, int head_dim, int G) {
  if (q_dtype == kF32 && kv_dtype == kF32)
    return head_dim == 64 ? resident_group<float, float, 64>(G) : resident_group<float, float, 128>(G);
  if (q_dtype == kBF16 && kv_dtype == kBF16)
    return head_dim == 64 ? resident_group<bf16_t, bf16_t, 64>(G)
                          : resident_group<bf16_t, bf16_t, 128>(G);
  return 1;
}

template <typename O, int D>
void launch_merge_t(const MergeArgs& a, hipStream_t stream) {
  // chunks of 8 pieces for calls of up to 8 pieces, 16 up to 16, else 32
  dim3 grid(cdiv(a.num_rows, 4));
  if (a.max_pieces <= 8) merge_pieces<O, D, 8><<<grid, 256, 0, stream>>>(a);
  else if (a.max_pieces <= 16) merge_pieces<O, D, 16><<<grid, 256, 0, stream>>>(a);
  else merge_pieces<O, D, 32><<<grid, 256, 0, stream>>>(a);
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.out_dtype == kF32) {
    if (a.head_dim == 64) launch_merge_t<float, 64>(a, stream);
    else launch_merge_t<float, 128>(a, stream);
  } else {
    if (a.head_dim == 64) launch_merge_t<bf16_t, 64>(a, stream);
    else launch_merge_t<bf16_t, 128>(a, stream);
  }
  return hipGetLastError();
}

hipError_t launch_decode_pass1(const DecodeArgs& a, bool append, hipStream_t stream) {
  const int G = a.q_heads / a.kv_heads;
  if (a.q_dtype == kF32 && a.kv_dtype == kF32) return dispatch_dim<float, float>(a, G, append, stream);
  if (a.q_dtype == kBF16 && a.kv_dtype == kBF16)
    return dispatch_dim<bf16_t, bf16_t>(a, G, append, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
