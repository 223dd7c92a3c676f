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
// online-softmax state for the key rows it sees (one per load), so the
// per-tile work needs no cross-row exchange; rows, then waves, are merged
// once at the end.
//
// With a single piece the workgroup writes the output row directly.  With
// several pieces it writes a normalised partial output and its log2-sum-exp
// to the workspace, and a merge pass combines the pieces of each row.  (A
// merge inside this kernel by the last workgroup to arrive needs agent-scope
// fences, which write back and invalidate the XCD's L2 and cost far more than
// the second launch.)
// Piece length is fixed per call (never derived from the lengths in the
// batch), so each sequence's arithmetic depends on its own length only.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
#ifdef PA_TIMING
__device__ unsigned long long g_times[8192 * 6];
#define PA_STAMP(k) do { if (threadIdx.x == 0 && blockIdx.x < 8192) { g_times[blockIdx.x * 6 + (k)] = __builtin_amdgcn_s_memrealtime(); if ((k) == 0) g_times[blockIdx.x * 6 + 5] = (unsigned long long)__builtin_amdgcn_s_getreg(4 | (31 << 11)) | ((unsigned long long)__builtin_amdgcn_s_getreg(20 | (31 << 11)) << 32); } } while (0)
#else
#define PA_STAMP(k) do { } while (0)
#endif
namespace {

// Byte k of x as a float; the backend selects v_cvt_f32_ubyte{k}.
template <int k>
__device__ __forceinline__ float ubyte_f32(uint32_t x) {
  return float((x >> (8 * k)) & 0xFFu);
}

template <typename KV, int D>
struct Geo {
  static constexpr int EPL = 16 / int(sizeof(KV));  // elements per lane per 16-byte load
  static constexpr int LPK = D / EPL;               // lanes per key row
  static constexpr int KPL = kWave / LPK;           // key rows per wave-wide load
  static constexpr int LPB = kBlockSize / KPL;      // wave-wide loads per 16-token tile
  static constexpr int TILE_BYTES = kBlockSize * D * int(sizeof(KV));
  static_assert(LPK >= 1 && LPK <= kWave && kBlockSize % KPL == 0, "unsupported geometry");
};

// ---------------------------------------------------------------------------
// Query registers and per-load dot products for each (q, cache) dtype pair.
// ---------------------------------------------------------------------------
template <typename Q, typename KV, int D, int G> struct QRegs;

// fp32 q, fp32 cache.
template <int D, int G> struct QRegs<float, float, D, G> {
  static constexpr int EPL = Geo<float, D>::EPL;
  float q[G][EPL];
  __device__ void load(const float* qrow, int c, int q_stride) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      u32x4 w = load16(qrow + size_t(h) * q_stride + c * EPL);
#pragma unroll
      for (int e = 0; e < 4; ++e) q[h][e] = __uint_as_float(w[e]);
    }
  }
  __device__ float dot(int h, u32x4 k) const {
    float s = q[h][0] * __uint_as_float(k[0]);
#pragma unroll
    for (int e = 1; e < 4; ++e) s = __builtin_fmaf(q[h][e], __uint_as_float(k[e]), s);
    return s;
  }
};

// bf16 q, bf16 cache: packed bf16 dot products into fp32.
template <int D, int G> struct QRegs<bf16_t, bf16_t, D, G> {
  uint32_t q[G][4];
  __device__ void load(const bf16_t* qrow, int c, int q_stride) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      u32x4 w = load16(qrow + size_t(h) * q_stride + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) q[h][e] = w[e];
    }
  }
  __device__ float dot(int h, u32x4 k) const {
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // Copy the element out first: a bit cast applied directly to an element
      // of a vector value reads element 0 with this compiler.
      const uint32_t kw = k[e];
      const uint32_t qw = q[h][e];
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw),
                                          __builtin_bit_cast(bf16x2, kw), s, false);
    }
    return s;
  }
};

// bf16 q, int8 cache.  Codes are biased to unsigned bytes (x ^ 0x80) so the
// hardware byte-to-float conversion applies; the bias is removed with the
// lane's precomputed sum of q (sum q*(u-128) = sum q*u - 128 * sum q).
template <int D, int G> struct QRegs<bf16_t, i8_t, D, G> {
  float q[G][16];
  float qsum[G];
  __device__ void load(const bf16_t* qrow, int c, int q_stride) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const bf16_t* p = qrow + size_t(h) * q_stride + c * 16;
      u32x4 w0 = load16(p);
      u32x4 w1 = load16(p + 8);
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        q[h][2 * e] = bf16_lo(w0[e]);
        q[h][2 * e + 1] = bf16_hi(w0[e]);
        q[h][8 + 2 * e] = bf16_lo(w1[e]);
        q[h][8 + 2 * e + 1] = bf16_hi(w1[e]);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) s += q[h][e];
      qsum[h] = s;
    }
  }
  __device__ static void widen(u32x4 k, float (&u)[16]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t x = k[w] ^ 0x80808080u;
      u[4 * w + 0] = ubyte_f32<0>(x);
      u[4 * w + 1] = ubyte_f32<1>(x);
      u[4 * w + 2] = ubyte_f32<2>(x);
      u[4 * w + 3] = ubyte_f32<3>(x);
    }
  }
  __device__ float dot_widened(int h, const float (&u)[16]) const {
    float s = -128.0f * qsum[h];
#pragma unroll
    for (int e = 0; e < 16; ++e) s = __builtin_fmaf(q[h][e], u[e], s);
    return s;
  }
};

// V tile values of one load, widened to fp32 (int8: biased, see above).
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
template <> struct VWiden<i8_t> {
  static constexpr int EPL = 16;
  __device__ static void run(u32x4 v, float (&o)[16]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t x = v[w] ^ 0x80808080u;
      o[4 * w + 0] = ubyte_f32<0>(x);
      o[4 * w + 1] = ubyte_f32<1>(x);
      o[4 * w + 2] = ubyte_f32<2>(x);
      o[4 * w + 3] = ubyte_f32<3>(x);
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
template <typename Q, typename KV, int D, int G, int NW, int DEPTH>
__global__ __launch_bounds__(NW * kWave, NW >= 8 ? (NW * 2) / 4 : 1) void decode_pass1(DecodeArgs a) {
  using GE = Geo<KV, D>;
  constexpr int EPL = GE::EPL, LPK = GE::LPK, KPL = GE::KPL, LPB = GE::LPB;
  constexpr bool kInt8 = __is_same(KV, i8_t);

  // 1-D grid, piece-major: ids 0 .. N*Hkv-1 are piece 0 of every (sequence,
  // KV head), then piece 1, ...  Consecutive ids go to different XCDs, so the
  // always-present first pieces spread evenly over the chip, and all pieces of
  // one (sequence, head) land on the same XCD whenever N*Hkv is a multiple of 8.
  PA_STAMP(0);
  const int pairs = a.num_seqs * a.kv_heads;
  const int piece = blockIdx.x / pairs;
  const int pair = blockIdx.x - piece * pairs;
  const int b = pair / a.kv_heads;
  const int g = pair - b * a.kv_heads;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPK;   // key row inside a load
  const int c = lane % LPK;   // 16-byte column of the key row
  const int split_blocks = a.split_tokens / kBlockSize;
  const int blk_begin = piece * split_blocks;

  // Issue the loads that do not depend on the context length first, so the
  // length, the block-table row and q arrive in one round trip: the piece's
  // table entries (at most 64, one per lane; a tile's physical block is then
  // read with readlane) and this group's query rows.
  const int32_t* bt = a.block_tables + size_t(b) * a.max_blocks_per_seq;
  const int tab = blk_begin + lane < a.max_blocks_per_seq ? bt[blk_begin + lane] : 0;
  const int q_stride = a.head_dim;  // elements between consecutive heads
  const Q* qrow = reinterpret_cast<const Q*>(a.q) + (size_t(b) * a.q_heads + size_t(g) * G) * D;
  QRegs<Q, KV, D, G> qr;
  qr.load(qrow, c, q_stride);

  // Lengths beyond the table are clamped so that no access leaves the
  // buffers (the result of such a call is unspecified).
  const int L = min(a.context_lens[b], a.max_blocks_per_seq * kBlockSize);
  const int n_pieces = min(L > 0 ? cdiv(L, a.split_tokens) : 1, a.max_pieces);
  if (piece >= n_pieces) return;
  PA_STAMP(1);

  const int blk_end = min(cdiv(L, kBlockSize), blk_begin + split_blocks);
  const size_t head_blocks = size_t(g) * a.num_blocks;
  const char* kbase = reinterpret_cast<const char*>(a.k_cache);
  const char* vbase = reinterpret_cast<const char*>(a.v_cache);
  const float sc_log2 = a.scale * kLog2e;

  float m[G], l[G], acc[G][EPL];
  float corr[kInt8 ? G : 1];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
    if constexpr (kInt8) corr[h] = 0.0f;
  }

  // Out-of-range table entries are clamped into the pool (unspecified
  // result, but no access outside the cache).
  const int lane_off = lane * 16;
  // A fetch with live == false (past the wave's last tile) keeps the
  // instruction stream, and so the wait counts, identical but reads nothing:
  // its buffer resource has zero records.
  auto fetch = [&](int blk, bool live, u32x4 (&kt)[LPB], u32x4 (&vt)[LPB], float& ks, float& vs) {
    const int phys = min(max(__builtin_amdgcn_readlane(tab, blk - blk_begin), 0), a.num_blocks - 1);
    const size_t tile = (head_blocks + size_t(phys)) * GE::TILE_BYTES;
    const int bytes = live ? GE::TILE_BYTES : 0;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + tile, bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + tile, bytes);
#pragma unroll
    for (int i = 0; i < LPB; ++i) kt[i] = buffer_load16_stream(kr, i * 1024 + lane_off);
#pragma unroll
    for (int i = 0; i < LPB; ++i) vt[i] = buffer_load16_stream(vr, i * 1024 + lane_off);
    if constexpr (kInt8) {
      ks = a.k_scale[head_blocks + phys];
      vs = a.v_scale[head_blocks + phys];
    } else {
      ks = 1.0f;
      vs = 1.0f;
    }
  };

  auto process = [&](int blk, u32x4 (&kt)[LPB], u32x4 (&vt)[LPB], float ks, float vs) {
    const bool partial = (blk + 1) * kBlockSize > L;  // uniform
    float s[G][LPB];
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
      if constexpr (kInt8) {
        float u[16];
        QRegs<Q, KV, D, G>::widen(kt[i], u);
#pragma unroll
        for (int h = 0; h < G; ++h) s[h][i] = qr.dot_widened(h, u);
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) s[h][i] = qr.dot(h, kt[i]);
      }
    }
    const float sc = kInt8 ? sc_log2 * ks : sc_log2;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < LPB; ++i) s[h][i] = group_sum<LPK>(s[h][i]) * sc;
    if (partial) {
#pragma unroll
      for (int i = 0; i < LPB; ++i) {
        const bool valid = blk * kBlockSize + i * KPL + r < L;
#pragma unroll
        for (int h = 0; h < G; ++h) s[h][i] = valid ? s[h][i] : kNegInf;
        // Rows past the context may hold anything (even NaN): zero them so a
        // zero weight really contributes nothing.
#pragma unroll
        for (int w = 0; w < 4; ++w) vt[i][w] = valid ? vt[i][w] : 0u;
      }
    }
    float vf[LPB][EPL];
#pragma unroll
    for (int i = 0; i < LPB; ++i) VWiden<KV>::run(vt[i], vf[i]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float smax = s[h][0];
#pragma unroll
      for (int i = 1; i < LPB; ++i) smax = fmaxf(smax, s[h][i]);
      const float mnew = fmaxf(m[h], smax);
      const float mref = mnew == kNegInf ? 0.0f : mnew;
      const float alpha = fast_exp2(m[h] - mref);
      m[h] = mnew;
      float p[LPB];
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < LPB; ++i) {
        p[i] = fast_exp2(s[h][i] - mref);
        psum += p[i];
      }
      l[h] = __builtin_fmaf(l[h], alpha, psum);
      if constexpr (kInt8) {
        float pv_sum = 0.0f;
#pragma unroll
        for (int i = 0; i < LPB; ++i) {
          p[i] *= vs;
          pv_sum += p[i];
        }
        corr[h] = __builtin_fmaf(corr[h], alpha, pv_sum);
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float x = acc[h][e] * alpha;
#pragma unroll
        for (int i = 0; i < LPB; ++i) x = __builtin_fmaf(p[i], vf[i][e], x);
        acc[h][e] = x;
      }
    }
  };

  // Each wave takes every NW-th tile of the piece.  Tiles go through a ring
  // of DEPTH + 1 register buffers: while tile j is reduced, tiles j+1 ..
  // j+DEPTH are in flight.  The loop is unrolled over the ring so every
  // buffer index is a compile-time constant (the buffers stay in VGPRs).
  // Fetches are issued unconditionally -- past the wave's last tile they read
  // nothing (see fetch) -- so every path through the loop has the same number
  // of loads outstanding and each wait covers exactly the tile about to be
  // reduced.
  const int first = blk_begin + wave;
  const int n_my = first < blk_end ? cdiv(blk_end - first, NW) : 0;
  if (n_my > 0) {
    const int last = n_my - 1;
    u32x4 kb[DEPTH + 1][LPB], vb[DEPTH + 1][LPB];
    float ksb[DEPTH + 1], vsb[DEPTH + 1];
#pragma unroll
    for (int u = 0; u < DEPTH; ++u)
      fetch(first + min(u, last) * NW, u <= last, kb[u], vb[u], ksb[u], vsb[u]);
    int j = 0;
    // Full turns of the ring: tiles j .. j+DEPTH all exist.  The only exit is
    // the loop test, so the loop head always sees DEPTH tiles in flight.
    for (; j + DEPTH <= last; j += DEPTH + 1) {
#pragma unroll
      for (int u = 0; u <= DEPTH; ++u) {
        const int nb = (u + DEPTH) % (DEPTH + 1);  // constant once unrolled
        fetch(first + min(j + u + DEPTH, last) * NW, j + u + DEPTH <= last, kb[nb], vb[nb],
              ksb[nb], vsb[nb]);
        process(first + (j + u) * NW, kb[u], vb[u], ksb[u], vsb[u]);
      }
    }
    // At most DEPTH tiles remain; they are already in flight in kb[0 ..].
#pragma unroll
    for (int u = 0; u < DEPTH; ++u)
      if (j + u <= last) process(first + (j + u) * NW, kb[u], vb[u], ksb[u], vsb[u]);
  }

  if constexpr (kInt8) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = __builtin_fmaf(-128.0f, corr[h], acc[h][e]);
  }

  PA_STAMP(2);
  // Merge the key rows of this wave (lanes c, c + LPK, c + 2 LPK, ...).
  if constexpr (LPK < kWave) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mw = stride_max<LPK>(m[h]);
      const float f = m[h] == kNegInf ? 0.0f : fast_exp2(m[h] - mw);
      l[h] = stride_sum<LPK>(l[h] * f);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = stride_sum<LPK>(acc[h][e] * f);
      m[h] = mw;
    }
  }

  // Merge the waves through LDS.
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_acc[NW][G][D];
  if (lane < LPK) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][h][c * EPL + e] = acc[h][e];
      if (c == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
  PA_STAMP(3);

  const int Hq = a.q_heads;
  for (int t = threadIdx.x; t < G * D; t += NW * kWave) {
    const int h = t / D, d = t % D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    float lsum = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = s_m[w][h] == kNegInf ? 0.0f : fast_exp2(s_m[w][h] - M);
      lsum = __builtin_fmaf(s_l[w][h], f, lsum);
      o = __builtin_fmaf(s_acc[w][h][d], f, o);
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
  PA_STAMP(4);
}

// ---------------------------------------------------------------------------
// Merge pass (only launched when a call has more than one piece): one wave per
// output row merges that row's pieces in piece order with the log2-sum-exp
// weights.  Rows of single-piece sequences were written by pass 1.
// rows_per_seq is q_heads for decode and T * q_heads for verify.
// ---------------------------------------------------------------------------
template <typename O, int D>
__global__ __launch_bounds__(256) void merge_pieces(MergeArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.num_rows) return;
  const int b = row / a.rows_per_seq;
  const int L = min(a.context_lens[b], a.max_len_clamp);
  const int n_pieces = min(L > 0 ? cdiv(L, a.split_tokens) : 1, a.max_pieces);
  if (n_pieces <= 1) return;
  const int lane = threadIdx.x & 63;
  const float* lse = a.part_lse + size_t(row) * a.max_pieces;
  const float* po = a.part_o + size_t(row) * a.max_pieces * D;
  // Each lane reads some of the row's log2-sum-exps; the maximum and the
  // weights are shared through wave reductions.
  float M = kNegInf;
  for (int s = lane; s < n_pieces; s += 64) M = fmaxf(M, lse[s]);
  M = stride_max<1>(M);
  constexpr int PER = D / 64;
  float o[PER] = {};
  float wsum = 0.0f;
  for (int s = 0; s < n_pieces; ++s) {
    const float ls = lse[s];
    const float w = ls == kNegInf ? 0.0f : fast_exp2(ls - M);
    wsum += w;
#pragma unroll
    for (int j = 0; j < PER; ++j) o[j] = __builtin_fmaf(w, po[size_t(s) * D + j * 64 + lane], o[j]);
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    store_out(reinterpret_cast<O*>(a.out) + size_t(row) * D + j * 64 + lane, o[j] * inv);
}

#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif
#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 1
#endif

template <typename Q, typename KV, int D, int G>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NW = PA_DECODE_WAVES;      // waves per workgroup
  constexpr int DEPTH = PA_DECODE_DEPTH;   // tiles in flight per wave beyond the one reduced
  const long wgs = long(a.max_pieces) * a.num_seqs * a.kv_heads;
  decode_pass1<Q, KV, D, G, NW, DEPTH><<<dim3(unsigned(wgs)), NW * kWave, 0, stream>>>(a);
  return hipGetLastError();
}

template <typename Q, typename KV, int D>
hipError_t dispatch_group(const DecodeArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_decode_t<Q, KV, D, 1>(a, stream);
    case 2: return launch_decode_t<Q, KV, D, 2>(a, stream);
    case 3: return launch_decode_t<Q, KV, D, 3>(a, stream);
    case 4: return launch_decode_t<Q, KV, D, 4>(a, stream);
    case 5: return launch_decode_t<Q, KV, D, 5>(a, stream);
    case 6: return launch_decode_t<Q, KV, D, 6>(a, stream);
    case 7: return launch_decode_t<Q, KV, D, 7>(a, stream);
    case 8: return launch_decode_t<Q, KV, D, 8>(a, stream);
    case 16: return launch_decode_t<Q, KV, D, 16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename Q, typename KV>
hipError_t dispatch_dim(const DecodeArgs& a, int G, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return dispatch_group<Q, KV, 64>(a, G, stream);
    case 128: return dispatch_group<Q, KV, 128>(a, G, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

#ifdef PA_TIMING
extern "C" int pa_debug_times(unsigned long long* host, int n) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_times), sizeof(unsigned long long) * n) == hipSuccess ? 0 : -1;
}
#endif

bool decode_group_supported(int G) { return (G >= 1 && G <= 8) || G == 16; }

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  dim3 grid(cdiv(a.num_rows, 4));
  if (a.out_dtype == kF32) {
    if (a.head_dim == 64) merge_pieces<float, 64><<<grid, 256, 0, stream>>>(a);
    else merge_pieces<float, 128><<<grid, 256, 0, stream>>>(a);
  } else {
    if (a.head_dim == 64) merge_pieces<bf16_t, 64><<<grid, 256, 0, stream>>>(a);
    else merge_pieces<bf16_t, 128><<<grid, 256, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_pass1(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.q_heads / a.kv_heads;
  if (a.q_dtype == kF32 && a.kv_dtype == kF32) return dispatch_dim<float, float>(a, G, stream);
  if (a.q_dtype == kBF16 && a.kv_dtype == kBF16) return dispatch_dim<bf16_t, bf16_t>(a, G, stream);
  if (a.q_dtype == kBF16 && a.kv_dtype == kI8) return dispatch_dim<bf16_t, i8_t>(a, G, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
