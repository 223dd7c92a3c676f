// Paged chunked prefill on the matrix cores: many new tokens per sequence,
// causal among themselves, over the paged cache -- the step before decode that
// "From 183 ms to 19 ms per decode step" names next in its "Limits" section.
// Sequence b's T_b new tokens are its last T_b positions (their K/V already in
// the cache); token t sees positions 0 .. L_b - T_b + t, as in verify.
//
// Work item: one workgroup of NW waves per (tile of 16 * RT * NW query rows,
// KV head, sequence).  Row r of a sequence is query token r / G of head
// g * G + r % G; wave w owns RT consecutive 16-row tiles (rows 16 RT w ..
// 16 RT (w + 1) - 1) over the whole visible context, so no partial results
// leave the workgroup.  The cache is
// walked in stages of KB blocks (32 positions): the workgroup stages a
// stage's K and V tiles in LDS with direct-to-LDS buffer loads (double
// buffered, the next stage in flight while this one is used), and every wave
// reads the shared tiles for its own rows.  A block's buffer resource covers
// only its rows inside the needed range, so positions past it arrive as zeros
// (finite: their weights are exactly 0) and cost no memory traffic.
//
// Per wave and 16-position tile the products are those of the verify kernel:
// scores S^T = K Q^T on 16x16x32 products (K from LDS as A, the query rows
// as B), P as the A operand of 16x16x16 products against V (bf16: transposed
// LDS reads; int8: codes turned by an identity product), the softmax per row
// with a reference maximum and delayed rescale.
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"
#include "pa_mfma.h"

// Shape of a workgroup, measured on 16 sequences x 512-token chunks after
// U{0..1536} prior positions, 16/8 heads, D = 128, bf16, with a work plan:
// four waves of two 16-row tiles each (128 rows; every K and V operand read
// from LDS serves two products), stages of two blocks, two stages in the ring,
// at most 168 VGPRs (three workgroups per CU): 92-94 us per call, against
// 105 us for eight waves of one row tile with four-block stages, 106-125 us
// for four-block stages with two row tiles (two workgroups per CU), 111 us
// with three stages in the ring and 146 us for two-wave workgroups.
#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 4
#endif
#ifndef PA_PREFILL_ROW_TILES
#define PA_PREFILL_ROW_TILES 2
#endif
#ifndef PA_PREFILL_STAGE_BLOCKS
#define PA_PREFILL_STAGE_BLOCKS 2
#endif
#ifndef PA_PREFILL_STAGES
#define PA_PREFILL_STAGES 2
#endif
// Register budget: at least two waves per SIMD asked of the compiler (the
// second launch bound is waves per SIMD), which then fits the bf16 and int8
// kernels (head_dim 128) in 168 VGPRs, i.e. three four-wave workgroups per
// CU; with no bound it spends 88 accumulation registers and gets two.  Asking
// for three spills.  At 168 the budget is full: any further per-row state
// costs the third workgroup.
#ifndef PA_PREFILL_MIN_WAVES_PER_SIMD
#define PA_PREFILL_MIN_WAVES_PER_SIMD 2
#endif

namespace pa {
namespace {

// f(integral_constant<int, i>) for i = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <typename KV, int D, int NW, int RT>
__global__ __launch_bounds__(NW * kWave, PA_PREFILL_MIN_WAVES_PER_SIMD) void prefill_rows(DecodeArgs a) {
  constexpr bool kInt8 = __is_same(KV, i8_t);
  constexpr int ROWB = D * int(sizeof(KV));      // bytes per key row
  constexpr int NL = ROWB / 64;                  // 1 KiB loads per 16-row tile
  constexpr int NQ = D / 32;                     // score products per tile
  constexpr int NT = D / 16;                     // output blocks of 16 dims
  constexpr int TILE_BYTES = kBlockSize * ROWB;
  // Cache blocks per stage (an even number: they are used in pairs), at least
  // enough for one load per wave.
  constexpr int KB = PA_PREFILL_STAGE_BLOCKS * 2 * NL >= NW ? PA_PREFILL_STAGE_BLOCKS : NW / (2 * NL);
  static_assert(KB % 2 == 0, "stages hold pairs of blocks");
  constexpr int NBUF = PA_PREFILL_STAGES;        // stage buffers in the ring
  constexpr int STAGE = 2 * KB * TILE_BYTES;     // K tiles, then V tiles
  constexpr int LOADS = 2 * KB * NL;             // 1 KiB loads per stage
  static_assert(LOADS % NW == 0, "stage loads must split evenly over the waves");
  constexpr int LPW = LOADS / NW;                // loads per wave per stage
  constexpr int CPR = ROWB / 16;                 // 16-byte chunks per key row
  constexpr int RPB = ROWB >= 256 ? 1 : 256 / ROWB;
  constexpr bool kSwizzleV = kInt8;
  using M = MOps<KV>;

  // Unit of this workgroup: rank r = blockIdx / kv_heads (the kv_heads
  // workgroups of a unit are consecutive, so they spread over the XCDs).
  // With a prefill work plan whose header matches the call, unit r of the
  // plan (longest first) and its offsets and lengths, in the round trip the
  // natural order spends on them; otherwise tiles of later rows (which see
  // more positions) first.  The order changes no bit of any result.
  constexpr int WROWS = RT * kRows;              // query rows per wave
  const int pairs = a.num_seqs * a.kv_heads;
  const int tiles = int(gridDim.x) / pairs;
  const int Hq = a.q_heads;
  const int G = Hq / a.kv_heads;
  const int g = int(blockIdx.x) % a.kv_heads;
  const int rank = int(blockIdx.x) / a.kv_heads;
  const int max_len = a.max_blocks_per_seq * kBlockSize;
  int b, tile, q0, T, L;
  bool planned = false;
  if (a.plan) {
    const int4 h0 = *reinterpret_cast<const int4*>(a.plan);
    const int4 h1 = *reinterpret_cast<const int4*>(a.plan + 4);
    const int32_t* row = a.plan + kPlanHeader + size_t(rank) * kPrefillPlanRow;
    const int4 r0 = *reinterpret_cast<const int4*>(row);
    const int r4 = row[4];
    planned = (h0.x == kPrefillPlanMagic) & (h0.y == a.num_seqs) & (h0.z == tiles) &
              (h0.w == NW * WROWS) & (h1.x == a.total_query_tokens) &
              (h1.y == a.num_query_tokens) & (h1.z == a.max_blocks_per_seq) & (h1.w == G);
    if (planned) {
      // clamped like the natural order's values: a corrupt row cannot address
      // outside the buffers
      b = min(max(r0.x, 0), a.num_seqs - 1);
      tile = min(max(r0.y, 0), tiles - 1);
      q0 = min(max(r0.z, 0), a.total_query_tokens);
      T = min(max(r0.w, 0), min(a.num_query_tokens, a.total_query_tokens - q0));
      L = min(r4, max_len);
    }
  }
  if (!planned) {
    tile = tiles - 1 - rank / a.num_seqs;
    b = rank % a.num_seqs;
    if (a.query_start) {
      const int s0 = a.query_start[b], s1 = a.query_start[b + 1];
      if (threadIdx.x == 0)
        check(s0 >= 0 && s1 >= s0 && s1 <= a.total_query_tokens && s1 - s0 <= a.num_query_tokens,
              kCheckQueryStart, a.check_status);
      q0 = min(max(s0, 0), a.total_query_tokens);
      T = min(max(s1 - s0, 0), min(a.num_query_tokens, a.total_query_tokens - q0));
    } else {
      // a fixed number of query tokens per sequence (a verify call with more
      // rows than the decode kernels take)
      T = a.num_query_tokens;
      q0 = b * T;
    }
    const int L_raw = a.context_lens[b];
    if (threadIdx.x == 0) check(L_raw >= 0 && L_raw <= max_len, kCheckContextTable, a.check_status);
    L = min(L_raw, max_len);
  }
  const int R = T * G;
  const int row0 = tile * NW * WROWS;
  if (row0 >= R) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;     // key row of an operand read / query row of S, P
  const int grp = lane >> 4;   // 8-dim group of a score product / key quad of S, P, O
  const int wrow0 = row0 + wave * WROWS;

  // Row tile i of this wave: rows wrow0 + 16i .. +15.  Query rows as the B
  // operand of score product c: lane (row n, group grp) holds
  // q[n][32c + 8grp .. +7] (fp16 for an int8 cache).
  // bf16 cache: a negative scale is carried by q's sign (exact), so that the
  // softmax below works with a positive factor.
  const uint32_t qflip = a.scale < 0.0f ? 0x80008000u : 0u;
  u32x4 qb[RT][NQ];
  float qsum[RT];
  int last_vis[RT];   // last position row n of tile i sees
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int row = wrow0 + i * kRows + n;
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
        qb[i][c] = w ^ qflip;
      }
    }
    qsum[i] = kInt8 ? add_xor32(add_xor16(qpart)) : 0.0f;
  }

  // Positions the workgroup needs (through its last row) and this wave needs.
  const int t_last = (min(row0 + NW * WROWS, R) - 1) / G;
  const int kend = min(max(L - T + t_last + 1, 0), L);
  const int w_kend = wrow0 < R ? min(max(L - T + (min(wrow0 + WROWS, R) - 1) / G + 1, 0), L) : 0;
  // Last position the wave's first row sees: every row sees at least this far.
  const int w_minvis = wrow0 < R ? L - T + wrow0 / G : -1;
  const int nblk = cdiv(kend, kBlockSize);
  const int nst = cdiv(nblk, KB);

  // The table row is read-only for this kernel: read through the constant
  // address space, its (uniform) entries come through scalar loads, which the
  // stage waits below (vector-memory counts) do not see.
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  const const_i32_ptr bt = (const_i32_ptr)(a.block_tables + size_t(b) * a.max_blocks_per_seq);
  const size_t head_blocks = size_t(g) * a.num_blocks;
  const char* kbase = reinterpret_cast<const char*>(a.k_cache);
  const char* vbase = reinterpret_cast<const char*>(a.v_cache);
  const float sc = a.scale * kLog2e;
  // The bf16 path's factor: |scale| log2(e), kept above zero so that a masked
  // (-inf) score still gives -inf (a zero scale then yields weights that round
  // to exactly 1, as it should).
  const float sc_pos = fmaxf(fabsf(sc), __FLT_MIN__);

  // A ring of NBUF stage buffers, each its own LDS object, so that waiting
  // for one stage's direct-to-LDS loads does not also wait for the others'.
  __shared__ __attribute__((aligned(16))) char s_st0[STAGE];
  __shared__ __attribute__((aligned(16))) char s_st1[STAGE];
  __shared__ __attribute__((aligned(16))) char s_st2[NBUF > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) char s_st3[NBUF > 3 ? STAGE : 16];
  auto ring = [&](auto u_tag) -> char* {
    constexpr int u = decltype(u_tag)::value;
    if constexpr (u == 0) return s_st0;
    else if constexpr (u == 1) return s_st1;
    else if constexpr (u == 2) return s_st2;
    else return s_st3;
  };
  auto sw = [](int r, int k) { return r * ROWB + 16 * (k ^ ((r / RPB) & (CPR - 1))); };
  // Source offsets of this lane's 16-byte LDS slots: K rows (and int8 V rows)
  // swizzled for the score operand reads, bf16 V rows for the transposed reads.
  int src_off[NL], src_off_v[NL];
#pragma unroll
  for (int c = 0; c < NL; ++c) {
    const int slot = 64 * c + lane;
    const int r = slot / CPR, p = slot % CPR;
    src_off[c] = r * ROWB + 16 * (p ^ ((r / RPB) & (CPR - 1)));
    src_off_v[c] = kSwizzleV ? src_off[c] : r * ROWB + 16 * (p ^ vswz<ROWB>(r));
  }
  // The physical blocks of stage st (and for int8 their scales), through
  // scalar loads: uniform addresses in the constant address space, outside
  // the vector-memory count the stage waits below rely on.  A stage's lookup
  // is issued one stage before its tile loads, so their latency overlaps the
  // previous stage's wait.
  auto lookup = [&](int st, int (&phys)[KB], float (&ks)[KB], float (&vs)[KB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int blk = st * KB + kb;
      const bool need = blk * kBlockSize < kend;
      const int entry = need ? bt[readfirstlane(blk)] : 0;
      if (threadIdx.x == 0) check(entry >= 0 && entry < a.num_blocks, kCheckTableEntry, a.check_status);
      // bf16: the raw entry, clamped where the fetch uses it, so that no wait
      // for the scalar load comes before then (clamped here, it was waited
      // for at once, twice per stage); int8: clamped here, it addresses the
      // block's scales
      phys[kb] = kInt8 ? min(max(entry, 0), a.num_blocks - 1) : entry;
      if constexpr (kInt8) {
        // a block past the needed range is fully masked: any finite, nonzero
        // scale keeps its zero weights zero (the row sum divides by the V scale)
        typedef const __attribute__((address_space(4))) float* const_f32_ptr;
        ks[kb] = need ? ((const_f32_ptr)a.k_scale)[head_blocks + phys[kb]] : 1.0f;
        vs[kb] = need ? ((const_f32_ptr)a.v_scale)[head_blocks + phys[kb]] : 1.0f;
      }
    }
  };
  // This wave's share of stage st's tile loads: loads wave*LPW .. +LPW-1 of
  // the stage's 2*KB*NL (K tiles, then V tiles; NL loads per tile).
  auto fetch = [&](int st, char* buf, const int (&phys)[KB]) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int li = wave * LPW + i;
      const bool isv = li >= KB * NL;
      const int kb = (li / NL) % KB;
      // c: the load's 1 KiB part of its tile (known at compile time when a
      // wave's share is whole tiles)
      const int c = LPW % NL == 0 ? i % NL : li % NL;
      const int blk = st * KB + kb;
      // (uniform; kept scalar so the buffer resource needs no per-lane loop)
      const int valid = readfirstlane(min(max(kend - blk * kBlockSize, 0), kBlockSize));
      const int pk = kInt8 ? phys[kb] : min(max(phys[kb], 0), a.num_blocks - 1);
      const size_t tile_off = (head_blocks + size_t(valid > 0 ? pk : 0)) * TILE_BYTES;
      const __amdgpu_buffer_rsrc_t r = make_rsrc((isv ? vbase : kbase) + tile_off, valid * ROWB);
      int off = 0;
      if constexpr (LPW % NL == 0) {
        off = isv ? src_off_v[c] : src_off[c];
      } else {
        // a run-time part: picked by selects, so the arrays stay in registers
#pragma unroll
        for (int k = 0; k < NL; ++k) off = c == k ? (isv ? src_off_v[k] : src_off[k]) : off;
      }
      buffer_load16_to_lds(r, buf + (isv ? KB + kb : kb) * TILE_BYTES + 1024 * c, off);
    }
  };

  u32x2 ident;
  {
    uint32_t e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = 4 * grp + j == n ? M::kOne : 0u;
    ident = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
  }
  const f32x4 vinit = {M::kVInit, M::kVInit, M::kVInit, M::kVInit};

  constexpr float kSlack = 8.0f;
  // Per row: the reference maximum m (log2 units); for bf16 caches also the
  // rescale threshold m + kSlack and the reference the exponents subtract
  // (m, or 0 while m is -inf), both changed only where m changes.
  float m[RT], thr[RT], mref[RT], lsum[RT];
  f32x4 o[RT][NT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    m[i] = thr[i] = kNegInf;
    mref[i] = 0.0f;
    lsum[i] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) o[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Two 16-position tiles (blocks blk, blk + 1, staged at kb, kb + 1 of buf)
  // for this wave's RT row tiles.  Lane (n, grp) holds row n's scores of keys
  // 4grp .. 4grp+3 of both blocks; read as keys 8grp .. 8grp+7 of one 32-key
  // product, with V's rows in the same order (the two blocks' transposed
  // reads side by side), P.V runs on 16x16x32 products.  Positions are masked
  // only where the pair crosses the wave's causal edge.
  // Scores of a pair (the products only; issued for every pair of a stage
  // before any softmax, so the matrix cores work on the next pair's scores
  // while the vector ALUs take the softmax of this one).
  // Both runs of matrix products (scores, then P.V) are issued at raised wave
  // priority: of the waves that share a SIMD, the one issuing products goes
  // first, and the others' softmax work fills the cycles between its
  // products.
  auto scores2 = [&](const char* buf, int kb, f32x4 (&s)[RT][2]) {
    const char* const sk0 = buf + kb * TILE_BYTES;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < RT; ++i) s[i][0] = s[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const char* const sk = sk0 + h * TILE_BYTES;
        u32x4 kop;
        if constexpr (kInt8) {
          const int k = (32 * c + 8 * grp) / 16;
          const uint2 w = *reinterpret_cast<const uint2*>(sk + sw(n, k) + 8 * (grp & 1));
          kop = codes8_f16(w.x, w.y);
        } else {
          kop = *reinterpret_cast<const u32x4*>(sk + sw(n, 4 * c + grp));
        }
#pragma unroll
        for (int i = 0; i < RT; ++i) s[i][h] = M::qk(kop, qb[i][c], s[i][h]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // The softmax of a pair: the packed weights of each row tile (the A
  // operands of its P.V products), the running maxima and sums updated.
  auto softmax2 = [&](int blk, f32x4 (&s)[RT][2], float ks0, float vs0, float ks1, float vs1,
                      u32x4 (&pa)[RT]) {
    const bool edge = (blk + 2) * kBlockSize - 1 > w_minvis;   // uniform per wave
    const float ssc[2] = {sc * ks0, sc * ks1};
    const float vsc[2] = {vs0, vs1};
    const float ivsc[2] = {kInt8 ? __builtin_amdgcn_rcpf(vs0) : 1.0f, kInt8 ? __builtin_amdgcn_rcpf(vs1) : 1.0f};
    if constexpr (!kInt8) {
      // bf16 cache: one factor for both blocks, so the row maximum is taken
      // over the raw scores and each weight is exp2 of one fused multiply-add;
      // the running sum adds the weights as rounded for the P.V product.
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        float r[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = s[i][e >> 2][e & 3];
        if (edge) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int pos = (blk + (e >> 2)) * kBlockSize + 4 * grp + (e & 3);
            r[e] = pos <= last_vis[i] ? r[e] : kNegInf;
          }
        }
        // The rescale test on this lane's own eight scores: rounding the
        // product by sc_pos > 0 is monotone, so some lane's maximum times
        // sc_pos passes the threshold exactly when the row's does, and the
        // row maximum (two lane exchanges) is taken on the rare path only.
        const float lmax = nmax8(r) * sc_pos;   // -inf stays -inf: sc_pos > 0
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(lmax > thr[i]) != 0, 0)) {   // rare
          const float tmax = nmax_xor32(nmax_xor16(lmax));
          const float mnew = fmaxf(m[i], tmax);
          const float alpha = mnew == kNegInf ? 1.0f : fast_exp2(m[i] - mnew);
          m[i] = mnew;
          thr[i] = mnew + kSlack;
          mref[i] = mnew == kNegInf ? 0.0f : mnew;
          lsum[i] *= alpha;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float ar = __shfl(alpha, 4 * grp + j);
#pragma unroll
            for (int t = 0; t < NT; ++t) o[i][t][j] *= ar;
          }
        }
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(r[e], sc_pos, -mref[i]));
        pa[i] = u32x4{pack_bf16_round(p[0], p[1]), pack_bf16_round(p[2], p[3]),
                      pack_bf16_round(p[4], p[5]), pack_bf16_round(p[6], p[7])};
        float ls = lsum[i];
#pragma unroll
        for (int w = 0; w < 4; ++w) ls = add_bf16_pair(pa[i][w], ls);
        lsum[i] = ls;
      }
    } else {
      // int8 cache: each block has its own K scale, so scores are scaled
      // before the maximum; P carries the block's V scale.
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = s[i][e >> 2][e & 3];
          x[e] = (v - kI8Bias * qsum[i]) * ssc[e >> 2];
        }
        if (edge) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int pos = (blk + (e >> 2)) * kBlockSize + 4 * grp + (e & 3);
            x[e] = pos <= last_vis[i] ? x[e] : kNegInf;
          }
        }
        // (the rescale test on this lane's own maximum, exact: the scores
        // are already scaled)
        const float lmax = nmax8(x);
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(lmax > m[i] + kSlack) != 0, 0)) {   // rare
          const float tmax = nmax_xor32(nmax_xor16(lmax));
          const float mnew = fmaxf(m[i], tmax);
          const float alpha = mnew == kNegInf ? 1.0f : fast_exp2(m[i] - mnew);
          m[i] = mnew;
          lsum[i] *= alpha;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float ar = __shfl(alpha, 4 * grp + j);
#pragma unroll
            for (int t = 0; t < NT; ++t) o[i][t][j] *= ar;
          }
        }
        const float mr = m[i] == kNegInf ? 0.0f : m[i];
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = fast_exp2(x[e] - mr);
        pa[i] = u32x4{pack_bf16_round(p[0] * vsc[0], p[1] * vsc[0]), pack_bf16_round(p[2] * vsc[0], p[3] * vsc[0]),
                      pack_bf16_round(p[4] * vsc[1], p[5] * vsc[1]), pack_bf16_round(p[6] * vsc[1], p[7] * vsc[1])};
        // the row sum adds the weights as rounded for the product, each block's
        // divided by its V scale again
        const float t0 = add_bf16_pair(pa[i][0], add_bf16_pair(pa[i][1], 0.0f));
        const float t1 = add_bf16_pair(pa[i][2], add_bf16_pair(pa[i][3], 0.0f));
        lsum[i] = __builtin_fmaf(t1, ivsc[1], __builtin_fmaf(t0, ivsc[0], lsum[i]));
      }
    }
  };
  // The P.V products of a pair (V tiles of blocks kb, kb + 1 of buf).
  auto pv2 = [&](const char* buf, int kb, const u32x4 (&pa)[RT]) {
    const char* const sv0 = buf + (KB + kb) * TILE_BYTES;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      u32x2 vb[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const char* const sv = sv0 + h * TILE_BYTES;
        if constexpr (kInt8) {
          const uint32_t u = *reinterpret_cast<const uint32_t*>(sv + sw(n, t) + 4 * grp) ^ 0x80808080u;
          const f32x4 tv = M::mm16(u32x2{f16pair_lo(u), f16pair_hi(u)}, ident, vinit);
          vb[h] = u32x2{pack_bf16_exact(tv[0], tv[1]), pack_bf16_exact(tv[2], tv[3])};
        } else {
          vb[h] = v_operand_tr<ROWB>(sv, t, lane);
        }
      }
      const u32x4 v8 = {vb[0][0], vb[0][1], vb[1][0], vb[1][1]};
#pragma unroll
      for (int i = 0; i < RT; ++i) o[i][t] = pv32(pa[i], v8, o[i][t]);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto softmax_pv2 = [&](const char* buf, int kb, int blk, f32x4 (&s)[RT][2], float ks0,
                         float vs0, float ks1, float vs1) {
    u32x4 pa[RT];
    softmax2(blk, s, ks0, vs0, ks1, vs1, pa);
    pv2(buf, kb, pa);
  };

  // Stage st lives in ring buffer st % NBUF; stages up to st + NBUF - 1 are
  // requested while stage st is used.  One barrier per stage both publishes
  // stage st (every wave has waited for its own share of its loads) and
  // frees buffer (st - 1) % NBUF, which the stage st + NBUF - 1 loads issued
  // right after it overwrite.  The loop is unrolled by NBUF so that buffers
  // and each stage's int8 scales are compile-time choices.
  float ks[NBUF][KB], vs[NBUF][KB];
#pragma unroll
  for (int u = 0; u < NBUF; ++u)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) ks[u][kb] = vs[u][kb] = 1.0f;
  int phys_next[KB] = {};
  auto wait_tiles = [&](int later) {   // stage st done; `later` stages may still load
    static_assert(NBUF - 2 <= 3 && (NBUF - 2) * LPW <= 63, "vmcnt range");
    if (later <= 0) __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(((LPW) & 15) | (((LPW) >> 4) << 14) | (7 << 4) | (15 << 8));
    else if (later == 2) __builtin_amdgcn_s_waitcnt(((2 * LPW) & 15) | (((2 * LPW) >> 4) << 14) | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt(((3 * LPW) & 15) | (((3 * LPW) >> 4) << 14) | (7 << 4) | (15 << 8));
    __asm__ __volatile__("" ::: "memory");
  };
  static_for<0, NBUF - 1>([&](auto u_tag) {
    constexpr int u = decltype(u_tag)::value;
    if (u < nst) {
      int phys[KB];
      lookup(u, phys, ks[u], vs[u]);
      fetch(u, ring(u_tag), phys);
    }
  });
  if (NBUF - 1 < nst) lookup(NBUF - 1, phys_next, ks[NBUF - 1], vs[NBUF - 1]);
  for (int st0 = 0; st0 < nst; st0 += NBUF) {
    static_for<0, NBUF>([&](auto u_tag) {
      constexpr int u = decltype(u_tag)::value;
      constexpr int nu = (u + NBUF - 1) % NBUF;   // ring slot of stage st + NBUF - 1
      const int st = st0 + u;
      if (st < nst) {
        wait_tiles(min(NBUF - 2, nst - 1 - st));
        __syncthreads();
        if (st + NBUF - 1 < nst) fetch(st + NBUF - 1, ring(std::integral_constant<int, nu>{}), phys_next);
        f32x4 sc2[KB / 2][RT][2];
#pragma unroll
        for (int kb = 0; kb < KB; kb += 2)
          if ((st * KB + kb) * kBlockSize < w_kend)   // uniform per wave
            scores2(ring(u_tag), kb, sc2[kb / 2]);
#pragma unroll
        for (int kb = 0; kb < KB; kb += 2) {
          const int blk = st * KB + kb;
          if (blk * kBlockSize < w_kend)
            softmax_pv2(ring(u_tag), kb, blk, sc2[kb / 2], kInt8 ? ks[u][kb] : 1.0f,
                        kInt8 ? vs[u][kb] : 1.0f, kInt8 ? ks[u][kb + 1] : 1.0f,
                        kInt8 ? vs[u][kb + 1] : 1.0f);
        }
        // the table entries (and scales) of the stage after next, into the
        // slot just used
        if (st + NBUF < nst) lookup(st + NBUF, phys_next, ks[u], vs[u]);
      }
    });
  }

  // Row totals, then O / l per row, rounded to bf16.
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const float lrow = add_xor32(add_xor16(lsum[i]));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wrow0 + i * kRows + 4 * grp + j;
      const float lr = __shfl(lrow, 4 * grp + j);
      const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
      if (r < R) {
        const int tq = r / G;
        const size_t orow = (size_t(q0) + tq) * Hq + size_t(g) * G + (r - tq * G);
        bf16_t* dst = reinterpret_cast<bf16_t*>(a.out) + orow * D + n;
#pragma unroll
        for (int t = 0; t < NT; ++t) dst[16 * t].bits = f32_to_bf16(o[i][t][j] * inv);
      }
    }
  }
}

template <typename KV>
hipError_t launch_prefill_t(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NW = PA_PREFILL_WAVES, RT = PA_PREFILL_ROW_TILES;
  const int G = a.q_heads / a.kv_heads;
  const long tiles = cdiv(a.num_query_tokens * G, NW * RT * kRows);
  const long wgs = tiles * a.num_seqs * a.kv_heads;
  if (a.head_dim == 128)
    prefill_rows<KV, 128, NW, RT><<<dim3(unsigned(wgs)), NW * kWave, 0, stream>>>(a);
  else
    prefill_rows<KV, 64, NW, RT><<<dim3(unsigned(wgs)), NW * kWave, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

int prefill_rows_per_workgroup() { return PA_PREFILL_WAVES * PA_PREFILL_ROW_TILES * kRows; }

bool prefill_supported(int q_dtype, int kv_dtype, int head_dim) {
  return q_dtype == kBF16 && (kv_dtype == kBF16 || kv_dtype == kI8) &&
         (head_dim == 64 || head_dim == 128);
}

hipError_t launch_prefill(const DecodeArgs& a, hipStream_t stream) {
  if (a.kv_dtype == kI8) return launch_prefill_t<i8_t>(a, stream);
  return launch_prefill_t<bf16_t>(a, stream);
}

}  // namespace pa
