// Device-side helpers shared by the libpa kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"

namespace pa {

constexpr int kWave = 64;
constexpr int kBlockSize = 16;   // tokens per cache block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

struct bf16_t { uint16_t bits; };   // storage tag for bfloat16 data
struct i8_t { int8_t v; };          // storage tag for int8 codes

template <typename T> struct Bytes { static constexpr int value = sizeof(T); };

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x.bits); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));  // v_cvt_pk_bf16_f32
}
// Two fp32 values as bf16 (round to nearest even) in one packed conversion.
__device__ __forceinline__ bf16x2 pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_convertvector(f32x2{lo, hi}, bf16x2);
}

// Exchange across 16-lane rows without LDS: permlane16_swap of a value with
// itself leaves row r's partner row (r ^ 1) in one of the two results, so
// combining both results reduces over lane ^ 16; permlane32_swap likewise
// over lane ^ 32.
__device__ __forceinline__ float add_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum that carries NaN through (IEEE 754-2019 maximum).  gfx950 has it as
// one three-operand instruction that takes its operands as they are, whereas
// fmaxf first quiets every operand the compiler cannot prove canonical (a
// matrix-product result, a lane exchange) with a move of its own: the row
// maximum of eight scores and its two lane exchanges take 9 instructions here,
// 19 with fmaxf.  For row maxima over scores only: a NaN score gives a NaN
// weight and a NaN row with either maximum, and the maximum of non-NaN
// numbers is the same number (the sign of a zero aside, which no exponent
// below depends on).
__device__ __forceinline__ float nmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float nmax3(float a, float b, float c) { return nmax(nmax(a, b), c); }
__device__ __forceinline__ float nmax8(const float (&r)[8]) {
  return nmax(nmax3(r[0], r[1], r[2]), nmax3(r[3], r[4], nmax3(r[5], r[6], r[7])));
}
__device__ __forceinline__ float nmax_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return nmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float nmax_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return nmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over groups of N consecutive lanes (N a power of two, N <= 64); every
// lane of a group receives the group's sum.  Inside a 16-lane DPP row the
// butterflies are quad_perm (lane ^ 1, lane ^ 2), then row_half_mirror and
// row_mirror, which after the quad steps pair each quad with the other
// quads of its half row and row.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += __builtin_amdgcn_update_dpp(0.0f, x, 0xB1, 0xF, 0xF, true);   // [1,0,3,2]
  if constexpr (N >= 4) x += __builtin_amdgcn_update_dpp(0.0f, x, 0x4E, 0xF, 0xF, true);   // [2,3,0,1]
  if constexpr (N >= 8) x += __builtin_amdgcn_update_dpp(0.0f, x, 0x141, 0xF, 0xF, true);  // row_half_mirror
  if constexpr (N >= 16) x += __builtin_amdgcn_update_dpp(0.0f, x, 0x140, 0xF, 0xF, true); // row_mirror
  if constexpr (N >= 32) x = add_xor16(x);
  if constexpr (N >= 64) x = add_xor32(x);
  return x;
}

// Maximum over groups of N consecutive lanes (N a power of two, N <= 16), by
// the butterflies of group_sum.
template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, __builtin_amdgcn_update_dpp(0.0f, x, 0xB1, 0xF, 0xF, true));
  if constexpr (N >= 4) x = fmaxf(x, __builtin_amdgcn_update_dpp(0.0f, x, 0x4E, 0xF, 0xF, true));
  if constexpr (N >= 8) x = fmaxf(x, __builtin_amdgcn_update_dpp(0.0f, x, 0x141, 0xF, 0xF, true));
  if constexpr (N >= 16) x = fmaxf(x, __builtin_amdgcn_update_dpp(0.0f, x, 0x140, 0xF, 0xF, true));
  static_assert(N <= 16, "group_max: at most one DPP row");
  return x;
}

// Reduction over the lanes that share lane % S (S a power of two < 64): every
// lane receives the result.  Within a row, rotations by S, 2S, ... < 16 gather
// the lanes of stride S (a rotation sum over a cyclic group covers each member
// once); rows are then combined with the permlane swaps.
template <int S>
__device__ __forceinline__ float stride_sum(float x) {
  if constexpr (S <= 1) x += __builtin_amdgcn_update_dpp(0.0f, x, 0x121, 0xF, 0xF, true);  // row_ror:1
  if constexpr (S <= 2) x += __builtin_amdgcn_update_dpp(0.0f, x, 0x122, 0xF, 0xF, true);  // row_ror:2
  if constexpr (S <= 4) x += __builtin_amdgcn_update_dpp(0.0f, x, 0x124, 0xF, 0xF, true);  // row_ror:4
  if constexpr (S <= 8) x += __builtin_amdgcn_update_dpp(0.0f, x, 0x128, 0xF, 0xF, true);  // row_ror:8
  if constexpr (S <= 16) x = add_xor16(x);
  if constexpr (S <= 32) x = add_xor32(x);
  return x;
}
template <int S>
__device__ __forceinline__ float stride_max(float x) {
  if constexpr (S <= 1) x = fmaxf(x, __builtin_amdgcn_update_dpp(0.0f, x, 0x121, 0xF, 0xF, true));
  if constexpr (S <= 2) x = fmaxf(x, __builtin_amdgcn_update_dpp(0.0f, x, 0x122, 0xF, 0xF, true));
  if constexpr (S <= 4) x = fmaxf(x, __builtin_amdgcn_update_dpp(0.0f, x, 0x124, 0xF, 0xF, true));
  if constexpr (S <= 8) x = fmaxf(x, __builtin_amdgcn_update_dpp(0.0f, x, 0x128, 0xF, 0xF, true));
  if constexpr (S <= 16) x = max_xor16(x);
  if constexpr (S <= 32) x = max_xor32(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// int8 codes as exact fp16: with u = c + 128 (the biased byte), placing u under
// the constant high byte 0x64 gives the fp16 number 1024 + u = c + 1152.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
constexpr uint32_t kMagic = 0x64646464u;   // fp16 high byte of 1024
constexpr float kI8Bias = 1152.0f;         // 1024 + 128
__device__ __forceinline__ uint32_t f16pair_lo(uint32_t u) {  // bytes 0,1 -> (1024+u0, 1024+u1)
  return __builtin_amdgcn_perm(kMagic, u, 0x04010400u);
}
__device__ __forceinline__ uint32_t f16pair_hi(uint32_t u) {  // bytes 2,3
  return __builtin_amdgcn_perm(kMagic, u, 0x04030402u);
}

__device__ __forceinline__ int readfirstlane(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Debug builds: record a violated precondition (ok == false) in the status
// word; callers pass conditions that are uniform across the calling lanes and
// call it from one lane.  Release builds: nothing.
__device__ __forceinline__ void check(bool ok, unsigned bit, unsigned* status) {
#if PA_DEVICE_CHECKS
  if (!ok && status) __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#else
  (void)ok;
  (void)bit;
  (void)status;
#endif
}

// The block-table entries of one piece, held across the wave: entry i of the
// piece sits in element i / 64 of lane i % 64 (a vector value, so it stays in
// registers).  NREG elements cover 64 * NREG blocks.
template <int NREG>
struct PieceTable {
  typedef int vec __attribute__((ext_vector_type(NREG)));
  vec e;
  // row: the sequence's table row; entries at or past `limit` are not read.
  __device__ void load(const int32_t* row, int begin, int limit, int lane) {
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
      const int j = begin + 64 * i + lane;
      e[i] = j < limit ? row[j] : 0;
    }
  }
  // Entry idx (the same idx in every lane of the wave).
  __device__ int at(int idx) const {
    if (idx < 64) return __builtin_amdgcn_readlane(e[0], idx);
    int v = e[0];
#pragma unroll
    for (int i = 1; i < NREG; ++i) {
      const int x = e[i];
      v = (idx >> 6) == i ? x : v;
    }
    return __builtin_amdgcn_readlane(v, idx & 63);
  }
};

// 16-byte streaming load (data read once: marked non-temporal).
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Buffer resource over [base, base + bytes): loads at offsets past `bytes`
// return zeros without a memory access (raw buffer, gfx9-family format word).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// 16-byte buffer load, non-temporal (the data is read once).
__device__ __forceinline__ u32x4 buffer_load16_stream(__amdgpu_buffer_rsrc_t r, int offset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 2));
}
// 16 bytes per lane from a buffer straight into LDS, non-temporal: lane i's
// bytes land at lds + 16 i (lds is the same in every lane).
typedef __attribute__((address_space(3))) void* lds_void_ptr;
__device__ __forceinline__ void buffer_load16_to_lds(__amdgpu_buffer_rsrc_t r, void* lds, int offset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)lds, 16, offset, 0, 0, 2);
}


// The work unit of this workgroup: sequence b, piece, KV head g, the
// sequence's context length L (clamped to the table), and the piece's
// block-table entries in `tab` (entry i = logical block piece * sb + i).
// With a work plan whose header matches the call, unit blockIdx / kv_heads of
// the plan is taken and its entries come from the plan row: one round trip,
// as the natural order's table-row load.  Otherwise (no plan, or a plan made
// for other sizes) the natural order: piece-major, then sequence, then head.
// Either way the unit's arithmetic is the same, so the order changes no bit
// of the result.  piece < 0 means no work.
struct WorkItem {
  int b, piece, g, L;
};
template <int NREG>
__device__ __forceinline__ WorkItem work_item(const DecodeArgs& a, PieceTable<NREG>& tab, int lane) {
  const int sb = a.split_tokens / kBlockSize;
  const int max_len = a.max_blocks_per_seq * kBlockSize;
  WorkItem it;
  if (a.plan) {
    const int unit = blockIdx.x / a.kv_heads;
    const int32_t* row = a.plan + kPlanHeader + size_t(unit) * plan_stride(a.split_tokens);
    tab.load(row + kPlanRowHead, 0, sb, lane);
    // Header and row head as two 16-byte loads issued together (a short-
    // circuit test would wait for each header word before asking for the next).
    const int4 h = *reinterpret_cast<const int4*>(a.plan);
    const int h4 = a.plan[4];
    const int4 r = *reinterpret_cast<const int4*>(row);
    const bool ok = (h.x == kPlanMagic) & (h.y == a.num_seqs) & (h.z == a.max_pieces) &
                    (h.w == a.split_tokens) & (h4 == a.max_blocks_per_seq);
    if (ok) {
      // Clamped so that a corrupt row cannot address outside the buffers.
      it.b = min(max(r.x, 0), a.num_seqs - 1);
      it.piece = r.w < 0 ? -1 : min(r.y, a.max_pieces - 1);
      it.g = blockIdx.x - unit * a.kv_heads;
      it.L = min(max(r.z, 0), max_len);
      if (threadIdx.x == 0) {
        check(r.z >= 0 && r.z <= max_len, kCheckContextTable, a.check_status);
        check(r.z <= a.max_pieces * a.split_tokens, kCheckContextMax, a.check_status);
      }
      return it;
    }
  }
  const int pairs = a.num_seqs * a.kv_heads;
  it.piece = blockIdx.x / pairs;
  const int pair = blockIdx.x - it.piece * pairs;
  it.b = pair / a.kv_heads;
  it.g = pair - it.b * a.kv_heads;
  const int begin = it.piece * sb;
  tab.load(a.block_tables + size_t(it.b) * a.max_blocks_per_seq, begin,
           min(a.max_blocks_per_seq, begin + sb), lane);
  const int L_raw = a.context_lens[it.b];
  it.L = min(L_raw, max_len);
  if (threadIdx.x == 0) {
    check(L_raw >= 0 && L_raw <= max_len, kCheckContextTable, a.check_status);
    check(L_raw <= a.max_pieces * a.split_tokens, kCheckContextMax, a.check_status);
  }
  return it;
}

}  // namespace pa
