// Matrix-core operand helpers shared by the kernels that run attention on
// the MFMA units (gfx950): products and conversions.
#pragma once

#include "pa_device.h"

namespace pa {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));

constexpr int kRows = 16;  // query rows of one matrix tile

// Score products (K tile on the left, query rows on the right) and the
// identity product that turns int8 V codes, per cache element type.
template <typename KV> struct MOps;
template <> struct MOps<bf16_t> {
  static constexpr uint32_t kOne = 0x3F80u;  // bf16 1.0
  static constexpr float kVInit = 0.0f;
  __device__ static f32x4 qk(u32x4 k, u32x4 q, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                  __builtin_bit_cast(bf16x8, q), c, 0, 0, 0);
  }
};
template <> struct MOps<i8_t> {
  static constexpr uint32_t kOne = 0x3C00u;  // fp16 1.0
  static constexpr float kVInit = -kI8Bias;
  __device__ static f32x4 qk(u32x4 k, u32x4 q, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h16x8, k),
                                                 __builtin_bit_cast(h16x8, q), c, 0, 0, 0);
  }
  __device__ static f32x4 mm16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h16x4, a),
                                                 __builtin_bit_cast(h16x4, b), c, 0, 0, 0);
  }
};

// P.V products, bf16 for every cache type: P is a softmax weight (times an
// int8 block's V scale), rounded to bf16, so its range is fp32's; V is a bf16
// cache value or an int8 code, exact in bf16.
__device__ __forceinline__ f32x4 pv16(u32x2 p, u32x2 v, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, p),
                                                   __builtin_bit_cast(s16x4, v), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 pv32(u32x4 p, u32x4 v, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, p),
                                                __builtin_bit_cast(bf16x8, v), c, 0, 0, 0);
}
// Two fp32 values that are bf16 numbers (int8 codes here): their high halves.
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
// Two fp32 values rounded to nearest even, in one packed conversion.
__device__ __forceinline__ uint32_t pack_bf16_round(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, pack_bf16x2(lo, hi));
}
// acc + the two bf16 values packed in w (one dot product against (1, 1); the
// products are exact).
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
  const bf16x2 ones = {__bf16(1.0f), __bf16(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, acc, false);
}

// bf16 V tiles staged in LDS for transposed reads.  16-byte chunk k of key
// row r sits at chunk position k ^ vswz(r): the rows an output block's read
// touches in one LDS pass (two chunks each) then fall on distinct banks.
template <int ROWB>
__device__ __forceinline__ int vswz(int r) {
  constexpr int CPR = ROWB / 16, RPB = ROWB >= 256 ? 1 : 256 / ROWB;
  return ((r / RPB) & (CPR / 2 - 1)) << 1;
}

// B operand of the P.V product for output dims 16t .. 16t+15 from a staged
// bf16 V tile (16 key rows): lane (n = lane % 16, grp = lane / 16) receives
// V[4grp + j][16t + n], j = 0..3.  One LDS transpose read: lane l addresses
// dims 16t + 4(l % 4) .. +3 of key row l / 4, and the hardware hands lane i
// of each 16-lane group element i % 4 of the chunks addressed by lanes
// i / 4 + 4j of that group, which are key rows 4grp + j.
template <int ROWB>
__device__ __forceinline__ u32x2 v_operand_tr(const char* sv, int t, int lane) {
  typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;
  const int r = lane >> 2;
  const int k = 2 * t + ((lane & 3) >> 1);
  const char* p = sv + r * ROWB + 16 * (k ^ vswz<ROWB>(r)) + 8 * (lane & 1);
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)p);
  return __builtin_bit_cast(u32x2, v);
}

// Byte offset of an LDS location inside the workgroup's LDS (p points into a
// __shared__ object).
typedef __attribute__((address_space(3))) const char* lds_cptr_t;
__device__ __forceinline__ uint32_t lds_offset(const char* p) {
  return (uint32_t)(uintptr_t)(lds_cptr_t)p;
}

// The LDS address v_operand_tr reads for output block t.
template <int ROWB>
__device__ __forceinline__ uint32_t v_tr_addr(const char* sv, int t, int lane) {
  const int r = lane >> 2;
  const int k = 2 * t + ((lane & 3) >> 1);
  return lds_offset(sv + r * ROWB + 16 * (k ^ vswz<ROWB>(r)) + 8 * (lane & 1));
}

// N transposed LDS reads (the operands of v_operand_tr at the given
// addresses) in one asm block that waits for them before it ends, so no read
// is left in flight when the block's outputs are handed back.  The builtin
// form cannot be used here: the compiler's waits for it do not tell a staged
// tile from the ring slot that direct-to-LDS loads are still filling, and it
// waited for every outstanding load (the next tile's too) before each tile's
// first transposed read.  The caller has already waited for the tile's own
// loads.
template <int N>
__device__ __forceinline__ void lds_read_tr(const uint32_t (&a)[N], u32x2 (&v)[N]);
template <>
__device__ __forceinline__ void lds_read_tr<2>(const uint32_t (&a)[2], u32x2 (&v)[2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2\n\t"
      "ds_read_b64_tr_b16 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1])
      : "v"(a[0]), "v"(a[1])
      : "memory");
}
template <>
__device__ __forceinline__ void lds_read_tr<4>(const uint32_t (&a)[4], u32x2 (&v)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}
template <>
__device__ __forceinline__ void lds_read_tr<8>(const uint32_t (&a)[8], u32x2 (&v)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// Two fp32 values as fp16, rounded to nearest even (values past fp16's range
// become infinite).
__device__ __forceinline__ f16x2 to_f16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_convertvector(f32x2{lo, hi}, f16x2);
}

// Eight codes (two words) as the fp16 numbers c + 1152.
__device__ __forceinline__ u32x4 codes8_f16(uint32_t w0, uint32_t w1) {
  const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
  return u32x4{f16pair_lo(u0), f16pair_hi(u0), f16pair_lo(u1), f16pair_hi(u1)};
}

}  // namespace pa
