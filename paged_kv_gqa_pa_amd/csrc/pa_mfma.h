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
