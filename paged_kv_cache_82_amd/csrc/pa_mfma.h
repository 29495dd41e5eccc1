// pa_mfma.h — 16x16x32 MFMA operand helpers shared by the decode and prefill kernels (gfx950).
//
// Layouts of v_mfma_f32_16x16x32_{bf16,f16} on a wave of 64 lanes, lane l = 16*gq + hh:
//   A (16 x 32):  lane l holds row hh, k = 8*gq .. 8*gq+7
//   B (32 x 16):  lane l holds column hh, k = 8*gq .. 8*gq+7
//   C (16 x 16):  lane l holds rows 4*gq .. 4*gq+3 of column hh
// Attention uses them transposed: S^T = K Q^T puts tokens on rows and query columns on
// columns, so a lane's four scores belong to one query column, and the softmax weights it
// computes are exactly its slice of the P^T operand of O^T += V^T P^T, once the k index of
// that product is paired with token 16*(e/4) + 4*gq + (e%4). The V^T operand is built from
// 16-byte V row loads by pairing M-tile mt, row r with head dimension (D/16)*r + mt.
#pragma once

#include "pa_device.h"

namespace pa {

template <DT dt>
struct MfmaT;
template <>
struct MfmaT<DT::BF16> {
  using vec8 = bf16x8;
  using scalar = __bf16;
  static __device__ __forceinline__ f32x4 mma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct MfmaT<DT::F16> {
  using vec8 = f16x8;
  using scalar = _Float16;
  static __device__ __forceinline__ f32x4 mma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to nearest-even 16-bit values, packed low/high (one v_cvt_pk_*_f32).
template <DT dt>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (dt == DT::BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
  }
}

// acc + lo + hi of a packed pair of 16-bit values (v_dot2c_f32_{f16,bf16} against (1, 1)):
// the softmax row sum taken over the weights exactly as the p.V MFMA sees them.
template <DT dt>
__device__ __forceinline__ float sum2(uint32_t pair, float acc) {
  if constexpr (dt == DT::BF16) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
  } else {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
  }
}

// V row fragment of one token: D/16 consecutive head dimensions (16 bytes for D = 128,
// 8 bytes for D = 64).
template <int D>
struct VFrag;
template <>
struct VFrag<128> {
  using T = u32x4;
  static constexpr int words = 4;
  static __device__ __forceinline__ T load_stream(const char* p) { return load16_stream(p); }
  static __device__ __forceinline__ T load_tile_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return load16_tile_stream(r, off);
  }
};
template <>
struct VFrag<64> {
  using T = u32x2;
  static constexpr int words = 2;
  static __device__ __forceinline__ T load_stream(const char* p) { return load8_stream(p); }
  static __device__ __forceinline__ T load_tile_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return load8_tile_stream(r, off);
  }
};

// 16-bit element `e` of a V fragment, as raw bits in the low half.
template <int D>
__device__ __forceinline__ uint32_t vfrag_elem(const typename VFrag<D>::T& f, int e) {
  const uint32_t w = f[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// The V registers of one 32-token step of one wave: loads of tile u hold V rows of tokens
// 16u + 4*gq + i (i < 4).
template <int D>
struct VRegs {
  typename VFrag<D>::T v[2][4];
};

}  // namespace pa
