// pa_device.h — device-side helpers shared by the libpa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace pa {

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>): unrolls a loop whose index
// must be a compile-time constant (register ring slots, LDS offsets in asm immediates).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// A register/LDS ring of NBUF slots over n steps, step k in slot k % NBUF: whole rounds of
// NBUF steps in a loop, step(k, integral_constant<int, k % NBUF>) each, then the last n % NBUF
// steps as last_step(k, ...), each inside the previous one's test. last_step issues no loads:
// every step it would prefetch lies past the end (and loads whose registers nothing reads would
// be removed by the compiler, which would upset a counted wait). A round that could stop
// part-way would give the loop a path back to its head with ring slots still loading; the
// compiler's wait insertion takes that path into account and waits for more loads than a step
// needs (a slot reused at the head then waits for every load in flight), which cuts the
// prefetch depth.
template <int U, int N, typename F>
__device__ __forceinline__ void ring_tail(int left, int k, F& f) {
  if constexpr (U < N) {
    if (U < left) {
      f(k + U, std::integral_constant<int, U>{});
      ring_tail<U + 1, N>(left, k, f);
    }
  }
}
template <int NBUF, typename F, typename G>
__device__ __forceinline__ void ring_loop(int n, F&& step, G&& last_step) {
  int k = 0;
  for (; k + NBUF <= n; k += NBUF)
    static_for<NBUF>([&](auto uc) { step(k + decltype(uc)::value, uc); });
  ring_tail<0, NBUF - 1>(n - k, k, last_step);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum class DT : int { F32 = 0, F16 = 1, BF16 = 2 };

template <DT dt>
struct Elem {
  static constexpr int bytes = (dt == DT::F32) ? 4 : 2;
};

constexpr float kLog2e = 1.4426950408889634f;  // log2(e): exp(x) = exp2(x * log2(e))
constexpr float kNegInf = -__builtin_inff();
// A score may exceed the reference maximum by this much (base 2) before a running softmax state
// is rescaled: weights stay below 2^8 = 256, well inside fp16/bf16 and fp32 sums.
constexpr float kSlack = 8.0f;

// ---- element access inside packed 32-bit words ------------------------------------------

// Widen 16-bit element `half` (0 = low, 1 = high) of word w to float.
template <DT dt>
__device__ __forceinline__ float widen16(uint32_t w, int half) {
  if constexpr (dt == DT::BF16) {
    return __uint_as_float(half ? (w & 0xffff0000u) : (w << 16));
  } else {
    f16x2 h = __builtin_bit_cast(f16x2, w);
    return half ? (float)h[1] : (float)h[0];
  }
}

// Element i of a chunk of 32-bit words holding `dt` values.
template <DT dt, int NWORDS>
__device__ __forceinline__ float elem_of(const uint32_t (&w)[NWORDS], int i) {
  if constexpr (dt == DT::F32) {
    return __uint_as_float(w[i]);
  } else {
    return widen16<dt>(w[i >> 1], i & 1);
  }
}

// Element idx of an array of `dt` values, widened to float.
template <DT dt>
__device__ __forceinline__ float load_elem(const void* base, int64_t idx) {
  if constexpr (dt == DT::F32) {
    return reinterpret_cast<const float*>(base)[idx];
  } else {
    const uint32_t w = reinterpret_cast<const uint16_t*>(base)[idx];
    return widen16<dt>(w, 0);
  }
}

// Round a float to the storage type (nearest, ties to even), returned as raw bits.
template <DT dt>
__device__ __forceinline__ uint32_t narrow_bits(float x) {
  if constexpr (dt == DT::F32) {
    return __float_as_uint(x);
  } else if constexpr (dt == DT::F16) {
    _Float16 h = (_Float16)x;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
  } else {
    __bf16 b = (__bf16)x;
    return (uint32_t)__builtin_bit_cast(uint16_t, b);
  }
}

template <DT dt>
__device__ __forceinline__ void store_elem(void* base, int64_t idx, float x) {
  if constexpr (dt == DT::F32) {
    reinterpret_cast<float*>(base)[idx] = x;
  } else {
    reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)narrow_bits<dt>(x);
  }
}

// ---- indices ----------------------------------------------------------------------------

// A physical block id clamped into the pool [0, n): a bad id reads the wrong block, never
// outside the pool.
__device__ __forceinline__ int64_t clamp_block(int32_t phys, int64_t n) {
  return phys < 0 ? 0 : (phys >= n ? n - 1 : (int64_t)phys);
}
// The same clamp in 32-bit scalar arithmetic, against id_max = last_block_id(num_blocks),
// computed once per wave.
__device__ __forceinline__ int last_block_id(int64_t n) {
  return n - 1 > 0x7fffffff ? 0x7fffffff : (int)(n - 1);
}
__device__ __forceinline__ int clamp_id(int32_t phys, int id_max) {
  const int lo = phys > 0 ? phys : 0;
  return lo < id_max ? lo : id_max;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Wave index inside the workgroup as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// ---- loads ------------------------------------------------------------------------------

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Non-temporal 16-byte load, for K/V tiles a launch reads once: the caches evict these lines
// first, which lets a stream of whole 128-byte lines run closer to the HBM rate. Do not re-read
// such a line later in the same launch and expect a cache hit.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 load8_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// ---- tile loads through buffer resources --------------------------------------------------
// A buffer resource spanning `bytes` bytes from `base` (untyped, stride 0). A load at an offset
// at or past `bytes` returns 0 and accesses no memory, so a resource with bytes = 0 makes inert
// loads: they keep their place in the instruction stream and in the wait counters, which lets
// a register ring prefetch unconditionally without reading anything past its last tile.
// Word 3 sets DATA_FORMAT = 32 bit (a zero data format reads as 0 on gfx9).
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kCachePolicyNt = 2;  // the instruction's nt bit: lines are evicted first
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4 load16_tile_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCachePolicyNt));
}
// One 16-byte-per-lane DMA load through a buffer resource, non-temporal, straight into LDS:
// lane L writes LDS bytes [lds + 16 L, lds + 16 L + 16) (lds wave-uniform). The LDS address is
// taken as a generic pointer (with an LDS-typed one in a kernel template, clang's host pass
// drops the kernel's stub).
__device__ __forceinline__ void load16_tile_stream_lds(__amdgpu_buffer_rsrc_t r, void* lds,
                                                       uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           off, 0, 0, kCachePolicyNt);
}
__device__ __forceinline__ u32x2 load8_tile_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2,
                            __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kCachePolicyNt));
}

// ---- cross-lane reductions ----------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i inside each group of 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i inside each row of 16

// Sum over aligned groups of N lanes (N = 1..64, power of two); every lane gets its group's
// sum. Uses DPP inside a row of 16 (after the quad steps every quad holds one value, so the
// mirrors pair up whole quads / halves) and lane shuffles across rows.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// exp2 via the hardware instruction (inputs here are <= 0 or -inf).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Weight of a state with maximum m against the merged maximum M, treating an empty state
// (m == -inf) as weight 0 even when M is -inf too.
__device__ __forceinline__ float rescale(float m, float M) {
  return (m == kNegInf) ? 0.0f : fast_exp2(m - M);
}

}  // namespace pa
