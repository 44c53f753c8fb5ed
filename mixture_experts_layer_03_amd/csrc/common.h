// Device helpers shared by the gfx950 kernels of the MoE layer (wave64, MFMA).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// round to nearest even (hardware v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

// 16x16 output tile, K = 32 bf16 per instruction.  Operand lane l: row/column l % 16,
// eight K-consecutive values of K-group l / 16.  Output lane l, register v:
// row 4 * (l / 16) + v, column l % 16.
__device__ __forceinline__ f32x4 mfma16_bf16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16x16 output tile, K = 4 fp32 per instruction (one value per lane, K = lane / 16).
__device__ __forceinline__ f32x4 mfma16_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal (streaming) hint, for data read exactly once.
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---- direct global -> LDS copies (global_load_lds_dwordx4), issued from inline asm so
// the compiler's wait insertion does not track (and drain) them; users wait explicitly.
// 16 bytes per lane from global memory to LDS at M0 + 16 * lane (M0 wave-uniform)
__device__ __forceinline__ void copy_to_lds(const void* src, const uint16_t* lds_dst) {
  const uint32_t m0 =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)lds_dst));
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}
// the same from a wave-uniform base plus a per-lane 32-bit byte offset
__device__ __forceinline__ void copy_to_lds(const char* base, uint32_t off, const uint16_t* lds_dst) {
  const uint32_t m0 =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)lds_dst));
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
}
// a pointer known to be the same in every lane, kept in scalar registers
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Wait until at most N of this wave's copies are outstanding and its LDS reads are
// done.  Followed by lds_barrier(): afterwards every wave's copies older than its last
// N have landed and no wave still reads a stage that is about to be refilled.
template <int N>
__device__ __forceinline__ void copy_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// copy_wait<min(ahead, A) * L>() for a runtime ahead >= 0
template <int L, int A>
__device__ __forceinline__ void copy_wait_ahead(int ahead) {
  if constexpr (A == 0) {
    copy_wait<0>();
  } else {
    if (ahead >= A)
      copy_wait<A * L>();
    else
      copy_wait_ahead<L, A - 1>(ahead);
  }
}

}  // namespace moe
