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

// ---- wavefront reductions on the DPP lane network (register to register; a shuffle
// through the LDS crossbar costs ~100 cycles per step)
// update_dpp: lane value moved by CTRL; lanes the instruction does not write (rows or
// banks masked off, source outside the row) return `old`
template <int CTRL, int ROWM = 0xf, int BANKM = 0xf>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWM, BANKM, false);
}
template <int CTRL, int ROWM = 0xf, int BANKM = 0xf>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(dpp_i<CTRL, ROWM, BANKM>(__float_as_int(old), __float_as_int(v)));
}
// gfx9 DPP controls
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// Fold `op` over all 64 lanes toward lane 63 (row prefix by shifts 1, 2, 4, 8, then the
// row totals by the row broadcasts), then broadcast lane 63.  `ident` is op's identity.
template <typename F>
__device__ __forceinline__ float wave_reduce(float v, float ident, F op) {
  v = op(v, dpp_f<kDppRowShr1>(ident, v));
  v = op(v, dpp_f<kDppRowShr2>(ident, v));
  v = op(v, dpp_f<kDppRowShr4, 0xf, 0xe>(ident, v));
  v = op(v, dpp_f<kDppRowShr8, 0xf, 0xc>(ident, v));
  v = op(v, dpp_f<kDppRowBcast15, 0xa, 0xf>(ident, v));
  v = op(v, dpp_f<kDppRowBcast31, 0xc, 0xf>(ident, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, 0.f, [](float x, float y) { return x + y; });
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, -__builtin_huge_valf(), [](float x, float y) { return fmaxf(x, y); });
}

// (v, i) with the largest v over the wavefront, equal v -> smaller i, in every lane,
// where the indices grow with the lane (every lane's i above all of a lower lane's): the
// largest v by a max fold, then the lowest lane holding it (one ballot) gives its i.
// Half the DPP moves of a fold that carries i through every step (measured in the
// one-token gate/up launch, whose routing runs eight such rounds: 0.6-1.9 us faster).
__device__ __forceinline__ void wave_argmax_lane_ordered(float& v, int& i) {
  const float m = wave_max(v);
  const unsigned long long hit = __ballot(v == m);
  const int src = hit ? __ffsll(static_cast<long long>(hit)) - 1 : 0;
  i = __builtin_amdgcn_readlane(i, src);
  v = m;
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
// The compiler's hazard recognizer does not look inside inline asm, so each block keeps
// the CDNA wait-state rules itself:
//  * a VMEM instruction reading an SGPR needs 5 wait states after a VALU write of it
//    (e.g. v_readlane restoring a spilled base); the base is therefore first copied by
//    s_mov_b64, an SALU read, which the hardware orders after any VALU write, and the
//    load reads the copy;
//  * a global load to LDS needs 1 wait state after an SALU write of M0 (the compiler
//    writes M0 right before the block): the s_mov_b64, or an s_nop, provides it.
// 16 bytes per lane from global memory to LDS at M0 + 16 * lane (M0 wave-uniform)
__device__ __forceinline__ void copy_to_lds(const void* src, const uint16_t* lds_dst) {
  const uint32_t m0 =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)lds_dst));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}
// the same from a wave-uniform base plus a per-lane 32-bit byte offset
__device__ __forceinline__ void copy_to_lds(const char* base, uint32_t off, const uint16_t* lds_dst) {
  const uint32_t m0 =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)lds_dst));
  const char* b;
  asm volatile("s_mov_b64 %0, %2\n\tglobal_load_lds_dwordx4 %1, %0"
               : "=&s"(b)
               : "v"(off), "s"(base), "{m0}"(m0)
               : "memory");
}
// 4 bytes per lane to LDS at M0 + 4 * lane (M0 wave-uniform)
__device__ __forceinline__ void copy4_to_lds(const void* src, const void* lds_dst) {
  const uint32_t m0 =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)lds_dst));
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(m0) : "memory");
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
