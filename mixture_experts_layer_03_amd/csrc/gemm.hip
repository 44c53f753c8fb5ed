// Tiled bf16 MFMA GEMM for large token batches (prefill): C = A B^T with both
// operands K-contiguous, as every product of the layer is:
//   router     logits[T,E]   = x[T,H]  W_r[E,H]^T                (fp32 out)
//   up         Hm[pos,I]     = silu(x W_g[e]^T) * (x W_u[e]^T)   (tokens gathered per expert)
//   down       r[slot,H]     = w_slot * Hm[pos] W_d[e]^T         (scattered to slot order)
//   shared     Hs[T,I_s], y  = Hs W_sd^T + sum_j r[t,j]          (combine fused)
// Expert weights are [out, in] per expert [mlxcel #838 "Validation checkpoint"], so
// the weight operand rows are the output features and K runs along memory.
//
// Block tile 128 (tokens) x BN (weight rows: 128 or 256) x 64 with BN/32 wavefronts,
// each owning a 64 x 64 sub-tile (a 4 x 4 grid of v_mfma_f32_16x16x32_bf16).  Two
// wavefronts share each SIMD, so one computes while the other waits on memory.  The
// wide tile halves the L2 -> LDS bytes per flop against a square 128 x 128 tile,
// which is what bounds a 128 x 128 tile on this chip.  Operands are staged global ->
// registers -> LDS (double buffered; 16-byte chunks XOR-swizzled by row so fragment
// reads do not collide on banks); the next K-step's global loads are issued before the
// current step's MFMAs.  u8 weights are dequantised to bf16 (s * (q - z), rounded to
// nearest even) on their way to LDS, eight codes per thread and chunk.  The epilogue
// stages 64-row halves of the tile through LDS as fp32 and writes 16-byte chunks, so
// every output, gather and scatter is coalesced.  Blocks are numbered so that
// consecutive tiles share an XCD (its L2 holds the shared A rows and weight panels).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = kTileM;

// Swizzled 16-byte chunk of (row, logical chunk) in an LDS tile of BK-element rows.
// 128-byte rows (BK = 64): XOR with row % 8.  64-byte rows (BK = 32): rows r and r + 4
// share banks, so XOR with (row / 4) % 4.  Either way every thread's staging rows and
// every fragment's rows keep the same XOR term, so one base address serves them all.
template <int BK>
__device__ __forceinline__ int phys_chunk(int row, int c) {
  return BK == 64 ? (c ^ (row & 7)) : (c ^ ((row >> 2) & 3));
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

template <int BN, int BK, WFmt WF, bool DUAL, AMode AM, Epi EPI>
__global__ __launch_bounds__(BN * 2) void k_tile(TileArgs a) {
  constexpr int NTHR = BN * 2;                  // BN/32 wavefronts
  constexpr int CPRK = BK / 8;                  // 16-byte chunks per LDS row
  constexpr int RSTEP = NTHR / CPRK;            // tile rows between one thread's chunks
  constexpr int AR = BM * CPRK / NTHR;          // A chunks per thread
  constexpr int BR = BN * CPRK / NTHR;          // B chunks per thread
  constexpr int WN = BN / 64;                   // wavefronts along N
  constexpr int STAGE_ELEMS = (BM + BN) * BK;   // bf16 elements per LDS stage
  constexpr int NCOL = DUAL ? BN / 2 : BN;      // output columns per tile
  constexpr int EPI_LD = NCOL + 4;              // fp32 epilogue row stride (bank spread)
  constexpr int SMEM_ELEMS = (64 * EPI_LD * 2 > 2 * STAGE_ELEMS) ? 64 * EPI_LD * 2 : 2 * STAGE_ELEMS;
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int NT = (a.N + NCOL - 1) / NCOL;
  const int per = gridDim.x / 8;
  const int KS = a.ksplit > 1 ? a.ksplit : 1;
  // logical tile order: consecutive blocks land on one XCD (hardware deals blocks
  // round-robin over the 8 XCDs); within a group of G consecutive M-tiles the N-tile
  // index varies slowest, so the G blocks that read the same weight panel run
  // together and share it through L2, and the group's G activation panels stay hot
  const int Lx = (blockIdx.x % 8) * per + blockIdx.x / 8;
  const int kp = Lx % KS, L = Lx / KS;
  const int G = a.group_m > 1 ? a.group_m : 1;
  const int grp = L / (G * NT), rem = L % (G * NT);
  const int mt = grp * G + rem % G, nt = rem / G;

  int e = 0, m_begin, m_rows;
  if (a.routed) {
    if (mt >= a.meta[1]) return;
    e = a.tiles[2 * mt];
    m_begin = a.tiles[2 * mt + 1];
    m_rows = min(BM, a.offsets[e + 1] - m_begin);
  } else {
    m_begin = mt * BM;
    if (m_begin >= a.M) return;
    m_rows = min(BM, a.M - m_begin);
  }
  const int K = a.K;
  const int kt0 = kp * (K / BK) / KS, kt1 = (kp + 1) * (K / BK) / KS;  // this block's K-steps

  // ---- staging: thread rows tid/8 + RSTEP*i (congruent mod 8, so one swizzled LDS
  // base plus immediate offsets), 16-byte chunk tid % 8 (8 elements: bf16, or 8 u8
  // codes for quantised weights).  A rows use 32-bit element offsets (the host keeps
  // rows * K below 2^32); rows past the tile's end are clamped (computed, never stored).
  const int sc = tid % CPRK, r0 = tid / CPRK;
  uint32_t a_off[AR];
#pragma unroll
  for (int i = 0; i < AR; ++i) {
    const int r = min(r0 + RSTEP * i, m_rows - 1);
    int row;
    if constexpr (AM == AMode::GATHER)
      row = a.perm[m_begin + r] / a.k;
    else
      row = m_begin + r;
    a_off[i] = static_cast<uint32_t>(row) * K + sc * 8;
  }
  constexpr int esz = WF == WFmt::U8 ? 1 : 2;
  const uint8_t* bp[BR];
  const uint16_t* bsp[BR];
  const uint16_t* bzp[BR];
#pragma unroll
  for (int i = 0; i < BR; ++i) {
    const int r = r0 + RSTEP * i;  // B tile row
    int n;
    bool second;
    if (DUAL) {
      // B tile rows in blocks of 32: gate, up, gate, up, ... so each wavefront's 64
      // rows are the gate and up rows of the same 32 output columns
      const int blk = r >> 5;
      second = blk & 1;
      n = nt * NCOL + (blk >> 1) * 32 + (r & 31);
    } else {
      second = false;
      n = min(nt * BN + r, a.N - 1);
    }
    const void* base = second ? a.B1 : a.B0;
    bp[i] = static_cast<const uint8_t*>(base) +
            (static_cast<int64_t>(e) * a.b_expert_stride + static_cast<int64_t>(n) * K + sc * 8) * esz;
    if constexpr (WF == WFmt::U8) {
      const int64_t ro = (static_cast<int64_t>(e) * a.N + n) * (K / 64);
      bsp[i] = (second ? a.B1s : a.B0s) + ro;
      bzp[i] = (second ? a.B1z : a.B0z) + ro;
    } else {
      bsp[i] = bzp[i] = nullptr;
    }
  }

  struct Regs {
    uint4 a[AR], b[WF == WFmt::U8 ? 1 : BR];
    uint2 q[WF == WFmt::U8 ? BR : 1];
    float s[WF == WFmt::U8 ? BR : 1], z[WF == WFmt::U8 ? BR : 1];
  };
  auto gload = [&](Regs& R, int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < AR; ++i) R.a[i] = ldg16(a.A + a_off[i] + k0);
#pragma unroll
    for (int i = 0; i < BR; ++i) {
      if constexpr (WF == WFmt::U8) {
        R.q[i] = *reinterpret_cast<const uint2*>(bp[i] + k0);
        R.s[i] = f16_to_f32(bsp[i][(kt * BK) >> 6]);
        R.z[i] = f16_to_f32(bzp[i][(kt * BK) >> 6]);
      } else {
        R.b[i] = ldg16(bp[i] + 2 * k0);
      }
    }
  };
  const int wr = r0 * BK + (phys_chunk<BK>(r0, sc) << 3);  // LDS write base (elements)
  auto sstore = [&](const Regs& R, int buf) {
    uint16_t* As = smem + buf * STAGE_ELEMS;
    uint16_t* Bs = As + BM * BK;
#pragma unroll
    for (int i = 0; i < AR; ++i) *reinterpret_cast<uint4*>(&As[wr + RSTEP * i * BK]) = R.a[i];
#pragma unroll
    for (int i = 0; i < BR; ++i) {
      uint4 v;
      if constexpr (WF == WFmt::U8) {
        const float s = R.s[i], z = R.z[i];
        const uint32_t lo = R.q[i].x, hi = R.q[i].y;
        v.x = pack_bf16x2(s * (static_cast<float>(lo & 0xffu) - z), s * (static_cast<float>((lo >> 8) & 0xffu) - z));
        v.y = pack_bf16x2(s * (static_cast<float>((lo >> 16) & 0xffu) - z), s * (static_cast<float>(lo >> 24) - z));
        v.z = pack_bf16x2(s * (static_cast<float>(hi & 0xffu) - z), s * (static_cast<float>((hi >> 8) & 0xffu) - z));
        v.w = pack_bf16x2(s * (static_cast<float>((hi >> 16) & 0xffu) - z), s * (static_cast<float>(hi >> 24) - z));
      } else {
        v = R.b[i];
      }
      *reinterpret_cast<uint4*>(&Bs[wr + RSTEP * i * BK]) = v;
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wm = w / WN, wn = w % WN;
  const int fr = lane & 15, fq = lane >> 4;
  // fragment read bases (the XOR term is the same for every sub-tile of a lane)
  const int a_rd = (wm * 64 + fr) * BK, b_rd = (wn * 64 + fr) * BK;
  auto compute = [&](int buf) {
    const uint16_t* As = smem + buf * STAGE_ELEMS;
    const uint16_t* Bs = As + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int cc = phys_chunk<BK>(fr, ks * 4 + fq) << 3;
      uint4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const uint4*>(&As[a_rd + cc + i * 16 * BK]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const uint4*>(&Bs[b_rd + cc + j * 16 * BK]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16_bf16(af[i], bf[j], acc[i][j]);
    }
  };

  // one register stage: the next K-step's loads are issued before this step's MFMAs.
  // (A second register stage to double the load lead time measured 1.6-1.9x slower on
  // the workloads: it either spills or halves the wavefronts per SIMD.)
  Regs R;
  if (kt0 < kt1) {
    gload(R, kt0);
    sstore(R, 0);
  }
  __syncthreads();
  for (int kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    if (kt + 1 < kt1) gload(R, kt + 1);
    compute(buf);
    if (kt + 1 < kt1) sstore(R, buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: two 64-row halves staged through LDS as fp32
  float* ep = reinterpret_cast<float*>(smem);
  constexpr int CPR = NCOL / 8;  // 8-column chunks per row
#pragma unroll 1
  for (int h = 0; h < 2; ++h) {
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = i * 16 + 4 * fq + v;
          if constexpr (DUAL) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
              ep[r * EPI_LD + wn * 32 + j * 16 + fr] = silu(acc[i][j][v]) * acc[i][j + 2][v];
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) ep[r * EPI_LD + wn * 64 + j * 16 + fr] = acc[i][j][v];
          }
        }
    }
    __syncthreads();
#pragma unroll 1
    for (int c = tid; c < 64 * CPR; c += NTHR) {
      const int r = c / CPR, c8 = (c % CPR) * 8;
      const int m = h * 64 + r;
      const int col = nt * NCOL + c8;
      if (m < m_rows && col < a.N) {
        const float4 v0 = *reinterpret_cast<const float4*>(&ep[r * EPI_LD + c8]);
        const float4 v1 = *reinterpret_cast<const float4*>(&ep[r * EPI_LD + c8 + 4]);
        float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        const int64_t orow = m_begin + m;
        if constexpr (EPI == Epi::F32) {
          float* out = static_cast<float*>(a.out) + kp * a.part_stride + orow * a.ldo + col;
          if (col + 8 <= a.N && (a.ldo & 3) == 0) {
            *reinterpret_cast<float4*>(out) = v0;
            *reinterpret_cast<float4*>(out + 4) = v1;
          } else {
            for (int q = 0; q < 8 && col + q < a.N; ++q) out[q] = f[q];
          }
        } else {
          int64_t drow = orow;
          if constexpr (EPI == Epi::SCALED_SLOT) {
            const int slot = a.perm[orow];
            const float ws = a.topk_w[slot];
#pragma unroll
            for (int q = 0; q < 8; ++q) f[q] *= ws;
            drow = slot;
          } else if constexpr (EPI == Epi::COMBINE) {
            for (int jj = 0; jj < a.k; ++jj) {
              const int64_t slot = orow * a.k + jj;
              const int ex = a.idx[slot];
              if (ex < 0 || ex >= a.E) continue;
              const uint4 rv = ldg16(a.r + slot * a.N + col);
              const uint32_t u[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                f[2 * q] += __uint_as_float(u[q] << 16);
                f[2 * q + 1] += __uint_as_float(u[q] & 0xffff0000u);
              }
            }
          }
          uint16_t* out = static_cast<uint16_t*>(a.out) + drow * a.ldo + col;
          *reinterpret_cast<uint4*>(out) = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
        }
      }
    }
    __syncthreads();
  }
}

template <int BN, int BK, WFmt WF, bool DUAL, AMode AM, Epi EPI>
hipError_t launch_one(const TileArgs& a, hipStream_t s) {
  constexpr int NCOL = DUAL ? BN / 2 : BN;
  const int NT = (a.N + NCOL - 1) / NCOL;
  const int G = a.group_m > 1 ? a.group_m : 1;
  const int64_t mt_pad = (a.mtiles_bound + G - 1) / G * G;  // whole groups (extra tiles exit)
  int64_t blocks = mt_pad * NT * (a.ksplit > 1 ? a.ksplit : 1);
  blocks = (blocks + 7) / 8 * 8;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_tile<BN, BK, WF, DUAL, AM, EPI>), dim3(static_cast<unsigned>(blocks)), dim3(BN * 2), 0, s, a);
  return hipGetLastError();
}

template <WFmt WF, bool DUAL, AMode AM, Epi EPI>
hipError_t launch_bn(const TileArgs& a, hipStream_t s) {
  // Single-matrix products take the wide 8-wavefront tile (half the L2 -> LDS bytes
  // per flop).  The gate/up product keeps the 4-wavefront 128 x 128 tile: measured
  // faster on the workloads' shapes (two blocks per CU instead of one).
  const bool wide = !DUAL && a.N >= 256;
  // K-step: 32 for the wide tile (48 KB of LDS, several blocks per CU), 64 for the
  // narrow one (measured best for each)
  if (wide) return launch_one<256, 32, WF, DUAL, AM, EPI>(a, s);
  return launch_one<128, 64, WF, DUAL, AM, EPI>(a, s);
}

}  // namespace

hipError_t launch_tile_gemm(const TileArgs& a, AMode am, WFmt wf, Epi epi, hipStream_t s) {
  // the combinations the layer uses
  if (epi == Epi::F32 && am == AMode::DENSE && wf == WFmt::BF16)
    return launch_one<128, 64, WFmt::BF16, false, AMode::DENSE, Epi::F32>(a, s);
  if (epi == Epi::SWIGLU && am == AMode::GATHER && wf == WFmt::BF16)
    return launch_bn<WFmt::BF16, true, AMode::GATHER, Epi::SWIGLU>(a, s);
  if (epi == Epi::SWIGLU && am == AMode::GATHER && wf == WFmt::U8)
    return launch_bn<WFmt::U8, true, AMode::GATHER, Epi::SWIGLU>(a, s);
  if (epi == Epi::SWIGLU && am == AMode::DENSE && wf == WFmt::BF16)
    return launch_bn<WFmt::BF16, true, AMode::DENSE, Epi::SWIGLU>(a, s);
  if (epi == Epi::SCALED_SLOT && am == AMode::DENSE && wf == WFmt::BF16)
    return launch_bn<WFmt::BF16, false, AMode::DENSE, Epi::SCALED_SLOT>(a, s);
  if (epi == Epi::SCALED_SLOT && am == AMode::DENSE && wf == WFmt::U8)
    return launch_bn<WFmt::U8, false, AMode::DENSE, Epi::SCALED_SLOT>(a, s);
  if (epi == Epi::COMBINE && am == AMode::DENSE && wf == WFmt::BF16)
    return launch_bn<WFmt::BF16, false, AMode::DENSE, Epi::COMBINE>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
