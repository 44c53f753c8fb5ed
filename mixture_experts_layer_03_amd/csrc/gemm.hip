// Tiled bf16 MFMA GEMM for large token batches (prefill): C = A B^T with both
// operands K-contiguous, as every product of the layer is:
//   router     logits[T,E]   = x[T,H]  W_r[E,H]^T                (fp32 out)
//   up         Hm[pos,I]     = silu(x W_g[e]^T) * (x W_u[e]^T)   (tokens gathered per expert)
//   down       r[slot,H]     = w_slot * Hm[pos] W_d[e]^T         (scattered to slot order)
//   shared     Hs[T,I_s], y  = Hs W_sd^T + sum_j r[t,j]          (combine fused)
// Expert weights are [out, in] per expert [mlxcel #838 "Validation checkpoint"], so
// the weight operand rows are the output features and K runs along memory.
//
// Block tile 128 (tokens) x BN (weight rows) x BK with BN/32 wavefronts, each owning a
// 64 x 64 sub-tile (a 4 x 4 grid of v_mfma_f32_16x16x32_bf16); the routed gate/up of
// the copy pipeline takes BN/64 wavefronts of 64 x 128 (4 x 8).  LDS tiles hold 16-byte
// chunks XOR-swizzled by row, so fragment reads do not collide on banks.
//
// bf16 weights (k_tile_dma): both operands go HBM/L2 -> LDS through the load unit's
// direct copy (global_load_lds_dwordx4), S LDS stages deep, with explicit waits.  The
// layer's products take 128 x 512 x 64 with two stages (160 KB of LDS, 16 wavefronts,
// four per SIMD; 8 wider ones for the routed gate/up): measured on this chip, the load
// path is what bounds these GEMMs, and
// per K-step it is paced by the number of wavefronts issuing copies and by the average
// L2 latency, so the tile moving the fewest bytes per flop with the most wavefronts
// wins.  Dense single-matrix products too small to fill the chip with such blocks take
// 128 x 256 x 64 with three stages, and so does a gate/up whose last 256-column tile
// would be mostly padding.  A routed gate/up whose last tile is at most half full
// (k_tile_dma_split) runs that tile's columns as 256 x 256 tiles over chunks of 256
// positions.  The router product (fp32 out, split over K) takes 128 x 128 x 64.
//
// u8 weights (k_tile_dma_q8) copy the codes and their group parameters to LDS the same
// way and dequantise each B fragment in registers; shapes it does not take (k_tile)
// stage them global -> registers -> LDS (double buffered), dequantised to bf16
// (s * (q - z), rounded to nearest even) on the way, eight codes per thread and chunk.
//
// Epilogues stage 64-row slices of the tile through LDS as fp32 and write 16-byte
// chunks, so every output, gather and scatter is coalesced.  Blocks are numbered so that
// consecutive tiles share an XCD (its L2 holds the shared activation rows and weight
// panels); the routed products group, for each N-tile, all M-tiles of one expert.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = kTileM;

// Swizzle term of a tile row: a row's 16-byte chunk c sits at chunk c ^ swz(row).
// 128-byte rows (BK = 64): row % 8, so the 8 rows a group of 8 lanes reads in one
// 16-byte fragment load hit 8 different bank groups.  64-byte rows (BK = 32): two rows
// share a 128-byte bank line, so rows r and r + 2 collide unless their terms differ:
// (row / 2) % 4.  Every thread's staging rows and every fragment's rows differ by
// multiples of 16, which keep the term, so one base address serves them all.
template <int BK>
__device__ __forceinline__ int swz(int row) {
  return BK == 64 ? (row & 7) : ((row >> 1) & 3);
}
template <int BK>
__device__ __forceinline__ int phys_chunk(int row, int c) {
  return c ^ swz<BK>(row);
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Position of this block's tile.  Logical tile order: consecutive blocks land on one
// XCD (hardware deals blocks round-robin over the 8 XCDs); within a group of G
// consecutive M-tiles the N-tile index varies slowest, so the G blocks that read the
// same weight panel run together and share it through L2, and the group's G
// activation panels stay hot.  Routed products with few tokens per expert
// (a.plain_order) keep the launch order instead and put an expert's N-tiles side by
// side: measured on the MI355X, with one or two M-tiles per expert there is little
// panel reuse to gain, and the tiles of one XCD crowding onto the same lines cost more
// (gate/up at 4096 tokens of the Ling-2.6-flash shape 1200 -> 1095 us, at 8192 of the
// Ling-3.0-flash shape 2146 -> 1930 us; Ling-lite, with 3-4 M-tiles per expert, is
// faster the XCD way, 384 against 422-435 us).  Returns false for a block past the
// last M-tile.
struct TilePos {
  int nt, kp, e, m_begin, m_rows, kt0, kt1;
};
// nblocks: the blocks of the launch that take such tiles (a multiple of 8, numbered
// from 0); NT: the N-tiles they cover (0: all of N).
template <int NCOL, int BK, int TBM = BM>
__device__ __forceinline__ bool tile_pos(const TileArgs& a, TilePos& p, int nblocks, int NT = 0) {
  if (NT <= 0) NT = (a.N + NCOL - 1) / NCOL;
  const int per = nblocks / 8;
  const int KS = a.ksplit > 1 ? a.ksplit : 1;
  const int Lx = a.plain_order ? static_cast<int>(blockIdx.x) : (blockIdx.x % 8) * per + blockIdx.x / 8;
  p.kp = Lx % KS;
  const int L = Lx / KS;
  int mt;
  if (a.routed && a.group_m <= 0) {
    // grouped by expert: for each N-tile, all M-tiles of one expert in a row, so the
    // blocks reading an expert's weight panel run together.  Tiles are stored in expert
    // order, so the logical range of expert e is [first_e * NT, (first_e + m_e) * NT)
    // and contains L exactly when M-tile L / NT belongs to e.
    const int q = L / NT;
    if (q >= a.meta[1]) return false;
    const int e = a.tiles[2 * q];
    const int first = q - (a.tiles[2 * q + 1] - a.offsets[e]) / TBM;
    const int me = (a.offsets[e + 1] - a.offsets[e] + TBM - 1) / TBM;
    const int local = L - first * NT;
    if (a.plain_order) {
      p.nt = local % NT;
      mt = first + local / NT;
    } else {
      p.nt = local / me;
      mt = first + local % me;
    }
  } else {
    const int G = a.group_m > 1 ? a.group_m : 1;
    const int grp = L / (G * NT), rem = L % (G * NT);
    mt = grp * G + rem % G;
    p.nt = rem / G;
  }
  p.e = 0;
  if (a.routed) {
    if (mt >= a.meta[1]) return false;
    p.e = a.tiles[2 * mt];
    p.m_begin = a.tiles[2 * mt + 1];
    p.m_rows = min(TBM, a.offsets[p.e + 1] - p.m_begin);
  } else {
    p.m_begin = mt * TBM;
    if (p.m_begin >= a.M) return false;
    p.m_rows = min(TBM, a.M - p.m_begin);
  }
  const int nk = a.K / BK;  // K-steps of this block's split
  p.kt0 = p.kp * nk / KS;
  p.kt1 = (p.kp + 1) * nk / KS;
  return true;
}

// Write-out of one epilogue pass: rows [h*RP, h*RP + RP) of the NCOL-column result,
// staged in LDS as fp32 (row stride NCOL + 4), go out as 16-byte chunks of 8 columns
// (fp32, or bf16 after the epilogue's scaling, scatter or combine).
template <int NTHR, int NCOL, int RP, Epi EPI>
__device__ __forceinline__ void epilogue_write(const TileArgs& a, const float* ep, int tid, int h, int nt, int kp,
                                               int m_begin, int m_rows) {
  constexpr int EPI_LD = NCOL + 4;
  constexpr int CPR = NCOL / 8;
#pragma unroll 1
  for (int c = tid; c < RP * CPR; c += NTHR) {
    const int r = c / CPR, c8 = (c % CPR) * 8;
    const int m = h * RP + r;
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
          // the k routed terms of the token in slot order, four slots per batch: their
          // indices, then their rows, are loaded together (one memory latency per batch)
          for (int j0 = 0; j0 < a.k; j0 += 4) {
            int ex[4];
            uint4 rv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) ex[q] = j0 + q < a.k ? a.idx[orow * a.k + j0 + q] : -1;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              rv[q] = ex[q] >= 0 && ex[q] < a.E ? ldg16(a.r + (orow * a.k + j0 + q) * a.N + col) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (ex[q] < 0 || ex[q] >= a.E) continue;
              const uint32_t u[4] = {rv[q].x, rv[q].y, rv[q].z, rv[q].w};
#pragma unroll
              for (int h = 0; h < 4; ++h) {
                f[2 * h] += __uint_as_float(u[h] << 16);
                f[2 * h + 1] += __uint_as_float(u[h] & 0xffff0000u);
              }
            }
          }
        }
        uint16_t* out = static_cast<uint16_t*>(a.out) + drow * a.ldo + col;
        *reinterpret_cast<uint4*>(out) = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                                    pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
      }
    }
  }
}

// Epilogue shared by the tile kernels: the TBM x NCOL result goes through LDS as fp32
// in passes of RP rows (RP = 64, 32 or 16, whatever the LDS area holds), then every
// thread writes 16-byte chunks of 8 columns.  Caller: all LDS reads of the main loop
// are finished (a barrier) before the first pass.
// A wavefront's result is NH 64 x 64 sub-tiles side by side along N (acc[hh]): sub-tile
// hh is placed as the 64-column band wn * NH + hh.
template <int NTHR, int BN, int RP, bool DUAL, Epi EPI, int TBM = BM, int NH = 1>
__device__ __forceinline__ void epilogue(const TileArgs& a, f32x4 (&acc)[NH][4][4], float* ep, int tid, int wm, int wn,
                                         int fr, int fq, int nt, int kp, int m_begin, int m_rows) {
  constexpr int NCOL = DUAL ? BN / 2 : BN;
  constexpr int EPI_LD = NCOL + 4;  // fp32 row stride (bank spread)
  static_assert(RP == 64 || RP == 32 || RP == 16, "rows per pass");
#pragma unroll 1
  for (int h = 0; h < TBM / RP && h * RP < m_rows; ++h) {
    // pass h covers tile rows [h*RP, h*RP + RP): 16-row fragments i0 .. i0 + RP/16 of
    // the wavefronts in 64-row band (h*RP)/64
    const int i0 = ((h * RP) & 63) >> 4;
    if (wm == (h * RP) >> 6) {
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const int band = wn * NH + hh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < i0 || i >= i0 + RP / 16) continue;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = (i - i0) * 16 + 4 * fq + v;
            if constexpr (DUAL) {
#pragma unroll
              for (int j = 0; j < 2; ++j)
                ep[r * EPI_LD + band * 32 + j * 16 + fr] = silu(acc[hh][i][j][v]) * acc[hh][i][j + 2][v];
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) ep[r * EPI_LD + band * 64 + j * 16 + fr] = acc[hh][i][j][v];
            }
          }
        }
      }
    }
    __syncthreads();
    epilogue_write<NTHR, NCOL, RP, EPI>(a, ep, tid, h, nt, kp, m_begin, m_rows);
    __syncthreads();
  }
}

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
  TilePos tp;
  if (!tile_pos<NCOL, BK>(a, tp, gridDim.x)) return;
  const int nt = tp.nt, kp = tp.kp, e = tp.e, m_begin = tp.m_begin, m_rows = tp.m_rows;
  const int K = a.K;
  const int kt0 = tp.kt0, kt1 = tp.kt1;

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
      n = min(nt * NCOL + (blk >> 1) * 32 + (r & 31), a.N - 1);  // past N: computed, never stored
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

  epilogue<NTHR, BN, 64, DUAL, EPI>(a, reinterpret_cast<f32x4(&)[1][4][4]>(acc), reinterpret_cast<float*>(smem), tid,
                                    wm, wn, fr, fq, nt, kp, m_begin, m_rows);
}

// ---------------------------------------------------------------------------------
// bf16 weights: the same tile, with both operands copied HBM/L2 -> LDS by the load
// unit itself (global_load_lds_dwordx4: each lane names a 16-byte source, the wave's
// 64 chunks land in 1 KB of consecutive LDS at M0), so no registers or VALU carry the
// staging and S LDS stages can be in flight at once.  The copies are issued from
// inline asm, which the compiler's wait insertion does not track (it would otherwise
// drain every copy in flight once per loop trip); the kernel waits for them itself:
// before the barrier of each K-step a wave lets at most the copies of the stages
// after the current one stay outstanding.  The compiler's own loads are unaffected:
// extra outstanding copies only make its vmcnt waits stricter.  A copy has no
// destination register, so nothing it writes can be reused early.
//
// A copy instruction covers 64 / (BK/8) whole tile rows; lane l takes row l / (BK/8)
// of them and logical chunk (l % (BK/8)) XOR the row's swizzle term, so the LDS image
// is the same swizzled tile the register-staged kernel writes.
// The stage image is BM + BN rows of BK elements: Q = (BM + BN) / RPI copy
// instructions of 1 KB (A rows first, then B rows), dealt round-robin to the NW
// wavefronts, so wave w issues instructions w, w + NW, ... and waits on its own count.
// LDS elements of a copy-pipeline tile shape: S stages, or the epilogue's 64 fp32 rows
template <int TBM, int BN, int BK, int S, bool DUAL>
constexpr int dma_smem_elems() {
  constexpr int NCOL = DUAL ? BN / 2 : BN;
  constexpr int STAGE_ELEMS = (TBM + BN) * BK;
  constexpr int EPI_ELEMS = 64 * (NCOL + 4) * 2;
  return S * STAGE_ELEMS > EPI_ELEMS ? S * STAGE_ELEMS : EPI_ELEMS;
}

// Wavefronts of a copy-pipeline tile: (TBM / 64) x (BN / WT), each 64 token rows x WT
// weight rows.
template <int TBM, int BN, int WT>
constexpr int dma_threads() {
  return (TBM / 64) * (BN / WT) * 64;
}

// One TBM x BN tile of the copy pipeline at position tp, with dma_threads() threads
// (the block's) and dma_smem_elems() elements of LDS at smem.  A wavefront computes
// 64 x WT (WT = 64 or 128: 4 x 4 or 4 x 8 MFMA tiles).  Per K-step a wavefront reads
// (64 + WT) rows of fragments from LDS, so the wider tile reads a quarter less of the
// LDS per flop, with half as many wavefronts issuing copies.
template <int TBM, int BN, int BK, int S, bool DUAL, AMode AM, Epi EPI, int WT = 64>
__device__ __forceinline__ void tile_dma_body(const TileArgs& a, const TilePos& tp, uint16_t* smem) {
  constexpr int NH = WT / 64;                   // 64-column sub-tiles per wavefront
  constexpr int WN = BN / WT;
  constexpr int NW = (TBM / 64) * WN;           // wavefronts
  constexpr int NTHR = NW * 64;
  constexpr int CPRK = BK / 8;                  // 16-byte chunks per LDS row
  constexpr int RPI = 64 / CPRK;                // tile rows per copy instruction
  constexpr int QA = TBM / RPI, Q = (TBM + BN) / RPI;
  constexpr int J = (Q + NW - 1) / NW;          // copy slots per wave
  constexpr int NHI = Q % NW == 0 ? NW : Q % NW;  // waves with J copies (the rest J - 1)
  constexpr int NCOL = DUAL ? BN / 2 : BN;
  constexpr int STAGE_ELEMS = (TBM + BN) * BK;
  static_assert(S >= 2 && TBM % 64 == 0 && TBM % RPI == 0 && BN % RPI == 0 && NTHR <= 1024, "pipeline shape");
  static_assert((WT == 64 || WT == 128) && BN % WT == 0, "wavefront tile");
  static_assert(J * (S - 1) < 64, "vmcnt range");

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nt = tp.nt, e = tp.e, m_begin = tp.m_begin, m_rows = tp.m_rows;
  const int K = a.K;

  // Weight row r of the B tile: matrix (gate or up for the gate/up product) and row.
  // Copy sources are 32-bit byte offsets from wave-uniform bases: the activation
  // matrix (the host keeps its size below 4 GB) or this block's expert matrix.
  auto weight_row = [&](int r, bool& second) {
    if (DUAL) {
      // rows in blocks of 32: gate, up, gate, up, ... (each wavefront's 64 rows are the
      // gate and up rows of the same 32 output columns)
      const int blk = r >> 5;
      second = blk & 1;
      return min(nt * NCOL + (blk >> 1) * 32 + (r & 31), a.N - 1);  // past N: computed, never stored
    }
    second = false;
    return min(nt * BN + r, a.N - 1);
  };
  const char* a_base = uniform_ptr(a.A);
  const char* b0_base = uniform_ptr(static_cast<const uint16_t*>(a.B0) + static_cast<int64_t>(e) * a.b_expert_stride);
  const char* b1_base =
      DUAL ? uniform_ptr(static_cast<const uint16_t*>(a.B1) + static_cast<int64_t>(e) * a.b_expert_stride) : b0_base;

  // ---- per-lane copy offsets: instruction q fills stage rows [RPI*q, RPI*q + RPI)
  const int lr = lane / CPRK;
  const int lc = (lane % CPRK) ^ swz<BK>(lr);   // logical chunk (RPI*q is a multiple of 8 or 16)
  uint32_t off[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int q = min(w + j * NW, Q - 1);       // slot past Q: never issued
    if (q < QA) {
      const int r = min(RPI * q + lr, m_rows - 1);  // clamped rows: computed, never stored
      int row;
      if constexpr (AM == AMode::GATHER)
        row = a.perm[m_begin + r] / a.k;
      else
        row = m_begin + r;
      off[j] = (static_cast<uint32_t>(row) * K + lc * 8) * 2;
    } else {
      bool second;
      off[j] = (static_cast<uint32_t>(weight_row(RPI * (q - QA) + lr, second)) * K + lc * 8) * 2;
    }
  }
  // the base of each of this wave's instructions (an instruction's RPI rows lie in one
  // 32-row block, so one matrix), in scalar registers
  const char* ibase[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int q = min(w + j * NW, Q - 1);
    bool second = false;
    if (q >= QA) weight_row(RPI * (q - QA), second);
    ibase[j] = uniform_ptr(q < QA ? a_base : second ? b1_base : b0_base);
  }
  auto issue = [&](int stage, int kt) {
    const uint16_t* st = smem + stage * STAGE_ELEMS;
    const int kb = kt * BK * 2;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int q = w + j * NW;
      if (j < J - 1 || w < NHI) copy_to_lds(ibase[j] + kb, off[j], st + q * 512);
    }
  };

  f32x4 acc[NH][4][4];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[hh][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wm = w / WN, wn = w % WN;
  const int fr = lane & 15, fq = lane >> 4;
  const int a_rd = (wm * 64 + fr) * BK, b_rd = (wn * WT + fr) * BK;
  // Compute of `stage` with the copies of a later stage spread over its MFMA groups.  A
  // wave's instructions issue in order, and the load unit takes a CU's copy instructions
  // one at a time (about 30 cycles each, from TA_TA_BUSY), so copies issued all at once
  // hold back the MFMAs behind them.  With three stages (two K-steps of slack) spreading
  // them lets both proceed: the Ling-3.0-tiny gate/up (128 x 256 x 64) 183 -> 173.5 us,
  // the Ling-lite shared down + combine 77 -> 74.5 us.  With two stages the copies must
  // land within one step, and spread they landed late (Ling-lite gate/up 382 -> 411 us),
  // so those kernels issue them all at the start of the step.
  constexpr int NG = (BK / 32) * NH * 4;  // MFMA groups (one row i of one sub-tile per group)
  auto compute_issue = [&](int stage, bool do_issue, int nstage, int kt) {
    const uint16_t* As = smem + stage * STAGE_ELEMS;
    const uint16_t* Bs = As + TBM * BK;
    const uint16_t* st = smem + nstage * STAGE_ELEMS;
    const int kb = kt * BK * 2;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int cc = ((ks * 4 + fq) ^ swz<BK>(fr)) << 3;
      uint4 af[4], bf[4 * NH];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const uint4*>(&As[a_rd + cc + i * 16 * BK]);
#pragma unroll
      for (int j = 0; j < 4 * NH; ++j) bf[j] = *reinterpret_cast<const uint4*>(&Bs[b_rd + cc + j * 16 * BK]);
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int g = (ks * NH + hh) * 4 + i;
#pragma unroll
          for (int jc = 0; jc < J; ++jc) {
            if (jc * NG / J == g && do_issue && (jc < J - 1 || w < NHI)) {
              __builtin_amdgcn_sched_barrier(0);
              copy_to_lds(ibase[jc] + kb, off[jc], st + (w + jc * NW) * 512);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[hh][i][j] = mfma16_bf16(af[i], bf[hh * 4 + j], acc[hh][i][j]);
        }
    }
  };
  auto compute = [&](int stage) { compute_issue(stage, false, 0, 0); };

  // K-step t lives in stage t % S.  Steps up to t + S - 2 are issued before step t is
  // consumed, so before the barrier of step t a wave lets min(S - 2, n - 1 - t) stages
  // of its copies stay outstanding.
  const int kt0 = tp.kt0, n = tp.kt1 - tp.kt0;
#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < n) issue(p, kt0 + p);
  int cur = 0, nxt = S - 1;  // stages of steps t and t + S - 1
  for (int t = 0; t < n; ++t) {
    const int ahead = n - 1 - t;
    if (w < NHI)
      copy_wait_ahead<J, S - 2>(ahead);
    else
      copy_wait_ahead<J - 1, S - 2>(ahead);
    lds_barrier();
    if constexpr (S >= 3) {
      compute_issue(cur, t + S - 1 < n, nxt, kt0 + t + S - 1);
    } else {
      if (t + S - 1 < n) issue(nxt, kt0 + t + S - 1);
      compute(cur);
    }
    cur = cur + 1 == S ? 0 : cur + 1;
    nxt = nxt + 1 == S ? 0 : nxt + 1;
  }
  copy_wait<0>();  // every wave is done reading the stages; all copies have landed
  lds_barrier();
  epilogue<NTHR, BN, 64, DUAL, EPI, TBM, NH>(a, acc, reinterpret_cast<float*>(smem), tid, wm, wn, fr, fq, nt, tp.kp,
                                         m_begin, m_rows);
}

template <int BN, int BK, int S, bool DUAL, AMode AM, Epi EPI, int WT>
__global__ __launch_bounds__((dma_threads<BM, BN, WT>())) void k_tile_dma(TileArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[dma_smem_elems<BM, BN, BK, S, DUAL>()];
  TilePos tp;
  if (!tile_pos<DUAL ? BN / 2 : BN, BK>(a, tp, gridDim.x)) return;
  tile_dma_body<BM, BN, BK, S, DUAL, AM, EPI, WT>(a, tp, smem);
}

// Routed gate/up (SwiGLU) whose last 256-column N-tile is at most half full (e.g. 1408
// = 5 x 256 + 128 columns).  Blocks [0, a.rem_first) take 128 x 512 tiles of the full
// N-tiles [0, N / 256); the blocks past it take the last N % 256 columns as 256 x 256
// tiles (128 columns of gate and of up) over chunks of 256 positions (tiles2), so
// those columns cost 512 rows of copies per K-step instead of 640 for half the useful
// work.  The remainder blocks come last, as the smallest units of the final round.
template <AMode AM, int WT>
__global__ __launch_bounds__((dma_threads<BM, 512, WT>())) void k_tile_dma_split(TileArgs a, int rem_first) {
  static_assert(dma_threads<BM, 512, WT>() == dma_threads<256, 256, WT>(), "one block size for both tile shapes");
  constexpr int SM_MAIN = dma_smem_elems<BM, 512, 64, 2, true>();
  constexpr int SM_REM = dma_smem_elems<256, 256, 64, 2, true>();
  __shared__ __attribute__((aligned(16))) uint16_t smem[SM_MAIN > SM_REM ? SM_MAIN : SM_REM];
  const int nt_main = a.N / 256;
  TilePos tp;
  if (static_cast<int>(blockIdx.x) < rem_first) {
    if (!tile_pos<256, 64>(a, tp, rem_first, nt_main)) return;
    tile_dma_body<BM, 512, 64, 2, true, AM, Epi::SWIGLU, WT>(a, tp, smem);
    return;
  }
  const int r = blockIdx.x - rem_first;
  if (r >= a.meta[3]) return;
  tp.e = a.tiles2[2 * r];
  tp.m_begin = a.tiles2[2 * r + 1];
  tp.m_rows = min(256, a.offsets[tp.e + 1] - tp.m_begin);
  tp.nt = 2 * nt_main;  // 128-column tiles: column base nt_main * 256
  tp.kp = 0;
  tp.kt0 = 0;
  tp.kt1 = a.K / 64;
  tile_dma_body<256, 256, 64, 2, true, AM, Epi::SWIGLU, WT>(a, tp, smem);
}

// ---------------------------------------------------------------------------------
// u8 weights through the copy pipeline: a 128 x 512 x 64 tile whose weight operand
// stays as codes in LDS.  Each of the 16 wavefronts owns all 128 token rows and 32
// weight rows (8 x 2 MFMA tiles), so every weight fragment is dequantised by exactly
// one wavefront; gate/up interleave gate and up rows in 16-row blocks, so a
// wavefront's two fragments are the gate and up rows of the same 16 output columns.
// Two stages of (bytes):
//   A   128 token rows x 128 B (bf16, 16-byte chunks XOR-swizzled by row % 8), 16 KB;
//   Bq  512 weight rows x 64 B of codes (16-byte chunk c of row r at slot
//       c ^ (r / 2) % 4, which spreads the 8-byte fragment reads of 16 rows over the
//       bank lines), 32 KB;
// and, double-buffered per window of 8 K-steps, the fp16 scales and zero points of the
// 512 rows for those 8 groups (16 bytes per row and kind, one copy lane each), 16 KB.
// Copying a row's parameters once per 8 K-steps keeps their line requests at an eighth
// of the rows per step (per-step copies touched one line per row, more lines than the
// codes and tokens together).  Each wavefront issues three copies per K-step (8 token
// rows, twice 16 code rows) and, at the first step of a window, one parameter copy for
// the next window (64 rows of scales or of zero points; those rows span gate and up
// blocks, so the lanes carry their own 64-bit addresses).  A fragment (16 rows x 8
// codes per lane) is dequantised in registers as s * (q - z), rounded to bf16 (the
// values the register-staged kernel stores), right before its MFMAs.
constexpr int kQ8Stage = 128 * 128 + 512 * 64;
constexpr int kQ8Params = 2 * 512 * 16;  // one window: scales, then zero points

template <bool DUAL, AMode AM, Epi EPI>
__global__ __launch_bounds__(1024) void k_tile_dma_q8(TileArgs a) {
  constexpr int TBM = BM, BN = 512, BK = 64, S = 2, WIN = 8, NTHR = 1024;
  constexpr int NCOL = DUAL ? BN / 2 : BN;
  constexpr int EPI_LD = NCOL + 4;
  constexpr int A_BYTES = TBM * BK * 2;
  static_assert(A_BYTES + BN * BK == kQ8Stage, "stage layout");
  constexpr int PIPE_BYTES = S * kQ8Stage + 2 * kQ8Params;
  constexpr int SMEM_BYTES = PIPE_BYTES > 64 * EPI_LD * 4 ? PIPE_BYTES : 64 * EPI_LD * 4;
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_BYTES / 2];
  char* const sm = reinterpret_cast<char*>(smem);
  char* const pm = sm + S * kQ8Stage;  // parameter windows

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  TilePos tp;
  if (!tile_pos<NCOL, BK>(a, tp, gridDim.x)) return;
  const int nt = tp.nt, e = tp.e, m_begin = tp.m_begin, m_rows = tp.m_rows;
  const int K = a.K, G = K / 64;

  // weight row of B tile row r (and whether it is an up row)
  auto weight_row = [&](int r, bool& second) {
    if (DUAL) {
      const int blk = r >> 4;
      second = blk & 1;
      return min(nt * NCOL + (blk >> 1) * 16 + (r & 15), a.N - 1);  // past N: computed, never stored
    }
    second = false;
    return min(nt * BN + r, a.N - 1);
  };
  const int64_t erow = static_cast<int64_t>(e) * a.N;  // first weight row of this expert
  const char* a_base = uniform_ptr(a.A);
  const char* q0_base = uniform_ptr(static_cast<const uint8_t*>(a.B0) + erow * K);
  const char* q1_base = DUAL ? uniform_ptr(static_cast<const uint8_t*>(a.B1) + erow * K) : q0_base;

  // copy 0: A rows 8w + l/8
  uint32_t a_off;
  {
    const int lr = lane >> 3, r = min(8 * w + lr, m_rows - 1);
    int row;
    if constexpr (AM == AMode::GATHER)
      row = a.perm[m_begin + r] / a.k;
    else
      row = m_begin + r;
    a_off = (static_cast<uint32_t>(row) * K + (((lane & 7) ^ (lr & 7)) << 3)) * 2;
  }
  // copies 1, 2: code rows 16 q + l/4 for q = w and 16 + w (one 16-row block: one matrix)
  uint32_t q_off[2];
  const char* q_base[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = 16 * h + w;
    const int r = 16 * q + (lane >> 2);
    bool second;
    const int n = weight_row(r, second);
    q_off[h] = static_cast<uint32_t>(n) * K + (((lane & 3) ^ ((r >> 1) & 3)) << 4);
    q_base[h] = second ? q1_base : q0_base;
  }
  // parameter copy: rows 64 (w % 8) + l, scales for w < 8, zero points otherwise
  const uint16_t* p_src;
  {
    const int r = 64 * (w & 7) + lane;
    bool second;
    const int n = weight_row(r, second);
    const uint16_t* arr = (w < 8) ? (second ? a.B1s : a.B0s) : (second ? a.B1z : a.B0z);
    p_src = arr + (erow + n) * G;
  }
  auto issue = [&](int stage, int kt) {
    char* st = sm + stage * kQ8Stage;
    copy_to_lds(a_base + kt * BK * 2, a_off, reinterpret_cast<uint16_t*>(st + w * 1024));
#pragma unroll
    for (int h = 0; h < 2; ++h)
      copy_to_lds(q_base[h] + kt * BK, q_off[h], reinterpret_cast<uint16_t*>(st + A_BYTES + (16 * h + w) * 1024));
  };
  auto issue_params = [&](int win) {  // groups [8 win, 8 win + 8)
    copy_to_lds(p_src + WIN * win, reinterpret_cast<uint16_t*>(pm + (win & 1) * kQ8Params + w * 1024));
  };

  f32x4 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fq = lane >> 4;
  auto compute = [&](int stage, int kt) {
    const char* st = sm + stage * kQ8Stage;
    const uint16_t* As = reinterpret_cast<const uint16_t*>(st);
    const char* Bq = st + A_BYTES;
    const uint16_t* Ps = reinterpret_cast<const uint16_t*>(pm + ((kt / WIN) & 1) * kQ8Params);
    const uint16_t* Pz = Ps + BN * WIN;
    float sf[2], zf[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 32 * w + 16 * j + fr;
      sf[j] = f16_to_f32(Ps[r * WIN + kt % WIN]);
      zf[j] = f16_to_f32(Pz[r * WIN + kt % WIN]);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int cc = ((ks * 4 + fq) ^ (fr & 7)) << 3;
      uint4 af[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) af[i] = *reinterpret_cast<const uint4*>(&As[(i * 16 + fr) * BK + cc]);
      const int o = ks * 4 + fq;  // 8-code group of the row
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 32 * w + 16 * j + fr;
        const uint2 c =
            *reinterpret_cast<const uint2*>(Bq + r * 64 + (((o >> 1) ^ ((r >> 1) & 3)) << 4) + ((o & 1) << 3));
        const float sj = sf[j], zj = zf[j];
        uint4 bfr;
        bfr.x = pack_bf16x2(sj * (static_cast<float>(c.x & 0xffu) - zj), sj * (static_cast<float>((c.x >> 8) & 0xffu) - zj));
        bfr.y = pack_bf16x2(sj * (static_cast<float>((c.x >> 16) & 0xffu) - zj), sj * (static_cast<float>(c.x >> 24) - zj));
        bfr.z = pack_bf16x2(sj * (static_cast<float>(c.y & 0xffu) - zj), sj * (static_cast<float>((c.y >> 8) & 0xffu) - zj));
        bfr.w = pack_bf16x2(sj * (static_cast<float>((c.y >> 16) & 0xffu) - zj), sj * (static_cast<float>(c.y >> 24) - zj));
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i][j] = mfma16_bf16(af[i], bfr, acc[i][j]);
      }
    }
  };

  // Two stages: the copies of K-step t + 1 (and, at the first step of a window, the next
  // window's parameters) are issued after the barrier of step t and have all landed
  // before the barrier of step t + 1.  A window's parameter buffer is refilled two
  // windows later, after every wave has passed the barrier of the step that follows its
  // last step.
  const int nk = tp.kt1 - tp.kt0;  // the whole K (no split): windows start at steps 0, 8, ..
  if (nk > 0) {
    issue_params(0);
    issue(0, 0);
  }
  for (int t = 0; t < nk; ++t) {
    copy_wait<0>();
    lds_barrier();
    if (t + 1 < nk) issue((t + 1) & 1, t + 1);
    if (t % WIN == 0 && t + WIN < nk) issue_params(t / WIN + 1);
    compute(t & 1, t);
  }
  copy_wait<0>();
  lds_barrier();
  // epilogue in two passes of 64 rows: every wavefront stages its 16 (SwiGLU) or 32
  // columns of the pass's rows, then the block writes them out
  float* ep = reinterpret_cast<float*>(smem);
#pragma unroll 1
  for (int h = 0; h < 2 && h * 64 < m_rows; ++h) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i >> 2) != h) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = (i - 4 * h) * 16 + 4 * fq + v;
        if constexpr (DUAL) {
          ep[r * EPI_LD + 16 * w + fr] = silu(acc[i][0][v]) * acc[i][1][v];
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) ep[r * EPI_LD + 32 * w + 16 * j + fr] = acc[i][j][v];
        }
      }
    }
    __syncthreads();
    epilogue_write<NTHR, NCOL, 64, EPI>(a, ep, tid, h, nt, tp.kp, m_begin, m_rows);
    __syncthreads();
  }
}

// blocks of a launch: whole groups of M-tiles (extra tiles exit) x N-tiles x K-splits,
// rounded up to the 8 XCDs (NT: the N-tiles, 0 for all of N)
inline int64_t grid_blocks(const TileArgs& a, int ncol, int NT = 0) {
  if (NT <= 0) NT = (a.N + ncol - 1) / ncol;
  const int G = a.group_m > 1 ? a.group_m : 1;  // (expert grouping: group_m <= 0, G = 1)
  const int64_t mt_pad = (a.mtiles_bound + G - 1) / G * G;
  const int64_t blocks = mt_pad * NT * (a.ksplit > 1 ? a.ksplit : 1);
  return (blocks + 7) / 8 * 8;
}

// Dense products (group_m <= 0): the M-tiles per block-order group.  Each XCD takes a
// contiguous eighth of the logical tile order (tile_pos), so with G M-tiles per group
// it reads about min(G, P) activation panels of BM rows and ceil(P / G) weight panels
// of `brows` rows (P tiles per XCD).  G is the power of two (padding the M-tiles by at
// most an eighth) that minimises those rows: for the Ling-lite shared gate/up at 4096
// tokens (32 M-tiles, 11 panels of 512 rows, 44 tiles per XCD) 16 instead of 4, which
// takes each XCD from all 11 weight panels to 3.
inline int dense_group_m(const TileArgs& a, int ncol, int brows) {
  const int64_t mt = a.mtiles_bound, NT = (a.N + ncol - 1) / ncol, KS = a.ksplit > 1 ? a.ksplit : 1;
  int best = 1;
  int64_t best_rows = -1;
  for (int G = 1; G <= 64 && G <= mt; G *= 2) {
    const int64_t mt_pad = (mt + G - 1) / G * G;
    if ((mt_pad - mt) * 8 > mt) continue;
    const int64_t P = (mt_pad * NT * KS + 7) / 8;
    const int64_t rows = std::min<int64_t>(G, P) * BM + (P + G - 1) / G * brows;
    if (best_rows < 0 || rows < best_rows) {
      best = G;
      best_rows = rows;
    }
  }
  return best;
}
inline TileArgs with_dense_group(const TileArgs& a, int ncol, int brows) {
  TileArgs b = a;
  if (!a.routed && a.group_m <= 0) b.group_m = dense_group_m(a, ncol, brows);
  return b;
}

template <int BN, int BK, WFmt WF, bool DUAL, AMode AM, Epi EPI>
hipError_t launch_one(const TileArgs& a0, hipStream_t s) {
  const TileArgs a = with_dense_group(a0, DUAL ? BN / 2 : BN, BN);
  const int64_t blocks = grid_blocks(a, DUAL ? BN / 2 : BN);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_tile<BN, BK, WF, DUAL, AM, EPI>), dim3(static_cast<unsigned>(blocks)), dim3(BN * 2), 0, s, a);
  return hipGetLastError();
}

// Wavefront tile width (weight rows).  The routed gate/up takes 64 x 128 wavefront
// tiles (8 wavefronts per 128 x 512 block, a quarter fewer LDS fragment reads per
// flop); measured against 64 x 64 tiles (16 wavefronts) on the MI355X: Ling-lite at
// 4096 tokens 419 -> 409 us, Ling-3.0-flash at 8192 tokens 2036-2061 -> 2028-2031 us.
// The single-matrix products keep 64 x 64 (routed down with 64 x 128: 224 -> 233 us
// and 673 -> 717 us on the Ling-lite and Ling-2.6-flash shapes), and so does the
// dense gate/up (the shared expert: 160 -> 165 us on the Ling-3.0-flash shape).
constexpr int kWaveGateUp = 128;
template <int BN, bool DUAL, AMode AM>
constexpr int wave_width() {
  return BN == 512 && DUAL && AM == AMode::GATHER ? kWaveGateUp : 64;
}

template <int BN, int BK, int S, bool DUAL, AMode AM, Epi EPI>
hipError_t launch_dma(const TileArgs& a0, hipStream_t s) {
  const TileArgs a = with_dense_group(a0, DUAL ? BN / 2 : BN, BN);
  constexpr int WT = wave_width<BN, DUAL, AM>();
  const int64_t blocks = grid_blocks(a, DUAL ? BN / 2 : BN);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_tile_dma<BN, BK, S, DUAL, AM, EPI, WT>), dim3(static_cast<unsigned>(blocks)),
                     dim3(dma_threads<BM, BN, WT>()), 0, s, a);
  return hipGetLastError();
}

// Tile shapes of the copy pipeline (bf16 weights): 128 token rows x 512 weight rows,
// K-step 64, two LDS stages (160 KB, one block per CU).  A dense
// single-matrix product with fewer such blocks than CUs, and a gate/up product whose
// last 256-column tile would be mostly padding, take 128 x 256 x 64 with three stages
// instead.
template <AMode AM>
hipError_t launch_split(const TileArgs& a, hipStream_t s) {
  const int64_t main_blocks = grid_blocks(a, 256, a.N / 256);
  const int64_t blocks = main_blocks + a.mtiles2_bound;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_tile_dma_split<AM, kWaveGateUp>), dim3(static_cast<unsigned>(blocks)),
                     dim3(dma_threads<BM, 512, kWaveGateUp>()), 0, s, a,
                     static_cast<int>(main_blocks));
  return hipGetLastError();
}

template <WFmt WF, bool DUAL, AMode AM, Epi EPI>
hipError_t launch_bn(const TileArgs& a, hipStream_t s) {
  if constexpr (WF == WFmt::BF16) {
    // dense products (the shared expert, the dense MLP) whose 128 x 512 blocks would not
    // fill the CUs take 128 x 256 x 64 with three stages (the Ling-2.6-flash shared
    // gate/up at 4096 tokens: 128 blocks of 512 columns, 144 -> 87 us)
    if (!a.routed && grid_blocks(a, DUAL ? 256 : 512) < a.ncu) return launch_dma<256, 64, 3, DUAL, AM, EPI>(a, s);
    // a routed gate/up whose experts average at most 192 tokens (one or two M-tiles
    // each, so a 512-column weight panel serves few tiles) takes the three-stage
    // 128 x 256 tile as well: Ling-2.6-flash at 4096 tokens 1089 -> 959 us (layer 1.81 ->
    // 1.72 ms), Ling-3.0-flash at 8192 tokens 1924 -> 1913 us; Ling-lite, 384 tokens per
    // expert, stays on 128 x 512 (385 against 395 us)
    if constexpr (DUAL && EPI == Epi::SWIGLU)
      if (a.routed && a.plain_order) return launch_dma<256, 64, 3, DUAL, AM, EPI>(a, s);
    // gate/up whose width leaves more than an eighth of the last 256-column tile empty
    // (e.g. 384 = 256 + 128) takes 128-column tiles
    if (DUAL && (a.N + 255) / 256 * 256 - a.N > a.N / 8) return launch_dma<256, 64, 3, DUAL, AM, EPI>(a, s);
    // routed gate/up whose last 256-column tile is at most half full (e.g. 1408 = 5 x 256
    // + 128): that tile over 256-position chunks (measured on the Ling-lite shape at 4096
    // tokens: 463 -> 420 us; the 384-wide tiny shape stays on 128-column tiles, 194 vs
    // 200 us)
    if constexpr (DUAL && EPI == Epi::SWIGLU)
      if (a.routed && a.tiles2 && a.N > 256 && a.N % 256 != 0 && a.N % 256 <= 128)
        return launch_split<AM>(a, s);
    return launch_dma<512, 64, 2, DUAL, AM, EPI>(a, s);
  } else {
    // u8 weights: codes through the copy pipeline (k_tile_dma_q8) when every row's
    // parameters of 8 groups can be copied as one aligned 16-byte chunk (K a multiple
    // of 512, 16-byte aligned parameter arrays); measured on the Ling-3.0-flash shape at
    // 8192 tokens: gate/up 3251 -> 2131 us, down 1462 -> 1236 us.  Otherwise the weights
    // are dequantised in registers on their way to LDS: single-matrix products take the
    // wide 8-wavefront tile with K-step 32, gate/up 128 x 128 x 64.
    {
      const bool al16 = (reinterpret_cast<uintptr_t>(a.B0s) | reinterpret_cast<uintptr_t>(a.B0z) |
                         (DUAL ? reinterpret_cast<uintptr_t>(a.B1s) | reinterpret_cast<uintptr_t>(a.B1z) : 0)) % 16 == 0;
      if (a.K % 512 == 0 && al16 && a.ksplit <= 1) {
        const int64_t blocks = grid_blocks(a, DUAL ? 256 : 512);
        if (blocks <= 0) return hipSuccess;
        hipLaunchKernelGGL((k_tile_dma_q8<DUAL, AM, EPI>), dim3(static_cast<unsigned>(blocks)), dim3(1024), 0, s, a);
        return hipGetLastError();
      }
    }
    if (!DUAL && a.N >= 256) return launch_one<256, 32, WF, DUAL, AM, EPI>(a, s);
    return launch_one<128, 64, WF, DUAL, AM, EPI>(a, s);
  }
}

}  // namespace

hipError_t launch_tile_gemm(const TileArgs& a, AMode am, WFmt wf, Epi epi, hipStream_t s) {
  // the combinations the layer uses
  if (epi == Epi::F32 && am == AMode::DENSE && wf == WFmt::BF16)
    return launch_dma<128, 64, 2, false, AMode::DENSE, Epi::F32>(a, s);
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
