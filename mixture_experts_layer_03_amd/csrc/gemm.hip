// Tiled bf16 MFMA GEMM for large token batches (prefill): C = A B^T with both
// operands K-contiguous, as every product of the layer is:
//   router     logits[T,E]   = x[T,H]  W_r[E,H]^T                (fp32 out)
//   up         Hm[pos,I]     = silu(x W_g[e]^T) * (x W_u[e]^T)   (tokens gathered per expert)
//   down       r[slot,H]     = w_slot * Hm[pos] W_d[e]^T         (scattered to slot order)
//   shared     Hs[T,I_s], y  = Hs W_sd^T + sum_j r[t,j]          (combine fused)
// Expert weights are [out, in] per expert [mlxcel #838 "Validation checkpoint"], so
// the weight operand rows are the output features and K runs along memory.
//
// Tile 128 (tokens) x 128 (weight rows) x 64, 256 threads as 2 x 2 wavefronts of
// 64 x 64, each a 4 x 4 grid of v_mfma_f32_16x16x32_bf16.  Operands are staged
// global -> registers -> LDS (double buffered, 16-byte chunks XOR-swizzled by row so
// fragment reads do not collide on banks).  u8 weights are dequantised to bf16
// (s * (q - z), rounded to nearest even) while being written to LDS.
// Blocks are numbered so that consecutive tiles share an XCD (its L2 holds the
// shared A rows and weight panels).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = kTileM, BN = 128, BK = 64;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

template <WFmt WF, bool DUAL, AMode AM, Epi EPI>
__global__ __launch_bounds__(256, 2) void k_tile(TileArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int NT = DUAL ? a.N / 64 : (a.N + BN - 1) / BN;
  const int per = gridDim.x / 8;
  const int L = (blockIdx.x % 8) * per + blockIdx.x / 8;
  const int mt = L / NT, nt = L % NT;

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

  // staging assignment: A rows r = tid/8 + 32 i, 16-byte chunk tid % 8
  const int sc = tid & 7;
  const uint16_t* arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min((tid >> 3) + 32 * i, m_rows - 1);
    int64_t row;
    if constexpr (AM == AMode::GATHER)
      row = a.perm[m_begin + r] / a.k;
    else
      row = m_begin + r;
    arow[i] = a.A + row * K + sc * 8;
  }

  // weight rows
  constexpr int BR = WF == WFmt::U8 ? 2 : 4;  // rows staged per thread
  const uint8_t* brow[BR];
  const uint16_t* bsrow[BR];
  const uint16_t* bzrow[BR];
  int brow_lds[BR];
  const int bchunk = WF == WFmt::U8 ? (tid & 3) : sc;
  const int esz = WF == WFmt::U8 ? 1 : 2;
#pragma unroll
  for (int i = 0; i < BR; ++i) {
    const int rb = WF == WFmt::U8 ? (tid >> 2) + 64 * i : (tid >> 3) + 32 * i;
    brow_lds[i] = rb;
    int n;
    const void* base;
    const uint16_t *bs, *bz;
    if (DUAL) {
      const int blk = rb >> 5;
      n = nt * 64 + (blk >> 1) * 32 + (rb & 31);
      base = (blk & 1) ? a.B1 : a.B0;
      bs = (blk & 1) ? a.B1s : a.B0s;
      bz = (blk & 1) ? a.B1z : a.B0z;
    } else {
      n = min(nt * BN + rb, a.N - 1);
      base = a.B0;
      bs = a.B0s;
      bz = a.B0z;
    }
    const int64_t ro = static_cast<int64_t>(e) * a.N + n;
    brow[i] = static_cast<const uint8_t*>(base) +
              (static_cast<int64_t>(e) * a.b_expert_stride + static_cast<int64_t>(n) * K) * esz +
              bchunk * 16;
    if constexpr (WF == WFmt::U8) {
      bsrow[i] = bs + ro * (K / 64);
      bzrow[i] = bz + ro * (K / 64);
    } else {
      bsrow[i] = nullptr;
      bzrow[i] = nullptr;
    }
  }

  uint4 ra[4], rbv[4];
  float rsc[BR], rzp[BR];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = ldg16(arow[i] + k0);
    if constexpr (WF == WFmt::U8) {
#pragma unroll
      for (int i = 0; i < BR; ++i) {
        rbv[i] = ldg16(brow[i] + k0);
        rsc[i] = f16_to_f32(bsrow[i][kt]);
        rzp[i] = f16_to_f32(bzrow[i][kt]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < BR; ++i) rbv[i] = ldg16(brow[i] + 2 * k0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&As[buf][swz((tid >> 3) + 32 * i, sc)]) = ra[i];
    if constexpr (WF == WFmt::U8) {
#pragma unroll
      for (int i = 0; i < BR; ++i) {
        const uint32_t q[4] = {rbv[i].x, rbv[i].y, rbv[i].z, rbv[i].w};
        uint32_t o[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float s = rsc[i], z = rzp[i];
          o[2 * c] = pack_bf16x2(s * (static_cast<float>(q[c] & 0xffu) - z),
                                 s * (static_cast<float>((q[c] >> 8) & 0xffu) - z));
          o[2 * c + 1] = pack_bf16x2(s * (static_cast<float>((q[c] >> 16) & 0xffu) - z),
                                     s * (static_cast<float>(q[c] >> 24) - z));
        }
        const int r = brow_lds[i];
        *reinterpret_cast<uint4*>(&Bs[buf][swz(r, 2 * bchunk)]) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(&Bs[buf][swz(r, 2 * bchunk + 1)]) = make_uint4(o[4], o[5], o[6], o[7]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < BR; ++i) *reinterpret_cast<uint4*>(&Bs[buf][swz(brow_lds[i], sc)]) = rbv[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wm = w >> 1, wn = w & 1;
  const int fr = lane & 15, fq = lane >> 4;
  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 64 + i * 16 + fr;
        af[i] = *reinterpret_cast<const uint4*>(&As[buf][swz(row, ks * 4 + fq)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 64 + j * 16 + fr;
        bf[j] = *reinterpret_cast<const uint4*>(&Bs[buf][swz(row, ks * 4 + fq)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16_bf16(af[i], bf[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[m][n], m = wm*64 + i*16 + 4*fq + v, n = wn*64 + j*16 + fr
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = wm * 64 + i * 16 + 4 * fq + v;
      if (m >= m_rows) continue;
      const int64_t orow = m_begin + m;
      if constexpr (EPI == Epi::SWIGLU) {
        uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = nt * 64 + wn * 32 + j * 16 + fr;
          out[orow * a.ldo + col] = f32_to_bf16(silu(acc[i][j][v]) * acc[i][j + 2][v]);
        }
      } else if constexpr (EPI == Epi::F32) {
        float* out = static_cast<float*>(a.out);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = nt * BN + wn * 64 + j * 16 + fr;
          if (col < a.N) out[orow * a.ldo + col] = acc[i][j][v];
        }
      } else if constexpr (EPI == Epi::SCALED_SLOT) {
        uint16_t* out = static_cast<uint16_t*>(a.out);
        const int slot = a.perm[orow];
        const float ws = a.topk_w[slot];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = nt * BN + wn * 64 + j * 16 + fr;
          if (col < a.N) out[static_cast<int64_t>(slot) * a.ldo + col] = f32_to_bf16(ws * acc[i][j][v]);
        }
      } else {  // COMBINE: y[t] = shared + sum_j r[t*k + j]
        uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = nt * BN + wn * 64 + j * 16 + fr;
          if (col >= a.N) continue;
          float s = acc[i][j][v];
          for (int jj = 0; jj < a.k; ++jj) {
            const int64_t slot = orow * a.k + jj;
            const int ex = a.idx[slot];
            if (ex >= 0 && ex < a.E) s += bf16_to_f32(a.r[slot * a.N + col]);
          }
          out[orow * a.ldo + col] = f32_to_bf16(s);
        }
      }
    }
  }
}

template <WFmt WF, bool DUAL, AMode AM, Epi EPI>
hipError_t launch_one(const TileArgs& a, hipStream_t s) {
  const int NT = DUAL ? a.N / 64 : (a.N + BN - 1) / BN;
  int64_t blocks = static_cast<int64_t>(a.mtiles_bound) * NT;
  blocks = (blocks + 7) / 8 * 8;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_tile<WF, DUAL, AM, EPI>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_gemm(const TileArgs& a, AMode am, WFmt wf, Epi epi, hipStream_t s) {
  // the combinations the layer uses
  if (epi == Epi::F32 && am == AMode::DENSE && wf == WFmt::BF16)
    return launch_one<WFmt::BF16, false, AMode::DENSE, Epi::F32>(a, s);
  if (epi == Epi::SWIGLU && am == AMode::GATHER && wf == WFmt::BF16)
    return launch_one<WFmt::BF16, true, AMode::GATHER, Epi::SWIGLU>(a, s);
  if (epi == Epi::SWIGLU && am == AMode::GATHER && wf == WFmt::U8)
    return launch_one<WFmt::U8, true, AMode::GATHER, Epi::SWIGLU>(a, s);
  if (epi == Epi::SWIGLU && am == AMode::DENSE && wf == WFmt::BF16)
    return launch_one<WFmt::BF16, true, AMode::DENSE, Epi::SWIGLU>(a, s);
  if (epi == Epi::SCALED_SLOT && am == AMode::DENSE && wf == WFmt::BF16)
    return launch_one<WFmt::BF16, false, AMode::DENSE, Epi::SCALED_SLOT>(a, s);
  if (epi == Epi::SCALED_SLOT && am == AMode::DENSE && wf == WFmt::U8)
    return launch_one<WFmt::U8, false, AMode::DENSE, Epi::SCALED_SLOT>(a, s);
  if (epi == Epi::COMBINE && am == AMode::DENSE && wf == WFmt::BF16)
    return launch_one<WFmt::BF16, false, AMode::DENSE, Epi::COMBINE>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
