// Weight-streaming kernels for small token batches (decode).
//
// Decode is bound by reading weights: only the selected experts' weights are read
// [Ling-3.0-flash-GGUF card, "Measured performance": decode is memory-bandwidth
// bound and only the selected experts are read].  Each wavefront owns 16 weight
// rows (one MFMA N-tile) and a range of the reduction axis, streams those rows once
// with 16-byte loads, and multiplies them against up to 64 tokens held as four
// 16-row MFMA M-tiles (tokens padded to 16; padded rows are computed and dropped).
//
// K ordering: the MFMA pairs A and B values by K-group (lane / 16) and position, so
// any permutation of k applied identically to both operands leaves the products
// unchanged.  Each 64-element step is mapped so that one load instruction covers 64
// contiguous bytes of every one of its 16 rows (bf16: two instructions per step,
// u8: one), i.e. whole cache-line halves.
#include <initializer_list>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

template <Act A>
struct ActType;
template <>
struct ActType<Act::BF16> {
  using T = uint16_t;
};
template <>
struct ActType<Act::F32> {
  using T = float;
};

template <WFmt F>
struct WType;
template <>
struct WType<WFmt::BF16> {
  using T = uint16_t;
};
template <>
struct WType<WFmt::F32> {
  using T = float;
};
template <>
struct WType<WFmt::U8> {
  using T = uint8_t;
};

// Per-lane operand pointers of one wavefront task.
template <Act ACT, WFmt WF, int NMAT, int MT>
struct Task {
  using AT = typename ActType<ACT>::T;
  using WT = typename WType<WF>::T;
  const AT* arow[MT];          // token row of lane (l % 16) in each M-tile (clamped valid)
  const WT* wrow[NMAT];        // weight row of lane (l % 16) (clamped valid)
  const uint16_t* srow[NMAT];  // u8: scale row (one per 64 elements)
  const uint16_t* zrow[NMAT];  // u8: zero-point row
  int mt_live;                 // M-tiles holding at least one real token
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 16 u8 codes -> 16 bf16 values (q - z), exact (integers in [-255, 255]).
__device__ __forceinline__ void dequant16(const uint4& q, float z, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float f0 = static_cast<float>(w[i] & 0xffu) - z;
    const float f1 = static_cast<float>((w[i] >> 8) & 0xffu) - z;
    const float f2 = static_cast<float>((w[i] >> 16) & 0xffu) - z;
    const float f3 = static_cast<float>(w[i] >> 24) - z;
    o[2 * i] = pack_bf16x2(f0, f1);
    o[2 * i + 1] = pack_bf16x2(f2, f3);
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// acc[mat][mt] += A(tokens) x W(rows)^T over elements [k0, k1) (multiples of 64).
// The weight loads of U steps are all issued before the first is used (they stream
// from HBM).
template <Act ACT, WFmt WF, int NMAT, int MT>
__device__ __forceinline__ void stream_rows(const Task<ACT, WF, NMAT, MT>& t, int k0, int k1,
                                            f32x4 (&acc)[NMAT][MT]) {
  const int q = lane_id() >> 4;
  if constexpr (ACT == Act::BF16 && WF == WFmt::BF16) {
    // K-group q of MFMA 0 takes elements [8q, 8q+8) of the 64-element step and of
    // MFMA 1 [32+8q, 40+8q): each load instruction reads 64 contiguous bytes per row.
    // U steps of weights are in flight per wavefront (4 with two matrices, 8 with one:
    // measured best), and the token rows of those U steps are loaded as one batch.
    constexpr int U = NMAT == 2 ? 4 : 8;
    int k = k0;
    for (; k + 64 * U <= k1; k += 64 * U) {
      uint4 w0[U][NMAT], w1[U][NMAT];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const uint16_t* p = t.wrow[m] + k + 64 * u + 8 * q;
          w0[u][m] = ld_stream(p);
          w1[u][m] = ld_stream(p + 32);
        }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt < t.mt_live) {
          uint4 a0[U], a1[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const uint16_t* p = t.arow[mt] + k + 64 * u + 8 * q;
            a0[u] = ld16(p);
            a1[u] = ld16(p + 32);
          }
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
              acc[m][mt] = mfma16_bf16(a0[u], w0[u][m], acc[m][mt]);
              acc[m][mt] = mfma16_bf16(a1[u], w1[u][m], acc[m][mt]);
            }
        }
      }
    }
    for (; k < k1; k += 64) {
      uint4 w0[NMAT], w1[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const uint16_t* p = t.wrow[m] + k + 8 * q;
        w0[m] = ld_stream(p);
        w1[m] = ld_stream(p + 32);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt < t.mt_live) {
          const uint16_t* p = t.arow[mt] + k + 8 * q;
          const uint4 a0 = ld16(p), a1 = ld16(p + 32);
#pragma unroll
          for (int m = 0; m < NMAT; ++m) {
            acc[m][mt] = mfma16_bf16(a0, w0[m], acc[m][mt]);
            acc[m][mt] = mfma16_bf16(a1, w1[m], acc[m][mt]);
          }
        }
      }
    }
  } else if constexpr (ACT == Act::BF16 && WF == WFmt::U8) {
    // one 64-element step = one quantisation group: exact (q - z) products per
    // group, then one fp32 scale per row and group.  Lane q holds codes
    // [16q, 16q+16) of the step (16 contiguous bytes; 64 per row per instruction).
    constexpr int U = 8;
    int k = k0;
    for (; k + 64 * U <= k1; k += 64 * U) {
      uint4 wq[U][NMAT];
      uint16_t sh[U][NMAT], zh[U][NMAT];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          wq[u][m] = ld_stream(t.wrow[m] + k + 64 * u + 16 * q);
          sh[u][m] = t.srow[m][(k >> 6) + u];
          zh[u][m] = t.zrow[m][(k >> 6) + u];
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          uint4 wl, wh;
          dequant16(wq[u][m], f16_to_f32(zh[u][m]), wl, wh);
          const float sc = f16_to_f32(sh[u][m]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if (mt < t.mt_live) {
              const uint16_t* p = t.arow[mt] + k + 64 * u + 16 * q;
              f32x4 g = {0.f, 0.f, 0.f, 0.f};
              g = mfma16_bf16(ld16(p), wl, g);
              g = mfma16_bf16(ld16(p + 8), wh, g);
              acc[m][mt] += sc * g;
            }
          }
        }
      }
    }
    for (; k < k1; k += 64) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const uint4 wq = ld_stream(t.wrow[m] + k + 16 * q);
        const float sc = f16_to_f32(t.srow[m][k >> 6]);
        const float zp = f16_to_f32(t.zrow[m][k >> 6]);
        uint4 wl, wh;
        dequant16(wq, zp, wl, wh);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (mt < t.mt_live) {
            const uint16_t* p = t.arow[mt] + k + 16 * q;
            f32x4 g = {0.f, 0.f, 0.f, 0.f};
            g = mfma16_bf16(ld16(p), wl, g);
            g = mfma16_bf16(ld16(p + 8), wh, g);
            acc[m][mt] += sc * g;
          }
        }
      }
    }
  } else {
    // fp32 activations and weights: 16 MFMA 16x16x4 per 64-element step
    for (int k = k0; k < k1; k += 64) {
      float4 w[NMAT][4];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          w[m][c] = *reinterpret_cast<const float4*>(t.wrow[m] + k + 16 * q + 4 * c);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt < t.mt_live) {
          float4 av[4];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            av[c] = *reinterpret_cast<const float4*>(t.arow[mt] + k + 16 * q + 4 * c);
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              acc[m][mt] = mfma16_f32(av[c].x, w[m][c].x, acc[m][mt]);
              acc[m][mt] = mfma16_f32(av[c].y, w[m][c].y, acc[m][mt]);
              acc[m][mt] = mfma16_f32(av[c].z, w[m][c].z, acc[m][mt]);
              acc[m][mt] = mfma16_f32(av[c].w, w[m][c].w, acc[m][mt]);
            }
        }
      }
    }
  }
}

// Split the 64-element units of [0, K) into `parts` near-equal ranges.
__device__ __forceinline__ void unit_range(int K, int part, int parts, int& k0, int& k1) {
  const int U = K >> 6;
  k0 = (part * U / parts) << 6;
  k1 = ((part + 1) * U / parts) << 6;
}

template <int NMAT, int MT>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[NMAT][MT]) {
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[m][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// K-split reduction across the 4 wavefronts of a block: afterwards wavefront w holds
// the full sums of M-tile w in acc[.][0].  Must be reached by the whole block.
template <int NMAT, int MT>
__device__ __forceinline__ void block_reduce(float* red, f32x4 (&acc)[NMAT][MT]) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f32x4*>(red + (((w * NMAT + m) * MT + mt) * 64 + lane) * 4) = acc[m][mt];
  __syncthreads();
  if (w < MT) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < 4; ++p) s += *reinterpret_cast<const f32x4*>(red + (((p * NMAT + m) * MT + w) * 64 + lane) * 4);
      acc[m][0] = s;
    }
  }
  __syncthreads();
}

template <Act ACT>
__device__ __forceinline__ void store_act(typename ActType<ACT>::T* p, float v) {
  if constexpr (ACT == Act::BF16)
    *p = f32_to_bf16(v);
  else
    *p = v;
}

// ------------------------------------------------------------------ router
template <Act ACT, int MT, int NWK>
__global__ __launch_bounds__(256) void k_skinny_router(SkinnyRouterArgs a) {
  using AT = typename ActType<ACT>::T;
  constexpr WFmt WF = ACT == Act::BF16 ? WFmt::BF16 : WFmt::F32;
  using WT = typename WType<WF>::T;
  constexpr int IPB = 4 / NWK;
  __shared__ float red[NWK > 1 ? 4 * MT * 256 : 1];
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int n = lane & 15;
  const int RC = (a.E + 15) / 16;
  const int nitems = RC * a.P;
  const AT* x = static_cast<const AT*>(a.x);
  const WT* W = static_cast<const WT*>(a.W);
  for (int base = blockIdx.x * IPB; base < nitems; base += gridDim.x * IPB) {
    const int item = base + w / NWK;
    const bool live = item < nitems;
    const int it = live ? item : 0;
    const int rc = it % RC, part = it / RC;
    const int row = min(rc * 16 + n, a.E - 1);
    int k0, k1;
    unit_range(a.H, part, a.P, k0, k1);
    if (NWK > 1) {
      const int kk0 = k0, span = k1 - k0;
      const int U = span >> 6, kp = w % NWK;
      k0 = kk0 + ((kp * U / NWK) << 6);
      k1 = kk0 + (((kp + 1) * U / NWK) << 6);
    }
    for (int t0 = 0; t0 < a.T; t0 += 16 * MT) {
      const int ntok = min(16 * MT, a.T - t0);
      Task<ACT, WF, 1, MT> tk;
      tk.wrow[0] = W + static_cast<int64_t>(row) * a.H;
      tk.mt_live = (ntok + 15) / 16;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = min(mt * 16 + n, ntok - 1);
        tk.arow[mt] = x + static_cast<int64_t>(t0 + m) * a.H;
      }
      f32x4 acc[1][MT];
      zero_acc(acc);
      if (live) stream_rows(tk, k0, k1, acc);
      int mt_lo = 0, mt_hi = MT;
      if constexpr (NWK > 1) {
        block_reduce<1, MT>(red, acc);
        mt_lo = w;
        mt_hi = w + 1;
      }
      if (live && (NWK == 1 || w < MT)) {
        const int col = rc * 16 + n;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (mt < mt_lo || mt >= mt_hi) continue;
          const int ai = NWK > 1 ? 0 : mt;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = mt * 16 + 4 * (lane >> 4) + v;
            if (m < ntok && col < a.E)
              a.out[(static_cast<int64_t>(part) * a.T + t0 + m) * a.E + col] = acc[0][ai][v];
          }
        }
      }
    }
  }
}

// ------------------------------------------------- routed + shared gate/up, SwiGLU
template <Act ACT, WFmt WF, int MT, int NWK>
__global__ __launch_bounds__(256) void k_skinny_up(SkinnyUpArgs a) {
  using AT = typename ActType<ACT>::T;
  using WT = typename WType<WF>::T;
  using ST = typename WType<ACT == Act::BF16 ? WFmt::BF16 : WFmt::F32>::T;  // shared weights
  constexpr int IPB = 4 / NWK;
  __shared__ float red[NWK > 1 ? 4 * 2 * MT * 256 : 1];
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int n = lane & 15;
  const int D = a.part == 2 ? 0 : a.meta[0];  // shared-only launches read no routing
  const int CH = a.I / 16, CHs = a.Is / 16;
  constexpr int TCH = 16 * MT;  // tokens per chunk
  const int TC = (a.T + TCH - 1) / TCH;
  const int n_routed = D * CH;
  const int nitems = n_routed + (a.part == 1 ? 0 : CHs * TC);
  const AT* x = static_cast<const AT*>(a.x);
  for (int base = blockIdx.x * IPB; base < nitems; base += gridDim.x * IPB) {
    const int item = base + w / NWK;
    const bool live = item < nitems;
    const int it = live ? item : 0;
    const bool shared = it >= n_routed;
    int k0 = 0, k1 = a.H;
    if (NWK > 1) unit_range(a.H, w % NWK, NWK, k0, k1);
    // item geometry
    int e = 0, off = 0, ntot, row0, tc_begin, tc_end;
    if (!shared) {
      e = a.active[it / CH];
      row0 = (it % CH) * 16;
      off = a.offsets[e];
      ntot = a.counts[e];
      tc_begin = 0;
      tc_end = (ntot + TCH - 1) / TCH;
    } else {
      const int si = it - n_routed;
      row0 = (si % CHs) * 16;
      tc_begin = si / CHs;
      tc_end = tc_begin + 1;
      ntot = a.T;
    }
    for (int tc = tc_begin; tc < tc_end; ++tc) {
      const int ntok = min(TCH, ntot - tc * TCH);
      Task<ACT, WF, 2, MT> tk;
      tk.mt_live = (ntok + 15) / 16;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = tc * TCH + min(mt * 16 + n, ntok - 1);
        const int tok = shared ? m : a.perm[off + m] / a.k;
        tk.arow[mt] = x + static_cast<int64_t>(tok) * a.H;
      }
      if (!shared) {
        const int64_t ro = static_cast<int64_t>(e) * a.I + row0 + n;
        tk.wrow[0] = static_cast<const WT*>(a.gate) + ro * a.H;
        tk.wrow[1] = static_cast<const WT*>(a.up) + ro * a.H;
        if constexpr (WF == WFmt::U8) {
          tk.srow[0] = a.gate_s + ro * (a.H / 64);
          tk.zrow[0] = a.gate_z + ro * (a.H / 64);
          tk.srow[1] = a.up_s + ro * (a.H / 64);
          tk.zrow[1] = a.up_z + ro * (a.H / 64);
        }
      }
      f32x4 acc[2][MT];
      zero_acc(acc);
      if (live) {
        if (!shared) {
          stream_rows(tk, k0, k1, acc);
        } else {
          // the shared expert keeps the activation dtype
          constexpr WFmt SF = ACT == Act::BF16 ? WFmt::BF16 : WFmt::F32;
          Task<ACT, SF, 2, MT> ts;
          ts.mt_live = tk.mt_live;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) ts.arow[mt] = tk.arow[mt];
          const int64_t ro = row0 + n;
          ts.wrow[0] = static_cast<const ST*>(a.sgate) + ro * a.H;
          ts.wrow[1] = static_cast<const ST*>(a.sup) + ro * a.H;
          stream_rows(ts, k0, k1, acc);
        }
      }
      int mt_lo = 0, mt_hi = MT;
      if constexpr (NWK > 1) {
        block_reduce<2, MT>(red, acc);
        mt_lo = w;
        mt_hi = w + 1;
      }
      if (live && (NWK == 1 || w < MT)) {
        AT* out = static_cast<AT*>(shared ? a.hs : a.hm);
        const int ld = shared ? a.Is : a.I;
        const int64_t rbase = shared ? 0 : off;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (mt < mt_lo || mt >= mt_hi) continue;
          const int ai = NWK > 1 ? 0 : mt;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = mt * 16 + 4 * (lane >> 4) + v;
            if (m < ntok) {
              const float h = silu(acc[0][ai][v]) * acc[1][ai][v];
              store_act<ACT>(out + (rbase + tc * TCH + m) * ld + row0 + n, h);
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------ routed + shared down
template <Act ACT, WFmt WF, int MT, int NWK>
__global__ __launch_bounds__(256) void k_skinny_down(SkinnyDownArgs a) {
  using AT = typename ActType<ACT>::T;
  using WT = typename WType<WF>::T;
  using ST = typename WType<ACT == Act::BF16 ? WFmt::BF16 : WFmt::F32>::T;
  constexpr int IPB = 4 / NWK;
  __shared__ float red[NWK > 1 ? 4 * MT * 256 : 1];
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int n = lane & 15;
  const int D = a.part == 2 ? 0 : a.meta[0];  // shared-only launches read no routing
  const int CH = a.H / 16;
  constexpr int TCH = 16 * MT;  // tokens per chunk
  const int TC = (a.T + TCH - 1) / TCH;
  const int n_routed = D * CH;
  const int nitems = n_routed + (a.Is > 0 && a.part != 1 ? CH * TC : 0);
  const AT* hm = static_cast<const AT*>(a.hm);
  const AT* hs = static_cast<const AT*>(a.hs);
  for (int base = blockIdx.x * IPB; base < nitems; base += gridDim.x * IPB) {
    const int item = base + w / NWK;
    const bool live = item < nitems;
    const int it = live ? item : 0;
    const bool shared = it >= n_routed;
    const int K = shared ? a.Is : a.I;
    int k0 = 0, k1 = K;
    if (NWK > 1) unit_range(K, w % NWK, NWK, k0, k1);
    int e = 0, off = 0, ntot, row0, tc_begin, tc_end;
    if (!shared) {
      e = a.active[it / CH];
      row0 = (it % CH) * 16;
      off = a.offsets[e];
      ntot = a.counts[e];
      tc_begin = 0;
      tc_end = (ntot + TCH - 1) / TCH;
    } else {
      const int si = it - n_routed;
      row0 = (si % CH) * 16;
      tc_begin = si / CH;
      tc_end = tc_begin + 1;
      ntot = a.T;
    }
    for (int tc = tc_begin; tc < tc_end; ++tc) {
      const int ntok = min(TCH, ntot - tc * TCH);
      f32x4 acc[1][MT];
      zero_acc(acc);
      const int mt_live = (ntok + 15) / 16;
      if (live) {
        if (!shared) {
          Task<ACT, WF, 1, MT> tk;
          tk.mt_live = mt_live;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            tk.arow[mt] = hm + static_cast<int64_t>(off + tc * TCH + min(mt * 16 + n, ntok - 1)) * a.I;
          const int64_t ro = static_cast<int64_t>(e) * a.H + row0 + n;
          tk.wrow[0] = static_cast<const WT*>(a.down) + ro * a.I;
          if constexpr (WF == WFmt::U8) {
            tk.srow[0] = a.down_s + ro * (a.I / 64);
            tk.zrow[0] = a.down_z + ro * (a.I / 64);
          }
          stream_rows(tk, k0, k1, acc);
        } else {
          constexpr WFmt SF = ACT == Act::BF16 ? WFmt::BF16 : WFmt::F32;
          Task<ACT, SF, 1, MT> ts;
          ts.mt_live = mt_live;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            ts.arow[mt] = hs + static_cast<int64_t>(tc * TCH + min(mt * 16 + n, ntok - 1)) * a.Is;
          ts.wrow[0] = static_cast<const ST*>(a.sdown) + static_cast<int64_t>(row0 + n) * a.Is;
          stream_rows(ts, k0, k1, acc);
        }
      }
      int mt_lo = 0, mt_hi = MT;
      if constexpr (NWK > 1) {
        block_reduce<1, MT>(red, acc);
        mt_lo = w;
        mt_hi = w + 1;
      }
      if (live && (NWK == 1 || w < MT)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (mt < mt_lo || mt >= mt_hi) continue;
          const int ai = NWK > 1 ? 0 : mt;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = mt * 16 + 4 * (lane >> 4) + v;
            if (m < ntok) {
              if (!shared) {
                const int slot = a.perm[off + tc * TCH + m];
                const float val = a.topk_w[slot] * acc[0][ai][v];
                const int64_t o = static_cast<int64_t>(slot) * a.H + row0 + n;
                if (a.r_bf16)
                  static_cast<uint16_t*>(a.r)[o] = f32_to_bf16(val);
                else
                  static_cast<float*>(a.r)[o] = val;
              } else {
                a.rs[static_cast<int64_t>(tc * TCH + m) * a.H + row0 + n] = acc[0][ai][v];
              }
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------- bf16 streaming through per-wave LDS rings
// The same work items as above (16 weight rows of one matrix set x one 16-token
// chunk), for bf16 activations and weights, with the operands brought in by direct
// global -> LDS copies of whole 128-byte lines: one copy instruction moves 8 rows x 128
// bytes (one 64-element K-step of 8 rows).  Each wavefront owns a ring of U K-steps in
// LDS holding its NMAT x 16 weight rows and its 16 token rows, keeps U - 1 steps in
// flight and reads MFMA fragments from the ring; wavefronts never wait for each other
// inside the K loop.  Token rows are read once per K-step and item (they are shared by
// the NMAT matrices), and every line of a weight row is requested once.
//
// Ring layout per step: rows [0, 16 NMAT) weights (matrix m: rows 16m ..), rows
// [16 NMAT, 16 NMAT + 16) tokens; 128-byte rows with 16-byte chunks XOR-swizzled by
// row % 8.  Lane l of a copy instruction covering rows [8h, 8h + 8) takes row 8h + l/8
// and logical chunk (l % 8) ^ (l / 8).
template <int NMAT>
struct RingGeom {
  static constexpr int ROWS = 16 * NMAT + 16;
  static constexpr int SLOT = ROWS * 64;      // bf16 elements per K-step
  static constexpr int CPS = 2 * NMAT + 2;    // copy instructions per K-step
};

// acc[m] += tokens x W_m^T over [k0, k1) (multiples of 64) with a U-step ring at `ring`.
// wbase[m]: wave-uniform byte address of weight row 0 of matrix m (rows H_row bytes
// apart, the stride folded into woff); woff[h]: this lane's byte offset of its row in
// copy h (row 8h + l/8) plus its chunk; abase / aoff[h]: the same for the token rows.
template <int NMAT, int U>
__device__ __forceinline__ void ring_stream(const char* const (&wbase)[NMAT], const uint32_t (&woff)[2],
                                            const char* abase, const uint32_t (&aoff)[2], int k0, int k1,
                                            uint16_t* ring, f32x4 (&acc)[NMAT]) {
  using G = RingGeom<NMAT>;
  const int lane = lane_id();
  const int n = (k1 - k0) >> 6;
  auto issue = [&](int slot, int step) {
    uint16_t* sl = ring + slot * G::SLOT;
    const int kb = (k0 + 64 * step) * 2;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int h = 0; h < 2; ++h) copy_to_lds(uniform_ptr(wbase[m] + kb), woff[h], sl + (16 * m + 8 * h) * 64);
#pragma unroll
    for (int h = 0; h < 2; ++h) copy_to_lds(uniform_ptr(abase + kb), aoff[h], sl + (16 * NMAT + 8 * h) * 64);
  };
  const int r = lane & 15, q = lane >> 4;
  auto compute = [&](int slot) {
    const uint16_t* sl = ring + slot * G::SLOT;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int cc = ((ks * 4 + q) ^ (r & 7)) << 3;
      const uint4 a = *reinterpret_cast<const uint4*>(sl + (16 * NMAT + r) * 64 + cc);
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const uint4 w = *reinterpret_cast<const uint4*>(sl + (16 * m + r) * 64 + cc);
        acc[m] = mfma16_bf16(a, w, acc[m]);
      }
    }
  };
#pragma unroll
  for (int p = 0; p < U - 1; ++p)
    if (p < n) issue(p, p);
  int cur = 0, nxt = U - 1;
  for (int t = 0; t < n; ++t) {
    // this wave's copies of step t have landed (later steps may still be in flight) and
    // its reads of the slot refilled next are done
    copy_wait_ahead<G::CPS, U - 2>(n - 1 - t);
    if (t + U - 1 < n) issue(nxt, t + U - 1);
    compute(cur);
    cur = cur + 1 == U ? 0 : cur + 1;
    nxt = nxt + 1 == U ? 0 : nxt + 1;
  }
  copy_wait<0>();
}

// per-lane ring offsets: copy h covers rows 8h + l/8, logical chunk (l % 8) ^ (l / 8)
__device__ __forceinline__ void ring_lane(int& row_in_copy, int& chunk) {
  const int lane = lane_id();
  row_in_copy = lane >> 3;
  chunk = (lane & 7) ^ (lane >> 3);
}

template <int U, int NWK>
__global__ __launch_bounds__(256) void k_stream_up(SkinnyUpArgs a) {
  using G = RingGeom<2>;
  constexpr int IPB = 4 / NWK;
  __shared__ __attribute__((aligned(16))) uint16_t rings[4 * U * G::SLOT];
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  uint16_t* ring = rings + w * U * G::SLOT;
  const int NQ = a.part == 2 ? 0 : a.meta[1];  // chunks; shared-only launches read no routing
  const int CH = a.I / 16, CHs = a.Is / 16;
  const int TC = (a.T + 15) / 16;
  const int n_routed = NQ * CH;
  const int nitems = n_routed + (a.part == 1 ? 0 : CHs * TC);
  int rr, ch;
  ring_lane(rr, ch);
  const char* xb = uniform_ptr(a.x);
  for (int base = blockIdx.x * IPB; base < nitems; base += gridDim.x * IPB) {
    const int item = base + w / NWK;
    const bool live = item < nitems;
    const int it = live ? item : 0;
    const bool shared = it >= n_routed;
    int k0 = 0, k1 = a.H;
    if (NWK > 1) unit_range(a.H, w % NWK, NWK, k0, k1);
    int e = 0, off = 0, ntot, row0, tc_begin, tc_end;
    if (!shared) {
      // one chunk of at most 16 positions.  Expert e's chunks are chunk-list entries
      // q0 .. q0 + nc - 1, and its items CH * q0 .. CH * (q0 + nc) - 1, ordered by row
      // block and then chunk: the items of one expert are contiguous (neighbouring row
      // blocks stream together) and a popular expert's chunks read the same rows side
      // by side.  Any entry of the expert, such as it / CH, names it and its q0.
      const int qa = it / CH;
      e = a.tiles[2 * qa];
      const int first = a.offsets[e];
      const int q0 = qa - (a.tiles[2 * qa + 1] - first) / kDecodeChunk;
      const int nc = (a.counts[e] + kDecodeChunk - 1) / kDecodeChunk;
      const int local = it - q0 * CH;
      const int c = local % nc;
      row0 = (local / nc) * 16;
      off = first + c * kDecodeChunk;
      ntot = a.counts[e] - c * kDecodeChunk;
      tc_begin = 0;
      tc_end = 1;
    } else {
      // shared item: the chunks of one row block are neighbours (they share its rows)
      const int si = it - n_routed;
      row0 = (si / TC) * 16;
      tc_begin = si % TC;
      tc_end = tc_begin + 1;
      ntot = a.T;
    }
    const char* wb[2];
    if (!shared) {
      const int64_t ro = static_cast<int64_t>(e) * a.I + row0;
      wb[0] = uniform_ptr(static_cast<const uint16_t*>(a.gate) + ro * a.H);
      wb[1] = uniform_ptr(static_cast<const uint16_t*>(a.up) + ro * a.H);
    } else {
      wb[0] = uniform_ptr(static_cast<const uint16_t*>(a.sgate) + static_cast<int64_t>(row0) * a.H);
      wb[1] = uniform_ptr(static_cast<const uint16_t*>(a.sup) + static_cast<int64_t>(row0) * a.H);
    }
    const uint32_t woff[2] = {static_cast<uint32_t>((rr * a.H + ch * 8) * 2),
                              static_cast<uint32_t>(((8 + rr) * a.H + ch * 8) * 2)};
    for (int tc = tc_begin; tc < tc_end; ++tc) {
      const int ntok = min(16, ntot - tc * 16);
      uint32_t aoff[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = tc * 16 + min(8 * h + rr, ntok - 1);  // padded rows repeat the last token
        const int tok = shared ? m : a.perm[off + m] / a.k;
        aoff[h] = static_cast<uint32_t>(tok) * a.H * 2 + ch * 16;
      }
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      if (live) ring_stream<2, U>(wb, woff, xb, aoff, k0, k1, ring, acc);
      if constexpr (NWK > 1) {
        // K-split: partial sums through the (now idle) rings; wavefront 0 adds them
        float* red = reinterpret_cast<float*>(rings);
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 2; ++m) *reinterpret_cast<f32x4*>(red + ((w * 2 + m) * 64 + lane) * 4) = acc[m];
        __syncthreads();
        if (w == 0) {
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 4; ++p) sum += *reinterpret_cast<const f32x4*>(red + ((p * 2 + m) * 64 + lane) * 4);
            acc[m] = sum;
          }
        }
        __syncthreads();
      }
      if (live && (NWK == 1 || w == 0)) {
        uint16_t* out = static_cast<uint16_t*>(shared ? a.hs : a.hm);
        const int ld = shared ? a.Is : a.I;
        const int64_t rbase = shared ? 0 : off;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 4 * (lane >> 4) + v;
          if (m < ntok) {
            const float h = silu(acc[0][v]) * acc[1][v];
            out[(rbase + tc * 16 + m) * ld + row0 + n] = f32_to_bf16(h);
          }
        }
      }
    }
  }
}

template <int U, int NWK>
__global__ __launch_bounds__(256) void k_stream_down(SkinnyDownArgs a) {
  using G = RingGeom<1>;
  constexpr int IPB = 4 / NWK;
  __shared__ __attribute__((aligned(16))) uint16_t rings[4 * U * G::SLOT];
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  uint16_t* ring = rings + w * U * G::SLOT;
  const int NQ = a.part == 2 ? 0 : a.meta[1];  // chunks; shared-only launches read no routing
  const int CH = a.H / 16;
  const int TC = (a.T + 15) / 16;
  const int n_routed = NQ * CH;
  const int nitems = n_routed + (a.Is > 0 && a.part != 1 ? CH * TC : 0);
  int rr, ch;
  ring_lane(rr, ch);
  for (int base = blockIdx.x * IPB; base < nitems; base += gridDim.x * IPB) {
    const int item = base + w / NWK;
    const bool live = item < nitems;
    const int it = live ? item : 0;
    const bool shared = it >= n_routed;
    const int K = shared ? a.Is : a.I;
    int k0 = 0, k1 = K;
    if (NWK > 1) unit_range(K, w % NWK, NWK, k0, k1);
    int e = 0, off = 0, ntot, row0, tc_begin, tc_end;
    if (!shared) {
      // one chunk of at most 16 positions.  Expert e's chunks are chunk-list entries
      // q0 .. q0 + nc - 1, and its items CH * q0 .. CH * (q0 + nc) - 1, ordered by row
      // block and then chunk: the items of one expert are contiguous (neighbouring row
      // blocks stream together) and a popular expert's chunks read the same rows side
      // by side.  Any entry of the expert, such as it / CH, names it and its q0.
      const int qa = it / CH;
      e = a.tiles[2 * qa];
      const int first = a.offsets[e];
      const int q0 = qa - (a.tiles[2 * qa + 1] - first) / kDecodeChunk;
      const int nc = (a.counts[e] + kDecodeChunk - 1) / kDecodeChunk;
      const int local = it - q0 * CH;
      const int c = local % nc;
      row0 = (local / nc) * 16;
      off = first + c * kDecodeChunk;
      ntot = a.counts[e] - c * kDecodeChunk;
      tc_begin = 0;
      tc_end = 1;
    } else {
      // shared item: the chunks of one row block are neighbours (they share its rows)
      const int si = it - n_routed;
      row0 = (si / TC) * 16;
      tc_begin = si % TC;
      tc_end = tc_begin + 1;
      ntot = a.T;
    }
    const char* wb[1];
    if (!shared)
      wb[0] = uniform_ptr(static_cast<const uint16_t*>(a.down) + (static_cast<int64_t>(e) * a.H + row0) * a.I);
    else
      wb[0] = uniform_ptr(static_cast<const uint16_t*>(a.sdown) + static_cast<int64_t>(row0) * a.Is);
    const uint32_t woff[2] = {static_cast<uint32_t>((rr * K + ch * 8) * 2),
                              static_cast<uint32_t>(((8 + rr) * K + ch * 8) * 2)};
    const char* ab = uniform_ptr(shared ? a.hs : a.hm);
    for (int tc = tc_begin; tc < tc_end; ++tc) {
      const int ntok = min(16, ntot - tc * 16);
      uint32_t aoff[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = tc * 16 + min(8 * h + rr, ntok - 1);
        const int row = shared ? m : off + m;
        aoff[h] = static_cast<uint32_t>(row) * K * 2 + ch * 16;
      }
      f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
      if (live) ring_stream<1, U>(wb, woff, ab, aoff, k0, k1, ring, acc);
      if constexpr (NWK > 1) {
        float* red = reinterpret_cast<float*>(rings);
        __syncthreads();
        *reinterpret_cast<f32x4*>(red + (w * 64 + lane) * 4) = acc[0];
        __syncthreads();
        if (w == 0) {
          f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < 4; ++p) sum += *reinterpret_cast<const f32x4*>(red + (p * 64 + lane) * 4);
          acc[0] = sum;
        }
        __syncthreads();
      }
      if (live && (NWK == 1 || w == 0)) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 4 * (lane >> 4) + v;
          if (m < ntok) {
            if (!shared) {
              const int slot = a.perm[off + tc * 16 + m];
              const float val = a.topk_w[slot] * acc[0][v];
              const int64_t o = static_cast<int64_t>(slot) * a.H + row0 + n;
              if (a.r_bf16)
                static_cast<uint16_t*>(a.r)[o] = f32_to_bf16(val);
              else
                static_cast<float*>(a.r)[o] = val;
            } else {
              a.rs[static_cast<int64_t>(tc * 16 + m) * a.H + row0 + n] = acc[0][v];
            }
          }
        }
      }
    }
  }
}

// ----------------------------------------------------- u8 weights through LDS rings
// One ring step covers 128 elements of K (two quantisation groups), so a weight row's
// codes for the step are one whole 128-byte line.  Slot layout (bytes): NMAT x 16 code
// rows of 128 B, two token images of 16 rows x 128 B (elements 0..63 and 64..127 of the
// step), then 256 B of group parameters: lane l of one 4-byte-per-lane copy brings the
// two fp16 values (groups 2t, 2t + 1) of matrix l / 32, kind (l / 16) % 2 (scale,
// zero), row l % 16.  Products per group are exact: codes minus the zero point are
// integers in [-255, 255], exact in bf16; the group scale multiplies the fp32 result.
template <int NMAT>
struct RingGeomU8 {
  static constexpr int W_BYTES = NMAT * 16 * 128;
  static constexpr int A_BYTES = 2 * 16 * 128;
  static constexpr int SLOT_BYTES = W_BYTES + A_BYTES + 256;
  static constexpr int CPS = 2 * NMAT + 4 + 1;  // copy instructions per step
};

// codes: 8 u8 in (lo, hi) minus zero point -> 8 bf16
__device__ __forceinline__ uint4 codes_minus_zero(uint2 c, float z) {
  const uint32_t w[2] = {c.x, c.y};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    o[2 * i] = pack_bf16x2(static_cast<float>(w[i] & 0xffu) - z, static_cast<float>((w[i] >> 8) & 0xffu) - z);
    o[2 * i + 1] = pack_bf16x2(static_cast<float>((w[i] >> 16) & 0xffu) - z, static_cast<float>(w[i] >> 24) - z);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// acc[m] += tokens x dequant(W_m)^T over [k0, k1) (multiples of 128).
// wbase[m]: wave-uniform byte address of code row 0 of matrix m; woff[h]: lane offset of
// its code row in copy h (row 8h + l/8, rows K bytes apart) plus its chunk.  sz_src: this
// lane's group-parameter address for group 0 of the range (4 bytes, 2 groups).
template <int NMAT, int U>
__device__ __forceinline__ void ring_stream_u8(const char* const (&wbase)[NMAT], const uint32_t (&woff)[2],
                                               const char* abase, const uint32_t (&aoff)[2], const uint16_t* sz_src,
                                               int k0, int k1, char* ring, f32x4 (&acc)[NMAT]) {
  using G = RingGeomU8<NMAT>;
  const int lane = lane_id();
  const int n = (k1 - k0) >> 7;
  auto issue = [&](int slot, int step) {
    char* sl = ring + slot * G::SLOT_BYTES;
    const int kc = k0 + 128 * step;  // element index = code byte offset
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        copy_to_lds(uniform_ptr(wbase[m] + kc), woff[h], reinterpret_cast<uint16_t*>(sl + (16 * m + 8 * h) * 128));
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        copy_to_lds(uniform_ptr(abase + (kc + 64 * half) * 2), aoff[h],
                    reinterpret_cast<uint16_t*>(sl + G::W_BYTES + half * 2048 + 8 * h * 128));
    copy4_to_lds(sz_src + (kc >> 6), sl + G::W_BYTES + G::A_BYTES);
  };
  const int r = lane & 15, q = lane >> 4;
  auto compute = [&](int slot) {
    const char* sl = ring + slot * G::SLOT_BYTES;
    const uint32_t* szp = reinterpret_cast<const uint32_t*>(sl + G::W_BYTES + G::A_BYTES);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      f32x4 part[NMAT];
      float zf[NMAT], sf[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        part[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint32_t sv = szp[m * 32 + r], zv = szp[m * 32 + 16 + r];
        sf[m] = f16_to_f32(static_cast<uint16_t>(g ? sv >> 16 : sv & 0xffffu));
        zf[m] = f16_to_f32(static_cast<uint16_t>(g ? zv >> 16 : zv & 0xffffu));
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c = ks * 4 + q;  // logical 16-byte chunk of the 64-element token image
        const uint4 av = *reinterpret_cast<const uint4*>(sl + G::W_BYTES + g * 2048 + r * 128 + ((c ^ (r & 7)) << 4));
        const int cw = 4 * g + (c >> 1);  // 16-byte chunk of the code row holding codes 8c .. of group g
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const uint2 cv =
              *reinterpret_cast<const uint2*>(sl + (16 * m + r) * 128 + ((cw ^ (r & 7)) << 4) + (c & 1) * 8);
          part[m] = mfma16_bf16(av, codes_minus_zero(cv, zf[m]), part[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m) acc[m] += sf[m] * part[m];
    }
  };
#pragma unroll
  for (int p = 0; p < U - 1; ++p)
    if (p < n) issue(p, p);
  int cur = 0, nxt = U - 1;
  for (int t = 0; t < n; ++t) {
    copy_wait_ahead<G::CPS, U - 2>(n - 1 - t);
    if (t + U - 1 < n) issue(nxt, t + U - 1);
    compute(cur);
    cur = cur + 1 == U ? 0 : cur + 1;
    nxt = nxt + 1 == U ? 0 : nxt + 1;
  }
  copy_wait<0>();
}

// ----------------------------------------------------- u4 weights through LDS rings
// One ring step again covers 128 elements of K (two quantisation groups); a weight row's
// codes for the step are 64 bytes, so one copy instruction moves all 16 rows of a
// matrix.  Slot layout (bytes): NMAT x 16 code rows of 64 B (16-byte chunks XOR-swizzled
// by (row / 4) % 4, which keeps the per-lane 4-byte fragment reads free of bank
// conflicts), TR token rows of 256 B (the step's 128 elements, chunks swizzled by the
// row), then the 256 B of group parameters laid out as for u8.  Only TR = 4, 8 or 16
// token rows are copied, the fewest that hold the chunk's live tokens; MFMA rows beyond
// TR reread row r % TR and their results are dropped.
//
// Dequantisation without per-element conversions: the bf16 pattern 0x4300 | q is the
// exact value 128 + q, so a code dword turns into four bf16 pairs with one mask-and-or
// each.  Taking elements (j, j + 4) into pair j fixes the order of the lane's 8 K values
// as 0 4 1 5 2 6 3 7; the token fragment is permuted the same way, which leaves the dot
// product unchanged.  Per group, sum_k a_k (q_k - z) = sum_k a_k (128 + q_k)
// - (128 + z) sum_k a_k, with sum_k a_k from one more MFMA against ones.
template <int NMAT, int TR>
struct RingGeomU4 {
  static constexpr int W_BYTES = NMAT * 16 * 64;
  static constexpr int A_BYTES = TR * 256;
  static constexpr int SLOT_BYTES = W_BYTES + A_BYTES + 256;
  static constexpr int CPS = NMAT + TR / 4 + 1;  // copy instructions per step
};
constexpr int kU4MaxSlot = RingGeomU4<2, 16>::SLOT_BYTES;

// code dword (8 nibbles, element j at bits 4j) -> bf16 pairs (128 + q_j, 128 + q_{j+4})
__device__ __forceinline__ uint4 nibbles_biased(uint32_t w) {
  constexpr uint32_t kMask = 0x000f000fu, kBias = 0x43004300u;
  return make_uint4((w & kMask) | kBias, ((w >> 4) & kMask) | kBias, ((w >> 8) & kMask) | kBias,
                    ((w >> 12) & kMask) | kBias);
}

// token fragment (a0 a1 | a2 a3 | a4 a5 | a6 a7) -> (a0 a4 | a1 a5 | a2 a6 | a3 a7)
__device__ __forceinline__ uint4 pair_j_j4(uint4 a) {
  return make_uint4((a.x & 0xffffu) | (a.z << 16), (a.x >> 16) | (a.z & 0xffff0000u), (a.y & 0xffffu) | (a.w << 16),
                    (a.y >> 16) | (a.w & 0xffff0000u));
}

// lane's code-row offset for the u4 ring: row l / 4 of the 16, logical chunk
// (l % 4) ^ (row / 4) % 4; rows `row_bytes` apart
__device__ __forceinline__ uint32_t u4_code_off(int row_bytes) {
  const int lane = lane_id();
  const int row = lane >> 2;
  return static_cast<uint32_t>(row * row_bytes + (((lane & 3) ^ ((row >> 2) & 3)) << 4));
}

// acc[m] += tokens x dequant(W_m)^T over [k0, k1) (multiples of 128), with a ring of as
// many steps (at most 8) as RB bytes hold: fewer token rows leave room for more steps in
// flight.  wbase[m]: wave-uniform byte address of code row 0 of matrix m; woff: this
// lane's offset (u4_code_off).  abase / aoff[i]: token rows of copy i (rows 4i + l/16;
// row byte offset plus 16 x logical chunk (l % 16) ^ row).  sz_src: as for the u8 ring.
template <int NMAT, int RB, int TR>
__device__ __forceinline__ void ring_stream_u4(const char* const (&wbase)[NMAT], uint32_t woff, const char* abase,
                                               const uint32_t (&aoff)[TR / 4], const uint16_t* sz_src, int k0,
                                               int k1, char* ring, f32x4 (&acc)[NMAT]) {
  using G = RingGeomU4<NMAT, TR>;
  constexpr int U = RB / G::SLOT_BYTES < 8 ? RB / G::SLOT_BYTES : 8;
  static_assert(U >= 2, "ring too small");
  const int lane = lane_id();
  const int n = (k1 - k0) >> 7;
  auto issue = [&](int slot, int step) {
    char* sl = ring + slot * G::SLOT_BYTES;
    const int kc = k0 + 128 * step;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
      copy_to_lds(uniform_ptr(wbase[m] + (kc >> 1)), woff, reinterpret_cast<uint16_t*>(sl + m * 1024));
#pragma unroll
    for (int i = 0; i < TR / 4; ++i)
      copy_to_lds(uniform_ptr(abase + kc * 2), aoff[i], reinterpret_cast<uint16_t*>(sl + G::W_BYTES + i * 1024));
    copy4_to_lds(sz_src + (kc >> 6), sl + G::W_BYTES + G::A_BYTES);
  };
  const int r = lane & 15, q = lane >> 4;
  const int tr = r & (TR - 1);
  const uint4 ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
  auto compute = [&](int slot) {
    const char* sl = ring + slot * G::SLOT_BYTES;
    const uint32_t* szp = reinterpret_cast<const uint32_t*>(sl + G::W_BYTES + G::A_BYTES);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      f32x4 part[NMAT];
      f32x4 asum = {0.f, 0.f, 0.f, 0.f};
      float zf[NMAT], sf[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        part[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint32_t sv = szp[m * 32 + r], zv = szp[m * 32 + 16 + r];
        sf[m] = f16_to_f32(static_cast<uint16_t>(g ? sv >> 16 : sv & 0xffffu));
        zf[m] = 128.f + f16_to_f32(static_cast<uint16_t>(g ? zv >> 16 : zv & 0xffffu));
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c = 8 * g + 4 * ks + q;  // 16-byte chunk of the 256-byte token row
        const uint4 av = *reinterpret_cast<const uint4*>(sl + G::W_BYTES + tr * 256 + ((c ^ tr) << 4));
        asum = mfma16_bf16(av, ones, asum);
        const uint4 ap = pair_j_j4(av);
        const int cw = 2 * g + ks;  // 16-byte chunk of the code row holding elements 32 cw ..
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const uint32_t cv =
              *reinterpret_cast<const uint32_t*>(sl + m * 1024 + r * 64 + ((cw ^ ((r >> 2) & 3)) << 4) + 4 * q);
          part[m] = mfma16_bf16(ap, nibbles_biased(cv), part[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m) acc[m] += sf[m] * (part[m] - zf[m] * asum);
    }
  };
#pragma unroll
  for (int p = 0; p < U - 1; ++p)
    if (p < n) issue(p, p);
  int cur = 0, nxt = U - 1;
  for (int t = 0; t < n; ++t) {
    copy_wait_ahead<G::CPS, U - 2>(n - 1 - t);
    if (t + U - 1 < n) issue(nxt, t + U - 1);
    compute(cur);
    cur = cur + 1 == U ? 0 : cur + 1;
    nxt = nxt + 1 == U ? 0 : nxt + 1;
  }
  copy_wait<0>();
}

// token-row copies of the u4 ring for the TR rows of a 16-token chunk: copy i, lane l
// brings row j = 4i + l/16 (the chunk's token min(j, ntok - 1), whose byte offset in the
// activation rows `row_of` gives), logical chunk (l % 16) ^ j
template <int TR, typename F>
__device__ __forceinline__ void u4_token_offsets(int ntok, F row_off, uint32_t (&aoff)[TR / 4]) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < TR / 4; ++i) {
    const int j = 4 * i + (lane >> 4);
    aoff[i] = row_off(min(j, ntok - 1)) + static_cast<uint32_t>(((lane & 15) ^ j) << 4);
  }
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

// calls f(IntC<TR>) with the fewest token rows (4, 8 or 16) covering ntok
template <typename F>
__device__ __forceinline__ void with_token_rows(int ntok, F f) {
  if (ntok <= 4)
    f(IntC<4>{});
  else if (ntok <= 8)
    f(IntC<8>{});
  else
    f(IntC<16>{});
}

// [k0, k1) of part `part` of `parts`, in 128-element units
__device__ __forceinline__ void unit_range128(int K, int part, int parts, int& k0, int& k1) {
  const int U = K >> 7;
  k0 = (part * U / parts) << 7;
  k1 = ((part + 1) * U / parts) << 7;
}

// lane's group-parameter source for the u8 ring: matrix l / 32 (NMAT = 2) or 0, scale
// (kind 0) or zero point (kind 1) of row l % 16
template <int NMAT>
__device__ __forceinline__ const uint16_t* u8_param_row(const uint16_t* const (&s)[NMAT], const uint16_t* const (&z)[NMAT],
                                                         int64_t row0, int K) {
  const int lane = lane_id();
  const int m = NMAT == 2 ? (lane >> 5) : 0;
  const int kind = (lane >> 4) & 1;
  const uint16_t* base = kind ? z[m] : s[m];
  return base + (row0 + (lane & 15)) * (K / 64);
}

// quantised routed experts (BITS = 8: u8 ring, 4: u4 ring); shared items stream bf16
template <int BITS, int U, int NWK>
__global__ __launch_bounds__(256) void k_stream_up_q(SkinnyUpArgs a) {
  constexpr int QSLOT = BITS == 8 ? RingGeomU8<2>::SLOT_BYTES : kU4MaxSlot;
  using GB = RingGeom<2>;
  constexpr int SLOTB = QSLOT > GB::SLOT * 2 ? QSLOT : GB::SLOT * 2;
  constexpr int IPB = 4 / NWK;
  __shared__ __attribute__((aligned(16))) char rings[4 * U * SLOTB];
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  char* ring = rings + w * U * SLOTB;
  const int NQ = a.part == 2 ? 0 : a.meta[1];  // chunks; shared-only launches read no routing
  const int CH = a.I / 16, CHs = a.Is / 16;
  const int TC = (a.T + 15) / 16;
  const int n_routed = NQ * CH;
  const int nitems = n_routed + (a.part == 1 ? 0 : CHs * TC);
  int rr, ch;
  ring_lane(rr, ch);
  const char* xb = uniform_ptr(a.x);
  for (int base = blockIdx.x * IPB; base < nitems; base += gridDim.x * IPB) {
    const int item = base + w / NWK;
    const bool live = item < nitems;
    const int it = live ? item : 0;
    const bool shared = it >= n_routed;
    int k0 = 0, k1 = a.H;
    if (NWK > 1) {
      if (shared)
        unit_range(a.H, w % NWK, NWK, k0, k1);
      else
        unit_range128(a.H, w % NWK, NWK, k0, k1);
    }
    int e = 0, off = 0, ntot, row0, tc_begin, tc_end;
    if (!shared) {
      // one chunk of at most 16 positions.  Expert e's chunks are chunk-list entries
      // q0 .. q0 + nc - 1, and its items CH * q0 .. CH * (q0 + nc) - 1, ordered by row
      // block and then chunk: the items of one expert are contiguous (neighbouring row
      // blocks stream together) and a popular expert's chunks read the same rows side
      // by side.  Any entry of the expert, such as it / CH, names it and its q0.
      const int qa = it / CH;
      e = a.tiles[2 * qa];
      const int first = a.offsets[e];
      const int q0 = qa - (a.tiles[2 * qa + 1] - first) / kDecodeChunk;
      const int nc = (a.counts[e] + kDecodeChunk - 1) / kDecodeChunk;
      const int local = it - q0 * CH;
      const int c = local % nc;
      row0 = (local / nc) * 16;
      off = first + c * kDecodeChunk;
      ntot = a.counts[e] - c * kDecodeChunk;
      tc_begin = 0;
      tc_end = 1;
    } else {
      // shared item: the chunks of one row block are neighbours (they share its rows)
      const int si = it - n_routed;
      row0 = (si / TC) * 16;
      tc_begin = si % TC;
      tc_end = tc_begin + 1;
      ntot = a.T;
    }
    const int64_t ro = static_cast<int64_t>(e) * a.I + row0;
    for (int tc = tc_begin; tc < tc_end; ++tc) {
      const int ntok = min(16, ntot - tc * 16);
      uint32_t aoff[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = tc * 16 + min(8 * h + rr, ntok - 1);
        const int tok = shared ? m : a.perm[off + m] / a.k;
        aoff[h] = static_cast<uint32_t>(tok) * a.H * 2 + ch * 16;
      }
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      if (live) {
        if (!shared) {
          const uint16_t* ss[2] = {a.gate_s, a.up_s};
          const uint16_t* zz[2] = {a.gate_z, a.up_z};
          const uint16_t* szs = u8_param_row<2>(ss, zz, ro, a.H);
          if constexpr (BITS == 8) {
            const char* wb[2] = {uniform_ptr(static_cast<const uint8_t*>(a.gate) + ro * a.H),
                                 uniform_ptr(static_cast<const uint8_t*>(a.up) + ro * a.H)};
            const uint32_t woff[2] = {static_cast<uint32_t>(rr * a.H + ch * 16),
                                      static_cast<uint32_t>((8 + rr) * a.H + ch * 16)};
            ring_stream_u8<2, U>(wb, woff, xb, aoff, szs, k0, k1, ring, acc);
          } else {
            const char* wb[2] = {uniform_ptr(static_cast<const uint8_t*>(a.gate) + ro * (a.H / 2)),
                                 uniform_ptr(static_cast<const uint8_t*>(a.up) + ro * (a.H / 2))};
            const uint32_t woff = u4_code_off(a.H / 2);
            const int* prow = a.perm + off + tc * 16;
            with_token_rows(ntok, [&](auto trc) {
              constexpr int TR = decltype(trc)::value;
              uint32_t ao[TR / 4];
              u4_token_offsets<TR>(ntok, [&](int j) { return static_cast<uint32_t>(prow[j] / a.k) * a.H * 2; }, ao);
              ring_stream_u4<2, U * SLOTB, TR>(wb, woff, xb, ao, szs, k0, k1, ring, acc);
            });
          }
        } else {
          const char* wb[2] = {uniform_ptr(static_cast<const uint16_t*>(a.sgate) + static_cast<int64_t>(row0) * a.H),
                               uniform_ptr(static_cast<const uint16_t*>(a.sup) + static_cast<int64_t>(row0) * a.H)};
          const uint32_t woff[2] = {static_cast<uint32_t>((rr * a.H + ch * 8) * 2),
                                    static_cast<uint32_t>(((8 + rr) * a.H + ch * 8) * 2)};
          ring_stream<2, U>(wb, woff, xb, aoff, k0, k1, reinterpret_cast<uint16_t*>(ring), acc);
        }
      }
      if constexpr (NWK > 1) {
        float* red = reinterpret_cast<float*>(rings);
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 2; ++m) *reinterpret_cast<f32x4*>(red + ((w * 2 + m) * 64 + lane) * 4) = acc[m];
        __syncthreads();
        if (w == 0) {
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 4; ++p) sum += *reinterpret_cast<const f32x4*>(red + ((p * 2 + m) * 64 + lane) * 4);
            acc[m] = sum;
          }
        }
        __syncthreads();
      }
      if (live && (NWK == 1 || w == 0)) {
        uint16_t* out = static_cast<uint16_t*>(shared ? a.hs : a.hm);
        const int ld = shared ? a.Is : a.I;
        const int64_t rbase = shared ? 0 : off;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 4 * (lane >> 4) + v;
          if (m < ntok) {
            const float h = silu(acc[0][v]) * acc[1][v];
            out[(rbase + tc * 16 + m) * ld + row0 + n] = f32_to_bf16(h);
          }
        }
      }
    }
  }
}

template <int BITS, int U, int NWK>
__global__ __launch_bounds__(256) void k_stream_down_q(SkinnyDownArgs a) {
  constexpr int QSLOT = BITS == 8 ? RingGeomU8<1>::SLOT_BYTES : RingGeomU4<1, 16>::SLOT_BYTES;
  using GB = RingGeom<1>;
  constexpr int SLOTB = QSLOT > GB::SLOT * 2 ? QSLOT : GB::SLOT * 2;
  constexpr int IPB = 4 / NWK;
  __shared__ __attribute__((aligned(16))) char rings[4 * U * SLOTB];
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  char* ring = rings + w * U * SLOTB;
  const int NQ = a.part == 2 ? 0 : a.meta[1];  // chunks; shared-only launches read no routing
  const int CH = a.H / 16;
  const int TC = (a.T + 15) / 16;
  const int n_routed = NQ * CH;
  const int nitems = n_routed + (a.Is > 0 && a.part != 1 ? CH * TC : 0);
  int rr, ch;
  ring_lane(rr, ch);
  for (int base = blockIdx.x * IPB; base < nitems; base += gridDim.x * IPB) {
    const int item = base + w / NWK;
    const bool live = item < nitems;
    const int it = live ? item : 0;
    const bool shared = it >= n_routed;
    const int K = shared ? a.Is : a.I;
    int k0 = 0, k1 = K;
    if (NWK > 1) {
      if (shared)
        unit_range(K, w % NWK, NWK, k0, k1);
      else
        unit_range128(K, w % NWK, NWK, k0, k1);
    }
    int e = 0, off = 0, ntot, row0, tc_begin, tc_end;
    if (!shared) {
      // one chunk of at most 16 positions.  Expert e's chunks are chunk-list entries
      // q0 .. q0 + nc - 1, and its items CH * q0 .. CH * (q0 + nc) - 1, ordered by row
      // block and then chunk: the items of one expert are contiguous (neighbouring row
      // blocks stream together) and a popular expert's chunks read the same rows side
      // by side.  Any entry of the expert, such as it / CH, names it and its q0.
      const int qa = it / CH;
      e = a.tiles[2 * qa];
      const int first = a.offsets[e];
      const int q0 = qa - (a.tiles[2 * qa + 1] - first) / kDecodeChunk;
      const int nc = (a.counts[e] + kDecodeChunk - 1) / kDecodeChunk;
      const int local = it - q0 * CH;
      const int c = local % nc;
      row0 = (local / nc) * 16;
      off = first + c * kDecodeChunk;
      ntot = a.counts[e] - c * kDecodeChunk;
      tc_begin = 0;
      tc_end = 1;
    } else {
      // shared item: the chunks of one row block are neighbours (they share its rows)
      const int si = it - n_routed;
      row0 = (si / TC) * 16;
      tc_begin = si % TC;
      tc_end = tc_begin + 1;
      ntot = a.T;
    }
    const char* ab = uniform_ptr(shared ? a.hs : a.hm);
    const int64_t ro = static_cast<int64_t>(e) * a.H + row0;
    for (int tc = tc_begin; tc < tc_end; ++tc) {
      const int ntok = min(16, ntot - tc * 16);
      uint32_t aoff[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = tc * 16 + min(8 * h + rr, ntok - 1);
        const int row = shared ? m : off + m;
        aoff[h] = static_cast<uint32_t>(row) * K * 2 + ch * 16;
      }
      f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
      if (live) {
        if (!shared) {
          const uint16_t* ss[1] = {a.down_s};
          const uint16_t* zz[1] = {a.down_z};
          const uint16_t* szs = u8_param_row<1>(ss, zz, ro, a.I);
          if constexpr (BITS == 8) {
            const char* wb[1] = {uniform_ptr(static_cast<const uint8_t*>(a.down) + ro * a.I)};
            const uint32_t woff[2] = {static_cast<uint32_t>(rr * a.I + ch * 16),
                                      static_cast<uint32_t>((8 + rr) * a.I + ch * 16)};
            ring_stream_u8<1, U>(wb, woff, ab, aoff, szs, k0, k1, ring, acc);
          } else {
            const char* wb[1] = {uniform_ptr(static_cast<const uint8_t*>(a.down) + ro * (a.I / 2))};
            const uint32_t woff = u4_code_off(a.I / 2);
            const int row0t = off + tc * 16;
            with_token_rows(ntok, [&](auto trc) {
              constexpr int TR = decltype(trc)::value;
              uint32_t ao[TR / 4];
              u4_token_offsets<TR>(ntok, [&](int j) { return static_cast<uint32_t>(row0t + j) * a.I * 2; }, ao);
              ring_stream_u4<1, U * SLOTB, TR>(wb, woff, ab, ao, szs, k0, k1, ring, acc);
            });
          }
        } else {
          const char* wb[1] = {uniform_ptr(static_cast<const uint16_t*>(a.sdown) + static_cast<int64_t>(row0) * a.Is)};
          const uint32_t woff[2] = {static_cast<uint32_t>((rr * K + ch * 8) * 2),
                                    static_cast<uint32_t>(((8 + rr) * K + ch * 8) * 2)};
          ring_stream<1, U>(wb, woff, ab, aoff, k0, k1, reinterpret_cast<uint16_t*>(ring), acc);
        }
      }
      if constexpr (NWK > 1) {
        float* red = reinterpret_cast<float*>(rings);
        __syncthreads();
        *reinterpret_cast<f32x4*>(red + (w * 64 + lane) * 4) = acc[0];
        __syncthreads();
        if (w == 0) {
          f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < 4; ++p) sum += *reinterpret_cast<const f32x4*>(red + (p * 64 + lane) * 4);
          acc[0] = sum;
        }
        __syncthreads();
      }
      if (live && (NWK == 1 || w == 0)) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 4 * (lane >> 4) + v;
          if (m < ntok) {
            if (!shared) {
              const int slot = a.perm[off + tc * 16 + m];
              const float val = a.topk_w[slot] * acc[0][v];
              const int64_t o = static_cast<int64_t>(slot) * a.H + row0 + n;
              if (a.r_bf16)
                static_cast<uint16_t*>(a.r)[o] = f32_to_bf16(val);
              else
                static_cast<float*>(a.r)[o] = val;
            } else {
              a.rs[static_cast<int64_t>(tc * 16 + m) * a.H + row0 + n] = acc[0][v];
            }
          }
        }
      }
    }
  }
}

// y[t] = sum_j r[t*k + j] (valid experts only, fixed j order) + rs[t]
template <Act ACT>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  using AT = typename ActType<ACT>::T;
  const int64_t nvec = static_cast<int64_t>(a.T) * (a.H / 4);
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < nvec; i += static_cast<int64_t>(gridDim.x) * 256) {
    const int t = static_cast<int>(i / (a.H / 4));
    const int h = static_cast<int>(i % (a.H / 4)) * 4;
    // the token's k indices, its k routed rows and its shared row are loaded together
    // (one memory latency; a row whose index is invalid is loaded but not added: its
    // slot holds no routed term), then added in slot order
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    const int64_t slot0 = static_cast<int64_t>(t) * a.k;
    int ex[kMaxTopK];
    float4 rv[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < a.k) ex[j] = a.idx[slot0 + j];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= a.k) continue;
      if (a.r_bf16) {
        const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.r) + (slot0 + j) * a.H + h);
        rv[j] = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                            __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
      } else {
        rv[j] = *reinterpret_cast<const float4*>(static_cast<const float*>(a.r) + (slot0 + j) * a.H + h);
      }
    }
    const float4 vs = a.rs ? *reinterpret_cast<const float4*>(a.rs + static_cast<int64_t>(t) * a.H + h)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= a.k || ex[j] < 0 || ex[j] >= a.E) continue;
      s.x += rv[j].x;
      s.y += rv[j].y;
      s.z += rv[j].z;
      s.w += rv[j].w;
    }
    if (a.rs) {
      s.x += vs.x;
      s.y += vs.y;
      s.z += vs.z;
      s.w += vs.w;
    }
    AT* y = static_cast<AT*>(a.y) + static_cast<int64_t>(t) * a.H + h;
    if constexpr (ACT == Act::BF16) {
      *reinterpret_cast<uint2*>(y) = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
    } else {
      *reinterpret_cast<float4*>(y) = s;
    }
  }
}

int pick_mt(int T) {
  const int t = T < 64 ? T : 64;
  return t <= 16 ? 1 : (t <= 32 ? 2 : 4);
}

int grid_for(int64_t items, int ipb, int ncu) {
  int64_t blocks = (items + ipb - 1) / ipb;
  const int64_t cap = static_cast<int64_t>(ncu) * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return static_cast<int>(blocks);
}

// K-steps per LDS ring (per wavefront) of the bf16 streaming kernels
constexpr int kUpRing = 3, kDownRing = 4;
// u8 gate/up: a two-step ring (two blocks per CU) split over the four wavefronts
// measured 3-6% faster than three steps unsplit on the Ling-3.0-flash shape at 1 to 64
// tokens (graph replay at 64 tokens 338.5 -> 317 us)
constexpr int kUpRingU8 = 2, kDownRingU8 = 3;
// u4 down: two steps (measured 3-5% faster than three on the Ling-3.0-flash u4 shape
// at 1 to 64 tokens, graph replay at 64 tokens 260.8 -> 248.4 us)
constexpr int kUpRingU4 = 3, kDownRingU4 = 2;
// the split u4 gate/up kernel: a two-slot budget (still 3-5 steps in flight with 4-8
// token rows) lets three blocks share a CU (measured 5-7% faster at 8-64 tokens)
constexpr int kUpRingSplitU4 = 2;

// work items of a launch covering `part` (see SkinnyUpArgs::part)
int64_t part_items(int part, int64_t routed, int64_t shared) {
  return (part == 2 ? 0 : routed) + (part == 1 ? 0 : shared);
}

// the u8 ring kernels copy two fp16 group parameters at a time (4-byte copies)
bool aligned4(std::initializer_list<const uint16_t*> ps) {
  for (const uint16_t* p : ps)
    if (reinterpret_cast<uintptr_t>(p) % 4) return false;
  return true;
}

// the ring kernels address activation rows with 32-bit byte offsets
bool stream_ok(int64_t rows, int64_t cols, int64_t rows2, int64_t cols2) {
  return rows * cols * 2 < (int64_t(1) << 31) && rows2 * cols2 * 2 < (int64_t(1) << 31);
}

// split: the four wavefronts of a block share one item's K; else one item each
template <int U, typename Args>
hipError_t launch_ring(void (*k1)(Args), void (*k4)(Args), int64_t items, bool split, int ncu, hipStream_t s,
                       const Args& a) {
  const int grid = grid_for(items, split ? 1 : 4, ncu);
  hipLaunchKernelGGL(split ? k4 : k1, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

#define MOE_DISPATCH_MT_NWK(KERNEL, ARGS, ITEMS, T_, SPLIT, ...)                                \
  do {                                                                                          \
    const int mt_ = pick_mt(T_);                                                                \
    const bool k4_ = (SPLIT);                                                                   \
    const int grid_ = grid_for((ITEMS), k4_ ? 1 : 4, ncu);                                      \
    if (k4_) {                                                                                  \
      if (mt_ == 1)                                                                             \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 1, 4>), dim3(grid_), dim3(256), 0, s, ARGS);    \
      else if (mt_ == 2)                                                                        \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 2, 4>), dim3(grid_), dim3(256), 0, s, ARGS);    \
      else                                                                                      \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 4, 4>), dim3(grid_), dim3(256), 0, s, ARGS);    \
    } else {                                                                                    \
      if (mt_ == 1)                                                                             \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 1, 1>), dim3(grid_), dim3(256), 0, s, ARGS);    \
      else if (mt_ == 2)                                                                        \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 2, 1>), dim3(grid_), dim3(256), 0, s, ARGS);    \
      else                                                                                      \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 4, 1>), dim3(grid_), dim3(256), 0, s, ARGS);    \
    }                                                                                           \
  } while (0)

hipError_t launch_skinny_router(const SkinnyRouterArgs& a, Act act, int ncu, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int64_t items = static_cast<int64_t>((a.E + 15) / 16) * a.P;
  const int64_t small = 4ll * ncu;
  if (act == Act::BF16)
    MOE_DISPATCH_MT_NWK(k_skinny_router, a, items, a.T, items < small, Act::BF16);
  else
    MOE_DISPATCH_MT_NWK(k_skinny_router, a, items, a.T, items < small, Act::F32);
  return hipGetLastError();
}

// Split decisions are taken from the item count of the whole layer (routed and shared
// items), never from `part`, so that a layer launched in one piece and one whose shared
// expert runs as a separate launch (a graph branch) do the same arithmetic.
hipError_t launch_skinny_up(const SkinnyUpArgs& a, Act act, WFmt wf, int ncu, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int64_t slots = static_cast<int64_t>(a.T) * a.k;
  const int64_t dmax = slots < a.E ? slots : a.E;
  const int tch = 16 * pick_mt(a.T);
  const int64_t shared_skinny = static_cast<int64_t>(a.Is / 16) * ((a.T + tch - 1) / tch);
  const int64_t items = part_items(a.part, dmax * (a.I / 16), shared_skinny);
  const int64_t small = 4ll * ncu;
  const bool split_skinny = part_items(0, dmax * (a.I / 16), shared_skinny) < small;
  // ring kernels: one item = 16 weight rows x one chunk of 16 tokens
  const int64_t shared_ring = static_cast<int64_t>(a.Is / 16) * ((a.T + 15) / 16);
  const int64_t ring = part_items(a.part, static_cast<int64_t>(a.mtiles) * (a.I / 16), shared_ring);
  const int64_t ring_all = part_items(0, static_cast<int64_t>(a.mtiles) * (a.I / 16), shared_ring);
  // Gate/up ring kernels split K over the four wavefronts of a block at every size
  // (measured faster on the bf16, u8 and u4 layers from 1 to 64 tokens: finer work units
  // even out the last round), except for the dense MLP, whose token chunks of one row
  // block share its rows best inside one block: it splits only when its items cannot
  // occupy the CUs otherwise.
  const bool split_ring = a.dense ? ring_all < small : true;
  if (wf == WFmt::U4) {
    // the only u4 kernel: the configuration checks guarantee its conditions
    if (act != Act::BF16 || a.H % 128 || !stream_ok(a.T, a.H, a.T, a.Is) || !aligned4({a.gate_s, a.gate_z, a.up_s, a.up_z}))
      return hipErrorInvalidValue;
    return launch_ring<kUpRingU4>(k_stream_up_q<4, kUpRingU4, 1>, k_stream_up_q<4, kUpRingSplitU4, 4>, ring,
                                  split_ring, ncu, s, a);
  }
  if (act == Act::F32)
    MOE_DISPATCH_MT_NWK(k_skinny_up, a, items, a.T, split_skinny, Act::F32, WFmt::F32);
  else if (wf == WFmt::U8 && a.H % 128 == 0 && stream_ok(a.T, a.H, 0, 0) &&
           aligned4({a.gate_s, a.gate_z, a.up_s, a.up_z}))
    return launch_ring<kUpRingU8>(k_stream_up_q<8, kUpRingU8, 1>, k_stream_up_q<8, kUpRingU8, 4>, ring, split_ring,
                                  ncu, s, a);
  else if (wf == WFmt::U8)
    MOE_DISPATCH_MT_NWK(k_skinny_up, a, items, a.T, split_skinny, Act::BF16, WFmt::U8);
  else if (stream_ok(a.T, a.H, a.T * a.k, a.I))
    return launch_ring<kUpRing>(k_stream_up<kUpRing, 1>, k_stream_up<kUpRing, 4>, ring, split_ring, ncu, s, a);
  else
    MOE_DISPATCH_MT_NWK(k_skinny_up, a, items, a.T, split_skinny, Act::BF16, WFmt::BF16);
  return hipGetLastError();
}

hipError_t launch_skinny_down(const SkinnyDownArgs& a, Act act, WFmt wf, int ncu, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int64_t slots = static_cast<int64_t>(a.T) * a.k;
  const int64_t dmax = slots < a.E ? slots : a.E;
  const int tch = 16 * pick_mt(a.T);
  const int64_t shared_skinny = a.Is > 0 ? static_cast<int64_t>(a.H / 16) * ((a.T + tch - 1) / tch) : 0;
  const int64_t items = part_items(a.part, dmax * (a.H / 16), shared_skinny);
  const int64_t small = 4ll * ncu;
  const bool split_skinny = part_items(0, dmax * (a.H / 16), shared_skinny) < small;
  const int64_t shared_ring = a.Is > 0 ? static_cast<int64_t>(a.H / 16) * ((a.T + 15) / 16) : 0;
  const int64_t ring = part_items(a.part, static_cast<int64_t>(a.mtiles) * (a.H / 16), shared_ring);
  // down, whose K is the expert width, splits only when its items cannot occupy the CUs
  const bool split_ring = part_items(0, static_cast<int64_t>(a.mtiles) * (a.H / 16), shared_ring) < small;
  if (wf == WFmt::U4) {
    if (act != Act::BF16 || a.I % 128 || !stream_ok(a.T * a.k, a.I, a.T, a.Is) || !aligned4({a.down_s, a.down_z}))
      return hipErrorInvalidValue;
    return launch_ring<kDownRingU4>(k_stream_down_q<4, kDownRingU4, 1>, k_stream_down_q<4, kDownRingU4, 4>, ring,
                                    split_ring, ncu, s, a);
  }
  if (act == Act::F32)
    MOE_DISPATCH_MT_NWK(k_skinny_down, a, items, a.T, split_skinny, Act::F32, WFmt::F32);
  else if (wf == WFmt::U8 && a.I % 128 == 0 && stream_ok(a.T * a.k, a.I, a.T, a.Is) &&
           aligned4({a.down_s, a.down_z}))
    return launch_ring<kDownRingU8>(k_stream_down_q<8, kDownRingU8, 1>, k_stream_down_q<8, kDownRingU8, 4>, ring,
                                    split_ring, ncu, s, a);
  else if (wf == WFmt::U8)
    MOE_DISPATCH_MT_NWK(k_skinny_down, a, items, a.T, split_skinny, Act::BF16, WFmt::U8);
  else if (stream_ok(a.T * a.k, a.I, a.T, a.Is))
    return launch_ring<kDownRing>(k_stream_down<kDownRing, 1>, k_stream_down<kDownRing, 4>, ring, split_ring, ncu, s,
                                  a);
  else
    MOE_DISPATCH_MT_NWK(k_skinny_down, a, items, a.T, split_skinny, Act::BF16, WFmt::BF16);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, Act act, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int64_t nvec = static_cast<int64_t>(a.T) * (a.H / 4);
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (act == Act::BF16)
    hipLaunchKernelGGL(k_combine<Act::BF16>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_combine<Act::F32>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
