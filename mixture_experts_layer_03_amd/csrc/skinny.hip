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
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "route_token.h"

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
// [16 NMAT, 16 NMAT + TR) tokens; 128-byte rows with 16-byte chunks XOR-swizzled by
// row % 8.  Lane l of a copy instruction covering rows [8h, 8h + 8) takes row 8h + l/8
// and logical chunk (l % 8) ^ (l / 8).  TR = 8 or 16 token rows: a chunk of at most 8
// live tokens copies 8 (MFMA rows 8..15 reread rows 0..7; their results are dropped),
// and the LDS it leaves holds more K-steps in flight within the same per-wavefront
// ring budget, so the same number of blocks fits on a CU.
template <int NMAT, int TR = 16>
struct RingGeom {
  static constexpr int ROWS = 16 * NMAT + TR;
  static constexpr int SLOT = ROWS * 64;         // bf16 elements per K-step
  static constexpr int CPS = 2 * NMAT + TR / 8;  // copy instructions per K-step
};
// K-steps in a ring of RB bytes with slots of SLOT_BYTES (at most 8)
constexpr int ring_depth(int rb, int slot_bytes) { return rb / slot_bytes < 8 ? rb / slot_bytes : 8; }

// acc[m] += tokens x W_m^T over [k0, k1) (multiples of 64) with a ring of RB bytes at
// `ring` (as many K-steps as fit, at most 8) and TR token rows.
// wbase[m]: wave-uniform byte address of weight row 0 of matrix m (rows H_row bytes
// apart, the stride folded into woff); woff[h]: this lane's byte offset of its row in
// copy h (row 8h + l/8) plus its chunk; abase / aoff[h]: the same for the token rows.
template <int NMAT, int RB, int TR>
__device__ __forceinline__ void ring_stream(const char* const (&wbase)[NMAT], const uint32_t (&woff)[2],
                                            const char* abase, const uint32_t (&aoff)[2], int k0, int k1,
                                            uint16_t* ring, f32x4 (&acc)[NMAT]) {
  using G = RingGeom<NMAT, TR>;
  constexpr int U = ring_depth(RB, G::SLOT * 2);
  static_assert(U >= 2 && G::CPS * (U - 1) < 64, "ring depth");
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
    for (int h = 0; h < TR / 8; ++h) copy_to_lds(uniform_ptr(abase + kb), aoff[h], sl + (16 * NMAT + 8 * h) * 64);
  };
  const int r = lane & 15, q = lane >> 4;
  auto compute = [&](int slot) {
    const uint16_t* sl = ring + slot * G::SLOT;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int cc = ((ks * 4 + q) ^ (r & 7)) << 3;
      const uint4 a = *reinterpret_cast<const uint4*>(sl + (16 * NMAT + (r & (TR - 1))) * 64 + cc);
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

// A work item of the ring kernels: CH routed items per chunk-list entry and n_shared
// items of the shared expert (row block si / TC, token chunk si % TC: the chunks of one
// row block are neighbours, they share its rows).  Expert e's entries are
// q0 .. q0 + nc - 1 and its items CH * q0 .. CH * (q0 + nc) - 1, ordered by row block and
// then chunk, so the items of one expert are contiguous (neighbouring row blocks stream
// together) and a popular expert's chunks read the same rows side by side.  Any entry
// of the expert names it and its q0, and the entry's 16-byte record carries the rest: a
// routed item waits for one load (the record, beside the chunk count) before its weight
// copies.
// shared_first: the shared items come first; they read no routing and start streaming
// at once (batches of one token chunk, where every item is short and the routing loads
// are a visible part of it).  Otherwise the routed items come first and the uniform
// shared items fill the last round (measured better once chunks are long).
// `item` must be below n_shared + (chunk bound) * CH, which keeps the record load in
// bounds; items past the live ones decode to an in-range routed item of offset 0 and
// one token, with live = false.
// slot[v] and routing weight wgt[v] of position p0 + m, m = 4 (lane / 16) + v (the
// rows this lane stores), for m < ntok
__device__ __forceinline__ void routed_slots(const int32_t* perm, const float* wpos, int p0, int ntok, int (&slot)[4],
                                             float (&wgt)[4]) {
  const int lane = lane_id();
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * (lane >> 4) + v;
    slot[v] = m < ntok ? perm[p0 + m] : 0;
    wgt[v] = m < ntok ? wpos[p0 + m] : 0.f;
  }
}

// Byte offsets of the ring kernels' token-row copies (copy h: chunk row 8h + rr, padded
// rows repeating the last live one) for rows [m0, m0 + ntok) of a shared chunk (tokens
// themselves) or of routed positions off + m0 .. (their tokens through the
// permutation; with one token, token 0).  Both permutation loads go out before either
// is used.
__device__ __forceinline__ void token_offsets(const SkinnyUpArgs& a, bool shared, int off, int m0, int ntok, int rr,
                                              int ch, uint32_t (&aoff)[2]) {
  int tok[2];
  if (shared || a.T == 1) {
#pragma unroll
    for (int h = 0; h < 2; ++h) tok[h] = shared ? m0 + min(8 * h + rr, ntok - 1) : 0;
  } else {
    int pv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) pv[h] = a.perm[off + m0 + min(8 * h + rr, ntok - 1)];
#pragma unroll
    for (int h = 0; h < 2; ++h) tok[h] = pv[h] / a.k;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) aoff[h] = static_cast<uint32_t>(tok[h]) * a.H * 2 + ch * 16;
}

// live items of a ring launch: the shared ones and CH per routed chunk (the chunk count
// is a device value; the grid covers the host's bound, and the loop stops at the live
// count, so blocks past it do no work)
template <typename Args>
__device__ __forceinline__ int live_items(const Args& a, int n_shared, int CH) {
  return n_shared + (a.part == 2 ? 0 : a.meta[1] * CH);
}

struct RingItem {
  bool live, shared;
  int e, off, ntot, row0, tc;
};

// Row block rb and chunk c of item `local` among CH row blocks x nc chunks, placed by
// groups of S row blocks: item g S nc + c S + j is chunk c of row block g S + j.
// With one item per block, blocks are dealt to the eight XCDs in turn (block b runs on
// XCD b % 8), so with S = 8 all chunks of a row block run on one XCD, 8 blocks apart,
// in the same window of 8 nc items, and that XCD's L2 fetches the rows once for all of
// them; items one after another would put them on different XCDs, each fetching the
// same rows.  With S = 1 the order is row block by row block, chunk innermost (with
// four items per block, a row block's chunks then share one block).
__device__ __forceinline__ void place_item(int local, int CH, int nc, int S, int& rb, int& c) {
  const int gs = S * nc, g = local / gs, rem = local - g * gs;
  const int R = min(S, CH - g * S);  // row blocks of this group (fewer in the last one)
  c = rem / R;
  rb = g * S + rem % R;
}

// S: as for place_item, applied to the routed items of each expert and to the shared
// items.
__device__ __forceinline__ RingItem ring_item(int item, int n_shared, int TC, int CH, int T, const int32_t* meta,
                                              const int4* chunks, bool shared_first, int S = 1) {
  RingItem r{};
  int it;  // routed item index
  const int CHs = n_shared / (TC > 0 ? TC : 1);
  if (shared_first) {
    if (item < n_shared) {
      r.live = r.shared = true;
      int rb;
      place_item(item, CHs, TC, S, rb, r.tc);
      r.row0 = rb * 16;
      r.ntot = T;
      return r;
    }
    it = item - n_shared;
  } else {
    const int nr = meta[1] * CH;
    if (item >= nr) {
      const int si = item - nr;
      r.live = si < n_shared;
      r.shared = true;
      r.ntot = T;
      if (n_shared > 0) {
        int rb;
        place_item(min(si, n_shared - 1), CHs, TC, S, rb, r.tc);
        r.row0 = rb * 16;
        return r;
      }
    }
    it = min(item, nr > 0 ? nr - 1 : 0);
  }
  const int qa = it / CH;
  int4 rec = chunks[qa];  // (expert, entry's first position, expert's first position, count)
  int nq = meta[1];
  // both loads are issued before this point, which needs them: one memory round trip
  asm volatile("" : "+v"(rec.x), "+v"(rec.y), "+v"(rec.z), "+v"(rec.w), "+v"(nq));
  r.live = qa < nq && (shared_first || item < nq * CH);
  const int first = r.live ? rec.z : 0, count = r.live ? rec.w : 1;
  const int q0 = r.live ? qa - (rec.y - rec.z) / kDecodeChunk : qa;
  const int nc = (count + kDecodeChunk - 1) / kDecodeChunk;
  int rb, c;
  place_item(it - q0 * CH, CH, nc, S, rb, c);
  r.e = r.live ? rec.x : 0;
  r.row0 = rb * 16;
  r.off = first + c * kDecodeChunk;
  r.ntot = count - c * kDecodeChunk;
  return r;
}

// One-token routing inside a gate/up launch (SkinnyUpArgs::fused_route).  Wave 0 routes
// the token (route_token) and ranks its k picks, which are distinct experts, by expert
// index: position p holds the p-th smallest valid pick, one chunk each, which is what
// the permutation kernels build for a single token.  Block 0 stores the routing (ta.idx,
// ta.w) and every table pa names; every block reads back the expert of its own item.
// Called by all threads of the block before any ring is in use (the scratch lies in
// the rings' LDS); returns the item as ring_item would for the shared-first order.
// EPL: experts per lane of route_token (a template argument of the one-token kernels
// only, so the other launches keep their registers).
template <int EPL>
__device__ RingItem one_token_item(const SkinnyUpArgs& a, char* scratch, int item, int n_shared, int CH) {
  int* s_slot_e = reinterpret_cast<int*>(scratch);           // [k] expert of slot j
  float* s_w = reinterpret_cast<float*>(s_slot_e + kMaxTopK);  // [k] weight of slot j
  int* s_pos_e = reinterpret_cast<int*>(s_w + kMaxTopK);       // [k] expert at position p
  int* s_kv = s_pos_e + kMaxTopK;                              // valid picks
  const bool publish = blockIdx.x == 0;
  const int tid = threadIdx.x;
  const int k = a.ta.k, E = a.ta.E;
  const PermuteArgs& pa = a.pa;
  if (tid < 64) {
    route_token<EPL>(a.ta, 0, s_slot_e, s_w, publish);
    one_token_tables(pa, k, E, s_slot_e, s_w, s_pos_e, s_kv, publish);
  }
  __syncthreads();
  const int kv = *s_kv;
  if (publish) one_token_counts(pa, E, s_pos_e, kv, tid, blockDim.x);
  RingItem r{};
  if (item < n_shared) {
    r.live = r.shared = true;
    r.row0 = item * 16;  // one token: one chunk per row block
    r.ntot = 1;
  } else {
    const int it = item - n_shared, qa = it / CH;
    r.live = qa < kv;
    r.e = r.live ? s_pos_e[qa] : 0;
    r.row0 = (it - qa * CH) * 16;
    r.off = r.live ? qa : 0;
    r.ntot = 1;
  }
  __syncthreads();  // every wave has read the scratch before a ring overwrites it
  return r;
}

// FEPL > 0: the one-token launch that routes its token itself (route_token<FEPL>)
template <int RB, int NWK, int FEPL = 0>
__global__ __launch_bounds__(256) void k_stream_up(SkinnyUpArgs a) {
  constexpr int IPB = 4 / NWK;
  __shared__ __attribute__((aligned(16))) uint16_t rings[4 * RB / 2];
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  uint16_t* ring = rings + w * (RB / 2);
  const int CH = a.I / 16, CHs = a.Is / 16;
  const int TC = (a.T + 15) / 16;
  const int n_shared = a.part == 1 ? 0 : CHs * TC;
  const int nbound = n_shared + (a.part == 2 ? 0 : a.mtiles * CH);  // routed: up to the chunk bound
  int rr, ch;
  ring_lane(rr, ch);
  const char* xb = uniform_ptr(a.x);
  // one token: this block routes it itself (the launch covers every item in one round)
  RingItem pre{};
  if constexpr (FEPL > 0)
    pre = one_token_item<FEPL>(a, reinterpret_cast<char*>(rings),
                               min(static_cast<int>(blockIdx.x) * IPB + w / NWK, nbound - 1), n_shared, CH);
  const bool sf = a.shared_first || a.part == 2;
  int nlive = FEPL == 0 && !sf ? live_items(a, n_shared, CH) : nbound;
  for (int base = blockIdx.x * IPB; base < nlive; base += gridDim.x * IPB) {
    if (FEPL == 0 && sf && base >= n_shared && nlive == nbound) {
      nlive = live_items(a, n_shared, CH);  // shared-first: loaded once a block reaches the routed items
      if (base >= nlive) break;
    }
    const int item = base + w / NWK;
    const RingItem itm = FEPL > 0 ? pre
                                  : ring_item(min(item, nbound - 1), n_shared, TC, CH, a.T, a.meta, a.chunks, sf, IPB == 1 ? 8 : 1);
    const bool live = item < nbound && itm.live, shared = itm.shared;
    const int e = itm.e, off = itm.off, ntot = itm.ntot, row0 = itm.row0, tc_begin = itm.tc, tc_end = itm.tc + 1;
    int k0 = 0, k1 = a.H;
    if (NWK > 1) unit_range(a.H, w % NWK, NWK, k0, k1);
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
      token_offsets(a, shared, off, tc * 16, ntok, rr, ch, aoff);
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      if (live) {
        if (ntok <= 8)
          ring_stream<2, RB, 8>(wb, woff, xb, aoff, k0, k1, ring, acc);
        else
          ring_stream<2, RB, 16>(wb, woff, xb, aoff, k0, k1, ring, acc);
      }
      if constexpr (NWK > 1) {
        // K-split: partial sums through the (now idle) rings; wavefront 0 adds them
        float* red = reinterpret_cast<float*>(rings);
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 2; ++m) *reinterpret_cast<f32x4*>(red + ((w * 2 + m) * 64 + lane) * 4) = acc[m];
        __syncthreads();
        if (w % NWK == 0) {  // the first wavefront of each item adds its item's partials
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < NWK; ++p) sum += *reinterpret_cast<const f32x4*>(red + (((w + p) * 2 + m) * 64 + lane) * 4);
            acc[m] = sum;
          }
        }
        __syncthreads();
      }
      if (live && (NWK == 1 || w % NWK == 0)) {
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

template <int RB, int NWK>
__global__ __launch_bounds__(256) void k_stream_down(SkinnyDownArgs a) {
  constexpr int IPB = 4 / NWK;
  __shared__ __attribute__((aligned(16))) uint16_t rings[4 * RB / 2];
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  uint16_t* ring = rings + w * (RB / 2);
  const int CH = a.H / 16;
  const int TC = (a.T + 15) / 16;
  const int n_shared = a.Is > 0 && a.part != 1 ? CH * TC : 0;
  const int nbound = n_shared + (a.part == 2 ? 0 : a.mtiles * CH);  // routed: up to the chunk bound
  int rr, ch;
  ring_lane(rr, ch);
  const bool sf = a.shared_first || a.part == 2;
  int nlive = sf ? nbound : live_items(a, n_shared, CH);
  for (int base = blockIdx.x * IPB; base < nlive; base += gridDim.x * IPB) {
    if (sf && base >= n_shared && nlive == nbound) {
      nlive = live_items(a, n_shared, CH);  // shared-first: loaded once a block reaches the routed items
      if (base >= nlive) break;
    }
    const int item = base + w / NWK;
    const RingItem itm = ring_item(min(item, nbound - 1), n_shared, TC, CH, a.T, a.meta, a.chunks, sf, IPB == 1 ? 8 : 1);
    const bool live = item < nbound && itm.live, shared = itm.shared;
    const int e = itm.e, off = itm.off, ntot = itm.ntot, row0 = itm.row0, tc_begin = itm.tc, tc_end = itm.tc + 1;
    const int K = shared ? a.Is : a.I;
    int k0 = 0, k1 = K;
    if (NWK > 1) unit_range(K, w % NWK, NWK, k0, k1);
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
      // the output slots and routing weights of this lane's rows, loaded before the
      // stream so that the store at its end waits for nothing
      int slot[4];
      float wgt[4];
      if (!shared) routed_slots(a.perm, a.wpos, off + tc * 16, ntok, slot, wgt);
      f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
      if (live) {
        if (ntok <= 8)
          ring_stream<1, RB, 8>(wb, woff, ab, aoff, k0, k1, ring, acc);
        else
          ring_stream<1, RB, 16>(wb, woff, ab, aoff, k0, k1, ring, acc);
      }
      if constexpr (NWK > 1) {
        float* red = reinterpret_cast<float*>(rings);
        __syncthreads();
        *reinterpret_cast<f32x4*>(red + (w * 64 + lane) * 4) = acc[0];
        __syncthreads();
        if (w % NWK == 0) {  // the first wavefront of each item adds its item's partials
          f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < NWK; ++p) sum += *reinterpret_cast<const f32x4*>(red + ((w + p) * 64 + lane) * 4);
          acc[0] = sum;
        }
        __syncthreads();
      }
      if (live && (NWK == 1 || w % NWK == 0)) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 4 * (lane >> 4) + v;
          if (m < ntok) {
            if (!shared) {
              const float val = wgt[v] * acc[0][v];
              const int64_t o = static_cast<int64_t>(slot[v]) * a.H + row0 + n;
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

// sum of eight bf16 products (two per step, fp32 accumulation) added to c
__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b, float c) {
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), __builtin_bit_cast(bf16x2, b.x), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, b.y), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, b.z), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, b.w), c, false);
  return c;
}

// sum over 16 u8 codes c_j of (c_j - z) * a_j, a_j the bf16 values in a0 (j < 8) and a1
// (each code minus the zero point is exact in fp32, and so is its product with a_j)
__device__ __forceinline__ float dot16_u8(const uint4& c, const uint4& a0, const uint4& a1, float z) {
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  const uint32_t aw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float cj = static_cast<float>((cw[j >> 2] >> (8 * (j & 3))) & 0xffu);
    const uint32_t w2 = aw[j >> 1];
    const float aj = __uint_as_float((j & 1) ? (w2 & 0xffff0000u) : (w2 << 16));
    acc = fmaf(cj - z, aj, acc);
  }
  return acc;
}

// the same for 16 u4 codes packed two per byte, element 2i in the low nibble of byte i
__device__ __forceinline__ float dot16_u4(const uint2& c, const uint4& a0, const uint4& a1, float z) {
  const uint32_t aw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float cj = static_cast<float>(((j < 8 ? c.x : c.y) >> (4 * (j & 7))) & 0xfu);
    const uint32_t w2 = aw[j >> 1];
    const float aj = __uint_as_float((j & 1) ? (w2 & 0xffff0000u) : (w2 << 16));
    acc = fmaf(cj - z, aj, acc);
  }
  return acc;
}

// ---------------------------------------- one token: gate/up, with or without routing
// With one token, column n of an expert's gated unit is silu(g_n . x) * (u_n . x): two
// dot products over H [Bailing MoE expert MLP: SwiGLU].  A wavefront takes one column at
// a time: it issues every 16-byte load of both rows (H / 512 per lane each) before using
// the first, and reduces the two sums across its lanes; each lane keeps its slice of x
// in registers (the same positions of every row).  The grid is sized so that every
// block is resident at once.  Waves 1 .. NW-1 of a block stream its share of the shared
// expert's columns while wave 0 finds the expert of each position: with FEPL > 0 it
// routes the token from the router's partial logits (route_token; block 0 also stores
// the routing and every table the permutation would build), with FEPL == 0 it reads
// them through the caller's permutation.  Then all waves stream the block's share of
// the selected experts' columns.  Lanes past the end of a row load its last vector
// again (same line) and add nothing, so no branch splits the loads.
constexpr int kUpOneWaves = 8;

// The experts by position of a one-token launch, found by one wavefront into LDS
// (s_pos_e[p], valid count *s_kv): FEPL > 0 routes the token from the router's partial
// logits (route_token, with `publish` storing the routing and every table the
// permutation would build); FEPL == 0 reads them through the caller's permutation
// (position p holds slot perm[p], the pick j of the one token; valid picks fill
// positions 0 .. kv - 1).
template <int FEPL>
__device__ __forceinline__ void up_one_picks(const SkinnyUpArgs& a, bool publish, int* s_slot_e, float* s_w,
                                             int* s_pos_e, int* s_kv) {
  if constexpr (FEPL > 0) {
    // 512 experts: the partial logits in two batches (the registers of one batch would
    // cost the launch half its blocks per CU)
    route_token<FEPL, FEPL >= 8 ? 32 : 64>(a.ta, 0, s_slot_e, s_w, publish);
    one_token_tables(a.pa, a.k, a.E, s_slot_e, s_w, s_pos_e, s_kv, publish);
  } else {
    const int lane = lane_id();
    const int jl = min(lane, a.k - 1);
    const int pslot = a.perm[jl];
    const int pidx = a.idx[jl];
    const int kv = __popcll(__ballot(lane < a.k && pidx >= 0 && pidx < a.E));
    const int pe = __shfl(pidx, min(max(pslot, 0), a.k - 1));
    if (lane < kv) s_pos_e[lane] = pe;
    if (lane == 0) *s_kv = kv;
  }
}

template <int NLH, int FEPL>
__global__ __launch_bounds__(64 * kUpOneWaves, 4) void k_up_one(SkinnyUpArgs a) {
  constexpr int NW = kUpOneWaves;
  __shared__ int s_slot_e[kMaxTopK], s_pos_e[kMaxTopK], s_kv;
  __shared__ float s_w[kMaxTopK];
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nvh = a.H / 8, nb = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
  // this lane's vectors of a row (byte offsets, clamped to the row); rows are addressed
  // as a wave-uniform base (scalar registers) plus these offsets
  uint32_t vo[NLH];
#pragma unroll
  for (int i = 0; i < NLH; ++i) vo[i] = 16u * static_cast<uint32_t>(min(lane + 64 * i, nvh - 1));
  // x in registers, loaded at once; with H = 4096 wave 0 loads it after routing (not
  // live across the routing, the launch keeps two blocks per CU)
  uint4 xv[NLH];
  auto load_x = [&]() {
    const char* xb = uniform_ptr(a.x);
#pragma unroll
    for (int i = 0; i < NLH; ++i) xv[i] = ld16(xb + vo[i]);
  };
  auto column = [&](const uint16_t* grow, const uint16_t* urow) {
    const char* gb = uniform_ptr(grow);
    const char* ub = uniform_ptr(urow);
    uint4 gv[NLH], uv[NLH];
#pragma unroll
    for (int i = 0; i < NLH; ++i) gv[i] = ld16(gb + vo[i]);
#pragma unroll
    for (int i = 0; i < NLH; ++i) uv[i] = ld16(ub + vo[i]);
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int i = 0; i < NLH; ++i) {
      const bool in = lane + 64 * i < nvh;
      const float tg = dot8_bf16(gv[i], xv[i], 0.f), tu = dot8_bf16(uv[i], xv[i], 0.f);
      g += in ? tg : 0.f;
      u += in ? tu : 0.f;
    }
    return silu(wave_sum(g)) * wave_sum(u);
  };
  if (NLH < 8 || w > 0) load_x();
  if (w > 0 && a.Is > 0) {
    const int s0 = static_cast<int>(static_cast<int64_t>(b) * a.Is / nb);
    const int s1 = static_cast<int>(static_cast<int64_t>(b + 1) * a.Is / nb);
    const uint16_t* sg = static_cast<const uint16_t*>(a.sgate);
    const uint16_t* su = static_cast<const uint16_t*>(a.sup);
    for (int n = s0 + w - 1; n < s1; n += NW - 1) {
      const int64_t ro = static_cast<int64_t>(n) * a.H;
      const float h = column(sg + ro, su + ro);
      if (lane == 0) static_cast<uint16_t*>(a.hs)[n] = f32_to_bf16(h);
    }
  }
  if (w == 0) up_one_picks<FEPL>(a, b == 0, s_slot_e, s_w, s_pos_e, &s_kv);
  __syncthreads();
  if (NLH >= 8 && w == 0) load_x();
  const int kv = s_kv;
  if constexpr (FEPL > 0)
    if (b == 0) one_token_counts(a.pa, a.E, s_pos_e, kv, threadIdx.x, blockDim.x);
  const int64_t nr = static_cast<int64_t>(kv) * a.I;
  const int r0 = static_cast<int>(static_cast<int64_t>(b) * nr / nb);
  const int r1 = static_cast<int>(static_cast<int64_t>(b + 1) * nr / nb);
  const uint16_t* gt = static_cast<const uint16_t*>(a.gate);
  const uint16_t* ut = static_cast<const uint16_t*>(a.up);
  for (int c = r0 + w; c < r1; c += NW) {
    const int p = c / a.I, n = c - p * a.I;
    const int64_t ro = (static_cast<int64_t>(s_pos_e[p]) * a.I + n) * a.H;
    const float h = column(gt + ro, ut + ro);
    if (lane == 0) static_cast<uint16_t*>(a.hm)[static_cast<int64_t>(p) * a.I + n] = f32_to_bf16(h);
  }
}

// The same with u8 routed experts (codes [E, I, H], fp16 scale and zero point per 64
// codes; the shared expert stays bf16).  A lane takes units of 16 elements, u = lane +
// 64 i (i < NU): one 16-byte load of codes, or two of bf16, per unit; the 64 groups of
// a row (H <= 4096) come in with one scale and one zero-point load per lane and reach
// the lanes that use them across the wavefront.  Per unit, sum_j (c_j - z) x_j is
// formed as sum_j c_j x_j - z sum_j x_j, the unit's sum of x taken once per launch.
template <int NU, int FEPL>
__global__ __launch_bounds__(64 * kUpOneWaves, 4) void k_up_one_q8(SkinnyUpArgs a) {
  constexpr int NW = kUpOneWaves;
  __shared__ int s_slot_e[kMaxTopK], s_pos_e[kMaxTopK], s_kv;
  __shared__ float s_w[kMaxTopK];
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nu = a.H / 16, ng = a.H / 64, nb = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
  int uc[NU];  // this lane's units (clamped to the row)
#pragma unroll
  for (int i = 0; i < NU; ++i) uc[i] = min(lane + 64 * i, nu - 1);
  uint4 xv[2 * NU];
  float sx[NU];
  auto load_x = [&]() {
    const char* xb = uniform_ptr(a.x);
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      xv[2 * i] = ld16(xb + 32 * uc[i]);
      xv[2 * i + 1] = ld16(xb + 32 * uc[i] + 16);
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const uint32_t v[8] = {xv[2 * i].x, xv[2 * i].y, xv[2 * i].z, xv[2 * i].w,
                             xv[2 * i + 1].x, xv[2 * i + 1].y, xv[2 * i + 1].z, xv[2 * i + 1].w};
      float t = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) t += __uint_as_float(v[j] << 16) + __uint_as_float(v[j] & 0xffff0000u);
      sx[i] = t;
    }
  };
  // a bf16 column (the shared expert)
  auto column16 = [&](const uint16_t* grow, const uint16_t* urow) {
    const char* gb = uniform_ptr(grow);
    const char* ub = uniform_ptr(urow);
    uint4 gv[2 * NU], uv[2 * NU];
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      gv[2 * i] = ld16(gb + 32 * uc[i]);
      gv[2 * i + 1] = ld16(gb + 32 * uc[i] + 16);
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      uv[2 * i] = ld16(ub + 32 * uc[i]);
      uv[2 * i + 1] = ld16(ub + 32 * uc[i] + 16);
    }
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const bool in = lane + 64 * i < nu;
      const float tg = dot8_bf16(gv[2 * i + 1], xv[2 * i + 1], dot8_bf16(gv[2 * i], xv[2 * i], 0.f));
      const float tu = dot8_bf16(uv[2 * i + 1], xv[2 * i + 1], dot8_bf16(uv[2 * i], xv[2 * i], 0.f));
      g += in ? tg : 0.f;
      u += in ? tu : 0.f;
    }
    return silu(wave_sum(g)) * wave_sum(u);
  };
  // a u8 column: rows r of gate and up (codes, and their group parameters)
  auto column8 = [&](int64_t r) {
    const char* gb = uniform_ptr(static_cast<const uint8_t*>(a.gate) + r * a.H);
    const char* ub = uniform_ptr(static_cast<const uint8_t*>(a.up) + r * a.H);
    const int gl = min(lane, ng - 1);
    const int64_t pr = r * ng + gl;
    uint4 gv[NU], uv[NU];
#pragma unroll
    for (int i = 0; i < NU; ++i) gv[i] = ld16(gb + 16 * uc[i]);
#pragma unroll
    for (int i = 0; i < NU; ++i) uv[i] = ld16(ub + 16 * uc[i]);
    const float gsc = f16_to_f32(a.gate_s[pr]), gzp = f16_to_f32(a.gate_z[pr]);
    const float usc = f16_to_f32(a.up_s[pr]), uzp = f16_to_f32(a.up_z[pr]);
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const bool in = lane + 64 * i < nu;
      const int src = uc[i] >> 2;  // the lane holding this unit's group
      const float gs_ = __shfl(gsc, src), gz_ = __shfl(gzp, src);
      const float us_ = __shfl(usc, src), uz_ = __shfl(uzp, src);
      const float tg = gs_ * (dot16_u8(gv[i], xv[2 * i], xv[2 * i + 1], 0.f) - gz_ * sx[i]);
      const float tu = us_ * (dot16_u8(uv[i], xv[2 * i], xv[2 * i + 1], 0.f) - uz_ * sx[i]);
      g += in ? tg : 0.f;
      u += in ? tu : 0.f;
    }
    return silu(wave_sum(g)) * wave_sum(u);
  };
  if (NU < 4 || w > 0) load_x();
  if (w > 0 && a.Is > 0) {
    const int s0 = static_cast<int>(static_cast<int64_t>(b) * a.Is / nb);
    const int s1 = static_cast<int>(static_cast<int64_t>(b + 1) * a.Is / nb);
    const uint16_t* sg = static_cast<const uint16_t*>(a.sgate);
    const uint16_t* su = static_cast<const uint16_t*>(a.sup);
    for (int n = s0 + w - 1; n < s1; n += NW - 1) {
      const int64_t ro = static_cast<int64_t>(n) * a.H;
      const float h = column16(sg + ro, su + ro);
      if (lane == 0) static_cast<uint16_t*>(a.hs)[n] = f32_to_bf16(h);
    }
  }
  if (w == 0) up_one_picks<FEPL>(a, b == 0, s_slot_e, s_w, s_pos_e, &s_kv);
  __syncthreads();
  if (NU >= 4 && w == 0) load_x();
  const int kv = s_kv;
  if constexpr (FEPL > 0)
    if (b == 0) one_token_counts(a.pa, a.E, s_pos_e, kv, threadIdx.x, blockDim.x);
  const int64_t nr = static_cast<int64_t>(kv) * a.I;
  const int r0 = static_cast<int>(static_cast<int64_t>(b) * nr / nb);
  const int r1 = static_cast<int>(static_cast<int64_t>(b + 1) * nr / nb);
  for (int c = r0 + w; c < r1; c += NW) {
    const int p = c / a.I, n = c - p * a.I;
    const float h = column8(static_cast<int64_t>(s_pos_e[p]) * a.I + n);
    if (lane == 0) static_cast<uint16_t*>(a.hm)[static_cast<int64_t>(p) * a.I + n] = f32_to_bf16(h);
  }
}

// ------------------------------------------ one token: down and combine in one launch
// With one token, element h of the layer output is a single dot product: the shared
// expert's down row h against its activation row, plus each selected expert's down row
// h against its own, scaled by the expert's routing weight [Bailing MoE block: the
// routed outputs are weighted, summed and added to the shared expert's output].  A
// wavefront owns one output element and issues every 16-byte load of its rows at once
// (2-23 KB per element, no ring needed): the routing first (an L2 round trip), the
// shared rows next (they need no routing), the selected experts' rows once the routing
// is in.  The block stages the activation rows (hs row 0, then hm positions 0..k-1) in
// LDS once for its NW elements.  No partial sum leaves the wavefront, so the weighted
// sum needs no second launch and no device-scope fence.
// NLS / NLR: loads per lane for a shared / routed row (Is / 512 and I / 512 rounded up
// for bf16; u8 and u4 routed rows take 16 codes per lane and load, I / 1024); K: top-k
// (position p of the one-token permutation holds a pick; with fewer valid picks than K
// the last valid row is loaded again and not added); QB: 0 for bf16 routed experts, 8
// or 4 for u8 or u4 codes with an fp16 scale and zero point per 64 (one group per four
// of a lane's 16-code vectors).
constexpr int kDownOneWaves = 8;

template <int NLS, int NLR, int K, int QB>
__global__ __launch_bounds__(64 * kDownOneWaves) void k_down_one(SkinnyDownArgs a) {
  constexpr int NW = kDownOneWaves, NT = 64 * NW;
  constexpr bool Q = QB != 0;  // u8 or u4 routed experts (16 codes per lane vector)
  constexpr int EPV = Q ? 16 : 8;  // routed-row elements per lane vector
  constexpr int NST = ((NLS + K * NLR * EPV / 8) * 64 + NT - 1) / NT;  // staging loads per thread
  __shared__ __attribute__((aligned(16))) uint16_t act[NST * NT * 8];
  // Every load is unconditional (lanes past a row's end load its last vector again, in
  // the same line, and add nothing), so no branch splits the loads and each use waits
  // only for the loads issued before its own.
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = static_cast<int>(blockIdx.x) * NW + w;
  const int hrow = min(h, a.H - 1);
  const int nvs = a.Is / 8, nvr = a.I / EPV, nst = nvs + K * (a.I / 8);
  // lane p: position p's slot (the pick j, one token) and weight; lane j: pick j's expert
  const int jl = min(lane, K - 1);
  const int pslot = a.perm[jl];
  const int pidx = a.idx[jl];
  const float pw = a.wpos[jl];
  __builtin_amdgcn_sched_barrier(0);
  const uint16_t* hs = static_cast<const uint16_t*>(a.hs);
  const uint16_t* hm = static_cast<const uint16_t*>(a.hm);
  uint4 st[NST];
#pragma unroll
  for (int i = 0; i < NST; ++i) {
    const int u = min(static_cast<int>(threadIdx.x) + NT * i, nst - 1);
    st[i] = ld16(u < nvs ? hs + 8 * u : hm + 8 * (u - nvs));
  }
  __builtin_amdgcn_sched_barrier(0);
  uint4 ws[NLS];
  const uint16_t* srow = static_cast<const uint16_t*>(a.sdown) + static_cast<int64_t>(hrow) * a.Is;
#pragma unroll
  for (int i = 0; i < NLS; ++i) ws[i] = ld16(srow + 8 * min(lane + 64 * i, nvs - 1));
  __builtin_amdgcn_sched_barrier(0);
  // valid picks fill positions 0 .. npos - 1 in expert order
  const int npos = __popcll(__ballot(lane < K && pidx >= 0 && pidx < a.E));
  const int pe = __shfl(pidx, min(max(pslot, 0), K - 1));
  uint4 wr[K][NLR];
  uint2 wq[QB == 4 ? K : 1][NLR];
  uint16_t gs[Q ? K : 1][NLR], gz[Q ? K : 1][NLR];  // u8 / u4: the group's fp16 scale, zero point
#pragma unroll
  for (int p = 0; p < K; ++p) {
    const int e = min(max(__builtin_amdgcn_readlane(pe, min(p, max(npos - 1, 0))), 0), a.E - 1);
    const int64_t r = static_cast<int64_t>(e) * a.H + hrow;
#pragma unroll
    for (int i = 0; i < NLR; ++i) {
      const int vc = min(lane + 64 * i, nvr - 1);
      if constexpr (QB == 8) wr[p][i] = ld16(static_cast<const uint8_t*>(a.down) + r * a.I + 16 * vc);
      if constexpr (QB == 4)
        wq[p][i] = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(a.down) + r * (a.I / 2) + 8 * vc);
      if constexpr (Q) {
        gs[p][i] = a.down_s[r * (a.I / 64) + vc / 4];
        gz[p][i] = a.down_z[r * (a.I / 64) + vc / 4];
      } else {
        wr[p][i] = ld16(static_cast<const uint16_t*>(a.down) + r * a.I + 8 * vc);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NST; ++i) {
    const int u = static_cast<int>(threadIdx.x) + NT * i;
    if (u < nst) *reinterpret_cast<uint4*>(act + 8 * u) = st[i];
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < NLS; ++i) {
    const int v = lane + 64 * i, vc = min(v, nvs - 1);
    const float t = dot8_bf16(ws[i], *reinterpret_cast<const uint4*>(act + 8 * vc), 0.f);
    acc += v < nvs ? t : 0.f;
  }
#pragma unroll
  for (int p = 0; p < K; ++p) {
    float sp = 0.f;
    const uint16_t* ap = act + 8 * nvs + p * a.I;  // position p's activation row
#pragma unroll
    for (int i = 0; i < NLR; ++i) {
      const int v = lane + 64 * i, vc = min(v, nvr - 1);
      float t;
      if constexpr (Q) {
        const uint4 a0 = *reinterpret_cast<const uint4*>(ap + 16 * vc);
        const uint4 a1 = *reinterpret_cast<const uint4*>(ap + 16 * vc + 8);
        const float z = f16_to_f32(gz[p][i]);
        t = f16_to_f32(gs[p][i]) * (QB == 8 ? dot16_u8(wr[p][i], a0, a1, z) : dot16_u4(wq[p][i], a0, a1, z));
      } else {
        t = dot8_bf16(wr[p][i], *reinterpret_cast<const uint4*>(ap + 8 * vc), 0.f);
      }
      sp += v < nvr ? t : 0.f;
    }
    const float wgt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw), p));
    acc = p < npos ? fmaf(wgt, sp, acc) : acc;
  }
  acc = wave_sum(acc);
  if (lane == 0 && h < a.H) static_cast<uint16_t*>(a.y)[h] = f32_to_bf16(acc);
}

// ----------------------------------------------------- u8 weights through LDS rings
// One ring step covers 128 elements of K (two quantisation groups), so a weight row's
// codes for the step are one whole 128-byte line.  Slot layout (bytes): NMAT x 16 code
// rows of 128 B, two token images of 16 rows x 128 B (elements 0..63 and 64..127 of the
// step), then 256 B of group parameters: lane l of one 4-byte-per-lane copy brings the
// two fp16 values (groups 2t, 2t + 1) of matrix l / 32, kind (l / 16) % 2 (scale,
// zero), row l % 16.  Products per group are exact: codes minus the zero point are
// integers in [-255, 255], exact in bf16; the group scale multiplies the fp32 result.
// PRE: the group parameters of the whole range are copied to their own area before the
// stream (ring_stream_u8), so a slot carries codes and token rows only.
template <int NMAT, int TR = 16, bool PRE = false>
struct RingGeomU8 {
  static constexpr int W_BYTES = NMAT * 16 * 128;
  static constexpr int A_BYTES = 2 * TR * 128;  // two token images of TR rows (8 or 16)
  static constexpr int SLOT_BYTES = W_BYTES + A_BYTES + (PRE ? 0 : 256);
  static constexpr int CPS = 2 * NMAT + 2 * (TR / 8) + (PRE ? 0 : 1);  // copy instructions per step
};
// LDS bytes of the preloaded group parameters: 32 * NMAT rows of scales or zero points,
// at most 16 groups (two 16-byte chunks) each
template <int NMAT>
constexpr int kU8ParamBytes = NMAT * 32 * 2 * 16;

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
// lane's group-parameter row (u8_param_row: scales or zero points of one row, group 0).
// Without PRE every step copies the step's two groups, 4 bytes per lane: one cache line
// per parameter row, so 32 NMAT line requests per step, as many as the codes and the
// token rows of a 16-token chunk together.  PRE (k1 - k0 a multiple of 512, at most
// 1024, parameter rows 16-byte aligned): before the stream the range's groups are copied
// once into kU8ParamBytes<NMAT> at `pa`, 16 bytes (8 groups) per lane and row, stored as
// chunk c = 16-byte piece j of parameter row rk at pa + 16 (j * 32 NMAT + rk); the whole
// range then costs 32 NMAT lines per 8 groups instead of per group pair.
template <int NMAT, int RB, int TR, bool PRE = false>
__device__ __forceinline__ void ring_stream_u8(const char* const (&wbase)[NMAT], const uint32_t (&woff)[2],
                                               const char* abase, const uint32_t (&aoff)[2], const uint16_t* sz_src,
                                               int k0, int k1, char* ring, f32x4 (&acc)[NMAT],
                                               char* pa = nullptr) {
  using G = RingGeomU8<NMAT, TR, PRE>;
  constexpr int U = ring_depth(RB, G::SLOT_BYTES);
  constexpr int NRK = 32 * NMAT;  // parameter rows: NMAT matrices x (scales, zero points) x 16 rows
  static_assert(U >= 2 && G::CPS * (U - 1) < 64, "ring depth");
  const int lane = lane_id();
  const int n = (k1 - k0) >> 7;
  if constexpr (PRE) {
    // lane l of copy i brings chunk c = 64 i + l: row c % NRK (that row is this lane's
    // sz_src row, since NRK divides 64), piece min(c / NRK, pieces - 1)
    const int pieces = (k1 - k0) >> 9;
#pragma unroll
    for (int i = 0; i < (2 * NRK + 63) / 64; ++i) {
      const int c = 64 * i + lane;
      if (i * 64 < pieces * NRK) copy_to_lds(sz_src + (k0 >> 6) + 8 * min(c / NRK, pieces - 1),
                                             reinterpret_cast<uint16_t*>(pa + 1024 * i));
    }
  }
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
      for (int h = 0; h < TR / 8; ++h)
        copy_to_lds(uniform_ptr(abase + (kc + 64 * half) * 2), aoff[h],
                    reinterpret_cast<uint16_t*>(sl + G::W_BYTES + half * TR * 128 + 8 * h * 128));
    if constexpr (!PRE) copy4_to_lds(sz_src + (kc >> 6), sl + G::W_BYTES + G::A_BYTES);
  };
  const int r = lane & 15, q = lane >> 4;
  auto compute = [&](int slot, int step) {
    const char* sl = ring + slot * G::SLOT_BYTES;
    const uint32_t* szp = reinterpret_cast<const uint32_t*>(sl + G::W_BYTES + G::A_BYTES);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      f32x4 part[NMAT];
      float zf[NMAT], sf[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        part[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (PRE) {
          const int gg = 2 * step + g;  // group within the range
          const uint16_t* pp = reinterpret_cast<const uint16_t*>(pa + 16 * ((gg >> 3) * NRK + m * 32 + r)) + (gg & 7);
          sf[m] = f16_to_f32(pp[0]);
          zf[m] = f16_to_f32(pp[128]);  // zero-point row m * 32 + 16 + r: 16 rows x 16 bytes further
        } else {
          const uint32_t sv = szp[m * 32 + r], zv = szp[m * 32 + 16 + r];
          sf[m] = f16_to_f32(static_cast<uint16_t>(g ? sv >> 16 : sv & 0xffffu));
          zf[m] = f16_to_f32(static_cast<uint16_t>(g ? zv >> 16 : zv & 0xffffu));
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c = ks * 4 + q;  // logical 16-byte chunk of the 64-element token image
        const uint4 av =
            *reinterpret_cast<const uint4*>(sl + G::W_BYTES + g * TR * 128 + (r & (TR - 1)) * 128 + ((c ^ (r & 7)) << 4));
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
    compute(cur, t);
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
template <int NMAT, int TR, bool PRE = false>
struct RingGeomU4 {
  static constexpr int W_BYTES = NMAT * 16 * 64;
  static constexpr int A_BYTES = TR * 256;
  static constexpr int SLOT_BYTES = W_BYTES + A_BYTES + (PRE ? 0 : 256);
  static constexpr int CPS = NMAT + TR / 4 + (PRE ? 0 : 1);  // copy instructions per step
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
// row byte offset plus 16 x logical chunk (l % 16) ^ row).  sz_src, PRE and pa: as for
// the u8 ring.
template <int NMAT, int RB, int TR, bool PRE = false>
__device__ __forceinline__ void ring_stream_u4(const char* const (&wbase)[NMAT], uint32_t woff, const char* abase,
                                               const uint32_t (&aoff)[TR / 4], const uint16_t* sz_src, int k0,
                                               int k1, char* ring, f32x4 (&acc)[NMAT], char* pa = nullptr) {
  using G = RingGeomU4<NMAT, TR, PRE>;
  constexpr int U = RB / G::SLOT_BYTES < 8 ? RB / G::SLOT_BYTES : 8;
  constexpr int NRK = 32 * NMAT;
  static_assert(U >= 2, "ring too small");
  const int lane = lane_id();
  const int n = (k1 - k0) >> 7;
  if constexpr (PRE) {
    const int pieces = (k1 - k0) >> 9;
#pragma unroll
    for (int i = 0; i < (2 * NRK + 63) / 64; ++i) {
      const int c = 64 * i + lane;
      if (i * 64 < pieces * NRK) copy_to_lds(sz_src + (k0 >> 6) + 8 * min(c / NRK, pieces - 1),
                                             reinterpret_cast<uint16_t*>(pa + 1024 * i));
    }
  }
  auto issue = [&](int slot, int step) {
    char* sl = ring + slot * G::SLOT_BYTES;
    const int kc = k0 + 128 * step;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
      copy_to_lds(uniform_ptr(wbase[m] + (kc >> 1)), woff, reinterpret_cast<uint16_t*>(sl + m * 1024));
#pragma unroll
    for (int i = 0; i < TR / 4; ++i)
      copy_to_lds(uniform_ptr(abase + kc * 2), aoff[i], reinterpret_cast<uint16_t*>(sl + G::W_BYTES + i * 1024));
    if constexpr (!PRE) copy4_to_lds(sz_src + (kc >> 6), sl + G::W_BYTES + G::A_BYTES);
  };
  const int r = lane & 15, q = lane >> 4;
  const int tr = r & (TR - 1);
  const uint4 ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
  auto compute = [&](int slot, int step) {
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
        if constexpr (PRE) {
          const int gg = 2 * step + g;
          const uint16_t* pp = reinterpret_cast<const uint16_t*>(pa + 16 * ((gg >> 3) * NRK + m * 32 + r)) + (gg & 7);
          sf[m] = f16_to_f32(pp[0]);
          zf[m] = 128.f + f16_to_f32(pp[128]);
        } else {
          const uint32_t sv = szp[m * 32 + r], zv = szp[m * 32 + 16 + r];
          sf[m] = f16_to_f32(static_cast<uint16_t>(g ? sv >> 16 : sv & 0xffffu));
          zf[m] = 128.f + f16_to_f32(static_cast<uint16_t>(g ? zv >> 16 : zv & 0xffffu));
        }
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
    compute(cur, t);
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

// Whether a u8 ring range [k0, k1) of rows K elements long takes the preloaded group
// parameters (ring_stream_u8 PRE): 8-group pieces that start on 16-byte boundaries
// (K, k0 and k1 multiples of 512, parameter arrays 16-byte aligned), at most 16 groups.
__device__ __forceinline__ bool u8_pre(int k0, int k1, int K, std::initializer_list<const uint16_t*> ps) {
  uintptr_t al = 0;
  for (const uint16_t* p : ps) al |= reinterpret_cast<uintptr_t>(p);
  return ((al & 15) | (K & 511) | (k0 & 511) | (k1 & 511)) == 0 && k1 - k0 <= 1024 && k1 > k0;
}

// quantised routed experts (BITS = 8: u8 ring, 4: u4 ring); shared items stream bf16
// RB: ring bytes per wavefront
// FEPL > 0: the one-token launch that routes its token itself (route_token<FEPL>)
template <int BITS, int RB, int NWK, int FEPL = 0>
__global__ __launch_bounds__(256) void k_stream_up_q(SkinnyUpArgs a) {
  constexpr int IPB = 4 / NWK;
  __shared__ __attribute__((aligned(16))) char rings[4 * RB];
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  char* ring = rings + w * RB;
  const int CH = a.I / 16, CHs = a.Is / 16;
  const int TC = (a.T + 15) / 16;
  const int n_shared = a.part == 1 ? 0 : CHs * TC;
  const int nbound = n_shared + (a.part == 2 ? 0 : a.mtiles * CH);  // routed: up to the chunk bound
  int rr, ch;
  ring_lane(rr, ch);
  const char* xb = uniform_ptr(a.x);
  // one token: this block routes it itself (the launch covers every item in one round)
  RingItem pre{};
  if constexpr (FEPL > 0)
    pre = one_token_item<FEPL>(a, reinterpret_cast<char*>(rings),
                               min(static_cast<int>(blockIdx.x) * IPB + w / NWK, nbound - 1), n_shared, CH);
  const bool sf = a.shared_first || a.part == 2;
  int nlive = FEPL == 0 && !sf ? live_items(a, n_shared, CH) : nbound;
  for (int base = blockIdx.x * IPB; base < nlive; base += gridDim.x * IPB) {
    if (FEPL == 0 && sf && base >= n_shared && nlive == nbound) {
      nlive = live_items(a, n_shared, CH);  // shared-first: loaded once a block reaches the routed items
      if (base >= nlive) break;
    }
    const int item = base + w / NWK;
    const RingItem itm = FEPL > 0 ? pre
                                  : ring_item(min(item, nbound - 1), n_shared, TC, CH, a.T, a.meta, a.chunks, sf, IPB == 1 ? 8 : 1);
    const bool live = item < nbound && itm.live, shared = itm.shared;
    const int e = itm.e, off = itm.off, ntot = itm.ntot, row0 = itm.row0, tc_begin = itm.tc, tc_end = itm.tc + 1;
    int k0 = 0, k1 = a.H;
    if (NWK > 1) {
      if (shared)
        unit_range(a.H, w % NWK, NWK, k0, k1);
      else
        unit_range128(a.H, w % NWK, NWK, k0, k1);
    }
    const int64_t ro = static_cast<int64_t>(e) * a.I + row0;
    for (int tc = tc_begin; tc < tc_end; ++tc) {
      const int ntok = min(16, ntot - tc * 16);
      uint32_t aoff[2];
      token_offsets(a, shared, off, tc * 16, ntok, rr, ch, aoff);
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
            if (u8_pre(k0, k1, a.H, {a.gate_s, a.gate_z, a.up_s, a.up_z})) {
              constexpr int PB = kU8ParamBytes<2>;
              if (ntok <= 8)
                ring_stream_u8<2, RB - PB, 8, true>(wb, woff, xb, aoff, szs, k0, k1, ring, acc, ring + RB - PB);
              else
                ring_stream_u8<2, RB - PB, 16, true>(wb, woff, xb, aoff, szs, k0, k1, ring, acc, ring + RB - PB);
            } else if (ntok <= 8) {
              ring_stream_u8<2, RB, 8>(wb, woff, xb, aoff, szs, k0, k1, ring, acc);
            } else {
              ring_stream_u8<2, RB, 16>(wb, woff, xb, aoff, szs, k0, k1, ring, acc);
            }
          } else {
            const char* wb[2] = {uniform_ptr(static_cast<const uint8_t*>(a.gate) + ro * (a.H / 2)),
                                 uniform_ptr(static_cast<const uint8_t*>(a.up) + ro * (a.H / 2))};
            const uint32_t woff = u4_code_off(a.H / 2);
            const int* prow = a.perm + off + tc * 16;
            with_token_rows(ntok, [&](auto trc) {
              constexpr int TR = decltype(trc)::value;
              uint32_t ao[TR / 4];
              u4_token_offsets<TR>(ntok, [&](int j) { return a.T == 1 ? 0u : static_cast<uint32_t>(prow[j] / a.k) * a.H * 2; }, ao);
              // preloaded parameters where their area leaves at least two slots (at most
              // 8 token rows)
              constexpr int PB = kU8ParamBytes<2>;
              bool done = false;
              if constexpr (TR <= 8) {
                if (u8_pre(k0, k1, a.H, {a.gate_s, a.gate_z, a.up_s, a.up_z})) {
                  ring_stream_u4<2, RB - PB, TR, true>(wb, woff, xb, ao, szs, k0, k1, ring, acc, ring + RB - PB);
                  done = true;
                }
              }
              if (!done) ring_stream_u4<2, RB, TR>(wb, woff, xb, ao, szs, k0, k1, ring, acc);
            });
          }
        } else {
          const char* wb[2] = {uniform_ptr(static_cast<const uint16_t*>(a.sgate) + static_cast<int64_t>(row0) * a.H),
                               uniform_ptr(static_cast<const uint16_t*>(a.sup) + static_cast<int64_t>(row0) * a.H)};
          const uint32_t woff[2] = {static_cast<uint32_t>((rr * a.H + ch * 8) * 2),
                                    static_cast<uint32_t>(((8 + rr) * a.H + ch * 8) * 2)};
          if (ntok <= 8)
            ring_stream<2, RB, 8>(wb, woff, xb, aoff, k0, k1, reinterpret_cast<uint16_t*>(ring), acc);
          else
            ring_stream<2, RB, 16>(wb, woff, xb, aoff, k0, k1, reinterpret_cast<uint16_t*>(ring), acc);
        }
      }
      if constexpr (NWK > 1) {
        float* red = reinterpret_cast<float*>(rings);
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 2; ++m) *reinterpret_cast<f32x4*>(red + ((w * 2 + m) * 64 + lane) * 4) = acc[m];
        __syncthreads();
        if (w % NWK == 0) {  // the first wavefront of each item adds its item's partials
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < NWK; ++p) sum += *reinterpret_cast<const f32x4*>(red + (((w + p) * 2 + m) * 64 + lane) * 4);
            acc[m] = sum;
          }
        }
        __syncthreads();
      }
      if (live && (NWK == 1 || w % NWK == 0)) {
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

// RB: ring bytes per wavefront
template <int BITS, int RB, int NWK>
__global__ __launch_bounds__(256) void k_stream_down_q(SkinnyDownArgs a) {
  constexpr int IPB = 4 / NWK;
  __shared__ __attribute__((aligned(16))) char rings[4 * RB];
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  char* ring = rings + w * RB;
  const int CH = a.H / 16;
  const int TC = (a.T + 15) / 16;
  const int n_shared = a.Is > 0 && a.part != 1 ? CH * TC : 0;
  const int nbound = n_shared + (a.part == 2 ? 0 : a.mtiles * CH);  // routed: up to the chunk bound
  int rr, ch;
  ring_lane(rr, ch);
  const bool sf = a.shared_first || a.part == 2;
  int nlive = sf ? nbound : live_items(a, n_shared, CH);
  for (int base = blockIdx.x * IPB; base < nlive; base += gridDim.x * IPB) {
    if (sf && base >= n_shared && nlive == nbound) {
      nlive = live_items(a, n_shared, CH);  // shared-first: loaded once a block reaches the routed items
      if (base >= nlive) break;
    }
    const int item = base + w / NWK;
    const RingItem itm = ring_item(min(item, nbound - 1), n_shared, TC, CH, a.T, a.meta, a.chunks, sf, IPB == 1 ? 8 : 1);
    const bool live = item < nbound && itm.live, shared = itm.shared;
    const int e = itm.e, off = itm.off, ntot = itm.ntot, row0 = itm.row0, tc_begin = itm.tc, tc_end = itm.tc + 1;
    const int K = shared ? a.Is : a.I;
    int k0 = 0, k1 = K;
    if (NWK > 1) {
      if (shared)
        unit_range(K, w % NWK, NWK, k0, k1);
      else
        unit_range128(K, w % NWK, NWK, k0, k1);
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
      int slot[4];
      float wgt[4];
      if (!shared) routed_slots(a.perm, a.wpos, off + tc * 16, ntok, slot, wgt);
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
            if (u8_pre(k0, k1, a.I, {a.down_s, a.down_z})) {
              constexpr int PB = kU8ParamBytes<1>;
              if (ntok <= 8)
                ring_stream_u8<1, RB - PB, 8, true>(wb, woff, ab, aoff, szs, k0, k1, ring, acc, ring + RB - PB);
              else
                ring_stream_u8<1, RB - PB, 16, true>(wb, woff, ab, aoff, szs, k0, k1, ring, acc, ring + RB - PB);
            } else if (ntok <= 8) {
              ring_stream_u8<1, RB, 8>(wb, woff, ab, aoff, szs, k0, k1, ring, acc);
            } else {
              ring_stream_u8<1, RB, 16>(wb, woff, ab, aoff, szs, k0, k1, ring, acc);
            }
          } else {
            const char* wb[1] = {uniform_ptr(static_cast<const uint8_t*>(a.down) + ro * (a.I / 2))};
            const uint32_t woff = u4_code_off(a.I / 2);
            const int row0t = off + tc * 16;
            with_token_rows(ntok, [&](auto trc) {
              constexpr int TR = decltype(trc)::value;
              uint32_t ao[TR / 4];
              u4_token_offsets<TR>(ntok, [&](int j) { return static_cast<uint32_t>(row0t + j) * a.I * 2; }, ao);
              // preloaded parameters where their area leaves at least two slots (at most
              // 8 token rows)
              constexpr int PB = kU8ParamBytes<1>;
              bool done = false;
              if constexpr (TR <= 8) {
                if (u8_pre(k0, k1, a.I, {a.down_s, a.down_z})) {
                  ring_stream_u4<1, RB - PB, TR, true>(wb, woff, ab, ao, szs, k0, k1, ring, acc, ring + RB - PB);
                  done = true;
                }
              }
              if (!done) ring_stream_u4<1, RB, TR>(wb, woff, ab, ao, szs, k0, k1, ring, acc);
            });
          }
        } else {
          const char* wb[1] = {uniform_ptr(static_cast<const uint16_t*>(a.sdown) + static_cast<int64_t>(row0) * a.Is)};
          const uint32_t woff[2] = {static_cast<uint32_t>((rr * K + ch * 8) * 2),
                                    static_cast<uint32_t>(((8 + rr) * K + ch * 8) * 2)};
          if (ntok <= 8)
            ring_stream<1, RB, 8>(wb, woff, ab, aoff, k0, k1, reinterpret_cast<uint16_t*>(ring), acc);
          else
            ring_stream<1, RB, 16>(wb, woff, ab, aoff, k0, k1, reinterpret_cast<uint16_t*>(ring), acc);
        }
      }
      if constexpr (NWK > 1) {
        float* red = reinterpret_cast<float*>(rings);
        __syncthreads();
        *reinterpret_cast<f32x4*>(red + (w * 64 + lane) * 4) = acc[0];
        __syncthreads();
        if (w % NWK == 0) {  // the first wavefront of each item adds its item's partials
          f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < NWK; ++p) sum += *reinterpret_cast<const f32x4*>(red + ((w + p) * 64 + lane) * 4);
          acc[0] = sum;
        }
        __syncthreads();
      }
      if (live && (NWK == 1 || w % NWK == 0)) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 4 * (lane >> 4) + v;
          if (m < ntok) {
            if (!shared) {
              const float val = wgt[v] * acc[0][v];
              const int64_t o = static_cast<int64_t>(slot[v]) * a.H + row0 + n;
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

// LDS ring bytes per wavefront of the streaming kernels (the K-steps a ring holds follow
// from its slot size, which depends on the token rows a chunk copies: 8 or 16).
// bf16 gate/up: 20 KB (three steps of 16 token rows, four of 8; 80 KB per block, two
// blocks per CU); bf16 down: 16 KB (four steps of 16 token rows, five of 8).
constexpr int kUpRingB = 20480, kDownRingB = 16384;
// u8 gate/up: two blocks per CU split over the four wavefronts (measured 3-6% faster
// than three steps unsplit on the Ling-3.0-flash shape at 1 to 64 tokens); 20 KB: two
// steps of 16 token rows, three of 8.  u8 down: three steps of 16 token rows, four of 8.
constexpr int kUpRingU8B = 20480, kDownRingU8B = 3 * RingGeomU8<1, 16, true>::SLOT_BYTES + kU8ParamBytes<1>;
// u4 (ring depth per the token rows inside ring_stream_u4): gate/up three slots of the
// largest u4 step, the split gate/up two (still 3-5 steps in flight with 4-8 token rows;
// three blocks share a CU, measured 5-7% faster at 8-64 tokens), down two slots
// (measured 3-5% faster than three at 1 to 64 tokens, graph replay at 64 tokens
// 260.8 -> 248.4 us)
constexpr int kUpRingU4B = 3 * kU4MaxSlot, kUpRingSplitU4B = 2 * kU4MaxSlot,
              kDownRingU4B = 2 * RingGeomU4<1, 16>::SLOT_BYTES;

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

// split: the NWKS wavefronts of an item share its K (4 / NWKS items per block); else
// one item per wavefront
template <int U, int NWKS = 4, typename Args>
hipError_t launch_ring(void (*k1)(Args), void (*k4)(Args), int64_t items, bool split, int ncu, hipStream_t s,
                       const Args& a) {
  const int grid = grid_for(items, split ? 4 / NWKS : 4, ncu);
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
// the gate/up launch takes a ring kernel (else a register-staged one)
static bool up_uses_ring(const SkinnyUpArgs& a, Act act, WFmt wf) {
  if (act != Act::BF16) return false;
  if (wf == WFmt::U4) return true;
  if (wf == WFmt::U8)
    return a.H % 128 == 0 && stream_ok(a.T, a.H, 0, 0) && aligned4({a.gate_s, a.gate_z, a.up_s, a.up_z});
  return stream_ok(a.T, a.H, a.T * a.k, a.I);
}

// Ring items of a gate/up launch (one item = 16 weight rows x one chunk of 16 tokens)
// and whether its blocks split K (one item per block).  Gate/up ring kernels split K
// over the four wavefronts of a block at every size (measured faster on the bf16, u8
// and u4 layers from 1 to 64 tokens: finer work units even out the last round), except
// for the dense MLP, whose token chunks of one row block share its rows inside one
// block unsplit: it splits when its items cannot occupy the CUs otherwise, or, with at
// most 4 chunks per row block, when split blocks fill the rounds of resident blocks (two
// per CU) better (unsplit, 64 tokens at intermediate 9216 are 576 blocks, a second round
// of 64; split, 2304 blocks in 4.5 rounds, a row block's chunks on one XCD: place_item).
// Measured on the Ling-2.6 layer-0 shape: 32 tokens 78.3 -> 64.9 us, 64 tokens 100.0 ->
// 95.7 us; split at 128 and 192 tokens (8 and 12 chunks) was slower, 160.8 -> 172.3 us
// and 218.4 -> 229.2 us.  Split decisions are taken from the whole layer's items, never
// from `part`.
static int64_t up_ring_items(const SkinnyUpArgs& a, int ncu, bool& split) {
  const int64_t shared_ring = static_cast<int64_t>(a.Is / 16) * ((a.T + 15) / 16);
  const int64_t routed = static_cast<int64_t>(a.mtiles) * (a.I / 16);
  if (a.dense) {
    const int64_t items = part_items(0, routed, shared_ring), slots = 2ll * ncu;
    // share of the block slots of its rounds that `blocks` blocks fill
    auto fill = [&](int64_t blocks) { return static_cast<double>(blocks) / (((blocks + slots - 1) / slots) * slots); };
    split = items < 4ll * ncu || ((a.T + 15) / 16 <= 4 && fill(items) > fill((items + 3) / 4));
  } else {
    split = true;
  }
  return part_items(a.part, routed, shared_ring);
}

// One-token routing inside the gate/up launch pays the routing chain (partial logits
// loaded, k rounds of arg-max) in every block that streams a routed item, before its
// first copy: it only gains where all blocks are resident at once, so that the chain
// is paid once per CU instead of once per round.  Measured at one token: Ling-3.0-tiny
// (216 blocks) 28.6 -> 26.1 us, Ling-3.0-flash u4 (576 blocks, three per CU) 53.7 ->
// 50.5 us; Ling-lite (704 blocks on 512 slots) no gain, Ling-2.6- and Ling-3.0-flash
// bf16 / u8 (576 blocks, two per CU) 2.6 to 4.3 us slower.  (One token with bf16
// weights now takes the one-token kernel, up_one_fits, before this rule is asked.)
bool skinny_up_can_route(const SkinnyUpArgs& a, Act act, WFmt wf, int ncu) {
  if (a.T != 1 || a.part != 0 || a.dense || a.k > kMaxTopK || a.E > 512 || !up_uses_ring(a, act, wf)) return false;
  bool split;
  const int64_t blocks = up_ring_items(a, ncu, split);
  const int64_t ring_bytes = 4ll * (wf == WFmt::U4 ? kUpRingSplitU4B : wf == WFmt::U8 ? kUpRingU8B : kUpRingB);
  const int64_t per_cu = (160 * 1024) / ring_bytes;  // blocks resident on a CU (LDS)
  return split && blocks <= per_cu * ncu;
}

// k_up_one instances by row loads per lane (H / 512 rounded up: 1, 2, 4, 8) and
// experts per lane of the routing (0: read the permutation; 1, 2, 4, 8)
namespace {
template <int NLH>
void (*up_one_kernel(int fepl))(SkinnyUpArgs) {
  switch (fepl) {
    case 0: return k_up_one<NLH, 0>;
    case 1: return k_up_one<NLH, 1>;
    case 2: return k_up_one<NLH, 2>;
    case 4: return k_up_one<NLH, 4>;
    default: return k_up_one<NLH, 8>;
  }
}
int up_one_nlh(int H) {
  const int n = (H / 8 + 63) / 64;
  return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : n <= 8 ? 8 : 0;
}
}  // namespace

template <int NU>
void (*up_one_q8_kernel(int fepl))(SkinnyUpArgs) {
  switch (fepl) {
    case 0: return k_up_one_q8<NU, 0>;
    case 1: return k_up_one_q8<NU, 1>;
    case 2: return k_up_one_q8<NU, 2>;
    case 4: return k_up_one_q8<NU, 4>;
    default: return k_up_one_q8<NU, 8>;
  }
}

bool up_one_fits(const SkinnyUpArgs& a, Act act, WFmt wf) {
  auto al16 = [](const void* q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  const bool q8 = wf == WFmt::U8;
  // u8: units of 16 elements, the row's groups one per lane (H <= 4096)
  const bool shape = q8 ? a.H % 64 == 0 && a.H <= 4096 && a.gate_s && a.gate_z && a.up_s && a.up_z
                        : a.H % 8 == 0 && up_one_nlh(a.H) > 0;
  return a.T == 1 && a.part == 0 && !a.dense && act == Act::BF16 && (wf == WFmt::BF16 || q8) && shape &&
         a.H > 0 && a.I > 0 && a.k <= kMaxTopK && a.E <= 512 && al16(a.x) && al16(a.gate) && al16(a.up) &&
         (a.Is == 0 || (al16(a.sgate) && al16(a.sup)));
}

// Resident blocks per CU of a one-token gate/up instance on the current device, asked
// of the runtime once per (instance, device) and kept; 1 if the query fails.
static int up_one_blocks_per_cu(void (*k)(SkinnyUpArgs)) {
  struct Entry {
    void (*k)(SkinnyUpArgs);
    int dev, per_cu;
  };
  static std::mutex mu;
  static Entry cache[128];
  static int n = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n; ++i)
      if (cache[i].k == k && cache[i].dev == dev) return cache[i].per_cu;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 64 * kUpOneWaves, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  std::lock_guard<std::mutex> lock(mu);
  if (n < 128) cache[n++] = Entry{k, dev, per_cu};
  return per_cu;
}

static hipError_t launch_up_one(const SkinnyUpArgs& a, WFmt wf, int ncu, hipStream_t s) {
  if (a.fused_route) {
    if (!a.ta.logits || !a.ta.idx || !a.ta.w || a.ta.E != a.E || a.ta.k != a.k || a.ta.T != 1 || !a.pa.perm ||
        !a.pa.slot_pos || !a.pa.wpos || !a.pa.chunks || !a.pa.tiles || !a.pa.active || !a.pa.meta ||
        !a.pa.counts || !a.pa.offsets)
      return hipErrorInvalidValue;
  } else if (!a.perm || !a.idx) {
    return hipErrorInvalidValue;
  }
  if (!a.hm || (a.Is > 0 && !a.hs)) return hipErrorInvalidValue;
  const int epl = (a.E + 63) / 64;
  const int fepl = !a.fused_route ? 0 : epl <= 1 ? 1 : epl <= 2 ? 2 : epl <= 4 ? 4 : 8;
  void (*k)(SkinnyUpArgs) = nullptr;
  if (wf == WFmt::U8) {
    const int nu = (a.H / 16 + 63) / 64;
    k = nu <= 1 ? up_one_q8_kernel<1>(fepl) : nu <= 2 ? up_one_q8_kernel<2>(fepl) : up_one_q8_kernel<4>(fepl);
  } else {
    switch (up_one_nlh(a.H)) {
      case 1: k = up_one_kernel<1>(fepl); break;
      case 2: k = up_one_kernel<2>(fepl); break;
      case 4: k = up_one_kernel<4>(fepl); break;
      default: k = up_one_kernel<8>(fepl); break;
    }
  }
  // every block resident at once (each finds the routing once), at most two per CU
  // (Ling-lite at one token: 20.3 us with two, 20.8 us with three); at least one block
  int per_cu = up_one_blocks_per_cu(k);
  if (per_cu > 2) per_cu = 2;
  const int64_t cols = static_cast<int64_t>(a.Is) + static_cast<int64_t>(a.k) * a.I;
  int64_t grid = static_cast<int64_t>(per_cu) * ncu;
  const int64_t need = (cols + kUpOneWaves - 1) / kUpOneWaves;
  if (grid > need) grid = need;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(grid)), dim3(64 * kUpOneWaves), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_skinny_up(const SkinnyUpArgs& a, Act act, WFmt wf, int ncu, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (up_one_fits(a, act, wf)) return launch_up_one(a, wf, ncu, s);
  // one-token routing inside the launch: only where skinny_up_can_route allows it, with
  // the shared-first order it assumes and every table it stores
  if (a.fused_route &&
      (!skinny_up_can_route(a, act, wf, ncu) || !a.shared_first || !a.ta.logits || !a.ta.idx || !a.ta.w ||
       a.ta.E != a.E || a.ta.k != a.k || !a.pa.perm || !a.pa.slot_pos || !a.pa.wpos || !a.pa.chunks ||
       !a.pa.tiles || !a.pa.active || !a.pa.meta || !a.pa.counts || !a.pa.offsets))
    return hipErrorInvalidValue;
  // routed items read the chunk records, the chunk count and the permutation
  if (a.part != 2 && !a.fused_route && (!a.chunks || !a.meta || !a.perm)) return hipErrorInvalidValue;
  const int64_t slots = static_cast<int64_t>(a.T) * a.k;
  const int64_t dmax = slots < a.E ? slots : a.E;
  const int tch = 16 * pick_mt(a.T);
  const int64_t shared_skinny = static_cast<int64_t>(a.Is / 16) * ((a.T + tch - 1) / tch);
  const int64_t items = part_items(a.part, dmax * (a.I / 16), shared_skinny);
  const int64_t small = 4ll * ncu;
  const bool split_skinny = part_items(0, dmax * (a.I / 16), shared_skinny) < small;
  bool split_ring;
  const int64_t ring = up_ring_items(a, ncu, split_ring);
  if (a.fused_route) {
    // one round of split blocks (skinny_up_can_route); the kernel that routes with
    // route_token<ceil(E / 64)>
    const int epl = (a.E + 63) / 64, grid = static_cast<int>(ring);
    void (*k)(SkinnyUpArgs) = nullptr;
    if (wf == WFmt::U4)
      k = epl <= 1 ? k_stream_up_q<4, kUpRingSplitU4B, 4, 1> : epl <= 2 ? k_stream_up_q<4, kUpRingSplitU4B, 4, 2>
        : epl <= 4 ? k_stream_up_q<4, kUpRingSplitU4B, 4, 4> : k_stream_up_q<4, kUpRingSplitU4B, 4, 8>;
    else if (wf == WFmt::U8)
      k = epl <= 1 ? k_stream_up_q<8, kUpRingU8B, 4, 1> : epl <= 2 ? k_stream_up_q<8, kUpRingU8B, 4, 2>
        : epl <= 4 ? k_stream_up_q<8, kUpRingU8B, 4, 4> : k_stream_up_q<8, kUpRingU8B, 4, 8>;
    else
      k = epl <= 1 ? k_stream_up<kUpRingB, 4, 1> : epl <= 2 ? k_stream_up<kUpRingB, 4, 2>
        : epl <= 4 ? k_stream_up<kUpRingB, 4, 4> : k_stream_up<kUpRingB, 4, 8>;
    if (!split_ring) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (wf == WFmt::U4) {
    // the only u4 kernel: the configuration checks guarantee its conditions
    if (act != Act::BF16 || a.H % 128 || !stream_ok(a.T, a.H, a.T, a.Is) || !aligned4({a.gate_s, a.gate_z, a.up_s, a.up_z}))
      return hipErrorInvalidValue;
    return launch_ring<0>(k_stream_up_q<4, kUpRingU4B, 1>, k_stream_up_q<4, kUpRingSplitU4B, 4>, ring, split_ring,
                          ncu, s, a);
  }
  if (act == Act::F32)
    MOE_DISPATCH_MT_NWK(k_skinny_up, a, items, a.T, split_skinny, Act::F32, WFmt::F32);
  else if (wf == WFmt::U8 && a.H % 128 == 0 && stream_ok(a.T, a.H, 0, 0) &&
           aligned4({a.gate_s, a.gate_z, a.up_s, a.up_z}))
    return launch_ring<0>(k_stream_up_q<8, kUpRingU8B, 1>, k_stream_up_q<8, kUpRingU8B, 4>, ring, split_ring, ncu,
                          s, a);
  else if (wf == WFmt::U8)
    MOE_DISPATCH_MT_NWK(k_skinny_up, a, items, a.T, split_skinny, Act::BF16, WFmt::U8);
  else if (stream_ok(a.T, a.H, a.T * a.k, a.I))
    return launch_ring<0>(k_stream_up<kUpRingB, 1>, k_stream_up<kUpRingB, 4>, ring, split_ring, ncu, s, a);
  else
    MOE_DISPATCH_MT_NWK(k_skinny_up, a, items, a.T, split_skinny, Act::BF16, WFmt::BF16);
  return hipGetLastError();
}

hipError_t launch_skinny_down(const SkinnyDownArgs& a, Act act, WFmt wf, int ncu, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  // routed items also store through the permutation with the weights by position
  if (a.part != 2 && (!a.chunks || !a.meta || !a.perm || !a.wpos)) return hipErrorInvalidValue;
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
    return launch_ring<0>(k_stream_down_q<4, kDownRingU4B, 1>, k_stream_down_q<4, kDownRingU4B, 4>, ring,
                          split_ring, ncu, s, a);
  }
  if (act == Act::F32)
    MOE_DISPATCH_MT_NWK(k_skinny_down, a, items, a.T, split_skinny, Act::F32, WFmt::F32);
  else if (wf == WFmt::U8 && a.I % 128 == 0 && stream_ok(a.T * a.k, a.I, a.T, a.Is) &&
           aligned4({a.down_s, a.down_z}))
    return launch_ring<0>(k_stream_down_q<8, kDownRingU8B, 1>, k_stream_down_q<8, kDownRingU8B, 4>, ring,
                          split_ring, ncu, s, a);
  else if (wf == WFmt::U8)
    MOE_DISPATCH_MT_NWK(k_skinny_down, a, items, a.T, split_skinny, Act::BF16, WFmt::U8);
  else if (stream_ok(a.T * a.k, a.I, a.T, a.Is))
    // split items share K between two wavefronts (two items per block): measured against
    // four on Ling-lite at 1 token (down 14.4 -> 13.7 us), the only split bf16 down of
    // the measured shapes
    return launch_ring<0, 2>(k_stream_down<kDownRingB, 1>, k_stream_down<kDownRingB, 2>, ring, split_ring, ncu, s, a);
  else
    MOE_DISPATCH_MT_NWK(k_skinny_down, a, items, a.T, split_skinny, Act::BF16, WFmt::BF16);
  return hipGetLastError();
}

// instances of k_down_one: (NLS, NLR, K, code bits: 0 for bf16), smallest first per K and
// format
namespace {
struct DownOneShape {
  int nls, nlr, k, qb;
  void (*fn)(SkinnyDownArgs);
};
const DownOneShape kDownOne[] = {
    {1, 1, 8, 0, k_down_one<1, 1, 8, 0>},
    {2, 2, 8, 0, k_down_one<2, 2, 8, 0>},
    {6, 3, 6, 0, k_down_one<6, 3, 6, 0>},
    {1, 1, 8, 8, k_down_one<1, 1, 8, 8>},
    {2, 1, 8, 8, k_down_one<2, 1, 8, 8>},
    {1, 1, 8, 4, k_down_one<1, 1, 8, 4>},
    {2, 1, 8, 4, k_down_one<2, 1, 8, 4>},
};
int down_one_qb(WFmt wf) { return wf == WFmt::U8 ? 8 : wf == WFmt::U4 ? 4 : 0; }
const DownOneShape* down_one_shape(const SkinnyDownArgs& a, WFmt wf) {
  const int qb = down_one_qb(wf);
  const int nls = (a.Is / 8 + 63) / 64, nlr = (a.I / (qb ? 16 : 8) + 63) / 64;
  for (const DownOneShape& d : kDownOne)
    if (d.qb == qb && d.k == a.k && nls <= d.nls && nlr <= d.nlr) return &d;
  return nullptr;
}
}  // namespace

bool down_one_fits(const SkinnyDownArgs& a, Act act, WFmt wf) {
  auto al16 = [](const void* q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  const bool q = wf == WFmt::U8 || wf == WFmt::U4;
  return a.T == 1 && a.part == 0 && act == Act::BF16 && (wf == WFmt::BF16 || q) && a.I % (q ? 64 : 8) == 0 &&
         a.Is % 8 == 0 && a.I > 0 && a.Is > 0 && a.H > 0 && al16(a.down) && al16(a.sdown) && al16(a.hm) &&
         al16(a.hs) && (!q || (a.down_s && a.down_z)) && down_one_shape(a, wf) != nullptr;
}

hipError_t launch_down_one(const SkinnyDownArgs& a, Act act, WFmt wf, hipStream_t s) {
  if (!down_one_fits(a, act, wf)) return hipErrorInvalidValue;
  if (!a.perm || !a.idx || !a.wpos || !a.y || !a.hm || !a.down || (a.Is > 0 && (!a.hs || !a.sdown)))
    return hipErrorInvalidValue;
  const int grid = (a.H + kDownOneWaves - 1) / kDownOneWaves;
  hipLaunchKernelGGL(down_one_shape(a, wf)->fn, dim3(grid), dim3(64 * kDownOneWaves), 0, s, a);
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
