// Router top-k (one wavefront per token) and token permutation by expert (LDS
// histograms, exclusive scans, scatter; one workgroup for small batches, a
// histogram pass and a scan-and-scatter pass over 2048-slot chunks otherwise).
//
// Routing semantics follow the model pages: scores are softmax over all experts or
// an elementwise sigmoid of the logits; the correction bias is added to a copy of
// the scores used for selection only; with grouping, each contiguous group is scored
// by the sum of its two largest biased scores, the topk_group best groups are kept
// and the other experts' selection scores are set to zero; the top_k experts by
// selection score are taken, their weights gathered from the unbiased scores,
// renormalised by (sum + 1e-20) when top_k > 1 and norm_topk_prob, and multiplied by
// routed_scaling_factor [mlxcel #838 "Router: selection uses biased scores, weights
// come from unbiased scores", "Architecture notes", "moe_router_enable_routed_scaling
// is dead code upstream"; Ling-2.6-flash-JANGTQ card, MoE routing paragraph].
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// Expert e lives in lane e / EPL, register e % EPL: each lane owns EPL consecutive
// experts, so a row of logits is read with contiguous per-lane runs.
// Routes token t with one wavefront (all 64 lanes active).
// (lds_idx, lds_w: optional copies of the token's k expert indices and weights in LDS,
// at [t * k + j])
template <int EPL>
__device__ void route_token(const TopkArgs& a, int t, int* lds_idx = nullptr, float* lds_w = nullptr) {
  const int lane = lane_id();
  const int E = a.E;

  float s[EPL], sel[EPL];
  bool valid[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    valid[i] = lane * EPL + i < E;
    s[i] = 0.f;
  }
  // both biases and the P partial logits are loaded together (one memory round trip
  // for P <= 8: a token's routing is a chain of dependent steps)
  float rb[EPL], eb[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    rb[i] = (valid[i] && a.router_bias) ? a.router_bias[lane * EPL + i] : 0.f;
    eb[i] = (valid[i] && a.use_ebias) ? a.expert_bias[lane * EPL + i] : 0.f;
  }
  const float* row = a.logits + static_cast<int64_t>(t) * E + lane * EPL;
  if (EPL % 4 == 0 && (E % 4) == 0 && lane * EPL + EPL <= E) {
    for (int q0 = 0; q0 < a.P; q0 += 8) {
      float4 v[8][EPL / 4 > 0 ? EPL / 4 : 1];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int c = 0; c < EPL / 4; ++c)
          v[u][c] = q0 + u < a.P ? *reinterpret_cast<const float4*>(row + (q0 + u) * a.part_stride + 4 * c)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int c = 0; c < EPL / 4; ++c) {
          s[4 * c] += v[u][c].x;
          s[4 * c + 1] += v[u][c].y;
          s[4 * c + 2] += v[u][c].z;
          s[4 * c + 3] += v[u][c].w;
        }
    }
  } else {
    for (int q0 = 0; q0 < a.P; q0 += 8) {
      float v[8][EPL];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < EPL; ++i) v[u][i] = (valid[i] && q0 + u < a.P) ? row[(q0 + u) * a.part_stride + i] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < EPL; ++i) s[i] += v[u][i];
    }
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) s[i] += rb[i];

  // scores
  if (a.score_sigmoid) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) s[i] = valid[i] ? 1.0f / (1.0f + expf(-s[i])) : 0.f;
  } else {
    float m = kNegInf;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (valid[i]) m = fmaxf(m, s[i]);
    m = wave_max(m);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      s[i] = valid[i] ? expf(s[i] - m) : 0.f;
      sum += s[i];
    }
    sum = wave_sum(sum);
#pragma unroll
    for (int i = 0; i < EPL; ++i) s[i] = s[i] / sum;
  }

  // selection copy (correction bias for selection only)
#pragma unroll
  for (int i = 0; i < EPL; ++i) sel[i] = valid[i] ? s[i] + eb[i] : kNegInf;

  // grouped mask: keep the g groups with the largest top-2 sums, zero the rest
  if (a.G > 1 && a.g < a.G) {
    const int gs = E / a.G;
    const int lpg = gs / EPL;  // lanes per group when a group spans whole lanes
    if (gs % EPL == 0 && (lpg == 1 || lpg == 2 || lpg == 4 || lpg == 8 || lpg == 16) && a.G * lpg <= kWave) {
      // each group is lpg consecutive lanes: top-2 per lane, then a butterfly inside the
      // group on the DPP network (xor 1, xor 2 within quads; the half-row and row
      // mirrors pair the 4- and 8-lane halves once those are uniform)
      float t1 = kNegInf, t2 = kNegInf;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const float x = valid[i] ? sel[i] : kNegInf;
        if (x > t1) {
          t2 = t1;
          t1 = x;
        } else if (x > t2) {
          t2 = x;
        }
      }
      auto merge = [&](float o1, float o2) {
        const float hi = fmaxf(t1, o1);
        t2 = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
        t1 = hi;
      };
      if (lpg >= 2) merge(dpp_f<kDppQuadXor1>(t1, t1), dpp_f<kDppQuadXor1>(t2, t2));
      if (lpg >= 4) merge(dpp_f<kDppQuadXor2>(t1, t1), dpp_f<kDppQuadXor2>(t2, t2));
      if (lpg >= 8) merge(dpp_f<kDppRowHalfMirror>(t1, t1), dpp_f<kDppRowHalfMirror>(t2, t2));
      if (lpg >= 16) merge(dpp_f<kDppRowMirror>(t1, t1), dpp_f<kDppRowMirror>(t2, t2));
      const float mine = t1 + t2;
      // rank of this lane's group among all groups (larger first, ties -> lower group)
      const int gme = lane / lpg;
      int rank = 0;
      for (int gr = 0; gr < a.G; ++gr) {
        const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), gr * lpg));
        rank += (o > mine || (o == mine && gr < gme)) ? 1 : 0;
      }
      if (rank >= a.g) {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (valid[i]) sel[i] = 0.0f;
      }
    } else {
      int grp[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) grp[i] = valid[i] ? (lane * EPL + i) / gs : -1;
      float sig_mine = kNegInf;
      for (int gr = 0; gr < a.G; ++gr) {
        float t1 = kNegInf, t2 = kNegInf;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          if (grp[i] == gr) {
            const float x = sel[i];
            if (x > t1) {
              t2 = t1;
              t1 = x;
            } else if (x > t2) {
              t2 = x;
            }
          }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const float o1 = __shfl_xor(t1, o, kWave), o2 = __shfl_xor(t2, o, kWave);
          const float hi = fmaxf(t1, o1);
          const float lo = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
          t1 = hi;
          t2 = lo;
        }
        if (lane == gr) sig_mine = t1 + t2;
      }
      int rank = 0;
      for (int gr = 0; gr < a.G; ++gr) {
        const float o = __shfl(sig_mine, gr, kWave);
        rank += (o > sig_mine || (o == sig_mine && gr < lane)) ? 1 : 0;
      }
      const unsigned long long kept = __ballot(lane < a.G && rank < a.g);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (grp[i] >= 0 && !((kept >> grp[i]) & 1ull)) sel[i] = 0.0f;
    }
  }

  // top-k: k rounds of wave arg-max, larger score first, equal scores -> lower index
  uint32_t taken = 0;
  int my_idx = 0x7fffffff;
  float my_w = 0.f;
  for (int j = 0; j < a.k; ++j) {
    float bv = kNegInf, bo = 0.f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (valid[i] && !((taken >> i) & 1u) && sel[i] > bv) {
        bv = sel[i];
        bi = lane * EPL + i;
        bo = s[i];
      }
    }
    const int own = bi;
    wave_argmax(bv, bi);
    // the unbiased score of the winner, from the lane that holds it
    const float wo = bi != 0x7fffffff ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bo), bi / EPL)) : 0.f;
    if (bi != 0x7fffffff && own == bi) taken |= 1u << (bi - lane * EPL);
    if (lane == j) {
      my_idx = bi;
      my_w = wo;
    }
  }

  const float tot = wave_sum(lane < a.k ? my_w : 0.f);
  if (a.k > 1 && a.norm) my_w = my_w / (tot + 1e-20f);
  my_w *= a.rsf;
  if (lane < a.k) {
    a.idx[static_cast<int64_t>(t) * a.k + lane] = my_idx;
    a.w[static_cast<int64_t>(t) * a.k + lane] = my_w;
    if (lds_idx) lds_idx[t * a.k + lane] = my_idx;
    if (lds_w) lds_w[t * a.k + lane] = my_w;
  }
}

template <int EPL>
__global__ __launch_bounds__(256) void k_topk(TopkArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;  // whole wavefront leaves; no block barrier here
  route_token<EPL>(a, t);
}

constexpr int kPermThreads = 1024;
constexpr int kPermUnroll = 4;

// Exclusive scans over the experts of: counts c[e], small-expert flags (1..small_max
// slots: handled by the streaming kernels), M-tiles of the larger experts and their
// chunks of BM2 positions.  Fills off[e] (LDS) with each expert's first position; when
// `write` is set, also stores counts, offsets, the small-expert list, both tile maps
// and meta.
// Called by all kPermThreads threads with c = this thread's expert count (0 past E).
__device__ void scan_experts(const PermuteArgs& a, int c, bool write, int* off, int (*wtot)[16], int* total_s) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int E = a.E;
  const int f = (c > 0 && c <= a.small_max) ? 1 : 0;
  const int nt = (a.BM > 0 && c > a.tile_min) ? (c + a.BM - 1) / a.BM : 0;
  const int nt2 = (a.BM2 > 0 && c > a.tile_min) ? (c + a.BM2 - 1) / a.BM2 : 0;
  int ci = c, fi = f, ti = nt, t2 = nt2;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(ci, o, kWave), y = __shfl_up(fi, o, kWave), z = __shfl_up(ti, o, kWave),
              u = __shfl_up(t2, o, kWave);
    if (lane >= o) {
      ci += x;
      fi += y;
      ti += z;
      t2 += u;
    }
  }
  if (lane == 63) {
    wtot[0][wv] = ci;
    wtot[1][wv] = fi;
    wtot[2][wv] = ti;
    wtot[3][wv] = t2;
  }
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int v = lane < 16 ? wtot[q][lane] : 0;
      int inc = v;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const int x = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += x;
      }
      if (lane < 16) wtot[q][lane] = inc - v;
    }
  }
  __syncthreads();
  const int ce = ci - c + wtot[0][wv];
  const int fe = fi - f + wtot[1][wv];
  const int te = ti - nt + wtot[2][wv];
  const int te2 = t2 - nt2 + wtot[3][wv];
  if (tid < E) {
    off[tid] = ce;
    if (write) {
      a.counts[tid] = c;
      a.offsets[tid] = ce;
      if (a.counts_copy) a.counts_copy[tid] = c;
      if (f) a.active[fe] = tid;
      for (int q = 0; q < nt; ++q) {
        a.tiles[2 * (te + q)] = tid;
        a.tiles[2 * (te + q) + 1] = ce + q * a.BM;
        if (a.chunks) a.chunks[te + q] = make_int4(tid, ce + q * a.BM, ce, c);
      }
      for (int q = 0; q < nt2; ++q) {
        a.tiles2[2 * (te2 + q)] = tid;
        a.tiles2[2 * (te2 + q) + 1] = ce + q * a.BM2;
      }
    }
  }
  if (tid == E - 1) {
    if (write) {
      a.offsets[E] = ce + c;
      a.meta[0] = fe + f;
      a.meta[1] = te + nt;
      a.meta[2] = ce + c;
      a.meta[3] = te2 + nt2;
    }
    *total_s = ce + c;
  }
  __syncthreads();
}

// Rank of each slot of [s0, s1) among the slots of its expert in that range (LDS
// atomics; the order inside an expert is not fixed), counts into cnt.
__device__ void rank_slots(const PermuteArgs& a, int s0, int s1, int* cnt) {
  const int tid = threadIdx.x;
  for (int base = s0; base < s1; base += kPermThreads * kPermUnroll) {
    int e[kPermUnroll];
#pragma unroll
    for (int u = 0; u < kPermUnroll; ++u) {
      const int s = base + u * kPermThreads + tid;
      e[u] = s < s1 ? a.idx[s] : -1;
    }
#pragma unroll
    for (int u = 0; u < kPermUnroll; ++u) {
      const int s = base + u * kPermThreads + tid;
      if (s < s1) {
        int p = -1;
        if (e[u] >= 0 && e[u] < a.E) p = atomicAdd(&cnt[e[u]], 1);
        a.slot_pos[s] = p;
      }
    }
  }
}

// Scatter slot ids of [s0, s1) to position base[e] + rank.
__device__ void scatter_slots(const PermuteArgs& a, int s0, int s1, const int* base) {
  const int tid = threadIdx.x;
  for (int b = s0; b < s1; b += kPermThreads * kPermUnroll) {
    int p[kPermUnroll], e[kPermUnroll];
#pragma unroll
    for (int u = 0; u < kPermUnroll; ++u) {
      const int s = b + u * kPermThreads + tid;
      p[u] = s < s1 ? a.slot_pos[s] : -1;
      e[u] = s < s1 ? a.idx[s] : -1;
    }
#pragma unroll
    for (int u = 0; u < kPermUnroll; ++u) {
      const int s = b + u * kPermThreads + tid;
      if (p[u] >= 0) {
        const int pos = base[e[u]] + p[u];
        a.perm[pos] = s;
        a.slot_pos[s] = pos;
        if (a.wpos) a.wpos[pos] = a.w[s];
      }
    }
  }
}

// One workgroup: histogram, scans, scatter (small slot counts).
__global__ __launch_bounds__(kPermThreads) void k_permute(PermuteArgs a) {
  __shared__ int cnt[1024];
  __shared__ int off[1024];
  __shared__ int wtot[4][16];
  __shared__ int total_s;
  const int tid = threadIdx.x;
  if (tid < a.E) cnt[tid] = 0;
  __syncthreads();
  rank_slots(a, 0, a.nslots, cnt);
  __syncthreads();
  scan_experts(a, tid < a.E ? cnt[tid] : 0, true, off, wtot, &total_s);
  scatter_slots(a, 0, a.nslots, off);
  for (int q = total_s + tid; q < a.nslots; q += kPermThreads) a.perm[q] = -1;
}

// Small batches: 16 wavefronts route the tokens, then the same workgroup permutes
// them (one launch instead of two on the decode critical path).
template <int EPL>
__global__ __launch_bounds__(kPermThreads) void k_route_permute(TopkArgs ta, PermuteArgs a) {
  // a.nslots <= kFusedSlots <= kPermThreads: thread s owns slot s, whose expert and
  // rank stay in registers (no round trip through global memory between the phases)
  __shared__ int cnt[1024];
  __shared__ int off[1024];
  __shared__ int wtot[4][16];
  __shared__ int total_s;
  __shared__ int s_idx[kFusedSlots];
  __shared__ float s_w[kFusedSlots];
  const int tid = threadIdx.x;
  for (int t = tid >> 6; t < ta.T; t += kPermThreads / 64) route_token<EPL>(ta, t, s_idx, s_w);
  if (tid < a.E) cnt[tid] = 0;
  __syncthreads();
  int e = -1, rank = -1;
  if (tid < a.nslots) {
    e = s_idx[tid];
    if (e >= 0 && e < a.E) rank = atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  scan_experts(a, tid < a.E ? cnt[tid] : 0, true, off, wtot, &total_s);
  if (rank >= 0) {
    const int pos = off[e] + rank;
    a.perm[pos] = tid;
    a.slot_pos[tid] = pos;
    if (a.wpos) a.wpos[pos] = s_w[tid];
  } else if (tid < a.nslots) {
    a.slot_pos[tid] = -1;
  }
  for (int q = total_s + tid; q < a.nslots; q += kPermThreads) a.perm[q] = -1;
}

// Multi-block form, pass 1: per-chunk histogram and in-chunk ranks.
__global__ __launch_bounds__(kPermThreads) void k_perm_count(PermuteArgs a) {
  __shared__ int cnt[1024];
  const int tid = threadIdx.x;
  if (tid < a.E) cnt[tid] = 0;
  __syncthreads();
  const int s0 = blockIdx.x * kPermChunk, s1 = min(a.nslots, s0 + kPermChunk);
  rank_slots(a, s0, s1, cnt);
  __syncthreads();
  if (tid < a.E) a.hist[static_cast<int64_t>(blockIdx.x) * a.E + tid] = cnt[tid];
}

// Pass 2: every block recomputes the expert totals and scans (block 0 publishes
// them), adds the counts of earlier chunks, and scatters its own chunk.
__global__ __launch_bounds__(kPermThreads) void k_perm_scatter(PermuteArgs a) {
  __shared__ int off[1024];
  __shared__ int wtot[4][16];
  __shared__ int total_s;
  const int tid = threadIdx.x;
  const int nb = gridDim.x, b = blockIdx.x;
  int tot = 0, pre = 0;
  if (tid < a.E) {
    for (int q = 0; q < nb; ++q) {
      const int h = a.hist[static_cast<int64_t>(q) * a.E + tid];
      tot += h;
      pre += q < b ? h : 0;
    }
  }
  scan_experts(a, tot, b == 0, off, wtot, &total_s);
  if (tid < a.E) off[tid] += pre;
  __syncthreads();
  const int s0 = b * kPermChunk, s1 = min(a.nslots, s0 + kPermChunk);
  scatter_slots(a, s0, s1, off);
  for (int q = max(s0, total_s) + tid; q < s1; q += kPermThreads) a.perm[q] = -1;
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const dim3 grid((a.T + 3) / 4), block(256);
  const int epl = (a.E + 63) / 64;
  if (epl <= 1)
    hipLaunchKernelGGL(k_topk<1>, grid, block, 0, s, a);
  else if (epl <= 2)
    hipLaunchKernelGGL(k_topk<2>, grid, block, 0, s, a);
  else if (epl <= 4)
    hipLaunchKernelGGL(k_topk<4>, grid, block, 0, s, a);
  else if (epl <= 8)
    hipLaunchKernelGGL(k_topk<8>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(k_topk<16>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_route_permute(const TopkArgs& t, const PermuteArgs& a, hipStream_t s) {
  if (a.nslots > kFusedSlots || a.E > kPermThreads) return hipErrorInvalidValue;
  const int epl = (t.E + 63) / 64;
  const dim3 g(1), b(kPermThreads);
  if (epl <= 1)
    hipLaunchKernelGGL(k_route_permute<1>, g, b, 0, s, t, a);
  else if (epl <= 2)
    hipLaunchKernelGGL(k_route_permute<2>, g, b, 0, s, t, a);
  else if (epl <= 4)
    hipLaunchKernelGGL(k_route_permute<4>, g, b, 0, s, t, a);
  else if (epl <= 8)
    hipLaunchKernelGGL(k_route_permute<8>, g, b, 0, s, t, a);
  else
    hipLaunchKernelGGL(k_route_permute<16>, g, b, 0, s, t, a);
  return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  if (a.nslots <= kPermSingleMax || a.hist == nullptr) {
    hipLaunchKernelGGL(k_permute, dim3(1), dim3(kPermThreads), 0, s, a);
    return hipGetLastError();
  }
  const int nb = (a.nslots + kPermChunk - 1) / kPermChunk;
  hipLaunchKernelGGL(k_perm_count, dim3(nb), dim3(kPermThreads), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_perm_scatter, dim3(nb), dim3(kPermThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
