// Router top-k (one wavefront per token) and token permutation by expert (LDS
// histograms, exclusive scans, scatter; one workgroup for small batches, a
// histogram pass and a scan-and-scatter pass over 2048-slot chunks otherwise).
// (routing semantics: route_token.h)
#include "common.h"
#include "kernels.h"
#include "route_token.h"

namespace moe {

namespace {

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

// One token: one wavefront routes it and stores every table of the permutation (the
// same tables k_route_permute builds, without its histogram, scans and block barriers).
template <int EPL>
__global__ __launch_bounds__(64) void k_route_one(TopkArgs ta, PermuteArgs a) {
  __shared__ int s_slot_e[kMaxTopK], s_pos_e[kMaxTopK], s_kv;
  __shared__ float s_w[kMaxTopK];
  route_token<EPL>(ta, 0, s_slot_e, s_w);
  one_token_tables(a, ta.k, ta.E, s_slot_e, s_w, s_pos_e, &s_kv, true);
  __syncthreads();  // one wavefront: orders the LDS writes above before the reads below
  one_token_counts(a, ta.E, s_pos_e, s_kv, threadIdx.x, 64);
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
  if (t.T == 1 && t.k <= kMaxTopK && a.wpos && a.chunks && !a.BM2) {
    // one token (the decode tables: chunk records and weights by position)
    const dim3 g1(1), b1(64);
    if (epl <= 1)
      hipLaunchKernelGGL(k_route_one<1>, g1, b1, 0, s, t, a);
    else if (epl <= 2)
      hipLaunchKernelGGL(k_route_one<2>, g1, b1, 0, s, t, a);
    else if (epl <= 4)
      hipLaunchKernelGGL(k_route_one<4>, g1, b1, 0, s, t, a);
    else if (epl <= 8)
      hipLaunchKernelGGL(k_route_one<8>, g1, b1, 0, s, t, a);
    else
      hipLaunchKernelGGL(k_route_one<16>, g1, b1, 0, s, t, a);
    return hipGetLastError();
  }
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
