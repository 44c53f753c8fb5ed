// Routing of one token by one wavefront, shared by the top-k kernels and the one-token
// gate/up launch.
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
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// Expert e lives in lane e / EPL, register e % EPL: each lane owns EPL consecutive
// experts, so a row of logits is read with contiguous per-lane runs.
// Routes token t with one wavefront (all 64 lanes active).
// (lds_idx, lds_w: optional copies of the token's k expert indices and weights in LDS,
// at [t * k + j]; store = false leaves a.idx and a.w alone; MAXF: partial logits a lane
// loads per batch, fewer registers for more round trips)
template <int EPL, int MAXF = 64>
__device__ void route_token(const TopkArgs& a, int t, int* lds_idx = nullptr, float* lds_w = nullptr, bool store = true) {
  const int lane = lane_id();
  const int E = a.E;

  float s[EPL], sel[EPL];
  bool valid[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    valid[i] = lane * EPL + i < E;
    s[i] = 0.f;
  }
  // both biases and the P partial logits are loaded together, PB partials per batch:
  // one memory round trip (a token's routing is a chain of dependent steps; the router's
  // split keeps P * EPL <= 64, so with MAXF = 64 one batch of PB = 64 / EPL, at most 16,
  // covers it)
  float rb[EPL], eb[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    rb[i] = (valid[i] && a.router_bias) ? a.router_bias[lane * EPL + i] : 0.f;
    eb[i] = (valid[i] && a.use_ebias) ? a.expert_bias[lane * EPL + i] : 0.f;
  }
  const float* row = a.logits + static_cast<int64_t>(t) * E + lane * EPL;
  constexpr int PB = EPL >= 4 ? MAXF / EPL : 16;
  if (EPL % 4 == 0 && (E % 4) == 0 && lane * EPL + EPL <= E) {
    for (int q0 = 0; q0 < a.P; q0 += PB) {
      float4 v[PB][EPL / 4 > 0 ? EPL / 4 : 1];
#pragma unroll
      for (int u = 0; u < PB; ++u)
#pragma unroll
        for (int c = 0; c < EPL / 4; ++c)
          v[u][c] = q0 + u < a.P ? *reinterpret_cast<const float4*>(row + (q0 + u) * a.part_stride + 4 * c)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < PB; ++u)
#pragma unroll
        for (int c = 0; c < EPL / 4; ++c) {
          s[4 * c] += v[u][c].x;
          s[4 * c + 1] += v[u][c].y;
          s[4 * c + 2] += v[u][c].z;
          s[4 * c + 3] += v[u][c].w;
        }
    }
  } else {
    for (int q0 = 0; q0 < a.P; q0 += PB) {
      float v[PB][EPL];
#pragma unroll
      for (int u = 0; u < PB; ++u)
#pragma unroll
        for (int i = 0; i < EPL; ++i) v[u][i] = (valid[i] && q0 + u < a.P) ? row[(q0 + u) * a.part_stride + i] : 0.f;
#pragma unroll
      for (int u = 0; u < PB; ++u)
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
    wave_argmax_lane_ordered(bv, bi);  // lane l holds experts l * EPL .. l * EPL + EPL - 1
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
    if (store) {
      a.idx[static_cast<int64_t>(t) * a.k + lane] = my_idx;
      a.w[static_cast<int64_t>(t) * a.k + lane] = my_w;
    }
    if (lds_idx) lds_idx[t * a.k + lane] = my_idx;
    if (lds_w) lds_w[t * a.k + lane] = my_w;
  }
}

// The tables of a single token's routing, by one wavefront (all 64 lanes).  Its k picks
// (expert of slot j in s_slot_e[j], weight in s_w[j], as route_token leaves them) are
// distinct experts; each valid one is ranked by expert index: position p holds the
// p-th smallest, one chunk each, which is what the permutation kernels build for one
// token.  Leaves the experts by position in s_pos_e and the valid count in *s_kv; with
// `publish`, stores perm, slot_pos, wpos, chunks, tiles, active and meta (the per-expert
// counts and offsets: one_token_counts).
__device__ __forceinline__ void one_token_tables(const PermuteArgs& pa, int k, int E, const int* s_slot_e,
                                                 const float* s_w, int* s_pos_e, int* s_kv, bool publish) {
  // the picks were written to LDS by other lanes of this wavefront: keep the reads after
  // those writes (LDS serves one wavefront's accesses in order)
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const int lane = lane_id();
  const int e = lane < k ? s_slot_e[lane] : -1;
  const bool valid = lane < k && e >= 0 && e < E;
  int rank = 0;
  for (int i = 0; i < k; ++i) {
    const int ei = s_slot_e[i];
    rank += (ei >= 0 && ei < E && ei < e) ? 1 : 0;
  }
  const int kv = __popcll(__ballot(valid));
  if (valid) s_pos_e[rank] = e;
  if (lane == 0) *s_kv = kv;
  if (publish && lane < k) {
    if (valid) {
      pa.perm[rank] = lane;
      pa.slot_pos[lane] = rank;
      pa.wpos[rank] = s_w[lane];
      pa.chunks[rank] = make_int4(e, rank, rank, 1);
      pa.tiles[2 * rank] = e;
      pa.tiles[2 * rank + 1] = rank;
      pa.active[rank] = e;
    } else {
      pa.slot_pos[lane] = -1;
    }
    if (lane >= kv) pa.perm[lane] = -1;
  }
  if (publish && lane == 0) {
    pa.meta[0] = kv;  // active experts
    pa.meta[1] = kv;  // chunks
    pa.meta[2] = kv;  // valid slots
    pa.meta[3] = 0;
    pa.offsets[E] = kv;
  }
}

// counts[e] and offsets[e] (experts before e's first position) of a single token's
// routing, over threads tid = t0, t0 + nthr, ... (the experts by position and their
// count from one_token_tables, visible to these threads)
__device__ __forceinline__ void one_token_counts(const PermuteArgs& pa, int E, const int* s_pos_e, int kv, int t0,
                                                 int nthr) {
  for (int e = t0; e < E; e += nthr) {
    int c = 0, before = 0;
    for (int p = 0; p < kv; ++p) {
      const int pe = s_pos_e[p];
      c += pe == e ? 1 : 0;
      before += pe < e ? 1 : 0;
    }
    pa.counts[e] = c;
    pa.offsets[e] = before;
    if (pa.counts_copy) pa.counts_copy[e] = c;
  }
}

}  // namespace
}  // namespace moe
