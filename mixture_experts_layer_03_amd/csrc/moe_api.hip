// Host side of the C ABI declared in include/moe.h: configuration checks, workspace
// layout, and the launch sequence of the layer's kernels on the caller's stream.
//
// Checks follow the pages' defensive rules [mlxcel #838 "Defensive requirements"]:
// magnitude ceilings on every architecture scalar before it is used, zero checks
// before divisibility checks, routing bounds (1 <= top_k <= experts; with groups,
// experts divisible by n_group and 1 <= topk_group <= n_group), sizes taken from
// the caller's real arguments, and no exception or abort ever crossing the ABI.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "moe.h"
#include "kernels.h"

using namespace moe;

// Fixed device scratch of moe_forward_noalloc (its address: noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512];

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

moe_status ok() {
  g_err[0] = 0;
  return MOE_OK;
}

constexpr int64_t kMaxH = 16384, kMaxE = 1024, kMaxI = 32768, kMaxT = int64_t(1) << 20, kMaxK = kMaxTopK;
constexpr int64_t kMaxGroupsGpu = 64;
constexpr int kDecodeMaxT = 64;
// The automatic path also streams (decode) while a batch averages at most
// min(20, 40960 / hidden) routed tokens per expert: T * top_k * max(hidden, 2048)
// <= 40960 * num_experts, i.e. 20 at hidden 2048 (and below) and 10 at hidden 4096.  There the
// tiled GEMMs' 128-row M-tiles are mostly padding and read the selected experts'
// weights at ~2 TB/s, while the streaming kernels read them at 5-6 TB/s.  Measured on
// the MI355X, the streaming path stays faster up to about 20 tokens per expert on the
// Ling-lite and Ling-3.0-tiny shapes (hidden 2048; T ~ 210 and ~ 320), 10-11 on the
// Ling-2.6-flash and Ling-3.0-flash shapes (hidden 4096; T ~ 330 and ~ 700) and 14 on
// the u8 Ling-3.0-flash shape; e.g. Ling-3.0-flash at 256 tokens: 0.92 ms streamed
// against 1.70 ms tiled.
constexpr int64_t kDecodeTokensTimesHidden = 40960, kDecodeHiddenFloor = 2048;
// The dense MLP streams up to this many tokens.  Measured on the MI355X at the
// Ling-2.6-flash layer-0 shape (H 4096, I 9216): streaming 99.5 / 149.6 / 163.4 /
// 219.6 / 284.5 us at 64 / 96 / 128 / 192 / 256 tokens against 243-261 us tiled (one
// or two 128-row M-tiles leave most CUs idle).
constexpr int kDenseDecodeMaxT = 192;
constexpr int kFusedRouteMaxT = 16;  // one workgroup routes and permutes up to this many tokens
// Streaming work order: the shared expert's items first up to this many tokens (one
// token chunk per item: their routing loads are a visible part of every short item),
// the routed items first above it (the uniform shared items then even out the last
// round).  Measured on the Ling shapes: 1 and 8 tokens faster shared-first (Ling-lite
// at 1 token 47.2 -> 43.7 us with the single-load chunk records), 64 tokens faster
// routed-first for gate/up.
constexpr int64_t kSharedFirstMaxT = 16;
constexpr int kGroupAuto = 0;  // dense tiled GEMMs: the launch picks the M-tiles per block-order group
// Routed GEMMs keep the launch order of their blocks (TileArgs::plain_order) when the
// experts average at most this many routed tokens (1.5 M-tiles of 128).
constexpr int64_t kPlainOrderMaxSlotsPerExpert = 192;

bool is_flag(int32_t v) { return v == 0 || v == 1; }

moe_status check_config(const moe_config* c) {
  if (!c) return fail(MOE_EINVAL_ARG, "cfg is null");
  // magnitudes first
  if (c->hidden < 1 || c->hidden > kMaxH) return fail(MOE_EINVAL_CONFIG, "hidden=%lld outside [1, %lld]", (long long)c->hidden, (long long)kMaxH);
  if (c->num_experts < 1 || c->num_experts > kMaxE)
    return fail(MOE_EINVAL_CONFIG, "num_experts=%lld outside [1, %lld]", (long long)c->num_experts, (long long)kMaxE);
  if (c->moe_intermediate < 1 || c->moe_intermediate > kMaxI)
    return fail(MOE_EINVAL_CONFIG, "moe_intermediate=%lld outside [1, %lld]", (long long)c->moe_intermediate, (long long)kMaxI);
  if (c->shared_intermediate < 0 || c->shared_intermediate > kMaxI)
    return fail(MOE_EINVAL_CONFIG, "shared_intermediate=%lld outside [0, %lld]", (long long)c->shared_intermediate, (long long)kMaxI);
  if (c->top_k < 1 || c->top_k > kMaxK || c->top_k > c->num_experts)
    return fail(MOE_EINVAL_CONFIG, "top_k=%lld outside [1, min(num_experts, %lld)]", (long long)c->top_k, (long long)kMaxK);
  // grouping: zero checks before divisibility
  if (c->n_group < 1 || c->n_group > c->num_experts)
    return fail(MOE_EINVAL_CONFIG, "n_group=%lld outside [1, num_experts]", (long long)c->n_group);
  if (c->topk_group < 1 || c->topk_group > c->n_group)
    return fail(MOE_EINVAL_CONFIG, "topk_group=%lld outside [1, n_group=%lld]", (long long)c->topk_group, (long long)c->n_group);
  if (c->n_group > 1) {
    if (c->num_experts % c->n_group != 0)
      return fail(MOE_EINVAL_CONFIG, "num_experts=%lld not divisible by n_group=%lld", (long long)c->num_experts, (long long)c->n_group);
    const int64_t gs = c->num_experts / c->n_group;
    if (gs < 2) return fail(MOE_EINVAL_CONFIG, "n_group=%lld leaves groups of %lld expert(s); a group score needs two", (long long)c->n_group, (long long)gs);
    if (c->top_k > c->topk_group * gs)
      return fail(MOE_EINVAL_CONFIG, "top_k=%lld exceeds the %lld experts of the kept groups", (long long)c->top_k, (long long)(c->topk_group * gs));
  }
  if (c->score_function != MOE_SCORE_SOFTMAX && c->score_function != MOE_SCORE_SIGMOID)
    return fail(MOE_EINVAL_CONFIG, "score_function=%d is neither softmax (0) nor sigmoid (1)", c->score_function);
  if (!std::isfinite(c->routed_scaling_factor) || !(c->routed_scaling_factor > 0.f))
    return fail(MOE_EINVAL_CONFIG, "routed_scaling_factor must be finite and > 0");
  if (!is_flag(c->norm_topk_prob)) return fail(MOE_EINVAL_CONFIG, "norm_topk_prob must be 0 or 1");
  if (!is_flag(c->use_expert_bias)) return fail(MOE_EINVAL_CONFIG, "use_expert_bias must be 0 or 1");
  if (c->act_dtype != MOE_DT_F32 && c->act_dtype != MOE_DT_BF16)
    return fail(MOE_EINVAL_CONFIG, "act_dtype=%d must be F32 or BF16", c->act_dtype);
  if (c->router_dtype != c->act_dtype) return fail(MOE_EINVAL_CONFIG, "router_dtype must equal act_dtype");
  if (c->shared_dtype != c->act_dtype) return fail(MOE_EINVAL_CONFIG, "shared_dtype must equal act_dtype");
  const bool quantised = c->expert_dtype == MOE_DT_U8_AFFINE || c->expert_dtype == MOE_DT_U4_AFFINE;
  if (c->expert_dtype != c->act_dtype && !(quantised && c->act_dtype == MOE_DT_BF16))
    return fail(MOE_EINVAL_CONFIG, "expert_dtype=%d must equal act_dtype or be U8_AFFINE/U4_AFFINE with BF16 activations", c->expert_dtype);
  if (quantised && c->quant_group != 64)
    return fail(MOE_EINVAL_CONFIG, "quant_group=%lld must be 64 for quantised experts", (long long)c->quant_group);
  if (c->path < MOE_PATH_AUTO || c->path > MOE_PATH_PREFILL) return fail(MOE_EINVAL_CONFIG, "path=%d unknown", c->path);
  // valid, but outside what the gfx950 kernels implement
  if (c->hidden % 64 || c->moe_intermediate % 64 || c->shared_intermediate % 64)
    return fail(MOE_EUNSUPPORTED, "hidden, moe_intermediate and shared_intermediate must be multiples of 64");
  if (c->n_group > kMaxGroupsGpu) return fail(MOE_EUNSUPPORTED, "n_group=%lld > %lld", (long long)c->n_group, (long long)kMaxGroupsGpu);
  if (c->expert_dtype == MOE_DT_U4_AFFINE && (c->hidden % 128 || c->moe_intermediate % 128))
    return fail(MOE_EUNSUPPORTED, "u4 experts need hidden and moe_intermediate multiples of 128");
  if (c->expert_dtype == MOE_DT_U4_AFFINE && c->path == MOE_PATH_PREFILL)
    return fail(MOE_EUNSUPPORTED, "u4 experts run the weight-streaming path only (path must be AUTO or DECODE)");
  if (c->path == MOE_PATH_PREFILL && c->act_dtype == MOE_DT_F32)
    return fail(MOE_EUNSUPPORTED, "the tiled MFMA path needs BF16 activations");
  return MOE_OK;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

WFmt expert_fmt(const moe_config& c, Act act) {
  if (c.expert_dtype == MOE_DT_U8_AFFINE) return WFmt::U8;
  if (c.expert_dtype == MOE_DT_U4_AFFINE) return WFmt::U4;
  return act == Act::F32 ? WFmt::F32 : WFmt::BF16;
}

struct Plan {
  bool decode;
  int P;
  int mtiles_bound;
  int mtiles2_bound;  // prefill: chunks of 256 positions (last N-tile of a half-full gate/up)
  size_t o_logits, o_idx, o_w, o_counts, o_offsets, o_perm, o_slotpos, o_active, o_meta, o_tiles, o_tiles2, o_hist,
      o_chunks, o_wpos, o_hm, o_hs, o_r, o_rs, total;
};

int router_parts(const moe_config& c) {
  const int rc = static_cast<int>((c.num_experts + 15) / 16);
  int p = 256 / rc;
  const int cap = static_cast<int>(c.hidden / 256) < 16 ? static_cast<int>(c.hidden / 256) : 16;
  if (p > cap) p = cap;
  if (p < 1) p = 1;
  return p;
}

// K-split of the tiled router GEMM: enough blocks to fill the chip when E is small.
int router_ksplit(const moe_config& c, int64_t T) {
  const int64_t mtiles = (T + kTileM - 1) / kTileM;
  const int64_t ntiles = (c.num_experts + 127) / 128;
  int64_t ks = (512 + mtiles * ntiles - 1) / (mtiles * ntiles);
  const int64_t cap = c.hidden / 256 < 8 ? c.hidden / 256 : 8;
  if (ks > cap) ks = cap;
  if (ks < 1) ks = 1;
  return static_cast<int>(ks);
}

void make_plan(const moe_config& c, int64_t T, Plan& p) {
  p.decode = c.path == MOE_PATH_DECODE || c.expert_dtype == MOE_DT_U4_AFFINE ||
             (c.path == MOE_PATH_AUTO && (T <= kDecodeMaxT || c.act_dtype == MOE_DT_F32 ||
                                          T * c.top_k * std::max(c.hidden, kDecodeHiddenFloor) <=
                                              kDecodeTokensTimesHidden * c.num_experts));
  const int64_t H = c.hidden, E = c.num_experts, k = c.top_k, I = c.moe_intermediate, Is = c.shared_intermediate;
  const size_t ab = c.act_dtype == MOE_DT_F32 ? 4 : 2;
  const int64_t slots = T * k;
  p.P = p.decode ? router_parts(c) : router_ksplit(c, T);
  const int64_t dmax = slots < E ? slots : E;
  const int64_t bm = p.decode ? kDecodeChunk : kTileM;
  p.mtiles_bound = static_cast<int>((slots + dmax * (bm - 1)) / bm);
  p.mtiles2_bound = p.decode ? 0 : static_cast<int>((slots + dmax * 255) / 256);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  p.o_logits = take(size_t(p.P) * T * E * 4);
  p.o_idx = take(slots * 4);
  p.o_w = take(slots * 4);
  p.o_counts = take(E * 4);
  p.o_offsets = take((E + 1) * 4);
  p.o_perm = take(slots * 4);
  p.o_slotpos = take(slots * 4);
  p.o_active = take(E * 4);
  p.o_meta = take(64);
  p.o_tiles = take(size_t(p.mtiles_bound) * 8);
  p.o_tiles2 = take(size_t(p.mtiles2_bound) * 8);
  p.o_hist = take(slots > kPermSingleMax ? size_t((slots + kPermChunk - 1) / kPermChunk) * E * 4 : 0);
  p.o_chunks = take(p.decode ? size_t(p.mtiles_bound) * 16 : 0);
  p.o_wpos = take(p.decode ? slots * 4 : 0);
  p.o_hm = take(slots * I * ab);
  p.o_hs = take(T * Is * ab);
  p.o_r = take(slots * H * (p.decode ? 4 : 2));
  p.o_rs = take(p.decode && Is > 0 ? T * H * 4 : 0);
  p.total = o;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// A second stream of this host thread on the current device (default priority,
// non-blocking) and two events, used to run the shared expert, which needs no routing,
// beside the router and the routed experts.  Created on first use outside stream
// capture; returns null when unavailable (the caller then runs everything in order).
struct AuxStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool ok = false;
};
AuxStream* aux_stream(hipStream_t user) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  thread_local AuxStream tab[64];
  AuxStream& a = tab[dev];
  if (!a.ok) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(user, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    if (!a.s && hipStreamCreateWithFlags(&a.s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (!a.fork && hipEventCreateWithFlags(&a.fork, hipEventDisableTiming) != hipSuccess) return nullptr;
    if (!a.join && hipEventCreateWithFlags(&a.join, hipEventDisableTiming) != hipSuccess) return nullptr;
    a.ok = true;
  }
  return &a;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------- kernel timing
struct ProfPair {
  hipEvent_t start, stop;
  int32_t stage;
};
struct Profiler {
  int32_t mask = 0;
  int32_t capacity = 0;
  int32_t used = 0;
  ProfPair* pool = nullptr;
};
Profiler g_prof;

struct ProfScope {
  ProfPair* pair = nullptr;
  hipStream_t stream;
  ProfScope(int32_t stage, hipStream_t s) : stream(s) {
    if ((g_prof.mask & stage) && g_prof.used < g_prof.capacity) {
      pair = &g_prof.pool[g_prof.used++];
      pair->stage = stage;
      if (hipEventRecord(pair->start, s) != hipSuccess) pair = nullptr;
    }
  }
  ~ProfScope() {
    if (pair) (void)hipEventRecord(pair->stop, stream);
  }
};

#define MOE_LAUNCH_STAGE(stage, stream, expr, what)    \
  do {                                                 \
    hipError_t e_;                                     \
    {                                                  \
      ProfScope ps_((stage), (stream));                \
      e_ = (expr);                                     \
    }                                                  \
    if (e_ != hipSuccess) return hip_fail(e_, what);   \
  } while (0)

moe_status check_T(int64_t T) {
  if (T < 0 || T > kMaxT) return fail(MOE_EINVAL_ARG, "T=%lld outside [0, %lld]", (long long)T, (long long)kMaxT);
  return MOE_OK;
}

moe_status check_ws(const moe_config& c, int64_t T, void* ws, size_t ws_bytes, Plan& p) {
  make_plan(c, T, p);
  if (!p.decode) {
    // the tiled kernels address activation rows with 32-bit byte offsets
    int64_t kmax = c.hidden > c.moe_intermediate ? c.hidden : c.moe_intermediate;
    if (c.shared_intermediate > kmax) kmax = c.shared_intermediate;
    if (T * c.top_k * kmax * 2 >= (int64_t(1) << 32))
      return fail(MOE_EUNSUPPORTED, "T * top_k * max(hidden, intermediate) * 2 bytes >= 2^32 on the tiled path; split the batch");
  }
  if (c.expert_dtype == MOE_DT_U4_AFFINE &&
      (T * c.hidden * 2 >= (int64_t(1) << 31) || T * c.top_k * c.moe_intermediate * 2 >= (int64_t(1) << 31) ||
       T * c.shared_intermediate * 2 >= (int64_t(1) << 31)))
    return fail(MOE_EUNSUPPORTED, "u4 experts: T too large for one call (activations above 2 GB); split the batch");
  if (ws_bytes < p.total) return fail(MOE_EWORKSPACE, "workspace of %zu bytes < %zu required", ws_bytes, p.total);
  if (p.total > 0 && (!ws || !aligned(ws, 256))) return fail(MOE_EWORKSPACE, "workspace must be non-null and 256-byte aligned");
  return MOE_OK;
}

#define REQUIRE_PTR(ptr, align, name)                                                           \
  do {                                                                                          \
    if (!(ptr)) return fail(MOE_EINVAL_ARG, "%s is null", name);                                \
    if (!aligned((ptr), (align))) return fail(MOE_EINVAL_ARG, "%s is not %d-byte aligned", name, (int)(align)); \
  } while (0)

TopkArgs topk_args(const moe_config& c, const Plan& p, int64_t T, void* ws, const float* router_bias,
                   const float* expert_bias, int32_t* idx, float* w);

// router logits (partials) into the workspace
moe_status run_logits(const moe_config& c, const Plan& p, int64_t T, const void* x, const void* router_w,
                      void* ws, hipStream_t s) {
  const Act act = c.act_dtype == MOE_DT_F32 ? Act::F32 : Act::BF16;
  float* logits = at<float>(ws, p.o_logits);
  if (p.decode) {
    SkinnyRouterArgs r{x, router_w, logits, static_cast<int>(T), static_cast<int>(c.hidden),
                       static_cast<int>(c.num_experts), p.P};
    MOE_LAUNCH_STAGE(MOE_STAGE_ROUTER, s, launch_skinny_router(r, act, device_cus(), s), "router logits");
  } else {
    TileArgs g{};
    g.A = static_cast<const uint16_t*>(x);
    g.K = static_cast<int>(c.hidden);
    g.B0 = router_w;
    g.b_expert_stride = 0;
    g.N = static_cast<int>(c.num_experts);
    g.routed = 0;
    g.M = static_cast<int>(T);
    g.out = logits;
    g.ldo = static_cast<int>(c.num_experts);
    g.mtiles_bound = static_cast<int>((T + kTileM - 1) / kTileM);
  g.group_m = kGroupAuto;
    g.ncu = device_cus();
    g.ksplit = p.P;
    g.part_stride = T * c.num_experts;
    MOE_LAUNCH_STAGE(MOE_STAGE_ROUTER, s, launch_tile_gemm(g, AMode::DENSE, WFmt::BF16, Epi::F32, s), "router logits (tiled)");
  }
  return MOE_OK;
}

// router: logits + top-k into (idx, w)
moe_status run_route(const moe_config& c, const Plan& p, int64_t T, const void* x, const void* router_w,
                     const float* router_bias, const float* expert_bias, int32_t* idx, float* w, void* ws,
                     hipStream_t s) {
  const moe_status st = run_logits(c, p, T, x, router_w, ws, s);
  if (st != MOE_OK) return st;
  TopkArgs t = topk_args(c, p, T, ws, router_bias, expert_bias, idx, w);
  MOE_LAUNCH_STAGE(MOE_STAGE_TOPK, s, launch_topk(t, s), "top-k");
  return MOE_OK;
}

TopkArgs topk_args(const moe_config& c, const Plan& p, int64_t T, void* ws, const float* router_bias,
                   const float* expert_bias, int32_t* idx, float* w) {
  float* logits = at<float>(ws, p.o_logits);
  TopkArgs t{};
  t.logits = logits;
  t.part_stride = T * c.num_experts;
  t.P = p.P;
  t.T = static_cast<int>(T);
  t.E = static_cast<int>(c.num_experts);
  t.k = static_cast<int>(c.top_k);
  t.G = static_cast<int>(c.n_group);
  t.g = static_cast<int>(c.topk_group);
  t.score_sigmoid = c.score_function == MOE_SCORE_SIGMOID;
  t.norm = c.norm_topk_prob;
  t.use_ebias = c.use_expert_bias;
  t.rsf = c.routed_scaling_factor;
  t.router_bias = router_bias;
  t.expert_bias = expert_bias;
  t.idx = idx;
  t.w = w;
  return t;
}

// w: the routing weights when the experts follow (decode also stores them by position), else null
PermuteArgs permute_args(const moe_config& c, const Plan& p, int64_t T, const int32_t* idx, const float* w,
                         int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* counts_copy, void* ws) {
  PermuteArgs a{};
  a.idx = idx;
  a.nslots = static_cast<int>(T * c.top_k);
  a.E = static_cast<int>(c.num_experts);
  // decode: every active expert is in the active list (register-staged kernels) and
  // cut into chunks of kDecodeChunk positions (ring kernels: one work item per chunk,
  // so a popular expert's chunks run side by side instead of one after another);
  // tiled path: every active expert gets M-tiles.  (Sending experts with few tokens to
  // the streaming kernels on the tiled path measured slower on the skewed workload:
  // inside one tiled launch their memory-bound blocks overlap the large experts'
  // MFMA-bound blocks.)
  a.BM = p.decode ? kDecodeChunk : kTileM;
  a.small_max = p.decode ? 0x7fffffff : 0;
  a.tile_min = 0;
  a.counts = counts;
  a.offsets = offsets;
  a.perm = perm;
  a.slot_pos = at<int32_t>(ws, p.o_slotpos);
  a.active = at<int32_t>(ws, p.o_active);
  a.tiles = at<int32_t>(ws, p.o_tiles);
  a.BM2 = p.mtiles2_bound > 0 ? 256 : 0;
  a.tiles2 = p.mtiles2_bound > 0 ? at<int32_t>(ws, p.o_tiles2) : nullptr;
  a.meta = at<int32_t>(ws, p.o_meta);
  a.counts_copy = counts_copy;
  a.hist = p.o_hist && T * c.top_k > kPermSingleMax ? at<int32_t>(ws, p.o_hist) : nullptr;
  a.chunks = p.decode ? at<int4>(ws, p.o_chunks) : nullptr;
  a.w = w;
  a.wpos = p.decode && w ? at<float>(ws, p.o_wpos) : nullptr;
  return a;
}

moe_status run_permute(const moe_config& c, const Plan& p, int64_t T, const int32_t* idx, const float* w, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* counts_copy, void* ws, hipStream_t s) {
  const PermuteArgs a = permute_args(c, p, T, idx, w, counts, offsets, perm, counts_copy, ws);
  MOE_LAUNCH_STAGE(MOE_STAGE_PERMUTE, s, launch_permute(a, s), "permutation");
  return MOE_OK;
}

// shared_join: the shared expert's first stages (decode: gate/up and down; prefill:
// gate/up) were launched on another stream that records this event when done; the
// routed stages here skip them and the stream waits for the event before using them.
// route_ta / route_pa (decode, small batches): the routing and permutation are still to
// be done, in one workgroup launch, or for one token inside the gate/up launch when
// skinny_up_can_route allows it (no launch of its own).
moe_status run_experts(const moe_config& c, const Plan& p, int64_t T, const void* x, const moe_weights* w,
                       const int32_t* idx, const float* topk_w, void* y, void* ws, hipStream_t s,
                       bool permuted = false, hipEvent_t shared_join = nullptr, const TopkArgs* route_ta = nullptr,
                       const PermuteArgs* route_pa = nullptr) {
  const Act act = c.act_dtype == MOE_DT_F32 ? Act::F32 : Act::BF16;
  const WFmt wf = expert_fmt(c, act);
  const int Ti = static_cast<int>(T), H = static_cast<int>(c.hidden), I = static_cast<int>(c.moe_intermediate),
            Is = static_cast<int>(c.shared_intermediate), k = static_cast<int>(c.top_k), E = static_cast<int>(c.num_experts);
  int32_t* counts = at<int32_t>(ws, p.o_counts);
  int32_t* offsets = at<int32_t>(ws, p.o_offsets);
  int32_t* perm = at<int32_t>(ws, p.o_perm);
  const int32_t* active = at<int32_t>(ws, p.o_active);
  const int32_t* meta = at<int32_t>(ws, p.o_meta);
  const int32_t* tiles = at<int32_t>(ws, p.o_tiles);
  void* hm = at<void>(ws, p.o_hm);
  void* hs = at<void>(ws, p.o_hs);
  void* r = at<void>(ws, p.o_r);
  float* rs = at<float>(ws, p.o_rs);
  if (!permuted) {
    const moe_status st = run_permute(c, p, T, idx, topk_w, counts, offsets, perm, nullptr, ws, s);
    if (st != MOE_OK) return st;
  }
  const int ncu = device_cus();
  if (route_ta && !p.decode)
    MOE_LAUNCH_STAGE(MOE_STAGE_TOPK, s, launch_route_permute(*route_ta, *route_pa, s), "top-k + permutation");
  if (p.decode) {
    SkinnyUpArgs u{};
    u.x = x;
    u.gate = w->gate;
    u.up = w->up;
    u.gate_s = w->gate_scale;
    u.gate_z = w->gate_zero;
    u.up_s = w->up_scale;
    u.up_z = w->up_zero;
    u.sgate = w->shared_gate;
    u.sup = w->shared_up;
    u.hm = hm;
    u.hs = hs;
    u.counts = counts;
    u.offsets = offsets;
    u.perm = perm;
    u.active = active;
    u.meta = meta;
    u.tiles = tiles;
    u.chunks = at<int4>(ws, p.o_chunks);
    u.mtiles = p.mtiles_bound;
    u.T = Ti;
    u.H = H;
    u.I = I;
    u.Is = Is;
    u.k = k;
    u.E = E;
    u.part = shared_join ? 1 : 0;
    u.shared_first = T <= kSharedFirstMaxT;
    u.idx = idx;
    if (route_ta) {
      if (up_one_fits(u, act, wf) || skinny_up_can_route(u, act, wf, ncu)) {
        u.fused_route = 1;
        u.ta = *route_ta;
        u.pa = *route_pa;
      } else {
        MOE_LAUNCH_STAGE(MOE_STAGE_TOPK, s, launch_route_permute(*route_ta, *route_pa, s), "top-k + permutation");
      }
    }
    MOE_LAUNCH_STAGE(MOE_STAGE_UP, s, launch_skinny_up(u, act, wf, ncu, s), "expert gate/up (streaming)");
    SkinnyDownArgs d{};
    d.hm = hm;
    d.hs = hs;
    d.down = w->down;
    d.down_s = w->down_scale;
    d.down_z = w->down_zero;
    d.sdown = w->shared_down;
    d.topk_w = topk_w;
    d.r = r;
    d.rs = rs;
    d.r_bf16 = 0;
    d.counts = counts;
    d.offsets = offsets;
    d.perm = perm;
    d.active = active;
    d.meta = meta;
    d.tiles = tiles;
    d.chunks = u.chunks;
    d.wpos = at<float>(ws, p.o_wpos);
    d.mtiles = p.mtiles_bound;
    d.T = Ti;
    d.H = H;
    d.I = I;
    d.Is = Is;
    d.k = k;
    d.E = E;
    d.part = shared_join ? 1 : 0;
    d.shared_first = T <= kSharedFirstMaxT;
    d.idx = idx;
    d.y = y;
    if (down_one_fits(d, act, wf)) {
      // one token: the down launch also forms the weighted sum (no combine launch)
      MOE_LAUNCH_STAGE(MOE_STAGE_DOWN, s, launch_down_one(d, act, wf, s), "expert down + combine (one token)");
      return MOE_OK;
    }
    MOE_LAUNCH_STAGE(MOE_STAGE_DOWN, s, launch_skinny_down(d, act, wf, ncu, s), "expert down (streaming)");
    if (shared_join) {
      const hipError_t e = hipStreamWaitEvent(s, shared_join, 0);
      if (e != hipSuccess) return hip_fail(e, "join of the shared expert");
    }
    CombineArgs cb{r, Is > 0 ? rs : nullptr, idx, y, Ti, H, k, E, 0};
    MOE_LAUNCH_STAGE(MOE_STAGE_COMBINE, s, launch_combine(cb, act, s), "combine");
    return MOE_OK;
  }
  // tiled MFMA path (bf16 activations)
  const int64_t slots = T * c.top_k;
  const int64_t dmax = slots < E ? slots : E;
  TileArgs g{};
  g.A = static_cast<const uint16_t*>(x);
  g.K = H;
  g.B0 = w->gate;
  g.B1 = w->up;
  g.B0s = w->gate_scale;
  g.B0z = w->gate_zero;
  g.B1s = w->up_scale;
  g.B1z = w->up_zero;
  g.b_expert_stride = static_cast<int64_t>(I) * H;
  g.N = I;
  g.routed = 1;
  g.tiles = at<int32_t>(ws, p.o_tiles);
  g.meta = meta;
  g.offsets = offsets;
  g.perm = perm;
  g.k = k;
  g.out = hm;
  g.ldo = I;
  g.mtiles_bound = p.mtiles_bound;
  g.tiles2 = p.mtiles2_bound > 0 ? at<int32_t>(ws, p.o_tiles2) : nullptr;
  g.mtiles2_bound = p.mtiles2_bound;
  g.group_m = 0;  // blocks grouped by expert
  g.plain_order = T * c.top_k <= kPlainOrderMaxSlotsPerExpert * c.num_experts;
  g.ncu = device_cus();
  MOE_LAUNCH_STAGE(MOE_STAGE_UP, s, launch_tile_gemm(g, AMode::GATHER, wf, Epi::SWIGLU, s), "expert gate/up (tiled)");
  TileArgs d{};
  d.A = static_cast<const uint16_t*>(hm);
  d.K = I;
  d.B0 = w->down;
  d.B0s = w->down_scale;
  d.B0z = w->down_zero;
  d.b_expert_stride = static_cast<int64_t>(H) * I;
  d.N = H;
  d.routed = 1;
  d.tiles = g.tiles;
  d.meta = meta;
  d.offsets = offsets;
  d.perm = perm;
  d.k = k;
  d.out = r;
  d.ldo = H;
  d.topk_w = topk_w;
  d.mtiles_bound = p.mtiles_bound;
  d.group_m = 0;
  d.plain_order = g.plain_order;
  d.ncu = g.ncu;
  MOE_LAUNCH_STAGE(MOE_STAGE_DOWN, s, launch_tile_gemm(d, AMode::DENSE, wf, Epi::SCALED_SLOT, s), "expert down (tiled)");
  (void)dmax;
  if (Is > 0) {
    if (shared_join) {
      const hipError_t e = hipStreamWaitEvent(s, shared_join, 0);
      if (e != hipSuccess) return hip_fail(e, "join of the shared expert");
    }
    TileArgs su{};
    su.A = static_cast<const uint16_t*>(x);
    su.K = H;
    su.B0 = w->shared_gate;
    su.B1 = w->shared_up;
    su.N = Is;
    su.routed = 0;
    su.M = Ti;
    su.out = hs;
    su.ldo = Is;
    su.mtiles_bound = static_cast<int>((T + kTileM - 1) / kTileM);
  su.group_m = kGroupAuto;
    su.ncu = device_cus();
    if (!shared_join)
      MOE_LAUNCH_STAGE(MOE_STAGE_SHARED_UP, s, launch_tile_gemm(su, AMode::DENSE, WFmt::BF16, Epi::SWIGLU, s), "shared gate/up (tiled)");
    TileArgs sd{};
    sd.A = static_cast<const uint16_t*>(hs);
    sd.K = Is;
    sd.B0 = w->shared_down;
    sd.N = H;
    sd.routed = 0;
    sd.M = Ti;
    sd.out = y;
    sd.ldo = H;
    sd.r = static_cast<const uint16_t*>(r);
    sd.idx = idx;
    sd.k = k;
    sd.E = E;
    sd.mtiles_bound = su.mtiles_bound;
  sd.group_m = kGroupAuto;
    sd.ncu = su.ncu;
    MOE_LAUNCH_STAGE(MOE_STAGE_SHARED_DOWN, s, launch_tile_gemm(sd, AMode::DENSE, WFmt::BF16, Epi::COMBINE, s), "shared down + combine (tiled)");
  } else {
    CombineArgs cb{r, nullptr, idx, y, Ti, H, k, E, 1};
    MOE_LAUNCH_STAGE(MOE_STAGE_COMBINE, s, launch_combine(cb, act, s), "combine");
  }
  return MOE_OK;
}

// The shared expert's stages that need no routing, on stream s: decode gate/up and
// down (into hs and rs), prefill gate/up (into hs).
moe_status run_shared(const moe_config& c, const Plan& p, int64_t T, const void* x, const moe_weights* w, void* ws,
                      hipStream_t s) {
  const Act act = c.act_dtype == MOE_DT_F32 ? Act::F32 : Act::BF16;
  const WFmt wf = expert_fmt(c, act);
  const int Ti = static_cast<int>(T), H = static_cast<int>(c.hidden), I = static_cast<int>(c.moe_intermediate),
            Is = static_cast<int>(c.shared_intermediate), k = static_cast<int>(c.top_k), E = static_cast<int>(c.num_experts);
  void* hs = at<void>(ws, p.o_hs);
  const int ncu = device_cus();
  if (p.decode) {
    SkinnyUpArgs u{};
    u.x = x;
    u.sgate = w->shared_gate;
    u.sup = w->shared_up;
    u.hs = hs;
    u.T = Ti;
    u.H = H;
    u.I = I;
    u.Is = Is;
    u.k = k;
    u.E = E;
    u.mtiles = p.mtiles_bound;  // the whole layer's counts decide the K split
    u.part = 2;
    MOE_LAUNCH_STAGE(MOE_STAGE_SHARED_UP, s, launch_skinny_up(u, act, wf, ncu, s), "shared gate/up (streaming)");
    SkinnyDownArgs d{};
    d.hs = hs;
    d.sdown = w->shared_down;
    d.rs = at<float>(ws, p.o_rs);
    d.T = Ti;
    d.H = H;
    d.I = I;
    d.Is = Is;
    d.k = k;
    d.E = E;
    d.mtiles = p.mtiles_bound;
    d.part = 2;
    MOE_LAUNCH_STAGE(MOE_STAGE_SHARED_DOWN, s, launch_skinny_down(d, act, wf, ncu, s), "shared down (streaming)");
    return MOE_OK;
  }
  TileArgs su{};
  su.A = static_cast<const uint16_t*>(x);
  su.K = H;
  su.B0 = w->shared_gate;
  su.B1 = w->shared_up;
  su.N = Is;
  su.routed = 0;
  su.M = Ti;
  su.out = hs;
  su.ldo = Is;
  su.mtiles_bound = static_cast<int>((T + kTileM - 1) / kTileM);
  su.group_m = kGroupAuto;
  su.ncu = ncu;
  MOE_LAUNCH_STAGE(MOE_STAGE_SHARED_UP, s, launch_tile_gemm(su, AMode::DENSE, WFmt::BF16, Epi::SWIGLU, s), "shared gate/up (tiled)");
  return MOE_OK;
}

moe_status check_weights(const moe_config& c, const moe_weights* w, bool need_router) {
  if (!w) return fail(MOE_EINVAL_ARG, "weights is null");
  if (need_router) REQUIRE_PTR(w->router, 16, "weights.router");
  if (w->router_bias && !aligned(w->router_bias, 4)) return fail(MOE_EINVAL_ARG, "weights.router_bias is not 4-byte aligned");
  if (need_router && c.use_expert_bias) REQUIRE_PTR(w->expert_bias, 4, "weights.expert_bias");
  REQUIRE_PTR(w->gate, 16, "weights.gate");
  REQUIRE_PTR(w->up, 16, "weights.up");
  REQUIRE_PTR(w->down, 16, "weights.down");
  if (c.expert_dtype == MOE_DT_U8_AFFINE || c.expert_dtype == MOE_DT_U4_AFFINE) {
    // u4: the kernels copy two fp16 group parameters at a time
    const int al = c.expert_dtype == MOE_DT_U4_AFFINE ? 4 : 2;
    REQUIRE_PTR(w->gate_scale, al, "weights.gate_scale");
    REQUIRE_PTR(w->gate_zero, al, "weights.gate_zero");
    REQUIRE_PTR(w->up_scale, al, "weights.up_scale");
    REQUIRE_PTR(w->up_zero, al, "weights.up_zero");
    REQUIRE_PTR(w->down_scale, al, "weights.down_scale");
    REQUIRE_PTR(w->down_zero, al, "weights.down_zero");
  }
  if (c.shared_intermediate > 0) {
    REQUIRE_PTR(w->shared_gate, 16, "weights.shared_gate");
    REQUIRE_PTR(w->shared_up, 16, "weights.shared_up");
    REQUIRE_PTR(w->shared_down, 16, "weights.shared_down");
  }
  return MOE_OK;
}

// ---- dense MLP (the shared expert's computation on its own)
moe_status check_dense(const moe_config* c, int64_t I) {
  if (!c) return fail(MOE_EINVAL_ARG, "cfg is null");
  if (c->hidden < 1 || c->hidden > kMaxH)
    return fail(MOE_EINVAL_CONFIG, "hidden=%lld outside [1, %lld]", (long long)c->hidden, (long long)kMaxH);
  if (c->act_dtype != MOE_DT_F32 && c->act_dtype != MOE_DT_BF16)
    return fail(MOE_EINVAL_CONFIG, "act_dtype=%d must be F32 or BF16", c->act_dtype);
  if (c->path < MOE_PATH_AUTO || c->path > MOE_PATH_PREFILL) return fail(MOE_EINVAL_CONFIG, "path=%d unknown", c->path);
  if (I < 1 || I > kMaxI) return fail(MOE_EINVAL_ARG, "intermediate=%lld outside [1, %lld]", (long long)I, (long long)kMaxI);
  if (c->hidden % 64 || I % 64) return fail(MOE_EUNSUPPORTED, "hidden and intermediate must be multiples of 64");
  if (c->path == MOE_PATH_PREFILL && c->act_dtype == MOE_DT_F32)
    return fail(MOE_EUNSUPPORTED, "the tiled MFMA path needs BF16 activations");
  return MOE_OK;
}

struct DensePlan {
  bool decode;
  size_t o_hs, o_rs, total;
};

void dense_plan(const moe_config& c, int64_t I, int64_t T, DensePlan& p) {
  p.decode = c.path == MOE_PATH_DECODE ||
             (c.path == MOE_PATH_AUTO && (T <= kDenseDecodeMaxT || c.act_dtype == MOE_DT_F32));
  const size_t ab = c.act_dtype == MOE_DT_F32 ? 4 : 2;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  p.o_hs = take(T * I * ab);                           // silu(x W_g^T) * (x W_u^T)
  p.o_rs = take(p.decode ? T * c.hidden * 4 : 0);      // fp32 output before rounding
  p.total = o;
}

moe_status run_dense(const moe_config& c, const DensePlan& p, int64_t T, int64_t I, const void* x, const void* gate,
                     const void* up, const void* down, void* y, void* ws, hipStream_t s) {
  const Act act = c.act_dtype == MOE_DT_F32 ? Act::F32 : Act::BF16;
  const WFmt wf = act == Act::F32 ? WFmt::F32 : WFmt::BF16;
  const int Ti = static_cast<int>(T), H = static_cast<int>(c.hidden), Id = static_cast<int>(I);
  void* hs = at<void>(ws, p.o_hs);
  const int ncu = device_cus();
  if (p.decode) {
    // the shared-expert items of the streaming kernels (part 2 reads no routing)
    SkinnyUpArgs u{};
    u.x = x;
    u.sgate = gate;
    u.sup = up;
    u.hs = hs;
    u.T = Ti;
    u.H = H;
    u.I = Id;
    u.Is = Id;
    u.k = 1;
    u.E = 1;
    u.part = 2;
    u.dense = 1;
    MOE_LAUNCH_STAGE(MOE_STAGE_SHARED_UP, s, launch_skinny_up(u, act, wf, ncu, s), "dense gate/up (streaming)");
    SkinnyDownArgs d{};
    d.hs = hs;
    d.sdown = down;
    d.rs = at<float>(ws, p.o_rs);
    d.T = Ti;
    d.H = H;
    d.I = Id;
    d.Is = Id;
    d.k = 1;
    d.E = 1;
    d.part = 2;
    MOE_LAUNCH_STAGE(MOE_STAGE_SHARED_DOWN, s, launch_skinny_down(d, act, wf, ncu, s), "dense down (streaming)");
    CombineArgs cb{nullptr, d.rs, nullptr, y, Ti, H, 0, 0, 0};  // no routed terms: y = rounded output
    MOE_LAUNCH_STAGE(MOE_STAGE_COMBINE, s, launch_combine(cb, act, s), "dense output");
    return MOE_OK;
  }
  TileArgs su{};
  su.A = static_cast<const uint16_t*>(x);
  su.K = H;
  su.B0 = gate;
  su.B1 = up;
  su.N = Id;
  su.routed = 0;
  su.M = Ti;
  su.out = hs;
  su.ldo = Id;
  su.mtiles_bound = static_cast<int>((T + kTileM - 1) / kTileM);
  su.group_m = kGroupAuto;
  su.ncu = ncu;
  MOE_LAUNCH_STAGE(MOE_STAGE_SHARED_UP, s, launch_tile_gemm(su, AMode::DENSE, WFmt::BF16, Epi::SWIGLU, s), "dense gate/up (tiled)");
  TileArgs sd{};
  sd.A = static_cast<const uint16_t*>(hs);
  sd.K = Id;
  sd.B0 = down;
  sd.N = H;
  sd.routed = 0;
  sd.M = Ti;
  sd.out = y;
  sd.ldo = H;
  sd.k = 0;  // the combine epilogue with no routed terms: y = rounded output
  sd.mtiles_bound = su.mtiles_bound;
  sd.group_m = kGroupAuto;
  sd.ncu = ncu;
  MOE_LAUNCH_STAGE(MOE_STAGE_SHARED_DOWN, s, launch_tile_gemm(sd, AMode::DENSE, WFmt::BF16, Epi::COMBINE, s), "dense down (tiled)");
  return MOE_OK;
}

// Argument checks of moe_forward and moe_forward_noalloc (everything but the workspace).
moe_status check_forward_args(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w, const void* y,
                              const int32_t* topk_idx_out, const float* topk_w_out,
                              const int32_t* expert_counts_out) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if ((s = check_T(T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x, 16, "x");
  REQUIRE_PTR(y, 16, "y");
  if (topk_idx_out && !aligned(topk_idx_out, 4)) return fail(MOE_EINVAL_ARG, "topk_idx_out is not 4-byte aligned");
  if (topk_w_out && !aligned(topk_w_out, 4)) return fail(MOE_EINVAL_ARG, "topk_w_out is not 4-byte aligned");
  if (expert_counts_out && !aligned(expert_counts_out, 4))
    return fail(MOE_EINVAL_ARG, "expert_counts_out is not 4-byte aligned");
  return check_weights(*cfg, w, true);
}

// ---- fixed scratch of moe_forward_noalloc, for callers that cannot allocate.
// A file-scope device array: every GPU the library runs on holds its own copy, at its
// own address, until the process ends.  In host code `scratch` names a host-side
// stand-in, so its device address is taken once per device with
// hipGetSymbolAddress (that device current) and only that address is used.
constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

moe_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(MOE_EUNSUPPORTED, "device %d: the fixed scratch covers devices 0..63", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned(ptr, 256)) return fail(MOE_EHIP, "the fixed scratch has no 256-byte aligned device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// The whole layer on stream st with a checked plan and workspace.  With `fork`, the
// prefill path runs the shared expert's gate/up on a second stream of this thread;
// without it every launch goes to st.
moe_status run_forward(const moe_config& c, const Plan& p, int64_t T, const void* x, const moe_weights* w, void* y,
                       int32_t* topk_idx_out, float* topk_w_out, int32_t* expert_counts_out, void* ws,
                       hipStream_t st, bool fork) {
  const moe_config* cfg = &c;
  moe_status s = MOE_OK;
  int32_t* idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, p.o_idx);
  float* wt = topk_w_out ? topk_w_out : at<float>(ws, p.o_w);
  const float* ebias = cfg->use_expert_bias ? w->expert_bias : nullptr;
  // prefill: the shared expert's gate/up GEMM, which needs no routing, runs on a second
  // stream beside the router, top-k, permutation and routed GEMMs (measured: the
  // Ling-lite shape at 4096 tokens 0.906 -> 0.873 ms).  Decode keeps one stream: there
  // the two extra launches and the join cost more than the overlap gains, eagerly and
  // as graph branches alike (Ling-lite at 1 token: graph replay 55 -> 72 us forked).
  hipEvent_t join = nullptr;
  AuxStream* aux = fork && cfg->shared_intermediate > 0 && !p.decode ? aux_stream(st) : nullptr;
  if (aux) {
    {
      hipError_t e = hipEventRecord(aux->fork, st);
      if (e == hipSuccess) e = hipStreamWaitEvent(aux->s, aux->fork, 0);
      if (e != hipSuccess) return hip_fail(e, "fork of the shared expert");
      if ((s = run_shared(*cfg, p, T, x, w, ws, aux->s)) != MOE_OK) return s;
      if ((e = hipEventRecord(aux->join, aux->s)) != hipSuccess) return hip_fail(e, "shared expert done");
      join = aux->join;
    }
  }
  if (p.decode && T <= kFusedRouteMaxT && T * cfg->top_k <= kFusedSlots) {
    // small batch: route and permute in one workgroup
    if ((s = run_logits(*cfg, p, T, x, w->router, ws, st)) != MOE_OK) return s;
    const TopkArgs ta = topk_args(*cfg, p, T, ws, w->router_bias, ebias, idx, wt);
    const PermuteArgs pa = permute_args(*cfg, p, T, idx, wt, at<int32_t>(ws, p.o_counts), at<int32_t>(ws, p.o_offsets),
                                          at<int32_t>(ws, p.o_perm), nullptr, ws);
    s = run_experts(*cfg, p, T, x, w, idx, wt, y, ws, st, true, join, &ta, &pa);
  } else {
    s = run_route(*cfg, p, T, x, w->router, w->router_bias, ebias, idx, wt, ws, st);
    if (s != MOE_OK) return s;
    s = run_experts(*cfg, p, T, x, w, idx, wt, y, ws, st, false, join);
  }
  if (s != MOE_OK) return s;
  if (expert_counts_out) {
    const hipError_t e = hipMemcpyAsync(expert_counts_out, at<int32_t>(ws, p.o_counts),
                                          sizeof(int32_t) * cfg->num_experts, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "expert counts copy");
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_config_default(moe_config* cfg) {
  if (!cfg) return fail(MOE_EINVAL_ARG, "cfg is null");
  std::memset(cfg, 0, sizeof *cfg);
  cfg->n_group = 1;
  cfg->topk_group = 1;
  cfg->score_function = MOE_SCORE_SOFTMAX;
  cfg->norm_topk_prob = 1;
  cfg->use_expert_bias = 0;
  cfg->routed_scaling_factor = 1.0f;
  cfg->act_dtype = cfg->router_dtype = cfg->expert_dtype = cfg->shared_dtype = MOE_DT_BF16;
  cfg->quant_group = 64;
  cfg->path = MOE_PATH_AUTO;
  return ok();
}

moe_status moe_validate_config(const moe_config* cfg) {
  try {
    const moe_status s = check_config(cfg);
    return s == MOE_OK ? ok() : s;
  } catch (...) {
    return fail(MOE_EINVAL_ARG, "internal error while validating");
  }
}

moe_status moe_workspace_size(const moe_config* cfg, int64_t T, size_t* bytes) {
  try {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    if ((s = check_T(T)) != MOE_OK) return s;
    if (!bytes) return fail(MOE_EINVAL_ARG, "bytes is null");
    Plan p;
    make_plan(*cfg, T, p);
    *bytes = p.total;
    return ok();
  } catch (...) {
    return fail(MOE_EINVAL_ARG, "internal error while sizing");
  }
}

moe_status moe_select_path(const moe_config* cfg, int64_t T, int32_t* path_out) {
  try {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    if ((s = check_T(T)) != MOE_OK) return s;
    if (!path_out) return fail(MOE_EINVAL_ARG, "path_out is null");
    Plan p;
    make_plan(*cfg, T, p);
    *path_out = p.decode ? MOE_PATH_DECODE : MOE_PATH_PREFILL;
    return ok();
  } catch (...) {
    return fail(MOE_EINVAL_ARG, "internal error while choosing the path");
  }
}

moe_status moe_route(const moe_config* cfg, int64_t T, const void* x, const void* router_w, const float* router_bias,
                     const float* expert_bias, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                     moe_stream_t stream) {
  try {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    if ((s = check_T(T)) != MOE_OK) return s;
    if (T == 0) return ok();
    REQUIRE_PTR(x, 16, "x");
    REQUIRE_PTR(router_w, 16, "router_w");
    if (router_bias && !aligned(router_bias, 4)) return fail(MOE_EINVAL_ARG, "router_bias is not 4-byte aligned");
    if (cfg->use_expert_bias) REQUIRE_PTR(expert_bias, 4, "expert_bias");
    REQUIRE_PTR(topk_idx, 4, "topk_idx");
    REQUIRE_PTR(topk_w, 4, "topk_w");
    Plan p;
    if ((s = check_ws(*cfg, T, ws, ws_bytes, p)) != MOE_OK) return s;
    s = run_route(*cfg, p, T, x, router_w, router_bias, cfg->use_expert_bias ? expert_bias : nullptr, topk_idx,
                  topk_w, ws, static_cast<hipStream_t>(stream));
    return s == MOE_OK ? ok() : s;
  } catch (...) {
    return fail(MOE_EINVAL_ARG, "internal error in moe_route");
  }
}

moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                       int32_t* perm, void* ws, size_t ws_bytes, moe_stream_t stream) {
  try {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    if ((s = check_T(T)) != MOE_OK) return s;
    if (T == 0) return ok();
    REQUIRE_PTR(topk_idx, 4, "topk_idx");
    REQUIRE_PTR(counts, 4, "counts");
    REQUIRE_PTR(offsets, 4, "offsets");
    REQUIRE_PTR(perm, 4, "perm");
    Plan p;
    if ((s = check_ws(*cfg, T, ws, ws_bytes, p)) != MOE_OK) return s;
    s = run_permute(*cfg, p, T, topk_idx, nullptr, counts, offsets, perm, nullptr, ws, static_cast<hipStream_t>(stream));
    return s == MOE_OK ? ok() : s;
  } catch (...) {
    return fail(MOE_EINVAL_ARG, "internal error in moe_permute");
  }
}

moe_status moe_experts(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w, const int32_t* topk_idx,
                       const float* topk_w, void* y, void* ws, size_t ws_bytes, moe_stream_t stream) {
  try {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    if ((s = check_T(T)) != MOE_OK) return s;
    if (T == 0) return ok();
    REQUIRE_PTR(x, 16, "x");
    REQUIRE_PTR(y, 16, "y");
    REQUIRE_PTR(topk_idx, 4, "topk_idx");
    REQUIRE_PTR(topk_w, 4, "topk_w");
    if ((s = check_weights(*cfg, w, false)) != MOE_OK) return s;
    Plan p;
    if ((s = check_ws(*cfg, T, ws, ws_bytes, p)) != MOE_OK) return s;
    s = run_experts(*cfg, p, T, x, w, topk_idx, topk_w, y, ws, static_cast<hipStream_t>(stream));
    return s == MOE_OK ? ok() : s;
  } catch (...) {
    return fail(MOE_EINVAL_ARG, "internal error in moe_experts");
  }
}

moe_status moe_forward(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w, void* y,
                       int32_t* topk_idx_out, float* topk_w_out, int32_t* expert_counts_out, void* ws,
                       size_t ws_bytes, moe_stream_t stream) {
  try {
    moe_status s = check_forward_args(cfg, T, x, w, y, topk_idx_out, topk_w_out, expert_counts_out);
    if (s != MOE_OK || T == 0) return s == MOE_OK ? ok() : s;
    Plan p;
    if ((s = check_ws(*cfg, T, ws, ws_bytes, p)) != MOE_OK) return s;
    s = run_forward(*cfg, p, T, x, w, y, topk_idx_out, topk_w_out, expert_counts_out, ws,
                    static_cast<hipStream_t>(stream), true);
    return s == MOE_OK ? ok() : s;
  } catch (...) {
    return fail(MOE_EINVAL_ARG, "internal error in moe_forward");
  }
}

moe_status moe_forward_noalloc(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w, void* y,
                               int32_t* topk_idx_out, float* topk_w_out, int32_t* expert_counts_out,
                               moe_stream_t stream) {
  try {
    moe_status s = check_forward_args(cfg, T, x, w, y, topk_idx_out, topk_w_out, expert_counts_out);
    if (s != MOE_OK || T == 0) return s == MOE_OK ? ok() : s;
    Plan p;
    make_plan(*cfg, T, p);
    if (p.total > kNoAllocScratchBytes)
      return fail(MOE_EWORKSPACE,
                  "T=%lld needs %zu bytes of scratch; moe_forward_noalloc holds at most %zu "
                  "(split the batch, or pass a workspace to moe_forward)",
                  (long long)T, p.total, kNoAllocScratchBytes);
    void* ws = nullptr;
    if ((s = noalloc_scratch(&ws)) != MOE_OK) return s;
    if ((s = check_ws(*cfg, T, ws, kNoAllocScratchBytes, p)) != MOE_OK) return s;
    s = run_forward(*cfg, p, T, x, w, y, topk_idx_out, topk_w_out, expert_counts_out, ws,
                    static_cast<hipStream_t>(stream), false);
    return s == MOE_OK ? ok() : s;
  } catch (...) {
    return fail(MOE_EINVAL_ARG, "internal error in moe_forward_noalloc");
  }
}

moe_status moe_dense_workspace_size(const moe_config* cfg, int64_t intermediate, int64_t T, size_t* bytes) {
  try {
    moe_status s = check_dense(cfg, intermediate);
    if (s != MOE_OK) return s;
    if ((s = check_T(T)) != MOE_OK) return s;
    if (!bytes) return fail(MOE_EINVAL_ARG, "bytes is null");
    DensePlan p;
    dense_plan(*cfg, intermediate, T, p);
    *bytes = p.total;
    return ok();
  } catch (...) {
    return fail(MOE_EINVAL_ARG, "internal error while sizing");
  }
}

moe_status moe_dense_mlp(const moe_config* cfg, int64_t intermediate, int64_t T, const void* x, const void* gate,
                         const void* up, const void* down, void* y, void* ws, size_t ws_bytes, moe_stream_t stream) {
  try {
    moe_status s = check_dense(cfg, intermediate);
    if (s != MOE_OK) return s;
    if ((s = check_T(T)) != MOE_OK) return s;
    if (T == 0) return ok();
    REQUIRE_PTR(x, 16, "x");
    REQUIRE_PTR(y, 16, "y");
    REQUIRE_PTR(gate, 16, "gate");
    REQUIRE_PTR(up, 16, "up");
    REQUIRE_PTR(down, 16, "down");
    DensePlan p;
    dense_plan(*cfg, intermediate, T, p);
    const int64_t kmax = cfg->hidden > intermediate ? cfg->hidden : intermediate;
    if (!p.decode && T * kmax * 2 >= (int64_t(1) << 32))
      return fail(MOE_EUNSUPPORTED, "T * max(hidden, intermediate) * 2 bytes >= 2^32 on the tiled path; split the batch");
    if (ws_bytes < p.total) return fail(MOE_EWORKSPACE, "workspace of %zu bytes < %zu required", ws_bytes, p.total);
    if (p.total > 0 && (!ws || !aligned(ws, 256))) return fail(MOE_EWORKSPACE, "workspace must be non-null and 256-byte aligned");
    if ((s = run_dense(*cfg, p, T, intermediate, x, gate, up, down, y, ws, static_cast<hipStream_t>(stream))) != MOE_OK)
      return s;
    return ok();
  } catch (...) {
    return fail(MOE_EINVAL_ARG, "internal error in moe_dense_mlp");
  }
}

moe_status moe_profile_enable(int32_t stage_mask, int32_t capacity) {
  try {
    if (capacity < 1 || capacity > (1 << 20)) return fail(MOE_EINVAL_ARG, "capacity must be in [1, 2^20]");
    moe_profile_disable();
    g_prof.pool = new ProfPair[capacity];
    for (int32_t i = 0; i < capacity; ++i) {
      hipError_t e = hipEventCreate(&g_prof.pool[i].start);
      if (e == hipSuccess) e = hipEventCreate(&g_prof.pool[i].stop);
      if (e != hipSuccess) {
        g_prof.capacity = i;
        moe_profile_disable();
        return hip_fail(e, "hipEventCreate");
      }
    }
    g_prof.capacity = capacity;
    g_prof.used = 0;
    g_prof.mask = stage_mask;
    return ok();
  } catch (...) {
    return fail(MOE_EINVAL_ARG, "internal error in moe_profile_enable");
  }
}

moe_status moe_profile_collect(int32_t stage, float* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return fail(MOE_EINVAL_ARG, "null output");
  float sum = 0.f;
  int32_t n = 0;
  for (int32_t i = 0; i < g_prof.used; ++i) {
    ProfPair& p = g_prof.pool[i];
    if (p.stage != stage) continue;
    hipError_t e = hipEventSynchronize(p.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.start, p.stop);
    if (e != hipSuccess) return hip_fail(e, "event timing");
    sum += ms;
    ++n;
  }
  *total_ms = sum;
  *launches = n;
  return ok();
}

moe_status moe_profile_disable(void) {
  if (g_prof.pool) {
    for (int32_t i = 0; i < g_prof.capacity; ++i) {
      (void)hipEventDestroy(g_prof.pool[i].start);
      (void)hipEventDestroy(g_prof.pool[i].stop);
    }
    delete[] g_prof.pool;
  }
  g_prof = Profiler{};
  return ok();
}

moe_status moe_profile_reset(void) {
  g_prof.used = 0;
  return ok();
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL_CONFIG: return "invalid configuration";
    case MOE_EINVAL_ARG: return "invalid argument";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_EUNSUPPORTED: return "valid layer not supported by the gfx950 kernels";
    case MOE_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_err; }

int32_t moe_abi_version(void) { return 1; }

}  // extern "C"
