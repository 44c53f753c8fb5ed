// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum class Act { F32 = 0, BF16 = 1 };
enum class WFmt { F32 = 0, BF16 = 1, U8 = 2, U4 = 3 };

// ------------------------------------------------------------------ routing
struct TopkArgs {
  const float* logits;      // [P][T][E] fp32 partial logits (summed over P)
  int64_t part_stride;      // elements between partials (T * E)
  int P;
  int T, E, k, G, g;
  int score_sigmoid, norm, use_ebias;
  float rsf;
  const float* router_bias;  // [E] or null
  const float* expert_bias;  // [E] or null
  int32_t* idx;              // [T, k]
  float* w;                  // [T, k]
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

struct PermuteArgs {
  const int32_t* idx;   // [nslots]
  int nslots, E, BM;    // BM > 0: also build the M-tile map (chunks of BM positions)
  int small_max;        // experts with 1..small_max slots go to the active list
  int tile_min;         // with BM > 0, experts with more than tile_min slots get M-tiles
  int32_t* counts;      // [E]
  int32_t* offsets;     // [E + 1]
  int32_t* perm;        // [nslots]  slot ids grouped by expert, -1 tail
  int32_t* slot_pos;    // [nslots]  position of each slot in perm, -1 if dropped
  int32_t* active;      // [E]       experts with 1..small_max slots, ascending
  int32_t* tiles;       // [max_tiles * 2] (expert, start position)
  int BM2;              // > 0: also a map of chunks of BM2 positions (tiles2, meta[3])
  int32_t* tiles2;      // [max_tiles2 * 2] (expert, start position)
  int32_t* meta;        // [4]: D, number of M-tiles, valid slots, number of BM2 chunks
  int32_t* counts_copy; // optional extra copy of counts (caller output) or null
  int32_t* hist;        // [ceil(nslots / kPermChunk)][E] per-block histograms (multi-block form)
  int4* chunks;         // optional: per entry of `tiles` one record (expert, first position of
                        // the entry, the expert's first position, the expert's count), so a
                        // streaming work item finds all it needs in one 16-byte load
  const float* w;       // [nslots] routing weights, with wpos: also store them by position
  float* wpos;          // [nslots] or null: wpos[perm position] = w[slot]
};
constexpr int kPermChunk = 2048;   // slots per workgroup in the multi-block permutation
constexpr int kPermSingleMax = 4096;  // up to this many slots one workgroup does everything
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
// top-k of every token and the permutation in one workgroup (a.nslots <= kFusedSlots)
constexpr int kFusedSlots = 256;
hipError_t launch_route_permute(const TopkArgs& t, const PermuteArgs& a, hipStream_t s);

// -------------------------------------------------- weight-streaming (decode) path
// C[m][n] = sum_k A[m][k] W[n][k] with the weight rows streamed from HBM once per
// group of <= 64 tokens.
struct SkinnyRouterArgs {
  const void* x;        // [T, H]
  const void* W;        // [E, H]
  float* out;           // [P][T][E]
  int T, H, E, P;
};
hipError_t launch_skinny_router(const SkinnyRouterArgs& a, Act act, int ncu, hipStream_t s);

// Decode work is cut into chunks of at most kDecodeChunk positions of one expert (one
// 16-row MFMA fragment of tokens), each chunk a separate work item.
constexpr int kDecodeChunk = 16;

struct SkinnyUpArgs {
  const void* x;           // [T, H]
  const void* gate;        // [E, I, H]
  const void* up;          // [E, I, H]
  const uint16_t *gate_s, *gate_z, *up_s, *up_z;  // u8 only: [E, I, H/64]
  const void* sgate;       // [Is, H] or null
  const void* sup;
  void* hm;                // [T*k, I] act, rows in permuted (position) order
  void* hs;                // [T, Is] act
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* active;
  const int32_t* meta;     // meta[0] active experts, meta[1] chunks in `tiles`
  const int32_t* tiles;    // chunks of kDecodeChunk positions: (expert, first position)
  const int4* chunks;      // the same chunks as records (PermuteArgs::chunks; ring kernels)
  int mtiles;              // upper bound on the chunks (grid sizing)
  int T, H, I, Is, k, E;
  int part;                // items: 0 routed and shared, 1 routed only, 2 shared only (reads no routing)
  int dense;               // 1: the dense MLP (shared items only, its own split rule)
  int shared_first;        // ring kernels: the shared expert's items before the routed ones
  // One token (T = 1): each block routes the token itself from the router's partial
  // logits (ta) instead of reading a permutation, and block 0 also stores the routing
  // and permutation tables (ta.idx, ta.w and everything pa names) for the stages after
  // it.  Taken by the one-token kernel (bf16 weights, up_one_fits) and by the u8 / u4
  // ring kernels where every item is in the first round of blocks (skinny_up_can_route).
  int fused_route;
  TopkArgs ta;
  PermuteArgs pa;
  const int32_t* idx;      // [T, k] routing (one-token kernel without fused_route: the expert
                           // of position p is idx[perm[p]])
};
hipError_t launch_skinny_up(const SkinnyUpArgs& a, Act act, WFmt wf, int ncu, hipStream_t s);
// whether the one-token gate/up kernel takes these arguments (bf16 weights, the whole
// layer); it routes the token itself when fused_route is set, for any expert count up
// to 512 and any number of blocks, so skinny_up_can_route does not apply to it
bool up_one_fits(const SkinnyUpArgs& a, Act act, WFmt wf);
// whether a gate/up launch with these arguments (fused_route aside) can route its one
// token itself: one token, the whole layer, a ring kernel, every item in one round
bool skinny_up_can_route(const SkinnyUpArgs& a, Act act, WFmt wf, int ncu);

struct SkinnyDownArgs {
  const void* hm;          // [T*k, I] position order
  const void* hs;          // [T, Is]
  const void* down;        // [E, H, I]
  const uint16_t *down_s, *down_z;  // u8 only: [E, H, I/64]
  const void* sdown;       // [H, Is] or null
  const float* topk_w;     // [T*k]
  void* r;                 // [T*k, H] fp32 (or bf16 when r_bf16), slot order, scaled by
                           // the routing weight
  float* rs;               // [T, H] fp32 shared expert output
  int r_bf16;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* active;
  const int32_t* meta;
  const int32_t* tiles;    // as SkinnyUpArgs
  const int4* chunks;      // as SkinnyUpArgs
  const float* wpos;       // [T*k] routing weight by position (ring kernels)
  int mtiles;
  int T, H, I, Is, k, E;
  int part;                // as SkinnyUpArgs::part
  int shared_first;        // as SkinnyUpArgs::shared_first
  // one token (launch_down_one): the layer output is written here, combined
  const int32_t* idx;      // [k] routing of the token (entries outside [0,E) skipped)
  void* y;                 // [1, H] act
};
hipError_t launch_skinny_down(const SkinnyDownArgs& a, Act act, WFmt wf, int ncu, hipStream_t s);
// One token, bf16 weights and activations, the whole layer (part 0): down of the shared
// and selected experts and their weighted sum in one launch, into y (no r, rs, combine).
// down_one_fits says whether launch_down_one takes these arguments.
bool down_one_fits(const SkinnyDownArgs& a, Act act, WFmt wf);
hipError_t launch_down_one(const SkinnyDownArgs& a, Act act, WFmt wf, hipStream_t s);

// largest top_k the library accepts (the combine kernel keeps a token's k terms in registers)
constexpr int kMaxTopK = 16;
struct CombineArgs {
  const void* r;            // [T*k, H] slot order (fp32 or bf16)
  const float* rs;          // [T, H] fp32 or null
  const int32_t* idx;       // [T*k] routing (entries outside [0,E) skipped)
  void* y;                  // [T, H] act
  int T, H, k, E;
  int r_bf16;
};
hipError_t launch_combine(const CombineArgs& a, Act act, hipStream_t s);

// ------------------------------------------------------------- tiled MFMA path
enum class AMode { DENSE = 0, GATHER = 1 };
enum class Epi { F32 = 0, SWIGLU = 1, SCALED_SLOT = 2, COMBINE = 3 };

struct TileArgs {
  // A operand rows (bf16, K contiguous)
  const uint16_t* A;      // DENSE: row r at A + r*K; GATHER: row = token perm[pos]/k
  int K;
  // B operand (weights, K contiguous): B0 (and B1 for SwiGLU) [experts][N][K]
  const void* B0;
  const void* B1;
  const uint16_t *B0s, *B0z, *B1s, *B1z;  // u8 scale / zero [experts][N][K/64]
  int64_t b_expert_stride;  // elements (codes) between experts
  int N;                    // weight rows per expert (output columns)
  // M tiling
  int routed;               // 1: tiles from the permutation's tile map
  int M;                    // dense: number of rows
  const int32_t* tiles;     // routed: (expert, start position) per M-tile
  const int32_t* meta;      // routed: meta[1] = number of M-tiles
  const int32_t* offsets;   // routed: expert position ranges
  const int32_t* perm;      // routed: slot of each position
  int k;                    // top_k (slot -> token)
  // epilogue
  void* out;                // F32: float [M][N]; SWIGLU: bf16 [pos|row][N]; SCALED_SLOT: bf16 [slot][N];
                            // COMBINE: bf16 y [T][N]
  int ldo;                  // output row stride (elements)
  const float* topk_w;      // SCALED_SLOT
  const uint16_t* r;        // COMBINE: routed terms bf16 [T*k][N]
  const int32_t* idx;       // COMBINE: routing
  int E;                    // COMBINE: expert count (validity of idx)
  int mtiles_bound;         // grid bound on M-tiles
  int ksplit;               // F32 epilogue only: K split into this many partial outputs
  int64_t part_stride;      // elements between partial outputs
  int group_m;              // M-tiles per block-order group (weight-panel reuse in L2)
  int plain_order;          // routed: 1 = blocks in launch order, an expert's N-tiles
                            // side by side; 0 = consecutive tiles on one XCD, an N-tile's
                            // M-tiles side by side (see tile_pos)
  int ncu;                  // compute units of the device (tile-shape choice)
  // routed SwiGLU products whose last 256-column N-tile is at most half full: that
  // tile's columns are computed over chunks of 256 positions (tiles2, count meta[3])
  const int32_t* tiles2;    // or null
  int mtiles2_bound;        // grid bound on the 256-position chunks
};
hipError_t launch_tile_gemm(const TileArgs& a, AMode am, WFmt wf, Epi epi, hipStream_t s);

constexpr int kTileM = 128;

}  // namespace moe
