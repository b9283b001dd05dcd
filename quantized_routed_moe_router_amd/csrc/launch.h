// Host-side launch wrappers of the ds4moe kernels (internal to the library).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ds4 {

// Optional per-kernel timing: start/stop events stamped by the kernel's own
// dispatch (hipExtLaunchKernelGGL); nullptr = plain launch.
struct Timing {
  hipEvent_t start, stop;
};

struct TileT {
  int32_t e, p0, n, pad;
};

// Small-batch (T <= 16) work item: one used expert, the tokens that chose it
// (bit t of tmask) and their routing weights (0 for other tokens).
struct DecTile {
  int32_t e;
  uint32_t tmask;
  int32_t pad0, pad1;
  float w[16];
};

// Activation preparation done per token next to the router: x -> fp16 and
// per-16-element sums (split into fp16 hi + lo) for the min term.
struct XPrep {
  const void *x;       // [T,H] x_dtype
  bool x_bf16;
  _Float16 *x16;       // [T,H]
  _Float16 *xs_hi;     // [T,H/16]
  _Float16 *xs_lo;     // [T,H/16]
  int32_t *xexp;       // [T] e of each token: x16 holds x * 2^-e (see token_exp)
  int32_t *xe16;       // [T][4] e again, one 16-byte row per token (nullable)
};

struct RouteOut {
  int32_t *idx;        // [T,k]
  float *w;            // [T,k]
  int32_t *counts;     // [E]
  int32_t *offsets;    // [E+1]
  int32_t *perm;       // [T*k]
  int32_t *pos;        // [T*k] inverse of perm (nullable)
  TileT *tiles;        // [max_tiles] (nullable)
  int32_t *ntiles;     // [2] tile count, first tile (0) (nullable)
  int tile_n;          // tokens per tile
  _Float16 *zeros;     // cleared here each call: read by GEMM lanes with no token
  int nzeros;          // halves
  const int32_t *xexp; // [T] token exponents (x16 = x * 2^-e): the decode tile
                       // weights carry 2^2e (nullable: no tiles)
  int32_t *pexp;       // [T*k] the exponent of each permuted position's token (nullable)
};

// Activations of a wide-tile grouped GEMM through one buffer window: rows of
// K fp16 values, then their per-16 sums (hi, lo) at byte offsets o_shi, o_slo.
struct GemmAct {
  const uint8_t *base;
  uint32_t len;
  uint32_t o_shi, o_slo;
  uint32_t row_bytes, srow_bytes;
  uint32_t o_xe;  // gate/up: 16-byte rows whose first word is the token's pre-scale exponent (else DS4_OOB)
};

// ways the 5..16-token down projection may split its tile list (workspace
// partials of T x H floats each)
constexpr int DEC_DOWN_SPLITS = 4;

struct GemmArgs {
  // routed experts
  const uint8_t *gate, *up, *down;   // packed, E matrices each
  size_t gu_bytes, d_bytes;          // bytes per expert matrix
  int bits;                          // code width of the gate/up codes: 2, 4, 5 or 6 (5: in 6-bit units)
  int bits_dn;                       // code width of the down codes: 2, 4, 5 or 6
  const TileT *tiles;
  const int32_t *ntiles;             // decode: [1] DecTiles; prefill: [2] tile count, first tile
  const int32_t *perm;
  int k, H, I, Ipad;
  const _Float16 *x16, *xs_hi, *xs_lo;
  const int32_t *xexp;               // [T] token exponents: x16 = x * 2^-e, h = silu(g) u * 2^-2e
  const int32_t *pexp;               // [T*k] prefill: exponent of each permuted position's token
  const int32_t *xe16;               // [T][4] prefill: the token exponents in 16-byte rows
  _Float16 *h, *hs_hi, *hs_lo;       // [T*k, Ipad], [T*k, Ipad/16]
  float *yp;                         // [T*k, H]
  const _Float16 *zeros;             // >= max(H, Ipad) zero halves
  // small batches: activations addressed as byte offsets inside the workspace
  const uint8_t *wsb;
  uint32_t ws_len;
  uint32_t o_x16, o_xs_hi, o_xs_lo, o_h, o_hs_hi, o_hs_lo;
  const DecTile *dtiles;
  int dt_cap;                        // decode: DecTile entries the tile buffer holds (>= any tile count)
  int T;
  int tile_n;                        // tokens per prefill tile (> 64: wide-tile GEMMs)
  // small batches of 5..16 tokens: the down projection's partial outputs
  // of the parts of the tile list [DEC_DOWN_SPLITS][T][H]
  float *dpart;
  const float *ysh;                  // [T,H] shared-expert output or nullptr
  float *y;                          // [T,H]
};

// Routed-expert cache state (device memory, inside the caller's cache buffer).
struct CacheHdr {
  uint32_t step;                    // calls since the reset (the stamp of the current call)
  uint32_t fill_n;                  // misses of the last call = length of its fill list
  unsigned long long calls, hits, misses;
};
struct CacheState {
  CacheHdr *hdr;
  int32_t *slot_expert;             // [S] expert held by each slot, -1 = empty
  int32_t *expert_slot;             // [E] slot of each expert, -1 = not cached
  uint32_t *stamp;                  // [S] step of the slot's last use (0 = never)
  int32_t *fill_e, *fill_s;         // [E] the last call's misses in batch order: expert, slot
  int32_t *frange;                  // [E][2] each batch's fill items [begin, end)
  int32_t *brange;                  // [E][2] each batch's prefill tiles: count, first
  uint8_t *gate, *up, *down;        // S slots of packed matrices each
};

hipError_t launch_cache_reset(const CacheState &c, int S, int E, hipStream_t s);
// after the small-batch routing: plan slots, rewrite each DecTile's expert as its slot
hipError_t launch_cache_plan(const CacheState &c, DecTile *dt, const int32_t *ntile, int S, int E, hipStream_t s,
                             const Timing *tm = nullptr);
// prefill: split the used experts into batches that fit the slots, plan each
// batch's slots and write the tile list in batch order with slots for experts
hipError_t launch_cache_plan_prefill(const CacheState &c, const int32_t *counts, const int32_t *offsets,
                                     TileT *tiles, int tile_n, int S, int E, hipStream_t s);
// copy the fill items [fr[0], fr[1]) from host memory (device-visible
// pointers) into their slots
hipError_t launch_cache_fill(const CacheState &c, const int32_t *fr, const void *hg, const void *hu, const void *hd,
                             size_t gu_bytes, size_t d_bytes, int max_items, hipStream_t s,
                             const Timing *tm = nullptr);

hipError_t launch_pack(void *dst, const void *canonical, int64_t n_mats, int64_t rows, int64_t cols, int bits,
                       hipStream_t s);
hipError_t launch_dequant(float *dst, const void *packed, int64_t n_mats, int64_t rows, int64_t cols, int bits,
                          hipStream_t s);

hipError_t launch_router_tiled(const void *x, bool x_bf16, const void *wr, bool w_bf16, const float *bias,
                               float *logits, int T, int E, int H, hipStream_t s, const Timing *tm = nullptr);
// large T: top-k + activation prep + per-chunk counts/ranks, scan, placement
int chunk_count(int T);
// an upper bound of chunk_count that never decreases with T (workspace sizing)
int chunk_count_max(int T);
hipError_t launch_route_chunked(const float *logits, int T, int E, int k, int H, const XPrep *xp, RouteOut ro,
                                int32_t *ccnt, int32_t *base, int32_t *lrank, hipStream_t s,
                                const Timing *tm_topk = nullptr, const Timing *tm_perm = nullptr);
// T <= 16: logits as fp64 partial sums per column slice [router_slices(H)][T][E],
// with the activation preparation (if xp != nullptr)
int router_slices(int H);
// batches of at most this many tokens: one expert per workgroup and a single
// slice (the whole row)
constexpr int ROUTER_ROWS_MAX_T = 4;
// slices the router of a T-token batch leaves in part[]
int router_nslice(int H, int T);
hipError_t launch_router_sliced(const void *x, bool x_bf16, const void *wr, bool w_bf16, double *part, int T,
                                int E, int H, const XPrep *xp, hipStream_t s, const Timing *tm = nullptr);
// one workgroup, T <= 16: slice sums + bias -> logits, top-k, counts, offsets,
// permutation and (dt != nullptr) the small-batch tiles
hipError_t launch_route_dec(const double *part, int nslice, const float *bias, float *logits, int T, int E, int k,
                            RouteOut ro, DecTile *dt, int32_t *ntile, hipStream_t s, const Timing *tm = nullptr);

// grouped GEMMs over the tile list (max_tiles = grid bound); tiles of more
// than 64 tokens take the wide-tile kernels, whose activation windows (x16 or
// h through the end of their sums) must fit 2 GiB
hipError_t launch_gateup(const GemmArgs &a, int max_tiles, hipStream_t s, const Timing *tm = nullptr);
hipError_t launch_down(const GemmArgs &a, int max_tiles, hipStream_t s, const Timing *tm = nullptr);
// Routing folded into the small-batch gate/up kernel (T <= 4): every
// workgroup routes the batch from the router's partial sums for itself;
// workgroup 0 also writes the routing outputs and the DecTile list.
struct DecRoute {
  const double *part;  // [nslice][T][E]
  int nslice;
  const float *bias;   // [E] or nullptr
  float *logits;       // [T,E]
  int E, k;
  RouteOut ro;
  DecTile *dt;
  int32_t *ntile;
};

// small batches: gate/up over the DecTile list (rr != nullptr: T <= 4 and
// the routing is done by the kernel itself), and down fused with the combine
// (writes y)
hipError_t launch_gateup_dec(const GemmArgs &a, int max_tiles, const DecRoute *rr, hipStream_t s,
                             const Timing *tm = nullptr);
hipError_t launch_down_combine_dec(const GemmArgs &a, hipStream_t s, const Timing *tm = nullptr,
                                   const Timing *tm_combine = nullptr);
hipError_t launch_combine(const float *yp, const int32_t *pos, const float *w, const int32_t *xexp, const float *ysh,
                          float *y, int T, int k, int H, hipStream_t s, const Timing *tm = nullptr);
// dense shared expert, bf16 weights.  From SHARED_DENSE_MIN_T tokens on the
// GEMMs read fp16 copies of the weights (w16: gate | up | down, 3*H*Is
// halves, written by launch_shared_convert in the same call)
constexpr int SHARED_DENSE_MIN_T = 65;
hipError_t launch_shared_convert(const uint16_t *wg, const uint16_t *wu, const uint16_t *wd, _Float16 *dst, int H,
                                 int Is, hipStream_t s, const Timing *tm = nullptr);
hipError_t launch_shared_gateup(const uint16_t *wg, const uint16_t *wu, const _Float16 *w16, const _Float16 *x16,
                                const int32_t *xexp, _Float16 *hs, int T, int H, int Is, hipStream_t s,
                                const Timing *tm = nullptr);
hipError_t launch_shared_down(const uint16_t *wd, const _Float16 *w16, const _Float16 *hs, const int32_t *xexp,
                              float *ysh, int T, int H, int Is, hipStream_t s, const Timing *tm = nullptr);

// Launch `kernel` plainly, or with dispatch-stamped timing events.
#define DS4_LAUNCH(tm, kernel, grid, block, shmem, stream, ...)                                                  \
  do {                                                                                                         \
    if (tm)                                                                                                    \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, (tm)->start, (tm)->stop, 0, __VA_ARGS__);      \
    else                                                                                                       \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                                     \
  } while (0)

}  // namespace ds4
