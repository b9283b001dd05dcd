// C ABI of the ds4moe library: argument validation (host only, before any
// launch), workspace layout, and the launch sequences of the three calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ds4moe.h"
#include "launch.h"

using namespace ds4;

namespace {

constexpr int kVersion = 300;  // 0.3.0: ds4moe_forward_prefill_cached
constexpr int kTileDecode = 16;
constexpr int kTilePrefill = 64;      // tokens per prefill tile (64-token GEMM kernels)
constexpr int kTilePrefillWide = 80;  // with the wide-tile GEMM kernels
constexpr int64_t kMaxTokens = 1 << 20;
// decode kernels address their activations as 32-bit byte offsets into the workspace
constexpr int64_t DS4_WS_WINDOW = (int64_t)1 << 31;

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int validate_dims(const ds4moe_dims *d) {
  if (!d) return DS4MOE_ERR_NULL;
  if (d->x_dtype != DS4MOE_F32 && d->x_dtype != DS4MOE_BF16) return DS4MOE_ERR_DTYPE;
  if (d->router_dtype != DS4MOE_F32 && d->router_dtype != DS4MOE_BF16) return DS4MOE_ERR_DTYPE;
  if (d->hidden < 256 || d->hidden > 65536 || d->hidden % 256) return DS4MOE_ERR_SHAPE;
  if (d->inter < 16 || d->inter > 32768 || d->inter % 16) return DS4MOE_ERR_SHAPE;
  if (d->inter % 256 && 256 % d->inter) return DS4MOE_ERR_SHAPE;
  if (d->top_k < 1 || d->top_k > 16) return DS4MOE_ERR_SHAPE;
  if (d->n_experts < d->top_k || d->n_experts > 256) return DS4MOE_ERR_SHAPE;
  if (d->shared_inter < 0 || d->shared_inter > 65536 || d->shared_inter % 32) return DS4MOE_ERR_SHAPE;
  auto width_ok = [](int b) { return b == 2 || b == 4 || b == 5 || b == 6; };
  if (!width_ok(d->expert_bits)) return DS4MOE_ERR_SHAPE;
  if (d->down_bits != 0 && !width_ok(d->down_bits)) return DS4MOE_ERR_SHAPE;
  return DS4MOE_OK;
}

// code width of the routed down matrices
inline int down_bits(const ds4moe_dims &d) { return d.down_bits ? d.down_bits : d.expert_bits; }

struct Layout {
  size_t logits, part, idx, w, counts, offsets, perm, pos, pexp, tiles, ntiles, ccnt, cbase, lrank, dpart;
  size_t x16, xs_hi, xs_lo, xexp, xe16, h, hs_hi, hs_lo, yp, hsh, ysh, shw, zeros;
  int nzeros;
  size_t total;
  int tile_n, max_tiles, Ipad;
  bool sliced;  // T <= 16 routing (sliced router + one-workgroup routing); else the chunked path
};

// Routing of small batches (decode, and route-only calls with T <= 16) uses
// the sliced router; prefill always uses the MFMA router and chunked top-k.
Layout make_layout(const ds4moe_dims &d, int64_t T, int mode) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const int64_t E = d.n_experts, k = d.top_k, H = d.hidden, Is = d.shared_inter;
  const int64_t A = T * k;
  L.sliced = T <= 16 && mode != DS4MOE_MODE_PREFILL;
  L.Ipad = d.inter % 256 ? 256 : d.inter;
  L.tile_n = mode == DS4MOE_MODE_PREFILL ? kTilePrefill : kTileDecode;
  if (mode == DS4MOE_MODE_PREFILL && d.inter % 256 == 0) {
    // wide tiles when the activation windows (x16, its hi/lo sums, the token
    // exponents and their 16-byte rows, or h and its hi/lo sums, contiguous
    // below) fit 2 GiB
    const int64_t xw = (int64_t)align256(2 * T * H) + 2 * (int64_t)align256(2 * T * (H / 16)) +
                       (int64_t)align256(4 * T) + 16 * T;
    const int64_t hw = (int64_t)align256(2 * A * L.Ipad) + (int64_t)align256(2 * A * (L.Ipad / 16)) +
                       2 * A * (L.Ipad / 16);
    if (xw <= ((int64_t)1 << 31) && hw <= ((int64_t)1 << 31)) L.tile_n = kTilePrefillWide;
  }
  L.max_tiles = mode == DS4MOE_MODE_DECODE ? (int)(A < E ? A : E) : (int)(A / L.tile_n + (A < E ? A : E));
  L.logits = take(sizeof(float) * T * E);
  // the sliced router's partial sums; reserved at T > 16 too, so that the
  // workspace never shrinks as T grows
  L.part = take(sizeof(double) * router_slices((int)H) * (T < 16 ? T : 16) * E);
  L.idx = take(sizeof(int32_t) * A);
  L.w = take(sizeof(float) * A);
  L.counts = take(sizeof(int32_t) * E);
  L.offsets = take(sizeof(int32_t) * (E + 1));
  L.perm = take(sizeof(int32_t) * A);
  if (!L.sliced) {
    const int64_t nch = chunk_count_max((int)T);  // the smallest chunk: sizes grow with T
    L.ccnt = take(sizeof(int32_t) * nch * E);
    L.cbase = take(sizeof(int32_t) * nch * E);
    L.lrank = take(sizeof(int32_t) * A);
  }
  if (mode != DS4MOE_MODE_ROUTE) {
    L.ntiles = take(16);
    L.x16 = take(2 * T * H);
    L.xs_hi = take(2 * T * (H / 16));
    L.xs_lo = take(2 * T * (H / 16));
    L.xexp = take(sizeof(int32_t) * T);
    if (mode == DS4MOE_MODE_PREFILL) L.xe16 = take(16 * T);
    // rows of h: assignments (prefill) or (tile, token) pairs (decode)
    const int64_t hrows = mode == DS4MOE_MODE_DECODE ? (int64_t)L.max_tiles * T : A;
    L.h = take(2 * hrows * L.Ipad);
    L.hs_hi = take(2 * hrows * (L.Ipad / 16));
    L.hs_lo = take(2 * hrows * (L.Ipad / 16));
    if (mode == DS4MOE_MODE_DECODE) {
      L.tiles = take(sizeof(DecTile) * (size_t)L.max_tiles);
      if (T > 4) L.dpart = take(sizeof(float) * DEC_DOWN_SPLITS * T * H);
    } else {
      L.tiles = take(sizeof(TileT) * (size_t)L.max_tiles);
      L.pos = take(sizeof(int32_t) * A);
      L.pexp = take(sizeof(int32_t) * A);
      L.yp = take(sizeof(float) * A * H);
      L.nzeros = (int)(H > L.Ipad ? H : L.Ipad);
      L.zeros = take(2 * (size_t)L.nzeros);
    }
    if (Is > 0) {
      L.hsh = take(2 * T * Is);
      L.ysh = take(sizeof(float) * T * H);
      // fp16 copies of the shared expert's weights for the dense GEMMs
      if (mode == DS4MOE_MODE_PREFILL && T >= SHARED_DENSE_MIN_T) L.shw = take(2 * 3 * H * Is);
    }
  }
  L.total = off;
  return L;
}

template <typename T>
T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off);
}

// Routed-expert cache buffer: header, slot tables, fill list and the
// batches' fill and tile ranges, then S slots of gate, up and down matrices.
struct CacheLayout {
  size_t hdr, slot_expert, expert_slot, stamp, fill_e, fill_s, frange, brange, gate, up, down, total;
  size_t gu_bytes, d_bytes;
};

CacheLayout make_cache_layout(const ds4moe_dims &d, int S) {
  CacheLayout C{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  C.gu_bytes = ds4moe_packed_bytes_bits(d.inter, d.hidden, d.expert_bits);
  C.d_bytes = ds4moe_packed_bytes_bits(d.hidden, d.inter, down_bits(d));
  C.hdr = take(sizeof(CacheHdr));
  C.slot_expert = take(4 * (size_t)S);
  C.expert_slot = take(4 * (size_t)d.n_experts);
  C.stamp = take(4 * (size_t)S);
  C.fill_e = take(4 * (size_t)d.n_experts);
  C.fill_s = take(4 * (size_t)d.n_experts);
  C.frange = take(8 * (size_t)d.n_experts);
  C.brange = take(8 * (size_t)d.n_experts);
  C.gate = take(C.gu_bytes * (size_t)S);
  C.up = take(C.gu_bytes * (size_t)S);
  C.down = take(C.d_bytes * (size_t)S);
  C.total = off;
  return C;
}

CacheState cache_state(void *cache, const CacheLayout &C) {
  CacheState c;
  c.hdr = at<CacheHdr>(cache, C.hdr);
  c.slot_expert = at<int32_t>(cache, C.slot_expert);
  c.expert_slot = at<int32_t>(cache, C.expert_slot);
  c.stamp = at<uint32_t>(cache, C.stamp);
  c.fill_e = at<int32_t>(cache, C.fill_e);
  c.fill_s = at<int32_t>(cache, C.fill_s);
  c.frange = at<int32_t>(cache, C.frange);
  c.brange = at<int32_t>(cache, C.brange);
  c.gate = at<uint8_t>(cache, C.gate);
  c.up = at<uint8_t>(cache, C.up);
  c.down = at<uint8_t>(cache, C.down);
  return c;
}

// a call through the cache: its state and the device-visible addresses of
// the host-resident experts
struct CacheCall {
  CacheState st;
  int S;
  const void *hg, *hu, *hd;
};

int validate_weights(const ds4moe_dims &d, const ds4moe_weights *w, bool experts) {
  if (!w) return DS4MOE_ERR_NULL;
  if (!w->router_w) return DS4MOE_ERR_NULL;
  if (!aligned(w->router_w, 16) || !aligned(w->router_bias, 4)) return DS4MOE_ERR_ALIGN;
  if (!experts) return DS4MOE_OK;
  if (!w->gate || !w->up || !w->down) return DS4MOE_ERR_NULL;
  if (!aligned(w->gate, 16) || !aligned(w->up, 16) || !aligned(w->down, 16)) return DS4MOE_ERR_ALIGN;
  if (d.shared_inter > 0) {
    if (!w->sh_gate || !w->sh_up || !w->sh_down) return DS4MOE_ERR_NULL;
    if (!aligned(w->sh_gate, 16) || !aligned(w->sh_up, 16) || !aligned(w->sh_down, 16)) return DS4MOE_ERR_ALIGN;
  }
  return DS4MOE_OK;
}

int validate_routing(const ds4moe_routing *r) {
  if (!r) return DS4MOE_OK;
  if (!aligned(r->topk_idx, 4) || !aligned(r->topk_w, 4) || !aligned(r->counts, 4) || !aligned(r->offsets, 4) ||
      !aligned(r->perm, 4) || !aligned(r->logits, 4))
    return DS4MOE_ERR_ALIGN;
  return DS4MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DS4MOE_OK : DS4MOE_ERR_HIP; }

#define TRY(expr)                          \
  do {                                     \
    const hipError_t _e = (expr);          \
    if (_e != hipSuccess) return DS4MOE_ERR_HIP; \
  } while (0)

// Common front half: validation shared by the three calls.
int check_call(const ds4moe_dims *dims, const ds4moe_weights *w, const void *x, int32_t T, const float *y,
               bool need_y, const ds4moe_routing *r, void *ws, size_t ws_bytes, int mode, Layout *L) {
  int st = validate_dims(dims);
  if (st) return st;
  if (T < 0 || T > kMaxTokens) return DS4MOE_ERR_SHAPE;
  if (mode == DS4MOE_MODE_DECODE && (T < 1 || T > 16)) return DS4MOE_ERR_SHAPE;
  st = validate_weights(*dims, w, mode != DS4MOE_MODE_ROUTE);
  if (st) return st;
  st = validate_routing(r);
  if (st) return st;
  if (T == 0) return DS4MOE_OK;
  if (!x || (need_y && !y)) return DS4MOE_ERR_NULL;
  if (!aligned(x, 16) || (need_y && !aligned(y, 16))) return DS4MOE_ERR_ALIGN;
  *L = make_layout(*dims, T, mode);
  if (!ws) return DS4MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return DS4MOE_ERR_ALIGN;
  if (ws_bytes < L->total) return DS4MOE_ERR_WORKSPACE;
  return DS4MOE_OK;
}

struct Ptrs {
  float *logits, *w;
  int32_t *idx, *counts, *offsets, *perm;
};

Ptrs routing_ptrs(void *ws, const Layout &L, const ds4moe_routing *r) {
  Ptrs p;
  p.logits = (r && r->logits) ? r->logits : at<float>(ws, L.logits);
  p.idx = (r && r->topk_idx) ? r->topk_idx : at<int32_t>(ws, L.idx);
  p.w = (r && r->topk_w) ? r->topk_w : at<float>(ws, L.w);
  p.counts = (r && r->counts) ? r->counts : at<int32_t>(ws, L.counts);
  p.offsets = (r && r->offsets) ? r->offsets : at<int32_t>(ws, L.offsets);
  p.perm = (r && r->perm) ? r->perm : at<int32_t>(ws, L.perm);
  return p;
}

// kernel slots of ds4moe_forward_timed
enum {
  SL_ROUTER = 0, SL_ROUTE, SL_PERMUTE, SL_GATEUP, SL_DOWN, SL_SHGATEUP, SL_SHDOWN, SL_COMBINE, SL_CPLAN, SL_CFILL,
  SL_SHCONV, SL_N
};
static_assert(SL_N == DS4MOE_N_TIMED_KERNELS, "timed kernel slots");

int forward(const ds4moe_dims *dims, const ds4moe_weights *w, const void *x, int32_t T, float *y,
            ds4moe_routing *route_out, void *ws, size_t ws_bytes, void *stream, int mode,
            const Timing *tms = nullptr, const CacheCall *cc = nullptr) {
  Layout L;
  int st = check_call(dims, w, x, T, y, true, route_out, ws, ws_bytes, mode, &L);
  if (st || T == 0) return st;
  const ds4moe_dims &d = *dims;
  hipStream_t s = (hipStream_t)stream;
  auto tm = [&](int slot) -> const Timing * { return tms ? tms + slot : nullptr; };
  const bool xb = d.x_dtype == DS4MOE_BF16, wb = d.router_dtype == DS4MOE_BF16;
  const Ptrs p = routing_ptrs(ws, L, route_out);

  XPrep xp{x, xb, at<_Float16>(ws, L.x16), at<_Float16>(ws, L.xs_hi), at<_Float16>(ws, L.xs_lo),
           at<int32_t>(ws, L.xexp), mode == DS4MOE_MODE_PREFILL ? at<int32_t>(ws, L.xe16) : nullptr};
  const bool dec = mode == DS4MOE_MODE_DECODE;
  RouteOut ro{p.idx, p.w, p.counts, p.offsets, p.perm, nullptr, nullptr, nullptr, L.tile_n, nullptr, 0, xp.xexp};
  if (!dec) {
    ro.pos = at<int32_t>(ws, L.pos);
    ro.pexp = at<int32_t>(ws, L.pexp);
    ro.tiles = at<TileT>(ws, L.tiles);
    ro.ntiles = at<int32_t>(ws, L.ntiles);
    ro.zeros = at<_Float16>(ws, L.zeros);
    ro.nzeros = L.nzeros;
  }
  DecTile *dtiles = nullptr;
  if (dec) dtiles = at<DecTile>(ws, L.tiles);
  int32_t *ntiles = at<int32_t>(ws, L.ntiles);
  // decode with T <= 4: the gate/up kernel routes the batch itself (not
  // through the cache, whose plan sits between routing and gate/up)
  const bool fused_route = dec && L.sliced && T <= 4 && !cc;
  DecRoute rr{at<double>(ws, L.part), router_nslice(d.hidden, T), w->router_bias, p.logits, d.n_experts, d.top_k, ro,
              dtiles, ntiles};
  if (L.sliced) {
    TRY(launch_router_sliced(x, xb, w->router_w, wb, at<double>(ws, L.part), T, d.n_experts, d.hidden, &xp, s,
                             tm(SL_ROUTER)));
    if (!fused_route)
      TRY(launch_route_dec(at<double>(ws, L.part), router_nslice(d.hidden, T), w->router_bias, p.logits, T,
                           d.n_experts, d.top_k, ro, dtiles, ntiles, s, tm(SL_ROUTE)));
  } else {
    TRY(launch_router_tiled(x, xb, w->router_w, wb, w->router_bias, p.logits, T, d.n_experts, d.hidden, s,
                            tm(SL_ROUTER)));
    TRY(launch_route_chunked(p.logits, T, d.n_experts, d.top_k, d.hidden, &xp, ro, at<int32_t>(ws, L.ccnt),
                             at<int32_t>(ws, L.cbase), at<int32_t>(ws, L.lrank), s, tm(SL_ROUTE), tm(SL_PERMUTE)));
  }

  GemmArgs ga{};
  ga.gate = (const uint8_t *)w->gate;
  ga.up = (const uint8_t *)w->up;
  ga.down = (const uint8_t *)w->down;
  ga.gu_bytes = ds4moe_packed_bytes_bits(d.inter, d.hidden, d.expert_bits);
  ga.d_bytes = ds4moe_packed_bytes_bits(d.hidden, d.inter, down_bits(d));
  if (cc) {  // experts through the cache: tiles name slots, the kernels read the slot arrays
    if (dec) {
      TRY(launch_cache_plan(cc->st, dtiles, ntiles, cc->S, d.n_experts, s, tm(SL_CPLAN)));
      TRY(launch_cache_fill(cc->st, cc->st.frange, cc->hg, cc->hu, cc->hd, ga.gu_bytes, ga.d_bytes,
                            L.max_tiles < cc->S ? L.max_tiles : cc->S, s, tm(SL_CFILL)));
    } else {
      TRY(launch_cache_plan_prefill(cc->st, p.counts, p.offsets, ro.tiles, L.tile_n, cc->S, d.n_experts, s));
    }
    ga.gate = cc->st.gate;
    ga.up = cc->st.up;
    ga.down = cc->st.down;
  }
  ga.bits = d.expert_bits;
  ga.bits_dn = down_bits(d);
  ga.tiles = ro.tiles;
  ga.ntiles = ntiles;
  ga.perm = p.perm;
  ga.k = d.top_k;
  ga.H = d.hidden;
  ga.I = d.inter;
  ga.Ipad = L.Ipad;
  ga.x16 = xp.x16;
  ga.xs_hi = xp.xs_hi;
  ga.xs_lo = xp.xs_lo;
  ga.xexp = xp.xexp;
  ga.pexp = dec ? nullptr : ro.pexp;
  ga.xe16 = xp.xe16;
  ga.h = at<_Float16>(ws, L.h);
  ga.hs_hi = at<_Float16>(ws, L.hs_hi);
  ga.hs_lo = at<_Float16>(ws, L.hs_lo);
  ga.yp = dec ? nullptr : at<float>(ws, L.yp);
  ga.zeros = ro.zeros;
  ga.dtiles = dtiles;
  ga.dt_cap = L.max_tiles;
  ga.wsb = (const uint8_t *)ws;
  ga.ws_len = (uint32_t)(L.total < (size_t)DS4_WS_WINDOW ? L.total : (size_t)DS4_WS_WINDOW);
  ga.o_x16 = (uint32_t)L.x16;
  ga.o_xs_hi = (uint32_t)L.xs_hi;
  ga.o_xs_lo = (uint32_t)L.xs_lo;
  ga.o_h = (uint32_t)L.h;
  ga.o_hs_hi = (uint32_t)L.hs_hi;
  ga.o_hs_lo = (uint32_t)L.hs_lo;
  ga.T = T;
  ga.tile_n = L.tile_n;
  ga.dpart = (dec && T > 4) ? at<float>(ws, L.dpart) : nullptr;
  ga.y = y;

  float *ysh = nullptr;
  auto shared = [&]() -> int {
    if (d.shared_inter <= 0) return DS4MOE_OK;
    _Float16 *hsh = at<_Float16>(ws, L.hsh);
    ysh = at<float>(ws, L.ysh);
    const uint16_t *sg = (const uint16_t *)w->sh_gate, *su = (const uint16_t *)w->sh_up,
                   *sd = (const uint16_t *)w->sh_down;
    _Float16 *w16 = nullptr;
    if (!dec && T >= SHARED_DENSE_MIN_T) {
      w16 = at<_Float16>(ws, L.shw);
      TRY(launch_shared_convert(sg, su, sd, w16, d.hidden, d.shared_inter, s, tm(SL_SHCONV)));
    }
    TRY(launch_shared_gateup(sg, su, w16, xp.x16, xp.xexp, hsh, T, d.hidden, d.shared_inter, s, tm(SL_SHGATEUP)));
    TRY(launch_shared_down(sd, w16, hsh, xp.xexp, ysh, T, d.hidden, d.shared_inter, s, tm(SL_SHDOWN)));
    return DS4MOE_OK;
  };
  if (dec) {
    TRY(launch_gateup_dec(ga, L.max_tiles, fused_route ? &rr : nullptr, s, tm(SL_GATEUP)));
    st = shared();
    if (st) return st;
    ga.ysh = ysh;
    TRY(launch_down_combine_dec(ga, s, tm(SL_DOWN), T > 4 ? tm(SL_COMBINE) : nullptr));
  } else if (cc) {
    // batch j: load its misses, then its tiles through gate/up and down; the
    // host launches the most batches the call can need, the plan leaves the
    // ones past the last empty (no fill items, no tiles)
    const int64_t A = (int64_t)T * d.top_k;
    const int used_max = (int)(A < d.n_experts ? A : d.n_experts);
    const int nb_max = (used_max + cc->S - 1) / cc->S;
    const int64_t cap64 = A / L.tile_n + (cc->S < used_max ? cc->S : used_max);
    const int cap = (int)(cap64 < L.max_tiles ? cap64 : L.max_tiles);  // tiles of one batch
    for (int j = 0; j < nb_max; ++j) {
      TRY(launch_cache_fill(cc->st, cc->st.frange + 2 * j, cc->hg, cc->hu, cc->hd, ga.gu_bytes, ga.d_bytes,
                            cc->S < used_max ? cc->S : used_max, s));
      GemmArgs gb = ga;
      gb.ntiles = cc->st.brange + 2 * j;
      TRY(launch_gateup(gb, cap, s));
      TRY(launch_down(gb, cap, s));
    }
    st = shared();
    if (st) return st;
    TRY(launch_combine(ga.yp, ro.pos, p.w, xp.xexp, ysh, y, T, d.top_k, d.hidden, s, tm(SL_COMBINE)));
  } else {
    TRY(launch_gateup(ga, L.max_tiles, s, tm(SL_GATEUP)));
    TRY(launch_down(ga, L.max_tiles, s, tm(SL_DOWN)));
    st = shared();
    if (st) return st;
    TRY(launch_combine(ga.yp, ro.pos, p.w, xp.xexp, ysh, y, T, d.top_k, d.hidden, s, tm(SL_COMBINE)));
  }
  return DS4MOE_OK;
}

// grid bounds of the pack (one workgroup per unit) and dequant (one thread
// per weight) launches: fewer than 2^39 padded weights in all
bool fits_grid(int64_t n_mats, int64_t rows, int64_t cols) {
  const int64_t per = rows * ((cols + 255) / 256) * 256;
  return n_mats <= (((int64_t)1 << 39) - 1) / per;
}

}  // namespace

extern "C" {

const char *ds4moe_status_str(int status) {
  switch (status) {
    case DS4MOE_OK: return "ok";
    case DS4MOE_ERR_NULL: return "required pointer is NULL";
    case DS4MOE_ERR_SHAPE: return "size out of the supported range";
    case DS4MOE_ERR_DTYPE: return "unknown dtype";
    case DS4MOE_ERR_ALIGN: return "pointer not aligned";
    case DS4MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case DS4MOE_ERR_UNSUPPORTED: return "unsupported request";
    case DS4MOE_ERR_HIP: return "HIP launch or runtime error";
    case DS4MOE_ERR_HOSTMEM: return "expert weights are not in pinned host memory";
    default: return "unknown status";
  }
}

int ds4moe_version(void) { return kVersion; }

size_t ds4moe_packed_bytes_bits(int64_t rows, int64_t cols, int32_t bits) {
  if (bits != 2 && bits != 4 && bits != 5 && bits != 6) return 0;
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % 16) return 0;
  if (cols % 256 && 256 % cols) return 0;
  if (rows > ((int64_t)1 << 31) || cols > ((int64_t)1 << 31)) return 0;
  const int64_t nchunks = (cols + 255) / 256;
  return (size_t)(rows / 16) * (size_t)nchunks * (bits == 2 ? 1344u : bits == 4 ? 2368u : 3392u);
}

size_t ds4moe_packed_bytes(int64_t rows, int64_t cols) { return ds4moe_packed_bytes_bits(rows, cols, 2); }

int ds4moe_pack(void *dst, const void *canonical, int64_t n_mats, int64_t rows, int64_t cols, int32_t bits,
                void *stream) {
  if (n_mats < 0) return DS4MOE_ERR_SHAPE;
  if (!ds4moe_packed_bytes_bits(rows, cols, bits) || !fits_grid(n_mats, rows, cols)) return DS4MOE_ERR_SHAPE;
  if (n_mats == 0) return DS4MOE_OK;
  if (!dst || !canonical) return DS4MOE_ERR_NULL;
  if (!aligned(dst, 16)) return DS4MOE_ERR_ALIGN;
  return hip_status(launch_pack(dst, canonical, n_mats, rows, cols, bits, (hipStream_t)stream));
}

int ds4moe_dequant(float *dst, const void *packed, int64_t n_mats, int64_t rows, int64_t cols, int32_t bits,
                   void *stream) {
  if (n_mats < 0) return DS4MOE_ERR_SHAPE;
  if (!ds4moe_packed_bytes_bits(rows, cols, bits) || !fits_grid(n_mats, rows, cols)) return DS4MOE_ERR_SHAPE;
  if (n_mats == 0) return DS4MOE_OK;
  if (!dst || !packed) return DS4MOE_ERR_NULL;
  if (!aligned(dst, 4) || !aligned(packed, 16)) return DS4MOE_ERR_ALIGN;
  return hip_status(launch_dequant(dst, packed, n_mats, rows, cols, bits, (hipStream_t)stream));
}

int ds4moe_pack_q2k(void *dst, const void *canonical, int64_t n_mats, int64_t rows, int64_t cols, void *stream) {
  return ds4moe_pack(dst, canonical, n_mats, rows, cols, 2, stream);
}

int ds4moe_dequant_q2k(float *dst, const void *packed, int64_t n_mats, int64_t rows, int64_t cols, void *stream) {
  return ds4moe_dequant(dst, packed, n_mats, rows, cols, 2, stream);
}

size_t ds4moe_workspace_bytes(const ds4moe_dims *dims, int32_t T, int32_t mode) {
  if (validate_dims(dims) != DS4MOE_OK) return 0;
  if (T < 0 || T > kMaxTokens) return 0;
  if (mode != DS4MOE_MODE_ROUTE && mode != DS4MOE_MODE_DECODE && mode != DS4MOE_MODE_PREFILL) return 0;
  if (T == 0) return 256;
  return make_layout(*dims, T, mode).total;
}

int ds4moe_route(const ds4moe_dims *dims, const ds4moe_weights *w, const void *x, int32_t T, ds4moe_routing *out,
                 void *ws, size_t ws_bytes, void *stream) {
  if (!out) return DS4MOE_ERR_NULL;
  Layout L;
  int st = check_call(dims, w, x, T, nullptr, false, out, ws, ws_bytes, DS4MOE_MODE_ROUTE, &L);
  if (st || T == 0) return st;
  const ds4moe_dims &d = *dims;
  hipStream_t s = (hipStream_t)stream;
  const bool xb = d.x_dtype == DS4MOE_BF16, wb = d.router_dtype == DS4MOE_BF16;
  const Ptrs p = routing_ptrs(ws, L, out);
  RouteOut ro{p.idx, p.w, p.counts, p.offsets, p.perm, nullptr, nullptr, nullptr, kTileDecode, nullptr, 0};
  if (L.sliced) {
    TRY(launch_router_sliced(x, xb, w->router_w, wb, at<double>(ws, L.part), T, d.n_experts, d.hidden, nullptr,
                             s));
    TRY(launch_route_dec(at<double>(ws, L.part), router_nslice(d.hidden, T), w->router_bias, p.logits, T, d.n_experts,
                         d.top_k, ro, nullptr, nullptr, s));
    return DS4MOE_OK;
  }
  TRY(launch_router_tiled(x, xb, w->router_w, wb, w->router_bias, p.logits, T, d.n_experts, d.hidden, s));
  TRY(launch_route_chunked(p.logits, T, d.n_experts, d.top_k, d.hidden, nullptr, ro, at<int32_t>(ws, L.ccnt),
                           at<int32_t>(ws, L.cbase), at<int32_t>(ws, L.lrank), s));
  return DS4MOE_OK;
}

int ds4moe_forward_decode(const ds4moe_dims *dims, const ds4moe_weights *w, const void *x, int32_t T, float *y,
                          ds4moe_routing *route_out, void *ws, size_t ws_bytes, void *stream) {
  return forward(dims, w, x, T, y, route_out, ws, ws_bytes, stream, DS4MOE_MODE_DECODE);
}

int ds4moe_forward_prefill(const ds4moe_dims *dims, const ds4moe_weights *w, const void *x, int32_t T, float *y,
                           ds4moe_routing *route_out, void *ws, size_t ws_bytes, void *stream) {
  return forward(dims, w, x, T, y, route_out, ws, ws_bytes, stream, DS4MOE_MODE_PREFILL);
}

size_t ds4moe_cache_bytes(const ds4moe_dims *dims, int32_t n_slots) {
  if (validate_dims(dims) != DS4MOE_OK) return 0;
  if (n_slots < 1 || n_slots > dims->n_experts) return 0;
  return make_cache_layout(*dims, n_slots).total;
}

namespace {
int check_cache(const ds4moe_dims *dims, int32_t n_slots, const void *cache, size_t cache_bytes, CacheLayout *C) {
  int st = validate_dims(dims);
  if (st) return st;
  if (n_slots < 1 || n_slots > dims->n_experts) return DS4MOE_ERR_SHAPE;
  if (!cache) return DS4MOE_ERR_NULL;
  if (!aligned(cache, 256)) return DS4MOE_ERR_ALIGN;
  *C = make_cache_layout(*dims, n_slots);
  if (cache_bytes < C->total) return DS4MOE_ERR_WORKSPACE;
  return DS4MOE_OK;
}

// device-visible address of pinned host memory (nullptr for anything else:
// device memory, pageable host memory)
const void *host_device_ptr(const void *h) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, h) != hipSuccess || a.type != hipMemoryTypeHost) {
    (void)hipGetLastError();  // clear the error the query left
    return nullptr;
  }
  void *d = nullptr;
  if (hipHostGetDevicePointer(&d, const_cast<void *>(h), 0) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return d;
}
}  // namespace

int ds4moe_cache_reset(const ds4moe_dims *dims, int32_t n_slots, void *cache, size_t cache_bytes, void *stream) {
  CacheLayout C;
  const int st = check_cache(dims, n_slots, cache, cache_bytes, &C);
  if (st) return st;
  return hip_status(launch_cache_reset(cache_state(cache, C), n_slots, dims->n_experts, (hipStream_t)stream));
}

int ds4moe_forward_decode_cached(const ds4moe_dims *dims, const ds4moe_weights *w, int32_t n_slots, void *cache,
                                 size_t cache_bytes, const void *x, int32_t T, float *y, ds4moe_routing *route_out,
                                 void *ws, size_t ws_bytes, void *const *events, void *stream) {
  CacheLayout C;
  int st = check_cache(dims, n_slots, cache, cache_bytes, &C);
  if (st) return st;
  if (T < 1 || T > 16) return DS4MOE_ERR_SHAPE;
  const int64_t used = (int64_t)T * dims->top_k < dims->n_experts ? (int64_t)T * dims->top_k : dims->n_experts;
  if (n_slots < used) return DS4MOE_ERR_SHAPE;  // every expert of the batch needs a slot at once
  st = validate_weights(*dims, w, true);
  if (st) return st;
  Layout L;
  st = check_call(dims, w, x, T, y, true, route_out, ws, ws_bytes, DS4MOE_MODE_DECODE, &L);
  if (st) return st;
  Timing tms[SL_N];
  if (events) {
    for (int i = 0; i < SL_N; ++i) {
      if (!events[2 * i] || !events[2 * i + 1]) return DS4MOE_ERR_NULL;
      tms[i].start = (hipEvent_t)events[2 * i];
      tms[i].stop = (hipEvent_t)events[2 * i + 1];
    }
  }
  CacheCall cc{cache_state(cache, C), n_slots, host_device_ptr(w->gate), host_device_ptr(w->up),
               host_device_ptr(w->down)};
  if (!cc.hg || !cc.hu || !cc.hd) return DS4MOE_ERR_HOSTMEM;
  return forward(dims, w, x, T, y, route_out, ws, ws_bytes, stream, DS4MOE_MODE_DECODE, events ? tms : nullptr,
                 &cc);
}

// Scratch memory of ds4moe_forward_decode_noalloc: a fixed array in every
// GPU's memory, in place of the caller's workspace.  In host code `scratch`
// names a host-side stand-in, never the device array: its device address is
// looked up once per device and only that address is handed to the kernels.
constexpr size_t kNoAllocScratchBytes = DS4MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kNoAllocMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[kNoAllocMaxDevices] = {};

// device address of `scratch` on the current device (looked up on the
// device's first call, with that device current)
int scratch_ptr(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DS4MOE_ERR_HIP;
  if (dev < 0 || dev >= kNoAllocMaxDevices) return DS4MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DS4MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DS4MOE_OK;
}
}  // namespace

int ds4moe_forward_decode_noalloc(const ds4moe_dims *dims, const ds4moe_weights *w, const void *x, int32_t T,
                                  float *y, ds4moe_routing *route_out, void *stream) {
  // every argument is checked before any HIP call: a stand-in workspace
  // address (aligned, never dereferenced) of the scratch size makes check_call
  // report a call whose workspace would not fit as DS4MOE_ERR_WORKSPACE
  Layout L;
  int st = check_call(dims, w, x, T, y, true, route_out, reinterpret_cast<void *>((uintptr_t)256),
                      kNoAllocScratchBytes, DS4MOE_MODE_DECODE, &L);
  if (st) return st;
  void *ws = nullptr;
  st = scratch_ptr(&ws);
  if (st) return st;
  return forward(dims, w, x, T, y, route_out, ws, kNoAllocScratchBytes, stream, DS4MOE_MODE_DECODE);
}

int ds4moe_forward_prefill_cached(const ds4moe_dims *dims, const ds4moe_weights *w, int32_t n_slots, void *cache,
                                  size_t cache_bytes, const void *x, int32_t T, float *y, ds4moe_routing *route_out,
                                  void *ws, size_t ws_bytes, void *stream) {
  CacheLayout C;
  int st = check_cache(dims, n_slots, cache, cache_bytes, &C);
  if (st) return st;
  st = validate_weights(*dims, w, true);
  if (st) return st;
  Layout L;
  st = check_call(dims, w, x, T, y, true, route_out, ws, ws_bytes, DS4MOE_MODE_PREFILL, &L);
  if (st || T == 0) return st;
  CacheCall cc{cache_state(cache, C), n_slots, host_device_ptr(w->gate), host_device_ptr(w->up),
               host_device_ptr(w->down)};
  if (!cc.hg || !cc.hu || !cc.hd) return DS4MOE_ERR_HOSTMEM;
  return forward(dims, w, x, T, y, route_out, ws, ws_bytes, stream, DS4MOE_MODE_PREFILL, nullptr, &cc);
}

int ds4moe_cache_stats(const ds4moe_dims *dims, int32_t n_slots, const void *cache, size_t cache_bytes,
                       uint64_t *out, void *stream) {
  CacheLayout C;
  const int st = check_cache(dims, n_slots, cache, cache_bytes, &C);
  if (st) return st;
  if (!out) return DS4MOE_ERR_NULL;
  const CacheHdr *h = reinterpret_cast<const CacheHdr *>(reinterpret_cast<const char *>(cache) + C.hdr);
  return hip_status(hipMemcpyAsync(out, &h->calls, 3 * sizeof(uint64_t), hipMemcpyDeviceToHost, (hipStream_t)stream));
}

int ds4moe_forward_timed(int32_t mode, const ds4moe_dims *dims, const ds4moe_weights *w, const void *x, int32_t T,
                         float *y, ds4moe_routing *route_out, void *ws, size_t ws_bytes, void *const *events,
                         void *stream) {
  static_assert(SL_N == DS4MOE_N_TIMED_KERNELS, "kernel slots");
  if (mode != DS4MOE_MODE_DECODE && mode != DS4MOE_MODE_PREFILL) return DS4MOE_ERR_SHAPE;
  if (!events) return DS4MOE_ERR_NULL;
  Timing tms[SL_N];
  for (int i = 0; i < SL_N; ++i) {
    if (!events[2 * i] || !events[2 * i + 1]) return DS4MOE_ERR_NULL;
    tms[i].start = (hipEvent_t)events[2 * i];
    tms[i].stop = (hipEvent_t)events[2 * i + 1];
  }
  return forward(dims, w, x, T, y, route_out, ws, ws_bytes, stream, mode, tms);
}

}  // extern "C"
