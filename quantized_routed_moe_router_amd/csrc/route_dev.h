// Device-side routing of small batches (T <= 16), shared by the routing
// kernel and by the gate/up kernel that routes for itself (T <= 4).
//
// Score: the router numeric test described on the opensource-hub.com
// "antirez/ds4" page (FAQ #1) shows log(1 + exp(x)) in fp32 losing precision
// near logit -12; the fix evaluates log1p by a four-term series when
// exp(x) < 1/32, with the series input clamped.  Here softplus(l) is
// max(l,0) + log1p(u), u = exp(-|l|) <= 1, which is the same thing for l <= 0
// and never overflows for large l.
#pragma once
#include "common.h"
#include "launch.h"

namespace ds4 {

// s = sqrt(max(l,0) + log1p(u)), u = exp(-|l|); log1p(u) by the series
// u - u^2/2 + u^3/3 - u^4/4 for u < 1/32 (series input clamped to 1/32),
// log(1 + u) otherwise.  Max relative error vs. the exact value < 3e-6.
__device__ __forceinline__ float router_score(float l) {
  const float u = expf(-fabsf(l));
  const float uc = fminf(u, 0.03125f);
  const float ser = uc * (1.0f - uc * (0.5f - uc * (0.33333334f - uc * 0.25f)));
  const float lp = (u < 0.03125f) ? ser : logf(1.0f + u);
  return sqrtf(fmaxf(l, 0.0f) + lp);
}

// order-preserving 32-bit key of a logit: larger logit -> larger key; every
// number maps to >= 0x007FFFFF, NaN to 1 (below every number), 0 = no expert
__device__ __forceinline__ uint32_t logit_key(float l) {
  if (l != l) return 1u;
  uint32_t u = __float_as_uint(l);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_logit(uint32_t key) {
  if (key == 1u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// exclusive prefix over the lanes of a wave of a small non-negative value
// (< 2^NB), and the wave total, by one ballot per bit
template <int NB>
__device__ __forceinline__ int wave_excl_prefix(int v, int &total) {
  int pre = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint64_t m = __ballot((v >> b) & 1);
    pre += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
    tot += __popcll(m) << b;
  }
  total = tot;
  return pre;
}

// compiler barrier between LDS accesses of one wave (the wave's LDS
// instructions execute in order)
__device__ __forceinline__ void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Top-k of one token by one wave from its E <= 256 logits in LDS, k <= 16.
// Composite 64-bit keys (logit key, then the inverted expert index; experts
// >= E get logit key 0) are unique and order experts by logit descending,
// ties to the lower index, NaN after every number.  Lane l holds experts
// 4l..4l+3.  The k-th largest of the 64 lane maxima is at most the k-th
// largest key, so the top-k are among the at most 4k keys at or above it;
// those are compacted into LDS and ranked by counting larger candidates.
// sm: 128 wave-private 64-bit LDS words.  Lane j < k ends with rank j:
// expert and normalised weight.
__device__ __forceinline__ void topk_wave(const float *__restrict__ lg, int E, int k, int &my_e, float &my_w,
                                          uint64_t *sm) {
  const int lane = threadIdx.x & 63;
  uint64_t K[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    const uint32_t kk = e < E ? logit_key(lg[e]) : 0u;
    K[i] = ((uint64_t)kk << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
  }
  uint64_t M = K[0] > K[1] ? K[0] : K[1];
  const uint64_t M2 = K[2] > K[3] ? K[2] : K[3];
  M = M > M2 ? M : M2;
  sm[lane] = M;
  wave_lds_order();
  int r = 0;  // lane maxima larger than this lane's
#pragma unroll 16
  for (int j = 0; j < 64; ++j) r += sm[j] > M ? 1 : 0;
  const uint64_t bt = __ballot(r == k - 1);
  const int lt = __ffsll((unsigned long long)bt) - 1;
  const uint32_t tlo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)M, lt);
  const uint32_t thi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(M >> 32), lt);
  const uint64_t tau = ((uint64_t)thi << 32) | tlo;
  int c = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) c += K[i] >= tau ? 1 : 0;
  int nc;
  int p = wave_excl_prefix<3>(c, nc);
  uint64_t *cand = sm + 64;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (K[i] >= tau) cand[p++] = K[i];
  wave_lds_order();
  const uint64_t mine = cand[lane];  // lanes >= nc: stale, not ranked
  int rank = 0;
  for (int j0 = 0; j0 < nc; j0 += 16) {  // j0 + 15 < 64: nc <= 64
#pragma unroll
    for (int j = 0; j < 16; ++j) rank += (j0 + j < nc && cand[j0 + j] > mine) ? 1 : 0;
  }
  if (lane >= nc) rank = 64;
  wave_lds_order();
  if (rank < k) sm[rank] = mine;  // the lane maxima are no longer read
  wave_lds_order();
  my_e = 0;
  float my_l = 0.0f;
  if (lane < k) {
    const uint64_t v = sm[lane];
    my_e = (int)(0xFFFFFFFFu - (uint32_t)v);
    my_l = key_to_logit((uint32_t)(v >> 32));
  }
  wave_lds_order();
  // sum of the k scores: lanes 0..15 (k <= 16), prefix sums inside row 0
  const float sc = lane < k ? router_score(my_l) : 0.0f;
  float S = sc;
  S += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(S), 0x111, 0xF, 0xF, true));  // row_shr:1
  S += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(S), 0x112, 0xF, 0xF, true));  // row_shr:2
  S += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(S), 0x114, 0xF, 0xF, true));  // row_shr:4
  S += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(S), 0x118, 0xF, 0xF, true));  // row_shr:8
  S = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(S), 15));
  my_w = sc / S;
}

// LDS of the small-batch routing of at most MAXT tokens.
template <int MAXT>
struct RouteLds {
  float lg[MAXT * 256];   // logits [T][E]
  int32_t idx[MAXT * 16];  // selected experts [T][k]
  float w[MAXT * 16];      // their weights
  uint32_t tm[256];        // per expert: mask of the tokens that chose it
  int32_t off[256];        // per expert: first position in the permutation
  int32_t tb[256];         // per used expert: its tile (used experts ascending)
  int32_t ntile;           // used experts
  uint64_t sel[MAXT][128];  // top-k scratch of the wave of token t
};

// One workgroup of NTH threads routes T <= MAXT tokens from the router's
// fp64 partial sums part[nslice][T][E]: the slices are added in slice order
// (+ bias) and rounded once to the fp32 logit; wave t picks the top-k of
// token t; then the per-expert token masks, counts and offsets (exclusive
// scan over experts), the stable permutation (tokens ascending within an
// expert) and one DecTile per used expert, in ascending expert order, with
// its token mask and the token's weight for each token that chose it (times
// 2^2e for a token pre-scaled by 2^-e, see token_exp; topk_w is unscaled).
// L.tm, L.tb and L.ntile are valid for every thread on return.  Global
// outputs (logits, ro, dt, ntile) are written only when `out` is set.
template <int NTH, int MAXT>
__device__ __forceinline__ void route_small_block(RouteLds<MAXT> &L, const double *__restrict__ part, int nslice,
                                                  const float *__restrict__ bias, float *__restrict__ logits,
                                                  int T, int E, int k, const RouteOut &ro,
                                                  DecTile *__restrict__ dt, int32_t *__restrict__ ntile, bool out) {
  static_assert(NTH % 64 == 0 && (MAXT * 256) % NTH == 0, "thread count");
  constexpr int Q = MAXT * 256 / NTH;
  constexpr int NW = NTH / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = T * E;
  for (int e = tid; e < 256; e += NTH) L.tm[e] = 0u;
  {
    double v[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) v[q] = 0.0;
    for (int s0 = 0; s0 < nslice; s0 += 4) {
      double pv[Q][4];
#pragma unroll
      for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = tid + NTH * q;
          pv[q][u] = (i < n && s0 + u < nslice) ? part[(int64_t)(s0 + u) * n + i] : 0.0;
        }
#pragma unroll
      for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (s0 + u < nslice) v[q] += pv[q][u];
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int i = tid + NTH * q;
      if (i < n) {
        double vv = v[q];
        if (bias) vv += (double)bias[i % E];
        const float l = (float)vv;
        L.lg[i] = l;
        if (out) logits[i] = l;
      }
    }
  }
  __syncthreads();
  for (int t = wave; t < T; t += NW) {
    int my_e;
    float my_w;
    topk_wave(L.lg + t * E, E, k, my_e, my_w, L.sel[wave]);
    if (lane < k) {
      const int a = t * k + lane;
      L.idx[a] = my_e;
      L.w[a] = my_w;
      if (out) {
        ro.idx[a] = my_e;
        ro.w[a] = my_w;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < T * k; i += NTH) atomicOr(&L.tm[L.idx[i]], 1u << (i / k));
  __syncthreads();
  if (wave == 0) {
    // exclusive scans over experts (4 per lane) of counts and of used flags
    int c[4], u[4], sc = 0, su = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      const uint32_t tm = e < E ? L.tm[e] : 0u;
      c[i] = __popc(tm);
      u[i] = tm != 0u;
      sc += c[i];
      su += u[i];
    }
    int ic, iu;  // totals
    int rc = wave_excl_prefix<7>(sc, ic), ru = wave_excl_prefix<3>(su, iu);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) {
        L.off[e] = rc;
        L.tb[e] = ru;
        if (out) {
          ro.counts[e] = c[i];
          ro.offsets[e] = rc;
        }
      }
      rc += c[i];
      ru += u[i];
    }
    if (lane == 0) {
      L.ntile = iu;
      if (out) {
        ro.offsets[E] = ic;
        if (ntile) *ntile = iu;
      }
    }
  }
  __syncthreads();
  if (!out) return;
  // tiles: header and zero weights for the tokens that did not choose the
  // expert; the weights of those that did are scattered per assignment below
  // (disjoint entries: a token picks an expert at most once)
  for (int e = tid; e < E && dt; e += NTH) {
    const uint32_t tm = L.tm[e];
    if (tm) {
      DecTile *d = dt + L.tb[e];
      d->e = e;
      d->tmask = tm;
      d->pad0 = 0;
      d->pad1 = 0;
#pragma unroll
      for (int t = 0; t < 16; ++t)
        if (!((tm >> t) & 1u)) d->w[t] = 0.0f;
    }
  }
  for (int i = tid; i < T * k; i += NTH) {
    const int e = L.idx[i], t = i / k;
    const int p = L.off[e] + __popc(L.tm[e] & ((1u << t) - 1u));
    ro.perm[p] = i;
    if (ro.pos) ro.pos[i] = p;
    if (dt) dt[L.tb[e]].w[t] = ro.xexp ? scale_2e(L.w[i], ro.xexp[t]) : L.w[i];
  }
}

// The same for one token (T = 1), with less machinery: every selected expert
// takes one assignment, so the k selected experts, ascending, are the tiles,
// each expert's count is 0 or 1 and its offset is the number of selected
// experts below it.  Returns the expert of tile `tile` (< k) to every thread.
template <int NTH>
__device__ __forceinline__ int route_one_token(RouteLds<4> &L, const double *__restrict__ part, int nslice,
                                               const float *__restrict__ bias, float *__restrict__ logits, int E,
                                               int k, const RouteOut &ro, DecTile *__restrict__ dt,
                                               int32_t *__restrict__ ntile, bool out, int tile) {
  static_assert(NTH >= 256 && NTH % 64 == 0, "one thread per expert");
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < E) {
    double v = 0.0;
    for (int s0 = 0; s0 < nslice; s0 += 4) {  // the slices in order, four loads in flight
      double pv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) pv[u] = s0 + u < nslice ? part[(int64_t)(s0 + u) * E + tid] : 0.0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (s0 + u < nslice) v += pv[u];
    }
    if (bias) v += (double)bias[tid];
    const float l = (float)v;
    L.lg[tid] = l;
    if (out) logits[tid] = l;
  }
  __syncthreads();
  if (tid < 64) {
    int my_e;
    float my_w;
    topk_wave(L.lg, E, k, my_e, my_w, L.sel[0]);
    int asc = 0;  // selected experts below this lane's (distinct experts)
    for (int j = 0; j < k; ++j) asc += __builtin_amdgcn_readlane(my_e, j) < my_e ? 1 : 0;
    if (lane < k) {
      L.tb[asc] = my_e;  // tile asc -> expert
      if (out) {
        ro.idx[lane] = my_e;
        ro.w[lane] = my_w;
        ro.perm[asc] = lane;
        if (ro.pos) ro.pos[lane] = asc;
        if (dt) {
          DecTile *d = dt + asc;
          d->e = my_e;
          d->tmask = 1u;
          d->pad0 = 0;
          d->pad1 = 0;
          d->w[0] = ro.xexp ? scale_2e(my_w, ro.xexp[0]) : my_w;
#pragma unroll
          for (int t = 1; t < 16; ++t) d->w[t] = 0.0f;
        }
      }
    }
    if (out && lane == 0) {
      ro.offsets[E] = k;
      if (ntile) *ntile = k;
    }
  }
  __syncthreads();
  if (out && tid < E) {
    int below = 0, sel = 0;
    for (int j = 0; j < k; ++j) {
      const int ej = L.tb[j];
      below += ej < tid ? 1 : 0;
      sel += ej == tid ? 1 : 0;
    }
    ro.counts[tid] = sel;
    ro.offsets[tid] = below;
  }
  return L.tb[tile];
}

}  // namespace ds4
