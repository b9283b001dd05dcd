// Router: fp64-accumulated logits, sqrt(softplus) scores, top-k by wavefront
// reductions, weight normalisation, activation preparation, and the
// token-to-expert histogram / scan / stable permutation.
//
// Score: the router numeric test described on the opensource-hub.com
// "antirez/ds4" page (FAQ #1) shows log(1 + exp(x)) in fp32 losing precision
// near logit -12; the fix evaluates log1p by a four-term series when
// exp(x) < 1/32, with the series input clamped.  Here softplus(l) is
// max(l,0) + log1p(u), u = exp(-|l|) <= 1, which is the same thing for l <= 0
// and never overflows for large l.
#include "common.h"
#include "launch.h"

namespace ds4 {

template <bool BF16>
__device__ __forceinline__ void load4_as_double(const void *p, int64_t idx, double out[4]) {
  if (BF16) {
    const u2 v = *reinterpret_cast<const u2 *>(reinterpret_cast<const uint16_t *>(p) + idx);
    out[0] = (double)bf16_bits_to_float((uint16_t)(v.x & 0xFFFF));
    out[1] = (double)bf16_bits_to_float((uint16_t)(v.x >> 16));
    out[2] = (double)bf16_bits_to_float((uint16_t)(v.y & 0xFFFF));
    out[3] = (double)bf16_bits_to_float((uint16_t)(v.y >> 16));
  } else {
    const f4 v = *reinterpret_cast<const f4 *>(reinterpret_cast<const float *>(p) + idx);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  }
}

// ---------------------------------------------------------------- logits, T <= 16, sliced
// Grid (E/4 expert groups) x (H/256 column slices): wave = one expert, lane =
// 4 columns of the slice, every token.  Partial sums of a slice are reduced
// over the 64 lanes in lane order through LDS and stored per slice in fp64;
// the routing kernel adds the slices in slice order.  Workgroups of expert
// group 0 also convert their slice of x to fp16 and form the 16-column sums.
template <bool XB, bool WB>
__global__ __launch_bounds__(256) void k_router_sliced(const void *__restrict__ x, const void *__restrict__ wr,
                                                       double *__restrict__ part, int T, int E, int H, XPrep xp,
                                                       bool do_x) {
  __shared__ double red[4][16][65];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 4 + wave;
  const int slice = blockIdx.y;
  const int h = slice * 256 + 4 * lane;
  double acc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) acc[t] = 0.0;
  if (e < E) {
    double w4[4];
    load4_as_double<WB>(wr, (int64_t)e * H + h, w4);
    double x4[16][4];
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (t < T) load4_as_double<XB>(x, (int64_t)t * H + h, x4[t]);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if (t < T) {
        acc[t] = fma(x4[t][0], w4[0], acc[t]);
        acc[t] = fma(x4[t][1], w4[1], acc[t]);
        acc[t] = fma(x4[t][2], w4[2], acc[t]);
        acc[t] = fma(x4[t][3], w4[3], acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 16; ++t)
    if (t < T) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (lane < T && e < E) {
    double v = 0.0;
    for (int l = 0; l < 64; ++l) v += red[wave][lane][l];
    part[((int64_t)slice * T + lane) * E + e] = v;
  }
  if (do_x && blockIdx.x == 0) {
    const int t = threadIdx.x >> 4, j = threadIdx.x & 15;  // token, sub-block of this slice
    if (t < T) {
      const int64_t base = (int64_t)t * H + slice * 256 + 16 * j;
      float v[16];
      if (xp.x_bf16) {
        const u4 a = *reinterpret_cast<const u4 *>(reinterpret_cast<const uint16_t *>(x) + base);
        const u4 b = *reinterpret_cast<const u4 *>(reinterpret_cast<const uint16_t *>(x) + base + 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16_bits_to_float((uint16_t)(a[i] & 0xFFFF));
          v[2 * i + 1] = bf16_bits_to_float((uint16_t)(a[i] >> 16));
          v[8 + 2 * i] = bf16_bits_to_float((uint16_t)(b[i] & 0xFFFF));
          v[8 + 2 * i + 1] = bf16_bits_to_float((uint16_t)(b[i] >> 16));
        }
      } else {
        const float *p = reinterpret_cast<const float *>(x) + base;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f4 a = *reinterpret_cast<const f4 *>(p + 4 * q);
          v[4 * q] = a[0]; v[4 * q + 1] = a[1]; v[4 * q + 2] = a[2]; v[4 * q + 3] = a[3];
        }
      }
      h8 o0, o1;
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        o0[i] = (half_t)v[i];
        sum += (float)o0[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        o1[i] = (half_t)v[8 + i];
        sum += (float)o1[i];
      }
      *reinterpret_cast<h8 *>(xp.x16 + base) = o0;
      *reinterpret_cast<h8 *>(xp.x16 + base + 8) = o1;
      const int nsub = H >> 4;
      const int jj = slice * 16 + j;
      const half_t hi = (half_t)sum;
      xp.xs_hi[(int64_t)t * nsub + jj] = hi;
      xp.xs_lo[(int64_t)t * nsub + jj] = (half_t)(sum - (float)hi);
    }
  }
}

// ---------------------------------------------------------------- logits, MFMA fp64
// 64 tokens x 64 experts per workgroup; wave w owns tokens 16w..16w+15 and
// all 64 experts (four 16x16 fp64 accumulators).  Operands are staged in LDS
// as fp32 (bf16 and fp32 inputs are exact there) and widened to fp64;
// v_mfma_f64_16x16x4_f64 accumulates in fp64, where every product of two
// fp32 numbers is exact.
typedef double d4 __attribute__((ext_vector_type(4)));

template <bool XB, bool WB>
__global__ __launch_bounds__(256) void k_router_mfma(const void *__restrict__ x, const void *__restrict__ wr,
                                                     const float *__restrict__ bias, float *__restrict__ logits,
                                                     int T, int E, int H) {
  __shared__ float xs[32][68];  // [k][token]
  __shared__ float ws[32][68];  // [k][expert]
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  d4 acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = (d4){0.0, 0.0, 0.0, 0.0};
  const int lrow = tid >> 2, lk = (tid & 3) * 8;
  for (int k0 = 0; k0 < H; k0 += 32) {
    {
      double v[8];
      const int t = t0 + lrow;
      if (t < T) {
        load4_as_double<XB>(x, (int64_t)t * H + k0 + lk, v);
        load4_as_double<XB>(x, (int64_t)t * H + k0 + lk + 4, v + 4);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) xs[lk + i][lrow] = (float)v[i];
      const int e = e0 + lrow;
      if (e < E) {
        load4_as_double<WB>(wr, (int64_t)e * H + k0 + lk, v);
        load4_as_double<WB>(wr, (int64_t)e * H + k0 + lk + 4, v + 4);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) ws[lk + i][lrow] = (float)v[i];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 32; kk += 4) {
      const double a = (double)xs[kk + g][16 * wave + r16];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const double b = (double)ws[kk + g][16 * n + r16];
        acc[n] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[n], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // D (fp64 16x16x4): lane holds rows (tokens) g, g+4, g+8, g+12 of the wave's 16,
  // column (expert) r16
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int e = e0 + 16 * n + r16;
    if (e >= E) continue;
    const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * wave + g + 4 * i;
      if (t < T) logits[(int64_t)t * E + e] = (float)(acc[n][i] + b);
    }
  }
}

// ---------------------------------------------------------------- score
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

// order-preserving key: larger logit first, then lower expert index; NaN last
__device__ __forceinline__ uint64_t rank_key(float l, int e) {
  uint32_t u = __float_as_uint(l);
  uint32_t ord;
  if (l != l) {
    ord = 0u;
  } else {
    if (u == 0x80000000u) u = 0u;  // -0 == +0
    ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  if (ord == 0u) return __uint_as_float(0x7FC00000u);
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  return __uint_as_float(u);
}

// max with the value DPP-shifted right by N lanes inside each 16-lane row
// (lanes with no source keep their own value)
template <int N>
__device__ __forceinline__ uint64_t dpp_max_shr(uint64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, 0x110 | N, 0xF, 0xF, false);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, 0x110 | N, 0xF, 0xF, false);
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > v ? o : v;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// wave-wide max: row prefix maxima by DPP, then the four row maxima
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_shr<1>(v);
  v = dpp_max_shr<2>(v);
  v = dpp_max_shr<4>(v);
  v = dpp_max_shr<8>(v);
  uint64_t m = readlane_u64(v, 15);
  const uint64_t m1 = readlane_u64(v, 31), m2 = readlane_u64(v, 47), m3 = readlane_u64(v, 63);
  m = m1 > m ? m1 : m;
  m = m2 > m ? m2 : m;
  m = m3 > m ? m3 : m;
  return m;
}

// Top-k of one token by one wave from the logits of experts lane + 64*i held
// in registers; lane j < k writes rank j (index and normalised weight) to
// global memory and, if s_row is given, the index to s_row[j] (LDS) as well.
__device__ void topk_select(const float lv[4], int t, int E, int k, RouteOut ro, int32_t *s_row) {
  const int lane = threadIdx.x & 63;
  uint64_t keys[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    keys[i] = e < E ? rank_key(lv[i], e) : 0ull;  // live keys are never 0
  }
  float sel_l[16];
  int sel_e[16];
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) best = keys[i] > best ? keys[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (keys[i] == best) keys[i] = 0ull;  // keys are unique: removes the winner
    sel_e[j] = e;
    sel_l[j] = key_logit(best);
  }
  float sc[16], S = 0.0f;
  for (int j = 0; j < k; ++j) {
    sc[j] = router_score(sel_l[j]);
    S += sc[j];
  }
  for (int j = 0; j < k; ++j) {
    if (lane == j) {
      ro.idx[(int64_t)t * k + j] = sel_e[j];
      ro.w[(int64_t)t * k + j] = sc[j] / S;
      if (s_row) s_row[j] = sel_e[j];
    }
  }
}

// x[t] -> fp16 and the per-16-element sums of the fp16 values (hi + lo), one wave.
__device__ void xprep_token(int t, int H, const void *xptr, bool x_bf16, _Float16 *x16, _Float16 *xs_hi,
                            _Float16 *xs_lo) {
  const int lane = threadIdx.x & 63;
  const int nsub = H >> 4;
  for (int j = lane; j < nsub; j += 64) {
    const int64_t base = (int64_t)t * H + 16 * j;
    float v[16];
    if (x_bf16) {
      const u4 a = *reinterpret_cast<const u4 *>(reinterpret_cast<const uint16_t *>(xptr) + base);
      const u4 b = *reinterpret_cast<const u4 *>(reinterpret_cast<const uint16_t *>(xptr) + base + 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_float((uint16_t)(a[i] & 0xFFFF));
        v[2 * i + 1] = bf16_bits_to_float((uint16_t)(a[i] >> 16));
        v[8 + 2 * i] = bf16_bits_to_float((uint16_t)(b[i] & 0xFFFF));
        v[8 + 2 * i + 1] = bf16_bits_to_float((uint16_t)(b[i] >> 16));
      }
    } else {
      const float *p = reinterpret_cast<const float *>(xptr) + base;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f4 a = *reinterpret_cast<const f4 *>(p + 4 * q);
        v[4 * q] = a[0]; v[4 * q + 1] = a[1]; v[4 * q + 2] = a[2]; v[4 * q + 3] = a[3];
      }
    }
    h8 o0, o1;
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o0[i] = (half_t)v[i];
      sum += (float)o0[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o1[i] = (half_t)v[8 + i];
      sum += (float)o1[i];
    }
    *reinterpret_cast<h8 *>(x16 + base) = o0;
    *reinterpret_cast<h8 *>(x16 + base + 8) = o1;
    const half_t hi = (half_t)sum;
    xs_hi[(int64_t)t * nsub + j] = hi;
    xs_lo[(int64_t)t * nsub + j] = (half_t)(sum - (float)hi);
  }
}

// Large T: one workgroup per chunk of 64 tokens (wave w: tokens 16w..16w+15).
// Besides top-k and the activation preparation it records, for the stable
// permutation, the chunk's count per expert and each assignment's rank among
// the chunk's assignments to the same expert (earlier tokens first).
constexpr int CHUNK = 64;

__global__ __launch_bounds__(256) void k_topk_chunk(const float *__restrict__ logits, int T, int E, int k, int H,
                                                    XPrep xp, bool do_x, RouteOut ro, int32_t *__restrict__ ccnt,
                                                    int32_t *__restrict__ lrank) {
  __shared__ int32_t s_idx[CHUNK * 16];
  __shared__ uint32_t s_mask[256 * 2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = blockIdx.x * CHUNK;
  for (int i = threadIdx.x; i < E * 2; i += 256) s_mask[i] = 0u;
  for (int q = 0; q < CHUNK / 4; ++q) {
    const int tl = 16 * wave + q;
    const int t = c0 + tl;
    if (t >= T) break;
    float lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lv[i] = (lane + 64 * i < E) ? logits[(int64_t)t * E + lane + 64 * i] : 0.0f;
    topk_select(lv, t, E, k, ro, s_idx + tl * k);
    if (do_x) xprep_token(t, H, xp.x, xp.x_bf16, xp.x16, xp.xs_hi, xp.xs_lo);
  }
  __syncthreads();
  const int nt = min(CHUNK, T - c0);
  for (int a = threadIdx.x; a < nt * k; a += 256) {
    const int tl = a / k;
    atomicOr(&s_mask[s_idx[a] * 2 + (tl >> 5)], 1u << (tl & 31));
  }
  __syncthreads();
  for (int a = threadIdx.x; a < nt * k; a += 256) {
    const int tl = a / k;
    const uint32_t *m = s_mask + s_idx[a] * 2;
    int r = __popc(m[tl >> 5] & ((1u << (tl & 31)) - 1u));
    if (tl >= 32) r += __popc(m[0]);
    lrank[(int64_t)c0 * k + a] = r;
  }
  for (int e = threadIdx.x; e < E; e += 256)
    ccnt[(int64_t)blockIdx.x * E + e] = __popc(s_mask[2 * e]) + __popc(s_mask[2 * e + 1]);
}

// One workgroup: per-expert exclusive prefix over chunks (base), counts,
// offsets, tile list, and the zero row for the GEMMs.
__global__ __launch_bounds__(1024) void k_scan_chunks(int T, int E, int k, int nchunk,
                                                      const int32_t *__restrict__ ccnt, int32_t *__restrict__ base,
                                                      RouteOut ro) {
  __shared__ int32_t s_cnt[256], s_off[256], s_tb[256];
  const int tid = threadIdx.x;
  if (ro.zeros)
    for (int i = tid; i < ro.nzeros; i += 1024) ro.zeros[i] = (half_t)0.0f;
  if (tid < E) {
    int run = 0;
    for (int c0 = 0; c0 < nchunk; c0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (c0 + u < nchunk) ? ccnt[(int64_t)(c0 + u) * E + tid] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c0 + u < nchunk) {
          base[(int64_t)(c0 + u) * E + tid] = run;
          run += v[u];
        }
    }
    s_cnt[tid] = run;
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    int c[4], nt[4], sc = 0, st = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      c[i] = e < E ? s_cnt[e] : 0;
      nt[i] = (ro.tiles && c[i] > 0) ? (c[i] + ro.tile_n - 1) / ro.tile_n : 0;
      sc += c[i];
      st += nt[i];
    }
    int ic = sc, it = st;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int oc = __shfl_up(ic, off), ot = __shfl_up(it, off);
      if (lane >= off) {
        ic += oc;
        it += ot;
      }
    }
    int rc = ic - sc, rt = it - st;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) {
        s_off[e] = rc;
        s_tb[e] = rt;
        ro.counts[e] = c[i];
        ro.offsets[e] = rc;
      }
      rc += c[i];
      rt += nt[i];
    }
    if (lane == 63) {
      ro.offsets[E] = ic;
      if (ro.ntiles) *ro.ntiles = it;
    }
  }
  __syncthreads();
  for (int e = tid; e < E && ro.tiles; e += 1024) {
    const int c = s_cnt[e];
    const int nt = (c + ro.tile_n - 1) / ro.tile_n;
    for (int i = 0; i < nt; ++i) {
      TileT tl;
      tl.e = e;
      tl.p0 = s_off[e] + i * ro.tile_n;
      tl.n = min(ro.tile_n, c - i * ro.tile_n);
      tl.pad = 0;
      ro.tiles[s_tb[e] + i] = tl;
    }
  }
}

// One workgroup per chunk: perm[offsets[e] + base[chunk][e] + rank] = a.
__global__ __launch_bounds__(256) void k_place_chunks(int T, int E, int k, const int32_t *__restrict__ base,
                                                      const int32_t *__restrict__ lrank, RouteOut ro) {
  const int c0 = blockIdx.x * CHUNK;
  const int nt = min(CHUNK, T - c0);
  for (int i = threadIdx.x; i < nt * k; i += 256) {
    const int64_t a = (int64_t)c0 * k + i;
    const int e = ro.idx[a];
    const int p = ro.offsets[e] + base[(int64_t)blockIdx.x * E + e] + lrank[a];
    ro.perm[p] = (int32_t)a;
    if (ro.pos) ro.pos[a] = p;
  }
}

// ---------------------------------------------------------------- permutation
// Whole workgroup (1024 threads).  Counts by LDS integer atomics (order does
// not matter for integers), exclusive scan by one wave, then a stable
// placement in chunks of 1024 tokens: for each expert a bitmask of the chunk's
// tokens that chose it; the rank of token t = number of set bits below t.
__device__ void permute_block(const int32_t *__restrict__ idx, int T, int E, int k, RouteOut ro,
                              int32_t *s_cnt, int32_t *s_base, int32_t *s_tbase, uint32_t *s_mask) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  if (ro.zeros)
    for (int i = tid; i < ro.nzeros; i += nthr) ro.zeros[i] = (half_t)0.0f;
  for (int e = tid; e < E; e += nthr) s_cnt[e] = 0;
  __syncthreads();
  const int64_t nA = (int64_t)T * k;
  for (int64_t a = tid; a < nA; a += nthr) atomicAdd(&s_cnt[idx[a]], 1);
  __syncthreads();
  if (tid < 64) {
    // exclusive scans of counts and of tiles per expert; 4 experts per lane
    const int lane = tid;
    int c[4], nt[4], sc = 0, st = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      c[i] = e < E ? s_cnt[e] : 0;
      nt[i] = (ro.tiles && c[i] > 0) ? (c[i] + ro.tile_n - 1) / ro.tile_n : 0;
      sc += c[i];
      st += nt[i];
    }
    int ic = sc, it = st;  // inclusive wave scans
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int oc = __shfl_up(ic, off), ot = __shfl_up(it, off);
      if (lane >= off) {
        ic += oc;
        it += ot;
      }
    }
    int rc = ic - sc, rt = it - st;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) {
        s_base[e] = rc;
        s_tbase[e] = rt;
        ro.counts[e] = c[i];
        ro.offsets[e] = rc;
      }
      rc += c[i];
      rt += nt[i];
    }
    if (lane == 63) {
      ro.offsets[E] = ic;
      if (ro.ntiles) *ro.ntiles = it;
    }
  }
  __syncthreads();
  if (ro.tiles) {
    for (int e = tid; e < E; e += nthr) {
      const int c = s_cnt[e];
      const int nt = (c + ro.tile_n - 1) / ro.tile_n;
      for (int i = 0; i < nt; ++i) {
        TileT tl;
        tl.e = e;
        tl.p0 = s_base[e] + i * ro.tile_n;
        tl.n = min(ro.tile_n, c - i * ro.tile_n);
        tl.pad = 0;
        ro.tiles[s_tbase[e] + i] = tl;
      }
    }
  }
  // stable placement, chunks of nthr tokens (nthr <= 1024, 32 words per expert)
  const int words = nthr / 32;
  for (int t0 = 0; t0 < T; t0 += nthr) {
    for (int i = tid; i < E * words; i += nthr) s_mask[i] = 0u;
    __syncthreads();
    const int t = t0 + tid;
    if (t < T)
      for (int j = 0; j < k; ++j) atomicOr(&s_mask[idx[(int64_t)t * k + j] * words + (tid >> 5)], 1u << (tid & 31));
    __syncthreads();
    if (t < T) {
      for (int j = 0; j < k; ++j) {
        const int e = idx[(int64_t)t * k + j];
        const uint32_t *m = s_mask + e * words;
        int rank = __popc(m[tid >> 5] & ((1u << (tid & 31)) - 1u));
        for (int w = 0; w < (tid >> 5); ++w) rank += __popc(m[w]);
        const int p = s_base[e] + rank;
        const int a = t * k + j;
        ro.perm[p] = a;
        if (ro.pos) ro.pos[a] = p;
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += nthr) {
      int c = 0;
      for (int w = 0; w < words; ++w) c += __popc(s_mask[e * words + w]);
      s_base[e] += c;
    }
    __syncthreads();
  }
}

// T <= 16: the whole block adds the slice partial sums of every (token,
// expert) in slice order plus the bias (loads of all slices in flight at
// once), then waves 0..T-1 route one token each from LDS, then the block
// permutes.
__global__ __launch_bounds__(1024) void k_route_small(const double *__restrict__ part, int nslice,
                                                      const float *__restrict__ bias, float *__restrict__ logits,
                                                      int T, int E, int k, RouteOut ro) {
  __shared__ int32_t s_cnt[256], s_base[256], s_tbase[256];
  __shared__ uint32_t s_mask[256 * 32];
  __shared__ int32_t s_idx[16 * 16];
  __shared__ float s_lg[16 * 256];
  const int n = T * E;
  for (int i = threadIdx.x; i < n; i += 1024) {
    // slices in increasing order; loads issued 8 at a time ahead of the adds
    double v = 0.0;
    for (int q0 = 0; q0 < nslice; q0 += 8) {
      double pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) pv[u] = (q0 + u < nslice) ? part[(int64_t)(q0 + u) * n + i] : 0.0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (q0 + u < nslice) v += pv[u];
    }
    const int e = i % E;
    if (bias) v += (double)bias[e];
    const float l = (float)v;
    s_lg[i] = l;
    logits[i] = l;
  }
  __syncthreads();
  const int t = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (t < T) {
    float lv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) lv[q] = (lane + 64 * q < E) ? s_lg[t * E + lane + 64 * q] : 0.0f;
    topk_select(lv, t, E, k, ro, s_idx + t * k);
  }
  __syncthreads();
  permute_block(s_idx, T, E, k, ro, s_cnt, s_base, s_tbase, s_mask);
}

// ---------------------------------------------------------------- launchers
template <bool XB, bool WB>
static hipError_t router_tiled_t(const void *x, const void *wr, const float *bias, float *logits, int T, int E,
                                 int H, hipStream_t s, const Timing *tm) {
  DS4_LAUNCH(tm, (k_router_mfma<XB, WB>), dim3((T + 63) / 64, (E + 63) / 64), dim3(256), 0, s, x, wr, bias,
             logits, T, E, H);
  return hipGetLastError();
}

hipError_t launch_router_tiled(const void *x, bool x_bf16, const void *wr, bool w_bf16, const float *bias,
                               float *logits, int T, int E, int H, hipStream_t s, const Timing *tm) {
  if (x_bf16 && w_bf16) return router_tiled_t<true, true>(x, wr, bias, logits, T, E, H, s, tm);
  if (x_bf16) return router_tiled_t<true, false>(x, wr, bias, logits, T, E, H, s, tm);
  if (w_bf16) return router_tiled_t<false, true>(x, wr, bias, logits, T, E, H, s, tm);
  return router_tiled_t<false, false>(x, wr, bias, logits, T, E, H, s, tm);
}

int chunk_count(int T) { return (T + CHUNK - 1) / CHUNK; }

hipError_t launch_route_chunked(const float *logits, int T, int E, int k, int H, const XPrep *xp, RouteOut ro,
                                int32_t *ccnt, int32_t *base, int32_t *lrank, hipStream_t s, const Timing *tm_topk,
                                const Timing *tm_perm) {
  const int nchunk = chunk_count(T);
  XPrep x = xp ? *xp : XPrep{nullptr, false, nullptr, nullptr, nullptr};
  DS4_LAUNCH(tm_topk, k_topk_chunk, dim3(nchunk), dim3(256), 0, s, logits, T, E, k, H, x, xp != nullptr, ro, ccnt,
             lrank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the permutation slot times the scan; the placement follows it directly
  DS4_LAUNCH(tm_perm, k_scan_chunks, dim3(1), dim3(1024), 0, s, T, E, k, nchunk, ccnt, base, ro);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_place_chunks, dim3(nchunk), dim3(256), 0, s, T, E, k, base, lrank, ro);
  return hipGetLastError();
}

hipError_t launch_route_small(const double *part, int nslice, const float *bias, float *logits, int T, int E,
                              int k, RouteOut ro, hipStream_t s, const Timing *tm) {
  DS4_LAUNCH(tm, k_route_small, dim3(1), dim3(1024), 0, s, part, nslice, bias, logits, T, E, k, ro);
  return hipGetLastError();
}

template <bool XB, bool WB>
static hipError_t router_sliced_t(const void *x, const void *wr, double *part, int T, int E, int H,
                                  const XPrep *xp, hipStream_t s, const Timing *tm) {
  XPrep xx = xp ? *xp : XPrep{nullptr, false, nullptr, nullptr, nullptr};
  DS4_LAUNCH(tm, (k_router_sliced<XB, WB>), dim3((E + 3) / 4, H / 256), dim3(256), 0, s, x, wr, part, T, E, H, xx,
             xp != nullptr);
  return hipGetLastError();
}

hipError_t launch_router_sliced(const void *x, bool x_bf16, const void *wr, bool w_bf16, double *part, int T,
                                int E, int H, const XPrep *xp, hipStream_t s, const Timing *tm) {
  if (x_bf16 && w_bf16) return router_sliced_t<true, true>(x, wr, part, T, E, H, xp, s, tm);
  if (x_bf16) return router_sliced_t<true, false>(x, wr, part, T, E, H, xp, s, tm);
  if (w_bf16) return router_sliced_t<false, true>(x, wr, part, T, E, H, xp, s, tm);
  return router_sliced_t<false, false>(x, wr, part, T, E, H, xp, s, tm);
}

}  // namespace ds4
