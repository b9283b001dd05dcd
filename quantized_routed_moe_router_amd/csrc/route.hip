// Router: fp64-accumulated logits, sqrt(softplus) scores, top-k by wavefront
// reductions, weight normalisation, activation preparation, and the
// token-to-expert histogram / scan / stable permutation.  The score
// (sqrt(softplus) with the stable log1p series) and the small-batch routing
// are in route_dev.h.
#include "common.h"
#include "launch.h"
#include "route_dev.h"

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

// 16 consecutive elements of x as fp32 (bf16 widening is exact)
__device__ __forceinline__ void load_x16(const void *xptr, bool x_bf16, int64_t base, float v[16]) {
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
}

// Token t of x -> x' = x * 2^-e in fp16 (max |x'| in [1, 2), see token_exp),
// the per-16-element sums of the fp16 values (hi + lo), and e.  NT threads
// cooperate (one wave, or a whole workgroup of NT threads with `red`: NT/64
// floats of LDS); tix is the thread's index among them.  e comes from the
// whole row; the conversion covers the 16-element chunks [j0, j1) (callers
// that split a row write e from the part with j0 = 0).
template <int NT>
__device__ void xprep_token(int t, int H, const XPrep &xp, int tix, float *red, int j0 = 0, int j1 = 1 << 30) {
  const int nsub = H >> 4;
  float amax = 0.0f;
  for (int j = tix; j < nsub; j += NT) {
    float v[16];
    load_x16(xp.x, xp.x_bf16, (int64_t)t * H + 16 * j, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if constexpr (NT > 64) {
    __syncthreads();  // the previous token's readers of red are done
    if ((tix & 63) == 0) red[tix >> 6] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) amax = fmaxf(amax, red[w]);
  }
  const int e = token_exp(amax);
  if (tix == 0 && j0 == 0) {
    xp.xexp[t] = e;
    if (xp.xe16) *reinterpret_cast<u4 *>(xp.xe16 + 4 * (int64_t)t) = (u4){(uint32_t)e, 0u, 0u, 0u};
  }
  for (int j = j0 + tix; j < min(j1, nsub); j += NT) {
    const int64_t base = (int64_t)t * H + 16 * j;
    float v[16];
    load_x16(xp.x, xp.x_bf16, base, v);
    h8 o0, o1;
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o0[i] = (half_t)ldexpf(v[i], -e);
      sum += (float)o0[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o1[i] = (half_t)ldexpf(v[8 + i], -e);
      sum += (float)o1[i];
    }
    *reinterpret_cast<h8 *>(xp.x16 + base) = o0;
    *reinterpret_cast<h8 *>(xp.x16 + base + 8) = o1;
    const half_t hi = (half_t)sum;
    xp.xs_hi[(int64_t)t * nsub + j] = hi;
    xp.xs_lo[(int64_t)t * nsub + j] = (half_t)(sum - (float)hi);
  }
}

// ---------------------------------------------------------------- logits, T <= 16, sliced
// Grid (E/4 expert groups) x (H/1024 column slices), 256 threads.  The slice
// of x (T tokens x up to 1024 columns) is staged in LDS as fp32; wave = one
// expert, lane = columns 4*lane + 256*i (i < 4).  Products of bf16/fp32
// inputs are exact in fp64, so the per-token sums over the lanes (a
// reduce-scatter butterfly) and over the slices (routing kernel, slice order)
// give the fp64 dot product up to fp64 rounding.  Workgroups also convert
// their column slice of x (token t in expert group t) to pre-scaled fp16 and
// form the 16-column sums.
constexpr int RSLICE = 1024;

template <bool XB, bool WB>
__global__ __launch_bounds__(256) void k_router_sliced(const void *__restrict__ x, const void *__restrict__ wr,
                                                       double *__restrict__ part, int T, int E, int H, XPrep xp,
                                                       bool do_x) {
  __shared__ float xs[16 * RSLICE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x * 4 + wave;
  const int slice = blockIdx.y;
  const int c0 = slice * RSLICE;
  const int cw = min(RSLICE, H - c0);  // multiple of 256
  // weights of this lane's columns (issued first)
  double w[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (e < E && 256 * i < cw) {
      load4_as_double<WB>(wr, (int64_t)e * H + c0 + 256 * i + 4 * lane, w[i]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) w[i][q] = 0.0;
    }
  }
  // stage x[0:T, c0:c0+cw] as fp32: 16-byte loads, all in flight
  {
    constexpr int V = XB ? 8 : 4;  // elements per 16-byte load
    constexpr int MAXL = 16 * RSLICE / V / 256;
    const int per_row = cw / V;
    const int nld = T * per_row;
    u4 v[MAXL];
#pragma unroll
    for (int q = 0; q < MAXL; ++q) {
      const int li = tid + 256 * q;
      if (li < nld) {
        const int t = li / per_row, c = (li - t * per_row) * V;
        const char *src = reinterpret_cast<const char *>(x) + ((int64_t)t * H + c0 + c) * (XB ? 2 : 4);
        v[q] = *reinterpret_cast<const u4 *>(src);
      }
    }
#pragma unroll
    for (int q = 0; q < MAXL; ++q) {
      const int li = tid + 256 * q;
      if (li < nld) {
        const int t = li / per_row, c = (li - t * per_row) * V;
        float *dst = xs + t * RSLICE + c;
        if (XB) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dst[2 * i] = bf16_bits_to_float((uint16_t)(v[q][i] & 0xFFFFu));
            dst[2 * i + 1] = bf16_bits_to_float((uint16_t)(v[q][i] >> 16));
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[i] = __uint_as_float(v[q][i]);
        }
      }
    }
  }
  __syncthreads();
  double acc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    acc[t] = 0.0;
    if (t < T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (256 * i < cw) {
          const f4 xv = *reinterpret_cast<const f4 *>(xs + t * RSLICE + 256 * i + 4 * lane);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[t] = fma((double)xv[q], w[i][q], acc[t]);
        }
      }
    }
  }
  // reduce-scatter over the 64 lanes: after the halving steps lane l holds
  // token ((l>>5)&1)*8 + ((l>>4)&1)*4 + ((l>>3)&1)*2 + ((l>>2)&1) summed over
  // 16 lanes; two more steps complete the sum over all 64
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool up = (lane >> 5) & 1;
    const double send = up ? acc[j] : acc[8 + j];
    const double keep = up ? acc[8 + j] : acc[j];
    acc[j] = keep + __shfl_xor(send, 32);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool up = (lane >> 4) & 1;
    const double send = up ? acc[j] : acc[4 + j];
    const double keep = up ? acc[4 + j] : acc[j];
    acc[j] = keep + __shfl_xor(send, 16);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bool up = (lane >> 3) & 1;
    const double send = up ? acc[j] : acc[2 + j];
    const double keep = up ? acc[2 + j] : acc[j];
    acc[j] = keep + __shfl_xor(send, 8);
  }
  {
    const bool up = (lane >> 2) & 1;
    const double send = up ? acc[0] : acc[1];
    const double keep = up ? acc[1] : acc[0];
    acc[0] = keep + __shfl_xor(send, 4);
  }
  acc[0] += __shfl_xor(acc[0], 2);
  acc[0] += __shfl_xor(acc[0], 1);
  const int tok = ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1);
  if ((lane & 3) == 0 && tok < T && e < E) part[((int64_t)slice * T + tok) * E + e] = acc[0];
  if (do_x) {
    // x -> pre-scaled fp16 and 16-column sums: token t by the workgroups of
    // expert group t (mod the groups), each converting its own column slice
    // (the exponent comes from the whole row)
    __shared__ float red[4];
    for (int t = blockIdx.x; t < T; t += gridDim.x)
      xprep_token<256>(t, H, xp, tid, red, c0 >> 4, (c0 + cw) >> 4);
  }
}

// ---------------------------------------------------------------- logits, T <= 4, one expert per workgroup
// Grid E, 256 threads: thread i takes the 8-column chunks i, i+256, ... of
// expert e's row and of the NT token rows of x (read from memory: they are
// small and every workgroup reads them), multiplies in fp64 (exact for
// bf16 / fp32 inputs) and sums its products in order; the 256 sums are added
// by a wave butterfly and then the four waves in order.  The result is the
// whole fp64 dot product of each token with the row (one "slice").  The
// first 4T workgroups also convert a quarter of a token's row of x each
// (pre-scaled fp16 and 16-column sums; the exponent from the whole row).
template <bool XB>
__device__ __forceinline__ void load8_as_double(const void *p, int64_t idx, double out[8]) {
  if (XB) {
    const u4 v = *reinterpret_cast<const u4 *>(reinterpret_cast<const uint16_t *>(p) + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = (double)bf16_bits_to_float((uint16_t)(v[i] & 0xFFFF));
      out[2 * i + 1] = (double)bf16_bits_to_float((uint16_t)(v[i] >> 16));
    }
  } else {
    const f4 a = *reinterpret_cast<const f4 *>(reinterpret_cast<const float *>(p) + idx);
    const f4 b = *reinterpret_cast<const f4 *>(reinterpret_cast<const float *>(p) + idx + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = a[i];
      out[4 + i] = b[i];
    }
  }
}

template <bool XB, bool WB, int NT>
__global__ __launch_bounds__(256) void k_router_rows(const void *__restrict__ x, const void *__restrict__ wr,
                                                     double *__restrict__ part, int T, int E, int H, XPrep xp,
                                                     bool do_x) {
  __shared__ double red[4][NT];
  __shared__ float xred[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x;
  const int nch = H >> 3;
  double acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.0;
  for (int ch = tid; ch < nch; ch += 256) {
    double w[8];
    load8_as_double<WB>(wr, (int64_t)e * H + 8 * ch, w);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < T) {
        double xv[8];
        load8_as_double<XB>(x, (int64_t)t * H + 8 * ch, xv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[t] = fma(xv[i], w[i], acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc[t] += __shfl_xor(acc[t], o);
    if (lane == 0) red[wave][t] = acc[t];
  }
  __syncthreads();
  if (tid < T) part[(int64_t)tid * E + e] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
  if (do_x)
    for (int q = blockIdx.x; q < 4 * T; q += gridDim.x) {
      const int t = q >> 2, j0 = (q & 3) * (H >> 6);
      xprep_token<256>(t, H, xp, tid, xred, j0, j0 + (H >> 6));
    }
}

// ---------------------------------------------------------------- logits, MFMA fp64
// 32 tokens x EW experts per workgroup (see the kernel).  Operands are
// staged in LDS as fp32 (bf16 and fp32 inputs are exact there) and widened to
// fp64;
// v_mfma_f64_16x16x4_f64 accumulates in fp64, where every product of two
// fp32 numbers is exact.
typedef double d4 __attribute__((ext_vector_type(4)));
// experts per tile: 32 gives T = 2048 twice the workgroups of 64 (one wave per
// SIMD left the fp64 MFMA latency exposed there) and leaves T = 8192 as it was
constexpr int ROUTER_EW = 32;

template <bool XB, bool WB, int EW>
__global__ __launch_bounds__(256) void k_router_mfma(const void *__restrict__ x, const void *__restrict__ wr,
                                                     const float *__restrict__ bias, float *__restrict__ logits,
                                                     int T, int E, int H) {
  // tile: 32 tokens x 32 experts; wave (tw, ew) = 16 tokens x 16 experts.
  // K-chunks of KC, staged in LDS as fp32 ([k][token], [k][expert], rows of
  // LS floats: LS = 16 mod 32 keeps the operand reads and the staging stores
  // free of bank conflicts) from raw registers loaded one chunk ahead;
  // double-buffered, one barrier per chunk.  Each accumulator takes its MFMAs
  // in ascending k, whatever KC is.
  static_assert(EW == 32, "expert tile");
  constexpr int KC = 64, LS = 48, PT = KC / 8;  // values staged per thread and chunk (x and w)
  __shared__ float xs[2][KC][LS];
  __shared__ float ws[2][KC][LS];
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * EW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int tw = wave & 1, ew = wave >> 1;
  d4 acc = (d4){0.0, 0.0, 0.0, 0.0};
  // staging: token / expert tid % 32, k (tid / 32) * PT (PT values)
  const int st = tid & 31, sk = (tid >> 5) * PT;
  const bool xv = t0 + st < T, wv = e0 + st < E;
  const int64_t xoff = (int64_t)(xv ? t0 + st : 0) * H + sk;
  const int64_t woff = (int64_t)(wv ? e0 + st : 0) * H + sk;
  constexpr int NR = PT / 4;   // 16-byte fp32 loads per operand (PT fp32 values)
  u4 rx[NR], rw[NR];            // bf16 operands use the first PT/8 (PT bf16 = PT/8 x 16 B)
  auto ld = [&](const void *p, int64_t off, bool v, bool bf, u4 (&r)[NR]) {
    if (bf && PT % 8) {  // PT = 4: one 8-byte load
      const u2 q = v ? *reinterpret_cast<const u2 *>(reinterpret_cast<const uint16_t *>(p) + off) : (u2){0u, 0u};
      r[0] = (u4){q.x, q.y, 0u, 0u};
    } else if (bf) {
#pragma unroll
      for (int i = 0; i < PT / 8; ++i)
        r[i] = v ? *reinterpret_cast<const u4 *>(reinterpret_cast<const uint16_t *>(p) + off + 8 * i) : (u4){0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int i = 0; i < NR; ++i)
        r[i] = v ? *reinterpret_cast<const u4 *>(reinterpret_cast<const float *>(p) + off + 4 * i) : (u4){0u, 0u, 0u, 0u};
    }
  };
  auto load = [&](int k0) {
    ld(x, xoff + k0, xv, XB, rx);
    ld(wr, woff + k0, wv, WB, rw);
  };
  auto val = [&](const u4 (&r)[NR], bool bf, int i) -> float {
    if (bf) {
      const uint32_t w = r[i / 8][(i / 2) & 3];
      return bf16_bits_to_float((uint16_t)((i & 1) ? (w >> 16) : (w & 0xFFFFu)));
    }
    return __uint_as_float(r[i / 4][i & 3]);
  };
  auto store = [&](int b) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      xs[b][sk + i][st] = val(rx, XB, i);
      ws[b][sk + i][st] = val(rw, WB, i);
    }
  };
  const int nk = H / KC;
  load(0);
  store(0);
  __syncthreads();
  for (int c = 0; c < nk; ++c) {
    const int b = c & 1;
    if (c + 1 < nk) load((c + 1) * KC);
#pragma unroll
    for (int kk = 0; kk < KC; kk += 4) {
      const double av = (double)xs[b][kk + g][16 * tw + r16];
      const double bv = (double)ws[b][kk + g][16 * ew + r16];
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
    }
    if (c + 1 < nk) store(b ^ 1);
    __syncthreads();
  }
  // D (fp64 16x16x4): lane holds rows (tokens) g, g+4, g+8, g+12 of the wave's 16,
  // column (expert) r16
  const int e = e0 + 16 * ew + r16;
  if (e < E) {
    const double bb = bias ? (double)bias[e] : 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * tw + g + 4 * i;
      if (t < T) logits[(int64_t)t * E + e] = (float)(acc[i] + bb);
    }
  }
}

// Large T: one workgroup per chunk of 16, 32 or 64 tokens (16 waves, each
// taking a run of the chunk's tokens).
// Besides top-k and the activation preparation it records, for the stable
// permutation, the chunk's count per expert and each assignment's rank among
// the chunk's assignments to the same expert (earlier tokens first).
// Tokens per chunk: 16 up to 2048 tokens (one token per wave: at T = 2048
// the top-k takes 14 rather than 22 us), 32 up to 4096, 64 above (the scan
// over chunks then grows faster than the top-k shrinks).
static int chunk_size(int T) { return T <= 2048 ? 16 : (T <= 4096 ? 32 : 64); }

// One workgroup of 16 waves per chunk of CHUNK tokens; wave w takes tokens
// TPW*w .. TPW*w+TPW-1 of the chunk: their logits are loaded together, staged in the
// wave's LDS row and ranked by topk_wave; then the per-expert token masks of
// the chunk give its counts and each assignment's rank inside the chunk.
template <int CHUNK>
__global__ __launch_bounds__(1024) void k_topk_chunk(const float *__restrict__ logits, int T, int E, int k, int H,
                                                     XPrep xp, bool do_x, RouteOut ro, int32_t *__restrict__ ccnt,
                                                     int32_t *__restrict__ lrank) {
  constexpr int TPW = CHUNK / 16;  // tokens per wave
  static_assert(CHUNK % 16 == 0 && CHUNK <= 64, "chunk: 16 waves, token masks of two words");
  __shared__ int32_t s_idx[CHUNK * 16];
  __shared__ uint32_t s_mask[256 * 2];
  __shared__ float s_lg[16][256];
  __shared__ uint64_t s_sel[16][128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = blockIdx.x * CHUNK;
  for (int i = tid; i < E * 2; i += 1024) s_mask[i] = 0u;
  float lv[TPW][4];
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int t = c0 + TPW * wave + q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      lv[q][i] = (t < T && e < E) ? logits[(int64_t)t * E + e] : 0.0f;
    }
  }
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int tl = TPW * wave + q;
    const int t = c0 + tl;
    if (t >= T) break;  // uniform per wave
#pragma unroll
    for (int i = 0; i < 4; ++i) s_lg[wave][4 * lane + i] = lv[q][i];
    wave_lds_order();
    int my_e;
    float my_w;
    topk_wave(s_lg[wave], E, k, my_e, my_w, s_sel[wave]);
    if (lane < k) {
      ro.idx[(int64_t)t * k + lane] = my_e;
      ro.w[(int64_t)t * k + lane] = my_w;
      s_idx[tl * k + lane] = my_e;
    }
    wave_lds_order();
  }
  if (do_x)
    for (int q = 0; q < TPW; ++q) {
      const int t = c0 + TPW * wave + q;
      if (t >= T) break;
      xprep_token<64>(t, H, xp, lane, nullptr);
    }
  __syncthreads();
  const int nt = min(CHUNK, T - c0);
  for (int a = tid; a < nt * k; a += 1024) {
    const int tl = a / k;
    atomicOr(&s_mask[s_idx[a] * 2 + (tl >> 5)], 1u << (tl & 31));
  }
  __syncthreads();
  for (int a = tid; a < nt * k; a += 1024) {
    const int tl = a / k;
    const uint32_t *m = s_mask + s_idx[a] * 2;
    int r = __popc(m[tl >> 5] & ((1u << (tl & 31)) - 1u));
    if (tl >= 32) r += __popc(m[0]);
    lrank[(int64_t)c0 * k + a] = r;
  }
  for (int e = tid; e < E; e += 1024)
    ccnt[(int64_t)blockIdx.x * E + e] = __popc(s_mask[2 * e]) + __popc(s_mask[2 * e + 1]);
}

// One workgroup: per-expert exclusive prefix over chunks (base), counts,
// offsets, tile list, and the zero row for the GEMMs.
__global__ __launch_bounds__(1024) void k_scan_chunks(int T, int E, int k, int nchunk,
                                                      const int32_t *__restrict__ ccnt, int32_t *__restrict__ base,
                                                      RouteOut ro) {
  __shared__ int32_t s_cnt[256], s_off[256], s_tb[256];
  __shared__ int32_t s_part[4][256];
  const int tid = threadIdx.x;
  if (ro.zeros)
    for (int i = tid; i < ro.nzeros; i += 1024) ro.zeros[i] = (half_t)0.0f;
  const int e = tid & 255, j = tid >> 8;
  const int per = (nchunk + 3) / 4;
  const int lo = min(nchunk, j * per), hi = min(nchunk, lo + per);
  // up to 128 chunks: four threads per expert, each with its part's counts in
  // registers (one round of loads, then the bases from the parts before it);
  // more chunks: one thread per expert in batches of 8
  if (per <= 32) {
    int v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) v[u] = (e < E && lo + u < hi) ? ccnt[(int64_t)(lo + u) * E + e] : 0;
    int sum = 0;
#pragma unroll
    for (int u = 0; u < 32; ++u) sum += v[u];
    s_part[j][e] = sum;
    __syncthreads();
    int r = 0;
    for (int jj = 0; jj < j; ++jj) r += s_part[jj][e];
#pragma unroll
    for (int u = 0; u < 32; ++u)
      if (e < E && lo + u < hi) {
        base[(int64_t)(lo + u) * E + e] = r;
        r += v[u];
      }
    if (j == 3 && e < E) s_cnt[e] = r;
  } else if (tid < E) {
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
      if (ro.ntiles) {  // the whole list: count, first tile
        ro.ntiles[0] = it;
        ro.ntiles[1] = 0;
      }
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
__global__ __launch_bounds__(256) void k_place_chunks(int T, int E, int k, int chunk, const int32_t *__restrict__ base,
                                                      const int32_t *__restrict__ lrank, RouteOut ro) {
  const int c0 = blockIdx.x * chunk;
  const int nt = min(chunk, T - c0);
  for (int i = threadIdx.x; i < nt * k; i += 256) {
    const int64_t a = (int64_t)c0 * k + i;
    const int e = ro.idx[a];
    const int p = ro.offsets[e] + base[(int64_t)blockIdx.x * E + e] + lrank[a];
    ro.perm[p] = (int32_t)a;
    if (ro.pos) ro.pos[a] = p;
    if (ro.pexp) ro.pexp[p] = ro.xexp[a / k];
  }
}

// ---------------------------------------------------------------- routing, T <= 16
// One workgroup: slice sums + bias -> logits, top-k of token t by wave t, then
// counts, offsets, the stable permutation and the small-batch tiles.
__global__ __launch_bounds__(1024) void k_route_dec(const double *__restrict__ part, int nslice,
                                                    const float *__restrict__ bias, float *__restrict__ logits, int T,
                                                    int E, int k, RouteOut ro, DecTile *__restrict__ dt,
                                                    int32_t *__restrict__ ntile) {
  __shared__ RouteLds<16> L;
  route_small_block<1024, 16>(L, part, nslice, bias, logits, T, E, k, ro, dt, ntile, true);
}

// ---------------------------------------------------------------- launchers
template <bool XB, bool WB>
static hipError_t router_tiled_t(const void *x, const void *wr, const float *bias, float *logits, int T, int E,
                                 int H, hipStream_t s, const Timing *tm) {
  DS4_LAUNCH(tm, (k_router_mfma<XB, WB, ROUTER_EW>), dim3((T + 31) / 32, (E + ROUTER_EW - 1) / ROUTER_EW), dim3(256), 0, s, x, wr, bias,
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

int chunk_count(int T) { return (T + chunk_size(T) - 1) / chunk_size(T); }

int chunk_count_max(int T) {
  const int a = ((T < 2048 ? T : 2048) + 15) / 16, b = (T + 31) / 32;  // 16-token chunks up to 2048 tokens
  return a > b ? a : b;
}

int router_slices(int H) { return (H + RSLICE - 1) / RSLICE; }

hipError_t launch_route_chunked(const float *logits, int T, int E, int k, int H, const XPrep *xp, RouteOut ro,
                                int32_t *ccnt, int32_t *base, int32_t *lrank, hipStream_t s, const Timing *tm_topk,
                                const Timing *tm_perm) {
  const int chunk = chunk_size(T), nchunk = chunk_count(T);
  XPrep x = xp ? *xp : XPrep{nullptr, false, nullptr, nullptr, nullptr};
  if (chunk == 16)
    DS4_LAUNCH(tm_topk, k_topk_chunk<16>, dim3(nchunk), dim3(1024), 0, s, logits, T, E, k, H, x, xp != nullptr, ro,
               ccnt, lrank);
  else if (chunk == 32)
    DS4_LAUNCH(tm_topk, k_topk_chunk<32>, dim3(nchunk), dim3(1024), 0, s, logits, T, E, k, H, x, xp != nullptr, ro,
               ccnt, lrank);
  else
    DS4_LAUNCH(tm_topk, k_topk_chunk<64>, dim3(nchunk), dim3(1024), 0, s, logits, T, E, k, H, x, xp != nullptr, ro,
               ccnt, lrank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the permutation slot times the scan; the placement follows it directly
  DS4_LAUNCH(tm_perm, k_scan_chunks, dim3(1), dim3(1024), 0, s, T, E, k, nchunk, ccnt, base, ro);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_place_chunks, dim3(nchunk), dim3(256), 0, s, T, E, k, chunk, base, lrank, ro);
  return hipGetLastError();
}

hipError_t launch_route_dec(const double *part, int nslice, const float *bias, float *logits, int T, int E, int k,
                            RouteOut ro, DecTile *dt, int32_t *ntile, hipStream_t s, const Timing *tm) {
  DS4_LAUNCH(tm, k_route_dec, dim3(1), dim3(1024), 0, s, part, nslice, bias, logits, T, E, k, ro, dt, ntile);
  return hipGetLastError();
}

template <bool XB, bool WB>
static hipError_t router_sliced_t(const void *x, const void *wr, double *part, int T, int E, int H,
                                  const XPrep *xp, hipStream_t s, const Timing *tm) {
  XPrep xx = xp ? *xp : XPrep{nullptr, false, nullptr, nullptr, nullptr};
  DS4_LAUNCH(tm, (k_router_sliced<XB, WB>), dim3((E + 3) / 4, router_slices(H)), dim3(256), 0, s, x, wr, part, T, E,
             H, xx,
             xp != nullptr);
  return hipGetLastError();
}

template <bool XB, bool WB>
static hipError_t router_rows_t(const void *x, const void *wr, double *part, int T, int E, int H, const XPrep *xp,
                                hipStream_t s, const Timing *tm) {
  const XPrep xv = xp ? *xp : XPrep{};
  switch (T) {
    case 1: DS4_LAUNCH(tm, (k_router_rows<XB, WB, 1>), dim3(E), dim3(256), 0, s, x, wr, part, T, E, H, xv, xp != nullptr); break;
    case 2: DS4_LAUNCH(tm, (k_router_rows<XB, WB, 2>), dim3(E), dim3(256), 0, s, x, wr, part, T, E, H, xv, xp != nullptr); break;
    default: DS4_LAUNCH(tm, (k_router_rows<XB, WB, 4>), dim3(E), dim3(256), 0, s, x, wr, part, T, E, H, xv, xp != nullptr);
  }
  return hipGetLastError();
}

int router_nslice(int H, int T) { return T <= ROUTER_ROWS_MAX_T ? 1 : router_slices(H); }

hipError_t launch_router_sliced(const void *x, bool x_bf16, const void *wr, bool w_bf16, double *part, int T,
                                int E, int H, const XPrep *xp, hipStream_t s, const Timing *tm) {
  if (T <= ROUTER_ROWS_MAX_T) {  // one expert per workgroup, the whole row
    if (x_bf16 && w_bf16) return router_rows_t<true, true>(x, wr, part, T, E, H, xp, s, tm);
    if (x_bf16) return router_rows_t<true, false>(x, wr, part, T, E, H, xp, s, tm);
    if (w_bf16) return router_rows_t<false, true>(x, wr, part, T, E, H, xp, s, tm);
    return router_rows_t<false, false>(x, wr, part, T, E, H, xp, s, tm);
  }
  if (x_bf16 && w_bf16) return router_sliced_t<true, true>(x, wr, part, T, E, H, xp, s, tm);
  if (x_bf16) return router_sliced_t<true, false>(x, wr, part, T, E, H, xp, s, tm);
  if (w_bf16) return router_sliced_t<false, true>(x, wr, part, T, E, H, xp, s, tm);
  return router_sliced_t<false, false>(x, wr, part, T, E, H, xp, s, tm);
}

}  // namespace ds4
