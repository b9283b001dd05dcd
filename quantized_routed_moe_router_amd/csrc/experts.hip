// Routed experts: dequant-fused grouped GEMMs on MFMA (gate/up with the SwiGLU
// epilogue, down), the weighted combine, and the dense bf16 shared expert.
//
// Exact-operand formulation of one packed super-block (256 columns, fp16 d and
// dmin, 16 sub-blocks j with 4-bit scale sc_j and min m_j, codes q):
//   sum_k w_k x_k = d * sum_k (sc_j(k) q_k) x_k  -  dmin * sum_j m_j X_j,
//   X_j = sum of x over sub-block j.
// sc*q (<= 45) and m (<= 15) are small integers, exact in fp16, so both MFMA
// operand sets are exact; only fp32 accumulation and the fp16 activations
// (x, or h between the two projections) round.  The min term is one extra
// 16x16x32 MFMA per super-block with X split into fp16 hi + lo.
//
// MFMA v_mfma_f32_16x16x32_f16, lane l = 16*g + r:
//   A: row r, 8 k's;  B: column r (token), the same 8 k's;  D: rows 4g..4g+3, column r.
// Per super-block the 8 steps s cover sub-block 4*(s/2) + g, half s%2, so a
// lane's 16-byte code vector holds 4 whole sub-blocks.
#include "common.h"
#include "launch.h"

namespace ds4 {

#define WAVES 4
#ifndef GEMM_R_GU
#define GEMM_R_GU 1
#endif
#ifndef GEMM_R_DN
#define GEMM_R_DN 2
#endif
#ifndef GEMM_NW_GU
#define GEMM_NW_GU 4
#endif
#ifndef GEMM_NW_DN
#define GEMM_NW_DN 4
#endif

struct UnitRegs {
  u4 code;   // 4 raw dwords: sub-blocks g, 4+g, 8+g, 12+g of row r
  u4 scale;  // row r: scale halfwords (bytes 0-7), min nibbles (bytes 8-15)
  u4 dd;     // rows 4g..4g+3: d | dmin<<16
};

__device__ __forceinline__ UnitRegs load_unit(const uint8_t *__restrict__ unit, int lane) {
  UnitRegs u;
  u.code = *reinterpret_cast<const u4 *>(unit + 16 * lane);
  u.scale = *reinterpret_cast<const u4 *>(unit + DS4_SCALE_OFF + 16 * (lane & 15));
  u.dd = *reinterpret_cast<const u4 *>(unit + DS4_DD_OFF + 16 * (lane >> 4));
  return u;
}

struct UnitDecoded {
  h2 sc[4];   // sub-block scales for q = 0..3 (sub-block 4q+g)
  h8 mfrag;   // min-MFMA A fragment: m of sub-blocks 8*(g&1) .. +7
  float d[4], dmin[4];
};

__device__ __forceinline__ UnitDecoded decode_unit(const UnitRegs &u, int g) {
  UnitDecoded o;
  const uint32_t sw = (g < 2) ? u.scale.x : u.scale.y;
  const uint32_t hw = (g & 1) ? (sw >> 16) : (sw & 0xFFFFu);
#pragma unroll
  for (int q = 0; q < 4; ++q) o.sc[q] = splat_h2((float)((hw >> (4 * q)) & 15u));
  o.mfrag = min_frag((g & 1) ? u.scale.w : u.scale.z);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o.d[i] = half_bits_to_float((uint16_t)(u.dd[i] & 0xFFFFu));
    o.dmin[i] = half_bits_to_float((uint16_t)(u.dd[i] >> 16));
  }
  return o;
}

template <int S>
__device__ __forceinline__ h8 step_frag(const UnitRegs &u, const UnitDecoded &dc) {
  return dequant_frag<(S & 1)>(u.code[S >> 1], dc.sc[S >> 1]);
}

// offset of the 8 activations a lane (group g) feeds at step S of a super-block
template <int S>
__device__ __forceinline__ int step_col(int g) {
  return 16 * (4 * (S >> 1) + g) + 8 * (S & 1);
}

// ------------------------------------------------------------------ prefill grouped GEMM
// Workgroup = one tile of up to 64 tokens x (WAVES*R*16) rows of NM packed
// matrices (NM = 2: gate and up with the SwiGLU epilogue; NM = 1: down).
// Per super-block the tile's activations (64 x 256 fp16) and their 16-column
// sums (hi, lo) are staged in LDS; the next super-block's activations and
// packed weights are already loading into registers while the current one
// is multiplied.  Each wave dequantizes its own rows' A fragments.
constexpr int GEMM_NT = 4;            // 16-token n-tiles per workgroup
constexpr int SB_STRIDE = 264;        // halves per staged token row (256 + pad)
constexpr int SS_STRIDE = 40;         // halves per staged sum row (32 + pad)

template <int NM>
struct GemmCtx {
  const uint8_t *W[NM];               // this wave's matrices, row tile rt0
  int nsb;
  size_t rt_stride;                   // bytes between consecutive row tiles
};

template <int NM, int R>
__device__ __forceinline__ void gemm_load_a(UnitRegs (&u)[R][NM], const GemmCtx<NM> &c, const int (&rts)[R], int sb,
                                            int lane) {
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < NM; ++m)
      u[r][m] = load_unit(c.W[m] + (size_t)rts[r] * c.rt_stride + (size_t)sb * DS4_UNIT_BYTES, lane);
}

// Activation staging: thread -> token row (tid/4)%64, chunk column tid%4;
// with NW waves each thread stages 8*4/NW of the row's 32 chunks of 8 halves
// (chunks lc + 4i), and threads of the first 256 also one chunk of sums
// (lc: hi 0-7, hi 8-15, lo 0-7, lo 8-15).
template <int NCH>
struct Stage {
  u4 b[NCH];
  u4 s;
};

template <int NCH, bool PADDED>
__device__ __forceinline__ void stage_load(Stage<NCH> &st, const half_t *brow, const half_t *shi, const half_t *slo,
                                           int sb, int lc, int part, int kreal, int jreal) {
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int col = sb * 256 + (lc + 4 * (part * NCH + i)) * 8;
    st.b[i] = (!PADDED || col < kreal) ? *reinterpret_cast<const u4 *>(brow + col) : (u4){0u, 0u, 0u, 0u};
  }
  if (part != 0) return;
  const int j0 = sb * 16 + 8 * (lc & 1);
  const half_t *sp = (lc >> 1) ? slo : shi;
  if (!PADDED) {
    st.s = *reinterpret_cast<const u4 *>(sp + j0);
    return;
  }
  u4 v = (u4){0u, 0u, 0u, 0u};
  if (j0 < jreal) {
    v = *reinterpret_cast<const u4 *>(sp + j0);
    if (j0 + 8 > jreal) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (j0 + 2 * q >= jreal) v[q] = 0u;
        else if (j0 + 2 * q + 1 >= jreal) v[q] &= 0xFFFFu;
      }
    }
  }
  st.s = v;
}

template <int NCH>
__device__ __forceinline__ void stage_store(const Stage<NCH> &st, half_t *sB, half_t *sS, int lr, int lc, int part) {
#pragma unroll
  for (int i = 0; i < NCH; ++i)
    *reinterpret_cast<u4 *>(sB + lr * SB_STRIDE + (lc + 4 * (part * NCH + i)) * 8) = st.b[i];
  if (part == 0) *reinterpret_cast<u4 *>(sS + lr * SS_STRIDE + lc * 8) = st.s;
}

template <int NM, int R>
__device__ __forceinline__ void gemm_compute_sb(const UnitRegs (&u)[R][NM], const half_t *sB, const half_t *sS,
                                                f4 (&y)[NM][R][GEMM_NT], int r16, int g) {
  UnitDecoded dc[R][NM];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < NM; ++m) dc[r][m] = decode_unit(u[r][m], g);
  f4 acc[NM][R][GEMM_NT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int nt = 0; nt < GEMM_NT; ++nt) acc[m][r][nt] = (f4){0.f, 0.f, 0.f, 0.f};
#define GEMM_STEP(S)                                                                          \
  {                                                                                           \
    h8 b[GEMM_NT];                                                                            \
    _Pragma("unroll") for (int nt = 0; nt < GEMM_NT; ++nt) b[nt] =                            \
        load_h8(sB + (16 * nt + r16) * SB_STRIDE + step_col<S>(g));                           \
    _Pragma("unroll") for (int r = 0; r < R; ++r) {                                           \
      _Pragma("unroll") for (int m = 0; m < NM; ++m) {                                        \
        const h8 A = step_frag<S>(u[r][m], dc[r][m]);                                         \
        _Pragma("unroll") for (int nt = 0; nt < GEMM_NT; ++nt) acc[m][r][nt] =                \
            mfma16(A, b[nt], acc[m][r][nt]);                                                  \
      }                                                                                       \
    }                                                                                         \
  }
  GEMM_STEP(0) GEMM_STEP(1) GEMM_STEP(2) GEMM_STEP(3) GEMM_STEP(4) GEMM_STEP(5) GEMM_STEP(6) GEMM_STEP(7)
#undef GEMM_STEP
  h8 bm[GEMM_NT];
#pragma unroll
  for (int nt = 0; nt < GEMM_NT; ++nt) bm[nt] = load_h8(sS + (16 * nt + r16) * SS_STRIDE + 8 * g);
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nt = 0; nt < GEMM_NT; ++nt) {
        const f4 mm = mfma16(dc[r][m].mfrag, bm[nt], (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          y[m][r][nt][q] = fmaf(dc[r][m].d[q], acc[m][r][nt][q], y[m][r][nt][q]);
          y[m][r][nt][q] = fmaf(-dc[r][m].dmin[q], mm[q], y[m][r][nt][q]);
        }
      }
}

template <int NM, int R, int NW, bool PADDED>
__global__ __launch_bounds__(64 * NW) void k_moe_gemm(GemmArgs a, int nrb) {
  __shared__ __attribute__((aligned(16))) half_t sB[64 * SB_STRIDE];
  __shared__ __attribute__((aligned(16))) half_t sS[64 * SS_STRIDE];
  const int tile_id = blockIdx.x / nrb;
  const int rb = blockIdx.x - tile_id * nrb;
  if (tile_id >= *a.ntiles) return;  // uniform over the workgroup
  const TileT tl = a.tiles[tile_id];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  constexpr bool GU = NM == 2;
  const int K = GU ? a.H : a.Ipad;
  const int kreal = GU ? a.H : a.I;
  const int jreal = kreal >> 4;
  const int nsb = K >> 8;
  const int n_rt = (GU ? a.I : a.H) >> 4;
  const int rt0 = (rb * NW + wave) * R;
  int rts[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rts[r] = min(rt0 + r, n_rt - 1);

  // activation rows staged by this thread
  constexpr int NCH = 32 / NW;
  const int lr = (tid >> 2) & 63, lc = tid & 3, part = tid >> 8;
  const bool lvalid = lr < tl.n;
  const half_t *brow, *shi, *slo;
  if (GU) {
    const int tok = a.perm[tl.p0 + (lvalid ? lr : 0)] / a.k;
    brow = a.x16 + (size_t)tok * a.H;
    shi = a.xs_hi + (size_t)tok * (a.H >> 4);
    slo = a.xs_lo + (size_t)tok * (a.H >> 4);
  } else {
    const size_t p = (size_t)(tl.p0 + (lvalid ? lr : 0));
    brow = a.h + p * a.Ipad;
    shi = a.hs_hi + p * (a.Ipad >> 4);
    slo = a.hs_lo + p * (a.Ipad >> 4);
  }
  if (!lvalid) brow = shi = slo = a.zeros;

  GemmCtx<NM> c;
  c.nsb = nsb;
  c.rt_stride = (size_t)nsb * DS4_UNIT_BYTES;
  if (GU) {
    c.W[0] = a.gate + (size_t)tl.e * a.gu_bytes;
    c.W[NM - 1] = a.up + (size_t)tl.e * a.gu_bytes;
  } else {
    c.W[0] = a.down + (size_t)tl.e * a.d_bytes;
  }

  f4 y[NM][R][GEMM_NT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int nt = 0; nt < GEMM_NT; ++nt) y[m][r][nt] = (f4){0.f, 0.f, 0.f, 0.f};

  Stage<NCH> st;
  UnitRegs ua[R][NM], ub[R][NM];
  stage_load<NCH, PADDED>(st, brow, shi, slo, 0, lc, part, kreal, jreal);
  gemm_load_a<NM, R>(ua, c, rts, 0, lane);
  for (int sb = 0; sb < nsb; sb += 2) {
    // even super-block: weights in ua, prefetch into ub
    __syncthreads();
    stage_store<NCH>(st, sB, sS, lr, lc, part);
    __syncthreads();
    if (sb + 1 < nsb) {
      stage_load<NCH, PADDED>(st, brow, shi, slo, sb + 1, lc, part, kreal, jreal);
      gemm_load_a<NM, R>(ub, c, rts, sb + 1, lane);
    }
    gemm_compute_sb<NM, R>(ua, sB, sS, y, r16, g);
    if (sb + 1 >= nsb) break;
    // odd super-block: weights in ub, prefetch into ua
    __syncthreads();
    stage_store<NCH>(st, sB, sS, lr, lc, part);
    __syncthreads();
    if (sb + 2 < nsb) {
      stage_load<NCH, PADDED>(st, brow, shi, slo, sb + 2, lc, part, kreal, jreal);
      gemm_load_a<NM, R>(ua, c, rts, sb + 2, lane);
    }
    gemm_compute_sb<NM, R>(ub, sB, sS, y, r16, g);
  }

  if (rt0 >= n_rt) return;
  if (GU) {
    const int nj = a.Ipad >> 4;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool rv = rt0 + r < n_rt;
      const int row0 = (rt0 + r) * 16 + 4 * g;
#pragma unroll
      for (int nt = 0; nt < GEMM_NT; ++nt) {
        const int col = 16 * nt + r16;
        const bool valid = col < tl.n;
        half_t hv[4];
        float ssum = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float gv = y[0][r][nt][q], uv = y[NM - 1][r][nt][q];
          hv[q] = (half_t)(gv / (1.0f + expf(-gv)) * uv);
          ssum += (float)hv[q];
        }
        ssum += __shfl_xor(ssum, 16);
        ssum += __shfl_xor(ssum, 32);
        if (valid && rv) {
          const size_t p = (size_t)(tl.p0 + col);
          uint2 pk;
          __builtin_memcpy(&pk, hv, 8);
          *reinterpret_cast<uint2 *>(a.h + p * a.Ipad + row0) = pk;
          if (g == 0) {
            const half_t hi = (half_t)ssum;
            a.hs_hi[p * nj + rt0 + r] = hi;
            a.hs_lo[p * nj + rt0 + r] = (half_t)(ssum - (float)hi);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (rt0 + r >= n_rt) continue;
      const int row0 = (rt0 + r) * 16 + 4 * g;
#pragma unroll
      for (int nt = 0; nt < GEMM_NT; ++nt) {
        const int col = 16 * nt + r16;
        if (col < tl.n) *reinterpret_cast<f4 *>(a.yp + (size_t)(tl.p0 + col) * a.H + row0) = y[0][r][nt];
      }
    }
  }
}

// ------------------------------------------------------------------ decode GEMV
// Small batches (<= 16 tokens per expert): bandwidth-bound weight streaming.
// Workgroup = one tile x one 16-row tile (of gate and up, or of down); its 4
// waves split the super-blocks of the reduction dimension, each wave issues
// the loads of a whole batch of SBW super-blocks before any arithmetic (so
// each wave keeps up to SBW*1344*matrices bytes in flight), and the four
// partial sums are added through LDS in wave order.
template <int SBW>
__global__ __launch_bounds__(256) void k_gateup_dec(GemmArgs a, int n_rt) {
  const int tile_id = blockIdx.x / n_rt;
  const int rt = blockIdx.x - tile_id * n_rt;
  if (tile_id >= *a.ntiles) return;  // uniform over the workgroup
  const TileT tl = a.tiles[tile_id];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int nsb = a.H >> 8;
  const int per = (nsb + WAVES - 1) / WAVES;
  const int sb0 = wave * per, sb1 = min(nsb, sb0 + per);
  const bool valid = r16 < tl.n;
  const int pidx = tl.p0 + (valid ? r16 : 0);
  const int tok = a.perm[pidx] / a.k;
  // lanes without a token read zeros instead of selecting per step
  const half_t *xrow = valid ? a.x16 + (size_t)tok * a.H : a.zeros;
  const half_t *xsrow = valid ? ((g >> 1) ? a.xs_lo : a.xs_hi) + (size_t)tok * (a.H >> 4) + 8 * (g & 1) : a.zeros;
  const uint8_t *G = a.gate + (size_t)tl.e * a.gu_bytes + (size_t)rt * nsb * DS4_UNIT_BYTES;
  const uint8_t *U = a.up + (size_t)tl.e * a.gu_bytes + (size_t)rt * nsb * DS4_UNIT_BYTES;
  f4 yg = (f4){0.f, 0.f, 0.f, 0.f}, yu = yg;
  for (int b0 = sb0; b0 < sb1; b0 += SBW) {
    UnitRegs ug[SBW], uu[SBW];
#pragma unroll
    for (int i = 0; i < SBW; ++i) {
      const int sb = min(b0 + i, sb1 - 1);
      ug[i] = load_unit(G + (size_t)sb * DS4_UNIT_BYTES, lane);
      uu[i] = load_unit(U + (size_t)sb * DS4_UNIT_BYTES, lane);
    }
#pragma unroll
    for (int i = 0; i < SBW; ++i) {
      if (b0 + i >= sb1) break;
      const int kb = (b0 + i) * 256;
      h8 b[9];
#pragma unroll
      for (int s = 0; s < 8; ++s) b[s] = load_h8(xrow + kb + 16 * (4 * (s >> 1) + g) + 8 * (s & 1));
      b[8] = load_h8(xsrow + (b0 + i) * 16);
      const UnitDecoded dg = decode_unit(ug[i], g);
      const UnitDecoded du = decode_unit(uu[i], g);
      f4 ag = (f4){0.f, 0.f, 0.f, 0.f}, au = ag;
#define DEC_STEP(S)                                   \
  ag = mfma16(step_frag<S>(ug[i], dg), b[S], ag);     \
  au = mfma16(step_frag<S>(uu[i], du), b[S], au);
      DEC_STEP(0) DEC_STEP(1) DEC_STEP(2) DEC_STEP(3) DEC_STEP(4) DEC_STEP(5) DEC_STEP(6) DEC_STEP(7)
#undef DEC_STEP
      const f4 z = (f4){0.f, 0.f, 0.f, 0.f};
      const f4 mg = mfma16(dg.mfrag, b[8], z);
      const f4 mu = mfma16(du.mfrag, b[8], z);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        yg[q] = fmaf(dg.d[q], ag[q], yg[q]);
        yg[q] = fmaf(-dg.dmin[q], mg[q], yg[q]);
        yu[q] = fmaf(du.d[q], au[q], yu[q]);
        yu[q] = fmaf(-du.dmin[q], mu[q], yu[q]);
      }
    }
  }
  __shared__ f4 red[2][WAVES][64];
  red[0][wave][lane] = yg;
  red[1][wave][lane] = yu;
  __syncthreads();
  if (wave != 0) return;
  yg = red[0][0][lane];
  yu = red[1][0][lane];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) {
    const f4 pg = red[0][w][lane], pu = red[1][w][lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      yg[q] += pg[q];
      yu[q] += pu[q];
    }
  }
  half_t hv[4];
  float ssum = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hv[q] = (half_t)(yg[q] / (1.0f + expf(-yg[q])) * yu[q]);
    ssum += (float)hv[q];
  }
  ssum += __shfl_xor(ssum, 16);
  ssum += __shfl_xor(ssum, 32);
  if (valid) {
    const int nj = a.Ipad >> 4;
    uint2 pk;
    __builtin_memcpy(&pk, hv, 8);
    *reinterpret_cast<uint2 *>(a.h + (size_t)pidx * a.Ipad + rt * 16 + 4 * g) = pk;
    if (g == 0) {
      const half_t hi = (half_t)ssum;
      a.hs_hi[(size_t)pidx * nj + rt] = hi;
      a.hs_lo[(size_t)pidx * nj + rt] = (half_t)(ssum - (float)hi);
    }
  }
}

template <int SBW>
__global__ __launch_bounds__(256) void k_down_dec(GemmArgs a, int n_rt) {
  const int tile_id = blockIdx.x / n_rt;
  const int rt = blockIdx.x - tile_id * n_rt;
  if (tile_id >= *a.ntiles) return;
  const TileT tl = a.tiles[tile_id];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int nsb = a.Ipad >> 8;
  const int nj = a.Ipad >> 4, nj_real = a.I >> 4;
  const int per = (nsb + WAVES - 1) / WAVES;
  const int sb0 = wave * per, sb1 = min(nsb, sb0 + per);
  const bool valid = r16 < tl.n;
  const int pidx = tl.p0 + (valid ? r16 : 0);
  const half_t *hrow = valid ? a.h + (size_t)pidx * a.Ipad : a.zeros;
  const half_t *hsrow = valid ? ((g >> 1) ? a.hs_lo : a.hs_hi) + (size_t)pidx * nj + 8 * (g & 1) : a.zeros;
  const bool padded = a.I != a.Ipad;
  const uint8_t *D = a.down + (size_t)tl.e * a.d_bytes + (size_t)rt * nsb * DS4_UNIT_BYTES;
  f4 y = (f4){0.f, 0.f, 0.f, 0.f};
  for (int b0 = sb0; b0 < sb1; b0 += SBW) {
    UnitRegs ud[SBW];
#pragma unroll
    for (int i = 0; i < SBW; ++i) ud[i] = load_unit(D + (size_t)min(b0 + i, sb1 - 1) * DS4_UNIT_BYTES, lane);
#pragma unroll
    for (int i = 0; i < SBW; ++i) {
      if (b0 + i >= sb1) break;
      const int kb = (b0 + i) * 256;
      h8 b[9];
      if (!padded) {
#pragma unroll
        for (int s = 0; s < 8; ++s) b[s] = load_h8(hrow + kb + 16 * (4 * (s >> 1) + g) + 8 * (s & 1));
        b[8] = load_h8(hsrow + (b0 + i) * 16);
      } else {  // reduction length not a multiple of 256: columns >= I read as zero
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int col = kb + 16 * (4 * (s >> 1) + g) + 8 * (s & 1);
          b[s] = col < a.I ? load_h8(hrow + col) : zero_h8();
        }
        const int j0 = (b0 + i) * 16 + 8 * (g & 1);
        h8 v = zero_h8();
        if (j0 < nj_real) {
          v = load_h8(hsrow + (b0 + i) * 16);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (j0 + e >= nj_real) v[e] = (half_t)0.0f;
        }
        b[8] = v;
      }
      const UnitDecoded dd = decode_unit(ud[i], g);
      f4 ac = (f4){0.f, 0.f, 0.f, 0.f};
#define DEC_STEP(S) ac = mfma16(step_frag<S>(ud[i], dd), b[S], ac);
      DEC_STEP(0) DEC_STEP(1) DEC_STEP(2) DEC_STEP(3) DEC_STEP(4) DEC_STEP(5) DEC_STEP(6) DEC_STEP(7)
#undef DEC_STEP
      const f4 mm = mfma16(dd.mfrag, b[8], (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        y[q] = fmaf(dd.d[q], ac[q], y[q]);
        y[q] = fmaf(-dd.dmin[q], mm[q], y[q]);
      }
    }
  }
  __shared__ f4 red[WAVES][64];
  red[wave][lane] = y;
  __syncthreads();
  if (wave != 0) return;
  y = red[0][lane];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) {
    const f4 p = red[w][lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] += p[q];
  }
  if (valid) *reinterpret_cast<f4 *>(a.yp + (size_t)pidx * a.H + rt * 16 + 4 * g) = y;
}

// ------------------------------------------------------------------ combine
// y[t] = sum_j w[t,j] * Yp[pos(t,j)] in rank order, then + shared output.
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ yp, const int32_t *__restrict__ pos,
                                                 const float *__restrict__ w, const float *__restrict__ ysh,
                                                 float *__restrict__ y, int T, int k, int H) {
  const int t = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  f4 acc = (f4){0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const f4 v = *reinterpret_cast<const f4 *>(yp + (size_t)pos[(size_t)t * k + j] * H + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
  }
  if (ysh) {
    const f4 v = *reinterpret_cast<const f4 *>(ysh + (size_t)t * H + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += v[i];
  }
  *reinterpret_cast<f4 *>(y + (size_t)t * H + c) = acc;
}

// ------------------------------------------------------------------ shared expert
// Dense bf16 weights -> fp16 operands (exact inside the binary16 range).
__device__ __forceinline__ h8 bf16x8_to_h8(u4 v) {
  h8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (half_t)bf16_bits_to_float((uint16_t)(v[i] & 0xFFFFu));
    r[2 * i + 1] = (half_t)bf16_bits_to_float((uint16_t)(v[i] >> 16));
  }
  return r;
}

template <int R, int NT>
__global__ __launch_bounds__(256) void k_shared_gateup(const uint16_t *__restrict__ wg,
                                                       const uint16_t *__restrict__ wu,
                                                       const half_t *__restrict__ x16, half_t *__restrict__ hs,
                                                       int T, int H, int Is) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n_rt = Is >> 4;
  const int rt0 = (blockIdx.x * WAVES + wave) * R;
  if (rt0 >= n_rt) return;
  const int t0 = blockIdx.y * 16 * NT;
  int tok[NT];
  bool valid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int t = t0 + 16 * nt + r16;
    valid[nt] = t < T;
    tok[nt] = valid[nt] ? t : 0;
  }
  f4 ag[R][NT], au[R][NT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      ag[r][nt] = (f4){0.f, 0.f, 0.f, 0.f};
      au[r][nt] = (f4){0.f, 0.f, 0.f, 0.f};
    }
  for (int k0 = 0; k0 < H; k0 += 32) {
    const int col = k0 + 8 * g;
    h8 b[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) b[nt] = valid[nt] ? load_h8(x16 + (size_t)tok[nt] * H + col) : zero_h8();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(rt0 + r, n_rt - 1) * 16 + r16;
      const h8 A0 = bf16x8_to_h8(*reinterpret_cast<const u4 *>(wg + (size_t)row * H + col));
      const h8 A1 = bf16x8_to_h8(*reinterpret_cast<const u4 *>(wu + (size_t)row * H + col));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        ag[r][nt] = mfma16(A0, b[nt], ag[r][nt]);
        au[r][nt] = mfma16(A1, b[nt], au[r][nt]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (rt0 + r >= n_rt) continue;
    const int row0 = (rt0 + r) * 16 + 4 * g;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (!valid[nt]) continue;
      half_t hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gv = ag[r][nt][i], uv = au[r][nt][i];
        hv[i] = (half_t)(gv / (1.0f + expf(-gv)) * uv);
      }
      uint2 pk;
      __builtin_memcpy(&pk, hv, 8);
      *reinterpret_cast<uint2 *>(hs + (size_t)tok[nt] * Is + row0) = pk;
    }
  }
}

template <int R, int NT>
__global__ __launch_bounds__(256) void k_shared_down(const uint16_t *__restrict__ wd, const half_t *__restrict__ hs,
                                                     float *__restrict__ ysh, int T, int H, int Is) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n_rt = H >> 4;
  const int rt0 = (blockIdx.x * WAVES + wave) * R;
  if (rt0 >= n_rt) return;
  const int t0 = blockIdx.y * 16 * NT;
  int tok[NT];
  bool valid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int t = t0 + 16 * nt + r16;
    valid[nt] = t < T;
    tok[nt] = valid[nt] ? t : 0;
  }
  f4 ac[R][NT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) ac[r][nt] = (f4){0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < Is; k0 += 32) {
    const int col = k0 + 8 * g;
    h8 b[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) b[nt] = valid[nt] ? load_h8(hs + (size_t)tok[nt] * Is + col) : zero_h8();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(rt0 + r, n_rt - 1) * 16 + r16;
      const h8 A0 = bf16x8_to_h8(*reinterpret_cast<const u4 *>(wd + (size_t)row * Is + col));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) ac[r][nt] = mfma16(A0, b[nt], ac[r][nt]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (rt0 + r >= n_rt) continue;
    const int row0 = (rt0 + r) * 16 + 4 * g;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      if (valid[nt]) *reinterpret_cast<f4 *>(ysh + (size_t)tok[nt] * H + row0) = ac[r][nt];
  }
}

// ------------------------------------------------------------------ launchers
// Decode batches (<= 16 tokens per expert): the split-reduction GEMV kernels.
// Prefill: four n-tiles (64 tokens) per workgroup.
hipError_t launch_gateup(const GemmArgs &a, int max_tiles, bool small, hipStream_t s, const Timing *tm) {
  if (max_tiles <= 0) return hipSuccess;
  if (small) {
    const int n_rt = a.I >> 4;
    DS4_LAUNCH(tm, (k_gateup_dec<4>), dim3((unsigned)((int64_t)n_rt * max_tiles)), dim3(256), 0, s, a, n_rt);
    return hipGetLastError();
  }
  constexpr int R = GEMM_R_GU, NW = GEMM_NW_GU;
  const int rows_per_wg = 16 * R * NW;
  const int nrb = (a.I + rows_per_wg - 1) / rows_per_wg;
  const dim3 grid((unsigned)((int64_t)nrb * max_tiles));
  DS4_LAUNCH(tm, (k_moe_gemm<2, R, NW, false>), grid, dim3(64 * NW), 0, s, a, nrb);
  return hipGetLastError();
}

hipError_t launch_down(const GemmArgs &a, int max_tiles, bool small, hipStream_t s, const Timing *tm) {
  if (max_tiles <= 0) return hipSuccess;
  if (small) {
    const int n_rt = a.H >> 4;
    DS4_LAUNCH(tm, (k_down_dec<2>), dim3((unsigned)((int64_t)n_rt * max_tiles)), dim3(256), 0, s, a, n_rt);
    return hipGetLastError();
  }
  constexpr int R = GEMM_R_DN, NW = GEMM_NW_DN;
  const int rows_per_wg = 16 * R * NW;
  const int nrb = (a.H + rows_per_wg - 1) / rows_per_wg;
  const dim3 grid((unsigned)((int64_t)nrb * max_tiles));
  if (a.I == a.Ipad)
    DS4_LAUNCH(tm, (k_moe_gemm<1, R, NW, false>), grid, dim3(64 * NW), 0, s, a, nrb);
  else
    DS4_LAUNCH(tm, (k_moe_gemm<1, R, NW, true>), grid, dim3(64 * NW), 0, s, a, nrb);
  return hipGetLastError();
}

hipError_t launch_combine(const float *yp, const int32_t *pos, const float *w, const float *ysh, float *y, int T,
                          int k, int H, hipStream_t s, const Timing *tm) {
  if (T <= 0) return hipSuccess;
  DS4_LAUNCH(tm, k_combine, dim3(T, (H + 1023) / 1024), dim3(256), 0, s, yp, pos, w, ysh, y, T, k, H);
  return hipGetLastError();
}

hipError_t launch_shared_gateup(const uint16_t *wg, const uint16_t *wu, const _Float16 *x16, _Float16 *hs, int T,
                                int H, int Is, hipStream_t s, const Timing *tm) {
  if (T <= 0) return hipSuccess;
  constexpr int R = 1, NT = 4;
  const dim3 grid((Is + 16 * R * WAVES - 1) / (16 * R * WAVES), (T + 16 * NT - 1) / (16 * NT));
  DS4_LAUNCH(tm, (k_shared_gateup<R, NT>), grid, dim3(256), 0, s, wg, wu, x16, hs, T, H, Is);
  return hipGetLastError();
}

hipError_t launch_shared_down(const uint16_t *wd, const _Float16 *hs, float *ysh, int T, int H, int Is,
                              hipStream_t s, const Timing *tm) {
  if (T <= 0) return hipSuccess;
  constexpr int R = 1, NT = 4;
  const dim3 grid((H + 16 * R * WAVES - 1) / (16 * R * WAVES), (T + 16 * NT - 1) / (16 * NT));
  DS4_LAUNCH(tm, (k_shared_down<R, NT>), grid, dim3(256), 0, s, wd, hs, ysh, T, H, Is);
  return hipGetLastError();
}

}  // namespace ds4
