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

// ------------------------------------------------------------------ gate/up
// Workgroup: one tile (expert, <= 16*NT tokens) x 64*R rows of gate and up.
// Wave w: row tiles (blockIdx.x*WAVES + w)*R .. +R-1.
template <int R, int NT>
__global__ __launch_bounds__(256) void k_gateup(GemmArgs a, int nrb) {
  const int tile_id = blockIdx.x / nrb;
  const int rb = blockIdx.x - tile_id * nrb;
  if (tile_id >= *a.ntiles) return;
  const TileT tl = a.tiles[tile_id];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n_rt = a.I >> 4;
  const int rt0 = (rb * WAVES + wave) * R;
  if (rt0 >= n_rt) return;
  const int nsb = a.H >> 8;
  const uint8_t *G = a.gate + (size_t)tl.e * a.gu_bytes;
  const uint8_t *U = a.up + (size_t)tl.e * a.gu_bytes;

  const half_t *xrow[NT];
  const half_t *xsrow[NT];
  bool valid[NT];
  int pidx[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = 16 * nt + r16;
    valid[nt] = c < tl.n;
    pidx[nt] = tl.p0 + (valid[nt] ? c : 0);
    const int tok = a.perm[pidx[nt]] / a.k;
    xrow[nt] = a.x16 + (size_t)tok * a.H;
    xsrow[nt] = ((g >> 1) ? a.xs_lo : a.xs_hi) + (size_t)tok * (a.H >> 4) + 8 * (g & 1);
  }
  int rts[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rts[r] = min(rt0 + r, n_rt - 1);

  f4 yg[R][NT], yu[R][NT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      yg[r][nt] = (f4){0.f, 0.f, 0.f, 0.f};
      yu[r][nt] = (f4){0.f, 0.f, 0.f, 0.f};
    }

  for (int sb = 0; sb < nsb; ++sb) {
    UnitRegs ug[R], uu[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const size_t off = ((size_t)rts[r] * nsb + sb) * DS4_UNIT_BYTES;
      ug[r] = load_unit(G + off, lane);
      uu[r] = load_unit(U + off, lane);
    }
    UnitDecoded dg[R], du[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      dg[r] = decode_unit(ug[r], g);
      du[r] = decode_unit(uu[r], g);
    }
    f4 ag[R][NT], au[R][NT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        ag[r][nt] = (f4){0.f, 0.f, 0.f, 0.f};
        au[r][nt] = (f4){0.f, 0.f, 0.f, 0.f};
      }
    const int kb = sb * 256;
#define GU_STEP(S)                                                                    \
  {                                                                                   \
    h8 b[NT];                                                                         \
    _Pragma("unroll") for (int nt = 0; nt < NT; ++nt) b[nt] =                         \
        valid[nt] ? load_h8(xrow[nt] + kb + step_col<S>(g)) : zero_h8();              \
    _Pragma("unroll") for (int r = 0; r < R; ++r) {                                   \
      const h8 A0 = step_frag<S>(ug[r], dg[r]);                                       \
      const h8 A1 = step_frag<S>(uu[r], du[r]);                                       \
      _Pragma("unroll") for (int nt = 0; nt < NT; ++nt) {                             \
        ag[r][nt] = mfma16(A0, b[nt], ag[r][nt]);                                     \
        au[r][nt] = mfma16(A1, b[nt], au[r][nt]);                                     \
      }                                                                               \
    }                                                                                 \
  }
    GU_STEP(0) GU_STEP(1) GU_STEP(2) GU_STEP(3) GU_STEP(4) GU_STEP(5) GU_STEP(6) GU_STEP(7)
#undef GU_STEP
    // min term
    h8 bm[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bm[nt] = valid[nt] ? load_h8(xsrow[nt] + sb * 16) : zero_h8();
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f4 z = (f4){0.f, 0.f, 0.f, 0.f};
        const f4 mg = mfma16(dg[r].mfrag, bm[nt], z);
        const f4 mu = mfma16(du[r].mfrag, bm[nt], z);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          yg[r][nt][i] = fmaf(dg[r].d[i], ag[r][nt][i], yg[r][nt][i]);
          yg[r][nt][i] = fmaf(-dg[r].dmin[i], mg[i], yg[r][nt][i]);
          yu[r][nt][i] = fmaf(du[r].d[i], au[r][nt][i], yu[r][nt][i]);
          yu[r][nt][i] = fmaf(-du[r].dmin[i], mu[i], yu[r][nt][i]);
        }
      }
  }

  // SwiGLU epilogue: h = silu(gate) * up -> fp16; per-16-row sums for the
  // down projection's min term (one sub-block of its reduction dimension).
  const int nj = a.Ipad >> 4;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool rv = rt0 + r < n_rt;
    const int row0 = (rt0 + r) * 16 + 4 * g;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      half_t hv[4];
      float ssum = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gv = yg[r][nt][i], uv = yu[r][nt][i];
        const float hh = gv / (1.0f + expf(-gv)) * uv;
        hv[i] = (half_t)hh;
        ssum += (float)hv[i];
      }
      ssum += __shfl_xor(ssum, 16);
      ssum += __shfl_xor(ssum, 32);
      if (valid[nt] && rv) {
        uint2 pk;
        __builtin_memcpy(&pk, hv, 8);
        *reinterpret_cast<uint2 *>(a.h + (size_t)pidx[nt] * a.Ipad + row0) = pk;
        if (g == 0) {
          const half_t hi = (half_t)ssum;
          a.hs_hi[(size_t)pidx[nt] * nj + rt0 + r] = hi;
          a.hs_lo[(size_t)pidx[nt] * nj + rt0 + r] = (half_t)(ssum - (float)hi);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ down
template <int R, int NT>
__global__ __launch_bounds__(256) void k_down(GemmArgs a, int nrb) {
  const int tile_id = blockIdx.x / nrb;
  const int rb = blockIdx.x - tile_id * nrb;
  if (tile_id >= *a.ntiles) return;
  const TileT tl = a.tiles[tile_id];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n_rt = a.H >> 4;
  const int rt0 = (rb * WAVES + wave) * R;
  if (rt0 >= n_rt) return;
  const int nsb = a.Ipad >> 8;
  const int nj = a.Ipad >> 4;       // h-sum row stride
  const int nj_real = a.I >> 4;
  const uint8_t *D = a.down + (size_t)tl.e * a.d_bytes;

  const half_t *hrow[NT];
  const half_t *hsrow[NT];
  bool valid[NT];
  int pidx[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = 16 * nt + r16;
    valid[nt] = c < tl.n;
    pidx[nt] = tl.p0 + (valid[nt] ? c : 0);
    hrow[nt] = a.h + (size_t)pidx[nt] * a.Ipad;
    hsrow[nt] = ((g >> 1) ? a.hs_lo : a.hs_hi) + (size_t)pidx[nt] * nj + 8 * (g & 1);
  }
  int rts[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rts[r] = min(rt0 + r, n_rt - 1);

  f4 y[R][NT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) y[r][nt] = (f4){0.f, 0.f, 0.f, 0.f};

  for (int sb = 0; sb < nsb; ++sb) {
    UnitRegs ud[R];
#pragma unroll
    for (int r = 0; r < R; ++r) ud[r] = load_unit(D + ((size_t)rts[r] * nsb + sb) * DS4_UNIT_BYTES, lane);
    UnitDecoded dd[R];
#pragma unroll
    for (int r = 0; r < R; ++r) dd[r] = decode_unit(ud[r], g);
    f4 ac[R][NT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) ac[r][nt] = (f4){0.f, 0.f, 0.f, 0.f};
    const int kb = sb * 256;
#define DN_STEP(S)                                                                    \
  {                                                                                   \
    const int col = kb + step_col<S>(g);                                              \
    h8 b[NT];                                                                         \
    _Pragma("unroll") for (int nt = 0; nt < NT; ++nt) b[nt] =                         \
        (valid[nt] && col < a.I) ? load_h8(hrow[nt] + col) : zero_h8();               \
    _Pragma("unroll") for (int r = 0; r < R; ++r) {                                   \
      const h8 A0 = step_frag<S>(ud[r], dd[r]);                                       \
      _Pragma("unroll") for (int nt = 0; nt < NT; ++nt) ac[r][nt] =                   \
          mfma16(A0, b[nt], ac[r][nt]);                                               \
    }                                                                                 \
  }
    DN_STEP(0) DN_STEP(1) DN_STEP(2) DN_STEP(3) DN_STEP(4) DN_STEP(5) DN_STEP(6) DN_STEP(7)
#undef DN_STEP
    h8 bm[NT];
    const int j0 = sb * 16 + 8 * (g & 1);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      h8 v = zero_h8();
      if (valid[nt] && j0 < nj_real) {
        v = load_h8(hsrow[nt] + sb * 16);
        if (j0 + 8 > nj_real) {
#pragma unroll
          for (int b = 0; b < 8; ++b)
            if (j0 + b >= nj_real) v[b] = (half_t)0.0f;
        }
      }
      bm[nt] = v;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f4 mm = mfma16(dd[r].mfrag, bm[nt], (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[r][nt][i] = fmaf(dd[r].d[i], ac[r][nt][i], y[r][nt][i]);
          y[r][nt][i] = fmaf(-dd[r].dmin[i], mm[i], y[r][nt][i]);
        }
      }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (rt0 + r >= n_rt) continue;
    const int row0 = (rt0 + r) * 16 + 4 * g;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      if (valid[nt]) *reinterpret_cast<f4 *>(a.yp + (size_t)pidx[nt] * a.H + row0) = y[r][nt];
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
  constexpr int R = 1;
  const int rows_per_wg = 16 * R * WAVES;
  const int nrb = (a.I + rows_per_wg - 1) / rows_per_wg;
  const dim3 grid((unsigned)((int64_t)nrb * max_tiles));
  DS4_LAUNCH(tm, (k_gateup<R, 4>), grid, dim3(256), 0, s, a, nrb);
  return hipGetLastError();
}

hipError_t launch_down(const GemmArgs &a, int max_tiles, bool small, hipStream_t s, const Timing *tm) {
  if (max_tiles <= 0) return hipSuccess;
  if (small) {
    const int n_rt = a.H >> 4;
    DS4_LAUNCH(tm, (k_down_dec<2>), dim3((unsigned)((int64_t)n_rt * max_tiles)), dim3(256), 0, s, a, n_rt);
    return hipGetLastError();
  }
  constexpr int R = 1;
  const int rows_per_wg = 16 * R * WAVES;
  const int nrb = (a.H + rows_per_wg - 1) / rows_per_wg;
  const dim3 grid((unsigned)((int64_t)nrb * max_tiles));
  DS4_LAUNCH(tm, (k_down<R, 4>), grid, dim3(256), 0, s, a, nrb);
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
