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
// The same holds for 4-bit codes (sc*q <= 225).
//
// MFMA v_mfma_f32_16x16x32_f16, lane l = 16*g + r:
//   A: row r, 8 k's;  B: column r (token), the same 8 k's;  D: rows 4g..4g+3, column r.
// Per super-block the 8 steps s cover sub-block 4*(s/2) + g, half s%2, so a
// lane's code vectors (16 bytes with 2-bit codes, 2 x 16 with 4-bit codes)
// hold 4 whole sub-blocks.  Every kernel is instantiated for both code widths
// B; only the unit size, the code loads and the fragment decode differ.
#include "common.h"
#include "launch.h"
#include "route_dev.h"

namespace ds4 {

#define WAVES 4
// Launch shapes and pipeline depths (each fixed by measurement on MI355X; the
// parity tests cover exactly these instantiations).
constexpr int GEMM_R_GU = 1;   // 64-token GEMMs: row tiles per wave, gate/up
constexpr int GEMM_R_DN = 2;   // ... down
constexpr int GEMM_NW_GU = 4;  // ... waves per workgroup, gate/up
constexpr int GEMM_NW_DN = 4;  // ... down
constexpr int DN_DEC_PD = 3;   // decode down with I below 256: pipeline depth
constexpr int GU_LDS_PD = 3;   // one-token gate/up: pipeline depth
constexpr int GU_LDS_KS = 2;   // ... waves sharing one row tile's reduction
constexpr int DN_LDS_PD = 4;   // decode down, T <= 4, I not a multiple of 512: pipeline depth
constexpr int GU_SH_PD = 2;    // gate/up of 5..16 tokens: pipeline depth
constexpr int GU_SH_NW = 4;    // ... waves (row tiles) per workgroup
// smallest batch that takes the shared-activation gate/up kernel (one token
// takes the per-wave kernel)
constexpr int GU_SH_MIN_T = 2;
constexpr int DN2_PD = 2;         // down of 5..16 tokens: pipeline depth
constexpr int DN2_R = 4;          // ... row tiles per wave
constexpr int DN2_NH = 4;         // ... ways the tile list is split
constexpr bool DN2_SDL = true;    // ... unit scales and d|dmin through LDS


// One lane's share of a packed unit.  Code plane p (1024 bytes at 1024*p)
// holds dwords 4p..4p+3 of every lane, 16 bytes per lane, so each plane is one
// fully coalesced load; dword S of a lane feeds MFMA step S with 4-bit codes,
// dword S/2 (both halves) with 2-bit codes.
template <int B>
struct UnitRegs {
  u4 code[B / 2];  // raw code dwords of sub-blocks g, 4+g, 8+g, 12+g of row r
  u4 scale;        // row r: scale halfwords (bytes 0-7), min nibbles (bytes 8-15)
  u4 dd;           // rows 4g..4g+3: d | dmin<<16
};

template <int B>
__device__ __forceinline__ UnitRegs<B> load_unit(const uint8_t *__restrict__ unit, int lane) {
  UnitRegs<B> u;
#pragma unroll
  for (int p = 0; p < B / 2; ++p) u.code[p] = *reinterpret_cast<const u4 *>(unit + 1024 * p + 16 * lane);
  u.scale = *reinterpret_cast<const u4 *>(unit + Unit<B>::SCALE_OFF + 16 * (lane & 15));
  u.dd = *reinterpret_cast<const u4 *>(unit + Unit<B>::DD_OFF + 16 * (lane >> 4));
  return u;
}

// The same unit through a buffer descriptor (offset out of range: all zeros,
// which decode to zero weights).
template <int B>
__device__ __forceinline__ UnitRegs<B> load_unit_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, int lane) {
  UnitRegs<B> u;
#pragma unroll
  for (int p = 0; p < B / 2; ++p)
    u.code[p] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 1024 * p + 16 * lane, 0, 0));
  u.scale = __builtin_bit_cast(
      u4, __builtin_amdgcn_raw_buffer_load_b128(r, off + Unit<B>::SCALE_OFF + 16 * (lane & 15), 0, 0));
  u.dd = __builtin_bit_cast(u4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off + Unit<B>::DD_OFF + 16 * (lane >> 4), 0, 0));
  return u;
}

struct UnitDecoded {
  h2 sc01, sc23;  // scales of sub-blocks (g, 4+g) and (8+g, 12+g)
  h8 mfrag;       // min-MFMA A fragment: m of sub-blocks 8*(g&1) .. +7
  uint32_t dd[4]; // rows 4g..4g+3: d | dmin<<16 (binary16)
};

__device__ __forceinline__ float dd_d(uint32_t v) { return half_bits_to_float((uint16_t)(v & 0xFFFFu)); }
__device__ __forceinline__ float dd_dmin(uint32_t v) { return half_bits_to_float((uint16_t)(v >> 16)); }

template <int B>
__device__ __forceinline__ UnitDecoded decode_unit(const UnitRegs<B> &u, int g) {
  UnitDecoded o;
  const uint32_t sw = (g < 2) ? u.scale.x : u.scale.y;
  const uint32_t hw = (g & 1) ? (sw >> 16) : sw;
  o.sc01 = CVT_FP8(hw & 0x0F0Fu, false);
  o.sc23 = CVT_FP8((hw >> 4) & 0x0F0Fu, false);
  const uint32_t mdw = (g & 1) ? u.scale.w : u.scale.z;
  const uint32_t lo = mdw & 0x0F0F0F0Fu, hi = (mdw >> 4) & 0x0F0F0F0Fu;
  o.mfrag = cat8(CVT_FP8(lo, false), CVT_FP8(lo, true), CVT_FP8(hi, false), CVT_FP8(hi, true));
#pragma unroll
  for (int i = 0; i < 4; ++i) o.dd[i] = u.dd[i];
  return o;
}

template <int S, int B>
__device__ __forceinline__ h8 step_frag(const UnitRegs<B> &u, const UnitDecoded &dc) {
  constexpr int Q = S >> 1;  // sub-block 4*Q + g
  const h2 pair = (Q < 2) ? dc.sc01 : dc.sc23;
  h2 sc2;
  sc2[0] = pair[Q & 1];
  sc2[1] = pair[Q & 1];
  if constexpr (B == 2) return dequant_frag<(S & 1)>(u.code[0][Q], sc2);
  else if constexpr (B == 4) return dequant_frag4(u.code[S >> 2][S & 3], sc2);
  else return dequant_frag6<(S & 1)>(u.code[S >> 2][S & 3], u.code[2][Q], sc2);
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

template <int NM, int R, int B>
__device__ __forceinline__ void gemm_load_a(UnitRegs<B> (&u)[R][NM], const GemmCtx<NM> &c, const int (&rts)[R],
                                            int sb, int lane) {
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < NM; ++m)
      u[r][m] = load_unit<B>(c.W[m] + (size_t)rts[r] * c.rt_stride + (size_t)sb * Unit<B>::BYTES, lane);
}

// The same loads in two parts: PART 0 every code plane but plane 1, PART 1
// plane 1, which steps 4-7 read (4- and 6-bit units: issued once the current
// super-block's plane 0, read by steps 0-3 only, is dead, so that the two
// super-blocks' units need few registers at once).  The scales and d/dmin go
// with PART 1 when NM == 1 (down: two row tiles, the larger register set),
// else with PART 0.
template <int PART, int NM, int R, int B>
__device__ __forceinline__ void gemm_load_a_part(UnitRegs<B> (&u)[R][NM], const GemmCtx<NM> &c, const int (&rts)[R],
                                                 int sb, int lane) {
  static_assert(B >= 4, "units with a second code plane");
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint8_t *unit = c.W[m] + (size_t)rts[r] * c.rt_stride + (size_t)sb * Unit<B>::BYTES;
      if (PART == 0) {
#pragma unroll
        for (int p = 0; p < B / 2; ++p)
          if (p != 1) u[r][m].code[p] = *reinterpret_cast<const u4 *>(unit + 1024 * p + 16 * lane);
      } else {
        u[r][m].code[1] = *reinterpret_cast<const u4 *>(unit + 1024 + 16 * lane);
      }
      if (PART == (NM == 1 ? 1 : 0)) {
        u[r][m].scale = *reinterpret_cast<const u4 *>(unit + Unit<B>::SCALE_OFF + 16 * (lane & 15));
        u[r][m].dd = *reinterpret_cast<const u4 *>(unit + Unit<B>::DD_OFF + 16 * (lane >> 4));
      }
    }
}

// Activation staging: thread -> 16-byte chunk column sc = tid % 32 of token
// rows tid/32 + SROWS*i (SROWS = threads/32), so 32 consecutive lanes move one
// row's 512 bytes (contiguous in memory and conflict-free in LDS); sums:
// thread -> row (tid%256)/4, quarter tid%4 (hi 0-7, hi 8-15, lo 0-7, lo 8-15).
template <int NR>
struct Stage {
  u4 b[NR];
  u4 s;
};

template <int NR, bool PADDED>
__device__ __forceinline__ void stage_load(Stage<NR> &st, const half_t *const (&rowp)[NR], const half_t *sp, int sb,
                                           int sc, int sq, int kreal, int jreal) {
  const int col = sb * 256 + 8 * sc;
#pragma unroll
  for (int i = 0; i < NR; ++i)
    st.b[i] = (!PADDED || col < kreal) ? *reinterpret_cast<const u4 *>(rowp[i] + col) : (u4){0u, 0u, 0u, 0u};
  if (!PADDED) {
    st.s = *reinterpret_cast<const u4 *>(sp + sb * 16);
    return;
  }
  const int j0 = sb * 16 + 8 * (sq & 1);
  u4 v = (u4){0u, 0u, 0u, 0u};
  if (j0 < jreal) {
    v = *reinterpret_cast<const u4 *>(sp + sb * 16);
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

template <int NR, int SROWS>
__device__ __forceinline__ void stage_store(const Stage<NR> &st, half_t *sB, half_t *sS, int sr0, int sc, int srow,
                                            int sq) {
#pragma unroll
  for (int i = 0; i < NR; ++i) *reinterpret_cast<u4 *>(sB + (sr0 + SROWS * i) * SB_STRIDE + 8 * sc) = st.b[i];
  *reinterpret_cast<u4 *>(sS + srow * SS_STRIDE + 8 * sq) = st.s;
}

template <int NM, int R, int B>
__device__ __forceinline__ void gemm_compute_sb(const UnitRegs<B> (&u)[R][NM], const half_t *sB, const half_t *sS,
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
        const h8 A = step_frag<S, B>(u[r][m], dc[r][m]);                                      \
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
          y[m][r][nt][q] = fmaf(dd_d(dc[r][m].dd[q]), acc[m][r][nt][q], y[m][r][nt][q]);
          y[m][r][nt][q] = fmaf(-dd_dmin(dc[r][m].dd[q]), mm[q], y[m][r][nt][q]);
        }
      }
}

// XCD-aware order of a grouped GEMM's (tile, row block) workgroups.  The
// hardware hands workgroups to the chip's 8 XCDs in turn (workgroup b to XCD
// b % 8), so workgroup b takes tile 8 * (slot / nrb) + b % 8 and row block
// slot % nrb, slot = b / 8: every row block of a tile runs on one XCD and
// reads the tile's activations through that XCD's L2 (one HBM read per tile
// instead of one per XCD).  The grid is a whole number of 8 * nrb workgroups
// (gemm_grid); tiles past the list exit at once.
constexpr int N_XCD = 8;
__device__ __forceinline__ void xcd_tile(int nrb, int &tile, int &rb) {
  const int b = blockIdx.x, slot = b / N_XCD, grp = slot / nrb;
  tile = N_XCD * grp + b % N_XCD;
  rb = slot - grp * nrb;
}
static dim3 gemm_grid(int nrb, int max_tiles) {
  return dim3((unsigned)((int64_t)nrb * ((max_tiles + N_XCD - 1) / N_XCD) * N_XCD));
}

template <int NM, int R, int NW, bool PADDED, int B>
__global__ __launch_bounds__(64 * NW) void k_moe_gemm(GemmArgs a, int nrb) {
  __shared__ __attribute__((aligned(16))) half_t sB[64 * SB_STRIDE];
  __shared__ __attribute__((aligned(16))) half_t sS[64 * SS_STRIDE];
  int tile_id, rb;
  xcd_tile(nrb, tile_id, rb);
  if (tile_id >= a.ntiles[0]) return;  // uniform over the workgroup
  const TileT tl = a.tiles[a.ntiles[1] + tile_id];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  constexpr bool GU = NM == 2;
  // gate/up epilogue: the pre-scale exponents of the tile's tokens, loaded
  // first and staged in LDS once the first prefetches are issued (visible
  // after the first barrier of the loop)
  __shared__ int32_t s_xe[16 * GEMM_NT];
  const int32_t xe_ld = (GU && tid < tl.n) ? a.pexp[tl.p0 + tid] : 0;
  const int K = GU ? a.H : a.Ipad;
  const int kreal = GU ? a.H : a.I;
  const int jreal = kreal >> 4;
  const int nsb = K >> 8;
  const int n_rt = (GU ? a.I : a.H) >> 4;
  const int rt0 = (rb * NW + wave) * R;
  int rts[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rts[r] = min(rt0 + r, n_rt - 1);

  // activation rows staged by this thread (rows without a token read zeros)
  constexpr int SROWS = 64 * NW / 32, NR = 64 / SROWS;
  const int sc = tid & 31, sr0 = tid >> 5;
  const int srow = (tid & 255) >> 2, sq = tid & 3;
  // source row of each staged row: token (gate/up) or assignment position (down);
  // the lookups are issued together, rows past the tile clamp to its first row
  int src[NR + 1];
#pragma unroll
  for (int i = 0; i <= NR; ++i) {
    const int row = i < NR ? sr0 + SROWS * i : srow;
    const int p = tl.p0 + (row < tl.n ? row : 0);
    src[i] = GU ? a.perm[p] : p;
  }
  const half_t *rowp[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const bool v = sr0 + SROWS * i < tl.n;
    rowp[i] = !v ? a.zeros : GU ? a.x16 + (size_t)(src[i] / a.k) * a.H : a.h + (size_t)src[i] * a.Ipad;
  }
  const half_t *sp = a.zeros;
  if (srow < tl.n) {
    const size_t sbase = GU ? (size_t)(src[NR] / a.k) * (a.H >> 4) : (size_t)src[NR] * (a.Ipad >> 4);
    sp = (GU ? ((sq >> 1) ? a.xs_lo : a.xs_hi) : ((sq >> 1) ? a.hs_lo : a.hs_hi)) + sbase + 8 * (sq & 1);
  }

  GemmCtx<NM> c;
  c.nsb = nsb;
  c.rt_stride = (size_t)nsb * Unit<B>::BYTES;
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

  // every prefetch is issued unconditionally (the last super-block is
  // reloaded at the end), so the load-counter waits are static
  Stage<NR> st;
  UnitRegs<B> ua[R][NM], ub[R][NM];
  stage_load<NR, PADDED>(st, rowp, sp, 0, sc, sq, kreal, jreal);
  gemm_load_a<NM, R, B>(ua, c, rts, 0, lane);
  if (GU && tid < tl.n) s_xe[tid] = xe_ld;
  for (int sb = 0; sb < nsb; sb += 2) {
    // even super-block: weights in ua, prefetch into ub
    __syncthreads();
    stage_store<NR, SROWS>(st, sB, sS, sr0, sc, srow, sq);
    __syncthreads();
    const int s1 = min(sb + 1, nsb - 1);
    stage_load<NR, PADDED>(st, rowp, sp, s1, sc, sq, kreal, jreal);
    gemm_load_a<NM, R, B>(ub, c, rts, s1, lane);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
    gemm_compute_sb<NM, R, B>(ua, sB, sS, y, r16, g);
    if (sb + 1 >= nsb) break;
    // odd super-block: weights in ub, prefetch into ua
    __syncthreads();
    stage_store<NR, SROWS>(st, sB, sS, sr0, sc, srow, sq);
    __syncthreads();
    const int s2 = min(sb + 2, nsb - 1);
    stage_load<NR, PADDED>(st, rowp, sp, s2, sc, sq, kreal, jreal);
    gemm_load_a<NM, R, B>(ua, c, rts, s2, lane);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
    gemm_compute_sb<NM, R, B>(ub, sB, sS, y, r16, g);
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
        const int e = valid ? s_xe[col] : 0;  // the token's pre-scale
        half_t hv[4];
        float ssum = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hv[q] = (half_t)swiglu_scaled(y[0][r][nt][q], y[NM - 1][r][nt][q], e);
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

// ------------------------------------------------------------------ prefill grouped GEMM, wide tiles
// Workgroup = one tile of up to 80 tokens x (8 waves * R * 16) rows of NM
// packed matrices.  Per super-block every token row of the tile (256 fp16
// activations and the 32 halves of their 16-column sums, hi then lo: 36
// chunks of 16 bytes, plus one pad chunk so that rows start on different
// banks) arrives through direct-to-LDS buffer loads into one of two ring
// slots; chunks of rows past the tile's tokens are out of range and arrive as
// zeros.  One barrier per super-block: after it every wave's loads of this
// super-block have landed and every wave has finished reading the other slot,
// which then takes the next super-block's activations while this one is
// multiplied (the packed weights of the next super-block load into the
// other register set meanwhile).  The multiply is instantiated for the tile's
// number of live 16-token n-tiles, so partial tiles issue no dead MFMAs.
constexpr int PT_NTM = 5;                                          // n-tiles per tile (80 tokens)
constexpr int PT_CH = 37;                                          // chunks per token row
constexpr int PT_NW = 8;                                           // waves per workgroup
constexpr int PT_SLOT_CH = ((PT_NTM * 16 * PT_CH + 64 * PT_NW - 1) / (64 * PT_NW)) * (64 * PT_NW);
constexpr int PT_LPW = PT_SLOT_CH / (64 * PT_NW);                  // load instructions per wave per slot
constexpr int PT_SLOT_BYTES = PT_SLOT_CH * 16;
static_assert(PT_LPW * 64 * PT_NW == PT_SLOT_CH, "slot chunks");

// chunk of the 8 activations a lane (group g) feeds at step S (see step_col)
template <int S>
__device__ __forceinline__ int step_chunk(int g) {
  return 2 * (4 * (S >> 1) + g) + (S & 1);
}

// 4-bit units: between steps 3 and 4, when the first code plane of `u` is
// dead, the rest of the next super-block's units (sb_next, if >= 0) is
// loaded into `nxt`
template <int NM, int R, int NTV, int B>
__device__ __forceinline__ void pt_compute_sb(const UnitRegs<B> (&u)[R][NM], const char *slot, f4 (&y)[NM][R][NTV],
                                              int r16, int g, UnitRegs<B> (&nxt)[R][NM], const GemmCtx<NM> &c,
                                              const int (&rts)[R], int sb_next, int lane) {
  UnitDecoded dc[R][NM];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < NM; ++m) dc[r][m] = decode_unit(u[r][m], g);
  f4 acc[NM][R][NTV];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) acc[m][r][nt] = (f4){0.f, 0.f, 0.f, 0.f};
  const char *rowb = slot + r16 * (PT_CH * 16);
  // mid(): 4-bit units, between steps 3 and 4 (see gemm_load_a_part)
  auto mid = [&]() {
    if constexpr (B >= 4) {
      __builtin_amdgcn_sched_barrier(0);
      if (sb_next >= 0) gemm_load_a_part<1, NM, R, B>(nxt, c, rts, sb_next, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if constexpr (NM == 2 && B == 2) {
    // gate/up, 2-bit: the A fragments of step S+1 are dequantized before the
    // MFMAs of step S (8 more registers; the other forms would spill)
    h8 A[2][R][NM];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < NM; ++m) A[0][r][m] = step_frag<0, B>(u[r][m], dc[r][m]);
#define PT_STEP(S)                                                                            \
  {                                                                                           \
    h8 b[NTV];                                                                                \
    _Pragma("unroll") for (int nt = 0; nt < NTV; ++nt) b[nt] =                                \
        *reinterpret_cast<const h8 *>(rowb + (16 * nt * PT_CH + step_chunk<S>(g)) * 16);       \
    if constexpr (S < 7) {                                                                    \
      _Pragma("unroll") for (int r = 0; r < R; ++r)                                           \
        _Pragma("unroll") for (int m = 0; m < NM; ++m)                                        \
          A[(S + 1) & 1][r][m] = step_frag<(S < 7 ? S + 1 : 7), B>(u[r][m], dc[r][m]);         \
    }                                                                                         \
    _Pragma("unroll") for (int r = 0; r < R; ++r) {                                           \
      _Pragma("unroll") for (int m = 0; m < NM; ++m) {                                        \
        _Pragma("unroll") for (int nt = 0; nt < NTV; ++nt) acc[m][r][nt] =                    \
            mfma16(A[S & 1][r][m], b[nt], acc[m][r][nt]);                                     \
      }                                                                                       \
    }                                                                                         \
  }
    PT_STEP(0) PT_STEP(1) PT_STEP(2) PT_STEP(3) PT_STEP(4) PT_STEP(5) PT_STEP(6) PT_STEP(7)
#undef PT_STEP
  } else {
#define PT_STEP(S)                                                                            \
  {                                                                                           \
    h8 b[NTV];                                                                                \
    _Pragma("unroll") for (int nt = 0; nt < NTV; ++nt) b[nt] =                                \
        *reinterpret_cast<const h8 *>(rowb + (16 * nt * PT_CH + step_chunk<S>(g)) * 16);       \
    _Pragma("unroll") for (int r = 0; r < R; ++r) {                                           \
      _Pragma("unroll") for (int m = 0; m < NM; ++m) {                                        \
        const h8 A = step_frag<S, B>(u[r][m], dc[r][m]);                                      \
        _Pragma("unroll") for (int nt = 0; nt < NTV; ++nt) acc[m][r][nt] =                    \
            mfma16(A, b[nt], acc[m][r][nt]);                                                  \
      }                                                                                       \
    }                                                                                         \
  }
    PT_STEP(0) PT_STEP(1) PT_STEP(2) PT_STEP(3)
    mid();
    PT_STEP(4) PT_STEP(5) PT_STEP(6) PT_STEP(7)
#undef PT_STEP
  }
  h8 bm[NTV];
#pragma unroll
  for (int nt = 0; nt < NTV; ++nt) bm[nt] = *reinterpret_cast<const h8 *>(rowb + (16 * nt * PT_CH + 32 + g) * 16);
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) {
        const f4 mm = mfma16(dc[r][m].mfrag, bm[nt], (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          y[m][r][nt][q] = fmaf(dd_d(dc[r][m].dd[q]), acc[m][r][nt][q], y[m][r][nt][q]);
          y[m][r][nt][q] = fmaf(-dd_dmin(dc[r][m].dd[q]), mm[q], y[m][r][nt][q]);
        }
      }
  // let the scheduler interleave the LDS fragment reads with the MFMAs
  if constexpr (NM == 2 && B == 2) __builtin_amdgcn_iglp_opt(0);
}

template <int NM, int R, int NTV, int B>
__device__ __forceinline__ void pt_tile(const GemmArgs &a, const GemmAct &xa, const TileT &tl, int rb, char *ring) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  constexpr bool GU = NM == 2;
  const int K = GU ? a.H : a.Ipad;
  const int nsb = K >> 8;
  const int n_rt = (GU ? a.I : a.H) >> 4;
  const int rt0 = (rb * PT_NW + wave) * R;
  int rts[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rts[r] = min(rt0 + r, n_rt - 1);

  // this lane's chunk of each of the wave's slot loads: token row u / PT_CH,
  // chunk u % PT_CH; the source row lookups are issued together
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(xa.base, xa.len);
  uint32_t src[PT_LPW], inc[PT_LPW];
  int srow[PT_LPW];
#pragma unroll
  for (int q = 0; q < PT_LPW; ++q) {
    const int u = 64 * (PT_LPW * wave + q) + lane;
    const int row = u / PT_CH;
    srow[q] = tl.p0 + (row < tl.n ? row : 0);
    if (GU) srow[q] = a.perm[srow[q]];
  }
#pragma unroll
  for (int q = 0; q < PT_LPW; ++q) {
    const int u = 64 * (PT_LPW * wave + q) + lane;
    const int row = u / PT_CH, c = u - row * PT_CH;
    const uint32_t sr = (uint32_t)(GU ? srow[q] / a.k : srow[q]);
    src[q] = DS4_OOB;
    inc[q] = 0;
    if (row < tl.n) {
      if (c < 32) {
        src[q] = sr * xa.row_bytes + 16u * c;
        inc[q] = 512;
      } else if (c < 36) {
        const int cc = c - 32;
        src[q] = ((cc >> 1) ? xa.o_slo : xa.o_shi) + sr * xa.srow_bytes + 16u * (cc & 1);
        inc[q] = 32;
      } else if (GU) {  // chunk 36: the token's pre-scale exponent, the same every super-block
        src[q] = xa.o_xe + 16u * sr;
      }
    }
  }
  auto issue = [&](int slot, int sb) {
    char *dst = ring + slot * PT_SLOT_BYTES + (PT_LPW * wave) * 1024;
#pragma unroll
    for (int q = 0; q < PT_LPW; ++q) buf_load_lds16(xr, dst + 1024 * q, src[q] + inc[q] * (uint32_t)sb);
  };

  GemmCtx<NM> c;
  c.nsb = nsb;
  c.rt_stride = (size_t)nsb * Unit<B>::BYTES;
  if (GU) {
    c.W[0] = a.gate + (size_t)tl.e * a.gu_bytes;
    c.W[NM - 1] = a.up + (size_t)tl.e * a.gu_bytes;
  } else {
    c.W[0] = a.down + (size_t)tl.e * a.d_bytes;
  }

  f4 y[NM][R][NTV];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) y[m][r][nt] = (f4){0.f, 0.f, 0.f, 0.f};

  UnitRegs<B> ua[R][NM], ub[R][NM];
  issue(0, 0);
  gemm_load_a<NM, R, B>(ua, c, rts, 0, lane);
  for (int sb = 0; sb < nsb; sb += 2) {
    // even super-block: slot 0, weights in ua; the next goes to slot 1 / ub
    wait_vm<0>();
    __syncthreads();
    if (sb + 1 < nsb) {
      issue(1, sb + 1);
      if constexpr (B >= 4) gemm_load_a_part<0, NM, R, B>(ub, c, rts, sb + 1, lane);
      else gemm_load_a<NM, R, B>(ub, c, rts, sb + 1, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    pt_compute_sb<NM, R, NTV, B>(ua, ring, y, r16, g, ub, c, rts, sb + 1 < nsb ? sb + 1 : -1, lane);
    if (sb + 1 >= nsb) break;
    // odd super-block: slot 1, weights in ub
    wait_vm<0>();
    __syncthreads();
    if (sb + 2 < nsb) {
      issue(0, sb + 2);
      if constexpr (B >= 4) gemm_load_a_part<0, NM, R, B>(ua, c, rts, sb + 2, lane);
      else gemm_load_a<NM, R, B>(ua, c, rts, sb + 2, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    pt_compute_sb<NM, R, NTV, B>(ub, ring + PT_SLOT_BYTES, y, r16, g, ua, c, rts, sb + 2 < nsb ? sb + 2 : -1, lane);
  }

  if (rt0 >= n_rt) return;
  if (GU) {
    const int nj = a.Ipad >> 4;
    // the last super-block's slot holds each token row's exponent in chunk 36
    const char *last = ring + ((nsb - 1) & 1) * PT_SLOT_BYTES;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool rv = rt0 + r < n_rt;
      const int row0 = (rt0 + r) * 16 + 4 * g;
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) {
        const int col = 16 * nt + r16;
        const bool valid = col < tl.n;
        const int e = valid ? *reinterpret_cast<const int32_t *>(last + (col * PT_CH + 36) * 16) : 0;
        half_t hv[4];
        float ssum = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hv[q] = (half_t)swiglu_scaled(y[0][r][nt][q], y[NM - 1][r][nt][q], e);
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
      for (int nt = 0; nt < NTV; ++nt) {
        const int col = 16 * nt + r16;
        if (col < tl.n) *reinterpret_cast<f4 *>(a.yp + (size_t)(tl.p0 + col) * a.H + row0) = y[0][r][nt];
      }
    }
  }
}

// One multiply instance per live n-tile count, so partial tiles issue no dead
// MFMAs.  The instances end in identical stores; the library is built with
// common-code sinking off (see build.py), which keeps those stores apart.
template <int NM, int R, int B>
__global__ __launch_bounds__(64 * PT_NW) void k_moe_gemm_wide(GemmArgs a, GemmAct xa, int nrb) {
  __shared__ __attribute__((aligned(16))) char ring[2 * PT_SLOT_BYTES];
  int tile_id, rb;
  xcd_tile(nrb, tile_id, rb);
  if (tile_id >= a.ntiles[0]) return;  // uniform over the workgroup
  const TileT tl = a.tiles[a.ntiles[1] + tile_id];
  switch ((tl.n + 15) >> 4) {  // 1..PT_NTM, uniform
    case 1: pt_tile<NM, R, 1, B>(a, xa, tl, rb, ring); break;
    case 2: pt_tile<NM, R, 2, B>(a, xa, tl, rb, ring); break;
    case 3: pt_tile<NM, R, 3, B>(a, xa, tl, rb, ring); break;
    case 4: pt_tile<NM, R, 4, B>(a, xa, tl, rb, ring); break;
    default: pt_tile<NM, R, 5, B>(a, xa, tl, rb, ring); break;
  }
}

// ------------------------------------------------------------------ small batches
// T <= 16 tokens: token t is MFMA column t of every tile (a zero column where
// the token did not choose the tile's expert), so h and y are indexed by
// token: h[(tile*T + t)*Ipad + row].  Weight bytes are streamed once per used
// expert through a PD-deep register pipeline: the loads of reduction step
// i+PD are in flight while step i is dequantized and multiplied.

// down fused with the combine, for an intermediate size below 256 (columns
// past I read as zeros).  Workgroup = one 16-row tile of y, 8 waves; wave w
// takes tiles w, w+8, ... (experts ascending), scales each tile's
// contribution to token t by the token's routing weight, and the eight
// partial sums are added in wave order, then the shared-expert output.
template <int PD, bool PADDED, int B>
__global__ __launch_bounds__(512) void k_down_dec(GemmArgs a) {
  const int rt = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  // lane L: expert and token mask of this wave's L-th tile (at most 32), read
  // together with the tile count from every entry the buffer holds; the lanes
  // past the count are cleared once it is known
  int e_l = 0;
  uint32_t m_l = 0u;
  if (lane < 32) {
    const int i = min(wave + 8 * lane, a.dt_cap - 1);
    e_l = a.dtiles[i].e;
    m_l = a.dtiles[i].tmask;
  }
  const int ntl = *a.ntiles;
  const int nsb = a.Ipad >> 8;
  const int nj = a.Ipad >> 4, nj_real = a.I >> 4;
  const int mt = wave < ntl ? (ntl - wave + 7) >> 3 : 0;  // tiles of this wave (<= 32)
  const int nit = mt * nsb;
  // wait for them here, before any weight load is in flight, so that the
  // pipelined loop below never has to drain the load counter for them
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (lane >= mt) {
    e_l = 0;
    m_l = 0u;
  }
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(a.wsb, a.ws_len);
  const uint32_t hs_base = ((g >> 1) ? a.o_hs_lo : a.o_hs_hi) + 2u * (8 * (g & 1));

  struct Stage {
    UnitRegs<B> wd;
    h8 b[9];
    float wt;
  };
  Stage st[PD];
  f4 y = (f4){0.f, 0.f, 0.f, 0.f};
  int lt = 0, lsb = 0;  // tile and super-block of the next load
  // every step issues the same loads (steps past the end read zeros), so the
  // load counter waits are static and the pipeline never drains
  auto load = [&](Stage &sg) {
    const bool in = lt < mt;
    const int tile = min(wave + 8 * lt, ntl - 1);
    const int e = __builtin_amdgcn_readlane(e_l, lt & 63);
    const uint32_t tmask = in ? (uint32_t)__builtin_amdgcn_readlane((int)m_l, lt & 63) : 0u;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.down + (size_t)e * a.d_bytes, (uint32_t)a.d_bytes);
    sg.wd = load_unit_buf<B>(wr, in ? ((uint32_t)rt * nsb + lsb) * Unit<B>::BYTES : DS4_OOB, lane);
    // h of token r16 if it chose the expert (zeros otherwise, weight 0)
    const bool routed = (tmask >> r16) & 1u;  // implies r16 < T
    const uint32_t p = (uint32_t)tile * a.T + r16;
    const uint32_t hoff = routed ? a.o_h + 2u * (p * a.Ipad + lsb * 256 + 16 * g) : DS4_OOB;
    const uint32_t soff = routed ? hs_base + 2u * (p * nj + lsb * 16) : DS4_OOB;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t o = hoff + 2u * (64 * (q >> 1) + 8 * (q & 1));
      if (PADDED && lsb * 256 + 16 * (4 * (q >> 1) + g) + 8 * (q & 1) >= a.I) o = DS4_OOB;  // columns >= I
      sg.b[q] = buf_load_h8(ws, o);
    }
    h8 v = buf_load_h8(ws, soff);
    if (PADDED) {
      const int j0 = lsb * 16 + 8 * (g & 1);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (j0 + q >= nj_real) v[q] = (half_t)0.0f;
    }
    sg.b[8] = v;
    sg.wt = a.dtiles[tile].w[r16];  // 0 for tokens that did not choose the expert
    if (++lsb == nsb) {
      lsb = 0;
      ++lt;
    }
  };
  auto compute = [&](const Stage &sg) {
    const UnitDecoded dd = decode_unit(sg.wd, g);
    f4 ac = (f4){0.f, 0.f, 0.f, 0.f};
#define DEC_STEP(S) ac = mfma16(step_frag<S, B>(sg.wd, dd), sg.b[S], ac);
    DEC_STEP(0) DEC_STEP(1) DEC_STEP(2) DEC_STEP(3) DEC_STEP(4) DEC_STEP(5) DEC_STEP(6) DEC_STEP(7)
#undef DEC_STEP
    const f4 mm = mfma16(dd.mfrag, sg.b[8], (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float v = fmaf(dd_d(dd.dd[q]), ac[q], -dd_dmin(dd.dd[q]) * mm[q]);
      y[q] = fmaf(sg.wt, v, y[q]);
    }
  };
#pragma unroll
  for (int sgi = 0; sgi < PD; ++sgi) load(st[sgi]);
  for (int i0 = 0; i0 < nit; i0 += PD) {
#pragma unroll
    for (int sgi = 0; sgi < PD; ++sgi) {
      compute(st[sgi]);
      load(st[sgi]);
    }
  }
  __shared__ f4 red[8][64];
  red[wave][lane] = y;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < 8; ++w) {
    const f4 p = red[w][lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] += p[q];
  }
  if (r16 < a.T) {
    const size_t o = (size_t)r16 * a.H + rt * 16 + 4 * g;
    if (a.ysh) {
      const f4 v = *reinterpret_cast<const f4 *>(a.ysh + o);
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] += v[q];
    }
    *reinterpret_cast<f4 *>(a.y + o) = y;
  }
}

// ------------------------------------------------------------------ small batches, T <= 4
// Variants of the two kernels above for batches of at most four tokens (the
// gate/up one is used for a single token, the down one up to four): the
// activations of each reduction step (x or h of the T tokens: 256 values and
// the 16-column sums, 36 chunks of 16 bytes per token, padded to 37) come in
// through one to three direct-to-LDS buffer loads per step instead of nine
// 64-lane register loads, into a per-wave ring of PD LDS slots filled at the
// same pipeline distance as the weights; the MFMA B fragments are read from
// the slot.  Chunks of tokens that did not choose the tile's expert are out
// of range and arrive as zeros.
constexpr int XCH = 37;  // 16-byte chunks per token per step (36 + 1 pad)

template <int NT>
struct SlotLoads {
  static constexpr int NI = (NT * XCH + 63) / 64;  // load instructions per step
};


// Routing folded into a small-batch gate/up workgroup of 256 threads: the
// workgroup routes the batch itself from the router's partial sums (one
// token: route_one_token; 2-4 tokens: route_small_block, one wave per token)
// in `lds` (the kernel's ring, before the ring is used) and takes the
// tile_id-th used expert; workgroup 0 writes the routing outputs and the
// tiles for the down kernel.  Returns false (uniformly) when the batch uses
// fewer than tile_id + 1 experts.
template <int NT>
__device__ __forceinline__ bool route_take_tile(char *lds, const DecRoute &rr, int T, int tile_id, int &e,
                                                uint32_t &tmask) {
  RouteLds<4> &L = *reinterpret_cast<RouteLds<4> *>(lds);
  const int lane = threadIdx.x & 63;
  if (NT == 1) {
    if (tile_id >= rr.k) return false;
    e = route_one_token<256>(L, rr.part, rr.nslice, rr.bias, rr.logits, rr.E, rr.k, rr.ro, rr.dt, rr.ntile,
                             blockIdx.x == 0, tile_id);
    tmask = 1u;
  } else {
    route_small_block<256, 4>(L, rr.part, rr.nslice, rr.bias, rr.logits, T, rr.E, rr.k, rr.ro, rr.dt, rr.ntile,
                              blockIdx.x == 0);
    if (tile_id >= L.ntile) return false;
    // the used expert whose tile index is tile_id (lowest e among equal tb: the used one)
    int sel = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ee = lane + 64 * i;
      const bool hit = ee < rr.E && L.tm[ee] != 0u && L.tb[ee] == tile_id;
      const uint64_t b = __ballot(hit);
      if (sel < 0 && b) sel = 64 * i + __ffsll((unsigned long long)b) - 1;
    }
    e = sel;
    tmask = L.tm[e];
  }
  __syncthreads();  // every wave has read the routing before the ring is filled
  return true;
}

// ROUTE: the workgroup routes the batch itself (route_take_tile).
template <int PD, int NT, bool ROUTE, int B, int KS>
__global__ __launch_bounds__(256) void k_gateup_dec_lds(GemmArgs a, int n_rt, DecRoute rr) {
  constexpr int NI = SlotLoads<NT>::NI;
  constexpr int SLOT = 64 * 16 * NI;  // bytes per ring slot
  constexpr int RPW = 4 / KS;         // row tiles per workgroup; KS waves split each one's reduction
  static_assert(KS == 1 || KS == 2 || KS == 4, "reduction splits");
  __shared__ __attribute__((aligned(16))) char ring_lds[4 * PD * SLOT];
  const int nrb = (n_rt + RPW - 1) / RPW;
  const int tile_id = blockIdx.x / nrb;
  const int rb = blockIdx.x - tile_id * nrb;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int e;
  uint32_t tmask;
  if constexpr (ROUTE) {
    static_assert(sizeof(RouteLds<4>) <= sizeof(ring_lds), "routing LDS must fit in the ring");
    if (!route_take_tile<NT>(ring_lds, rr, a.T, tile_id, e, tmask)) return;  // uniform over the workgroup
  } else {
    // the tile is read together with the count (the grid covers the buffer)
    const int ti = min(tile_id, a.dt_cap - 1);
    e = a.dtiles[ti].e;
    tmask = a.dtiles[ti].tmask;
    if (tile_id >= *a.ntiles) return;  // uniform over the workgroup
  }
  const int r16 = lane & 15, g = lane >> 4;
  const int rt = RPW * rb + wave / KS, kh = wave % KS;
  const int nsb = a.H >> 8;
  const int part = (nsb + KS - 1) / KS;
  const int sb0 = kh * part;
  const int nit = max(0, min(nsb, sb0 + part) - sb0);
  const uint32_t gub = (uint32_t)a.gu_bytes;
  const __amdgpu_buffer_rsrc_t gr = make_rsrc(a.gate + (size_t)e * a.gu_bytes, gub);
  const __amdgpu_buffer_rsrc_t ur = make_rsrc(a.up + (size_t)e * a.gu_bytes, gub);
  const uint32_t roff = ((uint32_t)min(rt, n_rt - 1) * nsb + sb0) * Unit<B>::BYTES;
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(a.wsb, a.ws_len);
  // chunk u = 64*q + lane of a slot: token u / XCH, chunk c = u % XCH
  uint32_t src[NI], inc[NI];
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int u = 64 * q + lane;
    const int t = u / XCH, c = u - t * XCH;
    src[q] = DS4_OOB;
    inc[q] = 0;
    if (t < NT && c < 36 && ((tmask >> t) & 1u)) {
      if (c < 32) {
        src[q] = a.o_x16 + 2u * ((uint32_t)t * a.H + (uint32_t)sb0 * 256 + 8 * c);
        inc[q] = 512;
      } else {
        const int cc = c - 32;
        src[q] = ((cc >> 1) ? a.o_xs_lo : a.o_xs_hi) + 2u * ((uint32_t)t * (a.H >> 4) + sb0 * 16 + 8 * (cc & 1));
        inc[q] = 32;
      }
    }
  }
  // B fragment of lane (r16, g): token r16 (columns r16 >= T read token 0 and are discarded)
  const uint32_t brow = (uint32_t)(r16 < NT ? r16 : 0) * (XCH * 16);
  char *ring = ring_lds + wave * (PD * SLOT);  // this wave's PD slots

  struct Stage {
    UnitRegs<B> wg, wu;
  };
  Stage st[PD];
  f4 yg = (f4){0.f, 0.f, 0.f, 0.f}, yu = yg;
  auto load = [&](Stage &sg, int slot, int i) {
    const bool in = i < nit;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): earlier reads of this slot are done
#pragma unroll
    for (int q = 0; q < NI; ++q)
      buf_load_lds16(ws, ring + slot * SLOT + 64 * 16 * q, in ? src[q] + inc[q] * (uint32_t)i : DS4_OOB);
    const uint32_t wo = in ? roff + (uint32_t)i * Unit<B>::BYTES : DS4_OOB;
    sg.wg = load_unit_buf<B>(gr, wo, lane);
    sg.wu = load_unit_buf<B>(ur, wo, lane);
  };
  auto compute = [&](const Stage &sg, int slot) {
    wait_vm<(PD - 1) * (NI + 2 * Unit<B>::LOADS)>();  // this step's loads (LDS and registers) have landed
    const char *base = ring + slot * SLOT + brow;
    h8 b[9];
#pragma unroll
    for (int S = 0; S < 8; ++S)
      b[S] = *reinterpret_cast<const h8 *>(base + 16 * (2 * (4 * (S >> 1) + g) + (S & 1)));
    b[8] = *reinterpret_cast<const h8 *>(base + 16 * (32 + 2 * (g >> 1) + (g & 1)));
    const UnitDecoded dg = decode_unit(sg.wg, g);
    const UnitDecoded du = decode_unit(sg.wu, g);
    f4 ag = (f4){0.f, 0.f, 0.f, 0.f}, au = ag;
#define DEC_STEP(S)                                  \
  ag = mfma16(step_frag<S, B>(sg.wg, dg), b[S], ag);    \
  au = mfma16(step_frag<S, B>(sg.wu, du), b[S], au);
    DEC_STEP(0) DEC_STEP(1) DEC_STEP(2) DEC_STEP(3) DEC_STEP(4) DEC_STEP(5) DEC_STEP(6) DEC_STEP(7)
#undef DEC_STEP
    const f4 z = (f4){0.f, 0.f, 0.f, 0.f};
    const f4 mg = mfma16(dg.mfrag, b[8], z);
    const f4 mu = mfma16(du.mfrag, b[8], z);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      yg[q] = fmaf(dd_d(dg.dd[q]), ag[q], yg[q]);
      yg[q] = fmaf(-dd_dmin(dg.dd[q]), mg[q], yg[q]);
      yu[q] = fmaf(dd_d(du.dd[q]), au[q], yu[q]);
      yu[q] = fmaf(-dd_dmin(du.dd[q]), mu[q], yu[q]);
    }
  };
#pragma unroll
  for (int sgi = 0; sgi < PD; ++sgi) load(st[sgi], sgi, sgi);
  for (int i0 = 0; i0 < nit; i0 += PD) {
#pragma unroll
    for (int sgi = 0; sgi < PD; ++sgi) {
      compute(st[sgi], sgi);
      load(st[sgi], sgi, i0 + sgi + PD);
    }
  }

  // [row tile of the workgroup][reduction part 1..KS-1][gate, up]
  __shared__ f4 red[RPW][KS > 1 ? KS - 1 : 1][2][64];
  const int rl = wave / KS;
  if (kh > 0) {
    red[rl][kh - 1][0][lane] = yg;
    red[rl][kh - 1][1][lane] = yu;
  }
  if constexpr (KS > 1) __syncthreads();
  if (kh > 0 || rt >= n_rt) return;  // uniform per wave
#pragma unroll
  for (int j = 0; j < KS - 1; ++j) {
    const f4 pg = red[rl][j][0][lane], pu = red[rl][j][1][lane];
    yg += pg;
    yu += pu;
  }
  const int xe = r16 < a.T ? a.xexp[r16] : 0;  // token r16's pre-scale
  half_t hv[4];
  float ssum = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hv[q] = (half_t)swiglu_scaled(yg[q], yu[q], xe);
    ssum += (float)hv[q];
  }
  ssum += __shfl_xor(ssum, 16);
  ssum += __shfl_xor(ssum, 32);
  if (r16 < a.T) {  // tokens that did not choose the expert get exact zeros
    const size_t p = (size_t)tile_id * a.T + r16;
    uint2 pk;
    __builtin_memcpy(&pk, hv, 8);
    *reinterpret_cast<uint2 *>(a.h + p * a.Ipad + rt * 16 + 4 * g) = pk;
    if (g == 0) {
      const int nj = a.Ipad >> 4;
      const half_t hi = (half_t)ssum;
      a.hs_hi[p * nj + rt] = hi;
      a.hs_lo[p * nj + rt] = (half_t)(ssum - (float)hi);
    }
  }
}

// down fused with the combine (I a multiple of 256), activations through LDS.
// Workgroup = one 16-row tile of y, 8 * KSP waves: wave w takes tiles w % 8,
// w % 8 + 8, ... (experts ascending) over super-blocks part w / 8 of KSP;
// the partial sums are added in wave order, then the shared output.
template <int PD, int NT, int B, int KSP>
__global__ __launch_bounds__(512 * KSP) void k_down_dec_lds(GemmArgs a) {
  constexpr int NI = SlotLoads<NT>::NI;
  constexpr int SLOT = 64 * 16 * NI;
  constexpr int NWV = 8 * KSP;  // KSP waves split each tile's reduction
  __shared__ __attribute__((aligned(16))) char ring_lds[NWV * PD * SLOT];
  const int rt = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wv = wave & 7, kh = wave >> 3;
  const int r16 = lane & 15, g = lane >> 4;
  // lane L: expert and token mask of this wave's L-th tile (a wave owns at
  // most 32).  They are read together with the tile count, from every entry
  // the buffer holds, and the lanes past the count are cleared once it is known.
  int e_l = 0;
  uint32_t m_l = 0u;
  if (lane < 32) {
    const int i = min(wv + 8 * lane, a.dt_cap - 1);
    e_l = a.dtiles[i].e;
    m_l = a.dtiles[i].tmask;
  }
  const int ntl = *a.ntiles;
  const int nsb = a.Ipad >> 8;
  const int nj = a.Ipad >> 4;
  const int mt = wv < ntl ? (ntl - wv + 7) >> 3 : 0;  // tiles of this wave (<= 32)
  const int nsw = nsb / KSP, sbb = kh * nsw;            // its super-blocks sbb .. sbb + nsw - 1 of each
  const int nit = mt * nsw;
  // wait for them here, before any weight load is in flight, so that the
  // pipelined loop below never has to drain the load counter for them
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (lane >= mt) {
    e_l = 0;
    m_l = 0u;
  }
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(a.wsb, a.ws_len);
  // chunk u = 64*q + lane of a slot: token u / XCH, chunk c = u % XCH
  // chunks c < 32: h[p][256*sb + 8c ...]; c = 32..35: sums hi/lo [p][16*sb + 8*(c&1) ...]
  uint32_t cbase[NI], crow[NI], cstep[NI];
  int ctok[NI];
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int u = 64 * q + lane;
    const int t = u / XCH, c = u - t * XCH;
    ctok[q] = (t < NT && c < 36) ? t : -1;
    if (c < 32) {
      cbase[q] = a.o_h + 2u * (8 * c);
      crow[q] = 2u * a.Ipad;
      cstep[q] = 512;
    } else {
      cbase[q] = (((c - 32) >> 1) ? a.o_hs_lo : a.o_hs_hi) + 2u * (8 * ((c - 32) & 1));
      crow[q] = 2u * nj;
      cstep[q] = 32;
    }
  }
  const uint32_t brow = (uint32_t)(r16 < NT ? r16 : 0) * (XCH * 16);
  char *ring = ring_lds + wave * (PD * SLOT);  // this wave's PD slots

  struct Stage {
    UnitRegs<B> wd;
    float wt;
  };
  Stage st[PD];
  f4 y = (f4){0.f, 0.f, 0.f, 0.f};
  int lt = 0, lsb = sbb;  // tile and super-block of the next load
  auto load = [&](Stage &sg, int slot) {
    const bool in = lt < mt;
    const int tile = min(wv + 8 * lt, ntl - 1);
    const int e = __builtin_amdgcn_readlane(e_l, lt & 63);
    const uint32_t tmask = in ? (uint32_t)__builtin_amdgcn_readlane((int)m_l, lt & 63) : 0u;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): earlier reads of this slot are done
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int t = ctok[q];
      const bool ok = t >= 0 && ((tmask >> t) & 1u);
      const uint32_t p = (uint32_t)tile * a.T + t;
      const uint32_t off = ok ? cbase[q] + crow[q] * p + cstep[q] * (uint32_t)lsb : DS4_OOB;
      buf_load_lds16(ws, ring + slot * SLOT + 64 * 16 * q, off);
    }
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.down + (size_t)e * a.d_bytes, (uint32_t)a.d_bytes);
    sg.wd = load_unit_buf<B>(wr, in ? ((uint32_t)rt * nsb + lsb) * Unit<B>::BYTES : DS4_OOB, lane);
    sg.wt = a.dtiles[tile].w[r16];  // 0 for tokens that did not choose the expert
    if (++lsb == sbb + nsw) {
      lsb = sbb;
      ++lt;
    }
  };
  auto compute = [&](const Stage &sg, int slot) {
    wait_vm<(PD - 1) * (NI + Unit<B>::LOADS + 1)>();  // this step's loads (LDS and registers) have landed
    const char *base = ring + slot * SLOT + brow;
    h8 b[9];
#pragma unroll
    for (int S = 0; S < 8; ++S)
      b[S] = *reinterpret_cast<const h8 *>(base + 16 * (2 * (4 * (S >> 1) + g) + (S & 1)));
    b[8] = *reinterpret_cast<const h8 *>(base + 16 * (32 + 2 * (g >> 1) + (g & 1)));
    const UnitDecoded dd = decode_unit(sg.wd, g);
    f4 ac = (f4){0.f, 0.f, 0.f, 0.f};
#define DEC_STEP(S) ac = mfma16(step_frag<S, B>(sg.wd, dd), b[S], ac);
    DEC_STEP(0) DEC_STEP(1) DEC_STEP(2) DEC_STEP(3) DEC_STEP(4) DEC_STEP(5) DEC_STEP(6) DEC_STEP(7)
#undef DEC_STEP
    const f4 mm = mfma16(dd.mfrag, b[8], (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float v = fmaf(dd_d(dd.dd[q]), ac[q], -dd_dmin(dd.dd[q]) * mm[q]);
      y[q] = fmaf(sg.wt, v, y[q]);
    }
  };
#pragma unroll
  for (int sgi = 0; sgi < PD; ++sgi) load(st[sgi], sgi);
  for (int i0 = 0; i0 < nit; i0 += PD) {
#pragma unroll
    for (int sgi = 0; sgi < PD; ++sgi) {
      compute(st[sgi], sgi);
      load(st[sgi], sgi);
    }
  }
  __shared__ f4 red[NWV][64];
  red[wave][lane] = y;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < NWV; ++w) {
    const f4 p = red[w][lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] += p[q];
  }
  if (r16 < a.T) {
    const size_t o = (size_t)r16 * a.H + rt * 16 + 4 * g;
    if (a.ysh) {
      const f4 v = *reinterpret_cast<const f4 *>(a.ysh + o);
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] += v[q];
    }
    *reinterpret_cast<f4 *>(a.y + o) = y;
  }
}

// ------------------------------------------------------------------ small batches, 2 <= T <= 16
// The activations of one reduction step (x or h of NT token slots, 37 chunks
// of 16 bytes each: 592 chunks for 16 slots, 148 for 4) are shared by the
// waves of a workgroup: they come in once per workgroup by direct-to-LDS
// buffer loads split across the waves into a PD-slot ring, with one barrier
// per step.  After that barrier every wave's loads of the step have landed
// (each wave waits for its own first) and every wave has finished reading the
// slot the step's prefetch then refills.  At T = 16 a wave issues 2-3
// activation loads per step instead of 9, which is what bounds these kernels
// there; at 2-4 tokens (four slots) one, and the per-wave ring kernel above
// is then 1.3-1.4x slower.  With 2-4 tokens the gate/up workgroup also
// routes the batch itself.
template <int NW, int NT>
struct ShRing {
  static constexpr int NI = (NT * XCH + 64 * NW - 1) / (64 * NW);  // load instructions per wave per step
  static constexpr int SLOT = NI * NW * 1024;                      // bytes per slot
};

// gate/up + SwiGLU: workgroup = one tile x NW 16-row tiles, the whole
// reduction per wave.
template <int PD, int NW, int B, int NT, bool ROUTE, bool SDL = false>
__global__ __launch_bounds__(64 * NW) void k_gateup_dec_sh(GemmArgs a, int n_rt, DecRoute rr) {
  constexpr int NI = ShRing<NW, NT>::NI;
  // SDL: each wave's gate and up scales + d|dmin (320 bytes per unit) land in
  // the slot after the activations by one 20-lane direct load per unit
  constexpr int SDW = SDL ? 640 : 0;
  constexpr int SLOT = ShRing<NW, NT>::SLOT + NW * SDW;
  constexpr int LPS = NI + (SDL ? B + 2 : 2 * Unit<B>::LOADS);  // vector memory instructions per step
  static_assert(PD >= 2, "ring depth");
  static_assert(!ROUTE || (NW == 4 && NT <= 4), "routing: 256 threads, at most 4 tokens");
  __shared__ __attribute__((aligned(16))) char ring[PD * SLOT];
  const int nrb = (n_rt + NW - 1) / NW;
  const int tile_id = blockIdx.x / nrb;
  const int rb = blockIdx.x - tile_id * nrb;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  int e;
  uint32_t tmask;
  if constexpr (ROUTE) {
    static_assert(sizeof(RouteLds<4>) <= sizeof(ring), "routing LDS must fit in the ring");
    if (!route_take_tile<NT>(ring, rr, a.T, tile_id, e, tmask)) return;  // uniform over the workgroup
  } else {
    // the tile is read together with the count (the grid covers the buffer)
    const int ti = min(tile_id, a.dt_cap - 1);
    e = a.dtiles[ti].e;
    tmask = a.dtiles[ti].tmask;
    if (tile_id >= *a.ntiles) return;  // uniform over the workgroup
  }
  const int rt = NW * rb + wave;
  const int nsb = a.H >> 8;
  const uint32_t gub = (uint32_t)a.gu_bytes;
  const __amdgpu_buffer_rsrc_t gr = make_rsrc(a.gate + (size_t)e * a.gu_bytes, gub);
  const __amdgpu_buffer_rsrc_t ur = make_rsrc(a.up + (size_t)e * a.gu_bytes, gub);
  const uint32_t roff = (uint32_t)min(rt, n_rt - 1) * nsb * Unit<B>::BYTES;
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(a.wsb, a.ws_len);
  // chunk u = 64*(NW*q + wave) + lane of a slot: token u / XCH, chunk u % XCH
  uint32_t src[NI], inc[NI];
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int u = 64 * (NW * q + wave) + lane;
    const int t = u / XCH, c = u - t * XCH;
    src[q] = DS4_OOB;
    inc[q] = 0;
    if (t < NT && c < 36 && ((tmask >> t) & 1u)) {  // tmask bits only below T
      if (c < 32) {
        src[q] = a.o_x16 + 2u * ((uint32_t)t * a.H + 8 * c);
        inc[q] = 512;
      } else {
        const int cc = c - 32;
        src[q] = ((cc >> 1) ? a.o_xs_lo : a.o_xs_hi) + 2u * ((uint32_t)t * (a.H >> 4) + 8 * (cc & 1));
        inc[q] = 32;
      }
    }
  }
  // B fragment of lane (r16, g): token slot r16 (columns r16 >= NT read slot 0 and are discarded)
  const uint32_t brow = (uint32_t)(r16 < NT ? r16 : 0) * (XCH * 16);

  struct Stage {
    UnitRegs<B> wg, wu;
  };
  Stage st[PD];
  f4 yg = (f4){0.f, 0.f, 0.f, 0.f}, yu = yg;
  auto load = [&](Stage &sg, int slot, int i) {
    const bool in = i < nsb;
#pragma unroll
    for (int q = 0; q < NI; ++q)
      buf_load_lds16(ws, ring + slot * SLOT + 1024 * (NW * q + wave), in ? src[q] + inc[q] * (uint32_t)i : DS4_OOB);
    const uint32_t wo = in ? roff + (uint32_t)i * Unit<B>::BYTES : DS4_OOB;
    if constexpr (SDL) {
      char *sd = ring + slot * SLOT + ShRing<NW, NT>::SLOT + wave * SDW;
      if (lane < 20) {  // 320 bytes: lane l's 16 land at sd + 16*l
        const uint32_t so = in ? wo + Unit<B>::SCALE_OFF + 16u * lane : DS4_OOB;
        buf_load_lds16(gr, sd, so);
        buf_load_lds16(ur, sd + 320, so);
      }
#pragma unroll
      for (int p = 0; p < B / 2; ++p) {
        sg.wg.code[p] =
            __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(gr, wo + 1024 * p + 16 * lane, 0, 0));
        sg.wu.code[p] =
            __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(ur, wo + 1024 * p + 16 * lane, 0, 0));
      }
    } else {
      sg.wg = load_unit_buf<B>(gr, wo, lane);
      sg.wu = load_unit_buf<B>(ur, wo, lane);
    }
  };
  auto compute = [&](const Stage &sg0, int slot) {
    Stage sg = sg0;
    if constexpr (SDL) {  // scales of row r16, d|dmin of rows 4g..4g+3 (the unit's byte layout)
      const char *sd = ring + slot * SLOT + ShRing<NW, NT>::SLOT + wave * SDW;
      sg.wg.scale = *reinterpret_cast<const u4 *>(sd + 16 * r16);
      sg.wg.dd = *reinterpret_cast<const u4 *>(sd + 256 + 16 * g);
      sg.wu.scale = *reinterpret_cast<const u4 *>(sd + 320 + 16 * r16);
      sg.wu.dd = *reinterpret_cast<const u4 *>(sd + 576 + 16 * g);
    }
    const char *base = ring + slot * SLOT + brow;
    h8 b[9];
#pragma unroll
    for (int S = 0; S < 8; ++S)
      b[S] = *reinterpret_cast<const h8 *>(base + 16 * (2 * (4 * (S >> 1) + g) + (S & 1)));
    b[8] = *reinterpret_cast<const h8 *>(base + 16 * (32 + 2 * (g >> 1) + (g & 1)));
    const UnitDecoded dg = decode_unit(sg.wg, g);
    const UnitDecoded du = decode_unit(sg.wu, g);
    f4 ag = (f4){0.f, 0.f, 0.f, 0.f}, au = ag;
#define DEC_STEP(S)                                  \
  ag = mfma16(step_frag<S, B>(sg.wg, dg), b[S], ag); \
  au = mfma16(step_frag<S, B>(sg.wu, du), b[S], au);
    DEC_STEP(0) DEC_STEP(1) DEC_STEP(2) DEC_STEP(3) DEC_STEP(4) DEC_STEP(5) DEC_STEP(6) DEC_STEP(7)
#undef DEC_STEP
    const f4 z = (f4){0.f, 0.f, 0.f, 0.f};
    const f4 mg = mfma16(dg.mfrag, b[8], z);
    const f4 mu = mfma16(du.mfrag, b[8], z);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      yg[q] = fmaf(dd_d(dg.dd[q]), ag[q], yg[q]);
      yg[q] = fmaf(-dd_dmin(dg.dd[q]), mg[q], yg[q]);
      yu[q] = fmaf(dd_d(du.dd[q]), au[q], yu[q]);
      yu[q] = fmaf(-dd_dmin(du.dd[q]), mu[q], yu[q]);
    }
  };
  // steps past the end load out of range (zeros): every step issues the same
  // loads, so the waits are static
#pragma unroll
  for (int sgi = 0; sgi < PD - 1; ++sgi) load(st[sgi], sgi, sgi);
  for (int i0 = 0; i0 < nsb; i0 += PD) {
#pragma unroll
    for (int sgi = 0; sgi < PD; ++sgi) {
      wait_vm<(PD - 2) * LPS>();  // this wave's loads of step i0+sgi have landed
      __syncthreads();                                  // ... and every wave's; slot sgi-1 is free
      load(st[(sgi + PD - 1) % PD], (sgi + PD - 1) % PD, i0 + sgi + PD - 1);
      compute(st[sgi], sgi);
    }
  }
  wait_vm<0>();  // the trailing out-of-range loads, before the workgroup's LDS is released
  if (rt >= n_rt) return;
  const int xe = r16 < a.T ? a.xexp[r16] : 0;  // token r16's pre-scale
  half_t hv[4];
  float ssum = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hv[q] = (half_t)swiglu_scaled(yg[q], yu[q], xe);
    ssum += (float)hv[q];
  }
  ssum += __shfl_xor(ssum, 16);
  ssum += __shfl_xor(ssum, 32);
  if (r16 < a.T) {  // tokens that did not choose the expert get exact zeros
    const size_t p = (size_t)tile_id * a.T + r16;
    uint2 pk;
    __builtin_memcpy(&pk, hv, 8);
    *reinterpret_cast<uint2 *>(a.h + p * a.Ipad + rt * 16 + 4 * g) = pk;
    if (g == 0) {
      const int nj = a.Ipad >> 4;
      const half_t hi = (half_t)ssum;
      a.hs_hi[p * nj + rt] = hi;
      a.hs_lo[p * nj + rt] = (half_t)(ssum - (float)hi);
    }
  }
}

// down for 5 <= T <= 16 (I a multiple of 256): workgroup = R 16-row tiles
// of y, all taken by every wave, so that one set of activation loads feeds R
// units; 8 waves, and the tile list split over NH workgroups (blockIdx.y):
// tile j goes to part j % NH and wave (j / NH) % 8, experts ascending within
// a wave.  Each workgroup adds its waves' partial sums in wave order and
// writes its part's partial; k_down_reduce adds the NH parts in order, then
// the shared-expert output.
template <int PD, int B, bool SDL, int R, int NH>
__global__ __launch_bounds__(512) void k_down_dec2(GemmArgs a) {
  // SDL: the R units' scales and d|dmin (320 bytes each) land in a
  // per-wave LDS slot by one 20-lane direct load per unit
  constexpr int LPS = 9 + (SDL ? R * (B / 2) + R : R * Unit<B>::LOADS);  // vector memory instructions per step
  constexpr int TS = 8 * NH;                                             // tile stride of a wave
  __shared__ __attribute__((aligned(16))) char sdl[SDL ? 8 * PD * R * 320 : 16];
  const int rt0 = R * blockIdx.x, half = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int j0 = half + NH * wave;  // this wave's first tile
  // lane L: expert and token mask of this wave's L-th tile (at most 16), read
  // together with the tile count from every entry the buffer holds; the lanes
  // past the count are cleared once it is known
  int e_l = 0;
  uint32_t m_l = 0u;
  if (lane < 16) {
    const int i = min(j0 + TS * lane, a.dt_cap - 1);
    e_l = a.dtiles[i].e;
    m_l = a.dtiles[i].tmask;
  }
  const int ntl = *a.ntiles;
  const int nsb = a.Ipad >> 8;
  const int nj = a.Ipad >> 4;
  const int mt = j0 < ntl ? (ntl - j0 + TS - 1) / TS : 0;  // its tiles j0, j0 + TS, ... (<= 16)
  const int nit = mt * nsb;
  // wait for them here, before any weight load is in flight, so that the
  // pipelined loop below never has to drain the load counter for them
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (lane >= mt) {
    e_l = 0;
    m_l = 0u;
  }
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(a.wsb, a.ws_len);
  const uint32_t hs_base = ((g >> 1) ? a.o_hs_lo : a.o_hs_hi) + 2u * (8 * (g & 1));
  const uint32_t ustride = (uint32_t)nsb * Unit<B>::BYTES;  // bytes per row tile

  struct Stage {
    UnitRegs<B> wd[R];
    h8 b[9];
    float wt;
  };
  Stage st[PD];
  f4 y[R];
#pragma unroll
  for (int r = 0; r < R; ++r) y[r] = (f4){0.f, 0.f, 0.f, 0.f};
  int lt = 0, lsb = 0;  // tile and super-block of the next load
  auto load = [&](Stage &sg, int slot) {
    const bool in = lt < mt;
    const int tile = min(j0 + TS * lt, ntl - 1);
    const int e = __builtin_amdgcn_readlane(e_l, lt & 63);
    const uint32_t tmask = in ? (uint32_t)__builtin_amdgcn_readlane((int)m_l, lt & 63) : 0u;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.down + (size_t)e * a.d_bytes, (uint32_t)a.d_bytes);
    const uint32_t wo = in ? (uint32_t)rt0 * ustride + (uint32_t)lsb * Unit<B>::BYTES : DS4_OOB;
    if constexpr (SDL) {
      char *sd = sdl + (wave * PD + slot) * (R * 320);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): earlier reads of this slot are done
      if (lane < 20) {  // 320 bytes per unit: lane l's 16 land at sd + 16*l
#pragma unroll
        for (int r = 0; r < R; ++r)
          buf_load_lds16(wr, sd + 320 * r, in ? wo + r * ustride + Unit<B>::SCALE_OFF + 16u * lane : DS4_OOB);
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int p = 0; p < B / 2; ++p)
          sg.wd[r].code[p] = __builtin_bit_cast(
              u4, __builtin_amdgcn_raw_buffer_load_b128(wr, (in ? wo + r * ustride : DS4_OOB) + 1024 * p + 16 * lane,
                                                        0, 0));
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) sg.wd[r] = load_unit_buf<B>(wr, in ? wo + r * ustride : DS4_OOB, lane);
    }
    // h of token r16 if it chose the expert (zeros otherwise, weight 0)
    const bool routed = (tmask >> r16) & 1u;  // implies r16 < T
    const uint32_t p = (uint32_t)tile * a.T + r16;
    const uint32_t hoff = routed ? a.o_h + 2u * (p * a.Ipad + lsb * 256 + 16 * g) : DS4_OOB;
    const uint32_t soff = routed ? hs_base + 2u * (p * nj + lsb * 16) : DS4_OOB;
#pragma unroll
    for (int q = 0; q < 8; ++q) sg.b[q] = buf_load_h8(ws, hoff + 2u * (64 * (q >> 1) + 8 * (q & 1)));
    sg.b[8] = buf_load_h8(ws, soff);
    sg.wt = a.dtiles[tile].w[r16];  // 0 for tokens that did not choose the expert
    if (++lsb == nsb) {
      lsb = 0;
      ++lt;
    }
  };
  auto compute = [&](const Stage &sg0, int slot) {
    Stage sg = sg0;
    if constexpr (SDL) {  // scales of row r16, d|dmin of rows 4g..4g+3 (the unit's byte layout)
      wait_vm<(PD - 1) * LPS>();  // this step's loads (LDS and registers) have landed
      const char *sd = sdl + (wave * PD + slot) * (R * 320);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        sg.wd[r].scale = *reinterpret_cast<const u4 *>(sd + 320 * r + 16 * r16);
        sg.wd[r].dd = *reinterpret_cast<const u4 *>(sd + 320 * r + 256 + 16 * g);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const UnitDecoded dd = decode_unit(sg.wd[r], g);
      f4 ac = (f4){0.f, 0.f, 0.f, 0.f};
#define DEC_STEP(S) ac = mfma16(step_frag<S, B>(sg.wd[r], dd), sg.b[S], ac);
      DEC_STEP(0) DEC_STEP(1) DEC_STEP(2) DEC_STEP(3) DEC_STEP(4) DEC_STEP(5) DEC_STEP(6) DEC_STEP(7)
#undef DEC_STEP
      const f4 mm = mfma16(dd.mfrag, sg.b[8], (f4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float v = fmaf(dd_d(dd.dd[q]), ac[q], -dd_dmin(dd.dd[q]) * mm[q]);
        y[r][q] = fmaf(sg.wt, v, y[r][q]);
      }
    }
  };
#pragma unroll
  for (int sgi = 0; sgi < PD; ++sgi) load(st[sgi], sgi);
  for (int i0 = 0; i0 < nit; i0 += PD) {
#pragma unroll
    for (int sgi = 0; sgi < PD; ++sgi) {
      compute(st[sgi], sgi);
      load(st[sgi], sgi);
    }
  }
  if constexpr (SDL) wait_vm<0>();  // the trailing loads into LDS, before the workgroup's LDS is released
  __shared__ f4 red[8][R][64];
#pragma unroll
  for (int r = 0; r < R; ++r) red[wave][r][lane] = y[r];
  __syncthreads();
  if (wave >= R) return;
  // wave r adds the 8 waves' sums of row tile rt0 + r in wave order
  f4 acc = red[0][wave][lane];
#pragma unroll
  for (int w = 1; w < 8; ++w) {
    const f4 v = red[w][wave][lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] += v[q];
  }
  if (r16 < a.T)
    *reinterpret_cast<f4 *>(a.dpart + ((size_t)half * a.T + r16) * a.H + (rt0 + wave) * 16 + 4 * g) = acc;
}

// y = the NH partials added in order (+ shared-expert output)
template <int NH>
__global__ __launch_bounds__(256) void k_down_reduce(const float *__restrict__ part, const float *__restrict__ ysh,
                                                     float *__restrict__ y, int T, int H) {
  const int i = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (i >= T * H) return;
  f4 v = *reinterpret_cast<const f4 *>(part + i);
#pragma unroll
  for (int h = 1; h < NH; ++h) {
    const f4 p = *reinterpret_cast<const f4 *>(part + (size_t)h * T * H + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += p[q];
  }
  if (ysh) {
    const f4 sv = *reinterpret_cast<const f4 *>(ysh + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += sv[q];
  }
  *reinterpret_cast<f4 *>(y + i) = v;
}

// ------------------------------------------------------------------ combine
// y[t] = 2^2e * sum_j w[t,j] * Yp[pos(t,j)] in rank order (e: the token's
// pre-scale), then + shared output.
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ yp, const int32_t *__restrict__ pos,
                                                 const float *__restrict__ w, const int32_t *__restrict__ xexp,
                                                 const float *__restrict__ ysh, float *__restrict__ y, int T, int k,
                                                 int H) {
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
  const int e = xexp[t];  // Yp carries the token's 2^-2e
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = scale_2e(acc[i], e);
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
                                                       const half_t *__restrict__ x16,
                                                       const int32_t *__restrict__ xexp, half_t *__restrict__ hs,
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
      const int e = xexp[tok[nt]];
      half_t hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[i] = (half_t)swiglu_scaled(ag[r][nt][i], au[r][nt][i], e);
      uint2 pk;
      __builtin_memcpy(&pk, hv, 8);
      *reinterpret_cast<uint2 *>(hs + (size_t)tok[nt] * Is + row0) = pk;
    }
  }
}

template <int R, int NT>
__global__ __launch_bounds__(256) void k_shared_down(const uint16_t *__restrict__ wd, const half_t *__restrict__ hs,
                                                     const int32_t *__restrict__ xexp, float *__restrict__ ysh, int T,
                                                     int H, int Is) {
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
    for (int nt = 0; nt < NT; ++nt) {
      if (!valid[nt]) continue;
      const int e = xexp[tok[nt]];  // h carries 2^-2e
      f4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = scale_2e(ac[r][nt][q], e);
      *reinterpret_cast<f4 *>(ysh + (size_t)tok[nt] * H + row0) = v;
    }
  }
}

// ------------------------------------------------------------------ shared expert, larger batches
// The shared expert's bf16 weights are first copied to fp16 (exact inside the
// binary16 range, the same conversion as the small-batch kernels), so the
// GEMM below has two fp16 operands and no conversion in its loop.
__global__ __launch_bounds__(256) void k_bf16_to_f16(const uint16_t *__restrict__ wg, const uint16_t *__restrict__ wu,
                                                     const uint16_t *__restrict__ wd, half_t *__restrict__ dst,
                                                     uint64_t n8) {  // 16-byte groups per matrix
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < 3 * n8; i += stride) {
    const uint16_t *src = i < n8 ? wg + 8 * i : i < 2 * n8 ? wu + 8 * (i - n8) : wd + 8 * (i - 2 * n8);
    *reinterpret_cast<h8 *>(dst + 8 * i) = bf16x8_to_h8(*reinterpret_cast<const u4 *>(src));
  }
}

// Dense C[rows, tokens] = W[rows, K] x X[tokens, K]^T, both fp16, fp32
// accumulation.  Workgroup = 4 waves, tile of 256 weight rows x 128 tokens.
// Per K-chunk of 32 both operands go from global memory straight into a
// 3-stage LDS ring (direct loads, two chunks ahead; no registers held, no
// stores); a row is 64 bytes and its 16-byte chunk c sits at position
// c ^ ((r >> 1) & 3), which spreads a fragment read over the banks.  One
// barrier per chunk.  Wave (wr, wc) holds 8 row n-tiles x 4 token n-tiles of
// 16x16 accumulators, so every LDS fragment feeds 4 or 8 MFMAs.  GU: the
// tile's rows are 128 gate rows and the same 128 up rows, a wave takes 64 of
// each, and the epilogue writes h = silu(gate)*up (fp16); otherwise the rows
// are 256 down rows, 128 per wave, and the epilogue writes fp32.  Rows past
// `rows` and tokens past T load as zeros and are not written.
constexpr int DG_KC = 32;  // K per chunk
constexpr int DG_ROWS = 256, DG_TOK = 128;
constexpr int DG_STAGES = 3;
constexpr int DG_A_BYTES = DG_ROWS * 2 * DG_KC, DG_X_BYTES = DG_TOK * 2 * DG_KC;
constexpr int DG_STAGE_BYTES = DG_A_BYTES + DG_X_BYTES;

__device__ __forceinline__ int dg_swz(int r) { return (r >> 1) & 3; }

template <bool GU>
__global__ __launch_bounds__(256) void k_dense_gemm(const half_t *__restrict__ wa, const half_t *__restrict__ wb,
                                                    const half_t *__restrict__ x, const int32_t *__restrict__ xexp,
                                                    void *__restrict__ out, int T, int K, int rows) {
  __shared__ __attribute__((aligned(16))) char ring[DG_STAGES * DG_STAGE_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int wr = wave >> 1, wc = wave & 1;
  const int row0 = blockIdx.x * (GU ? DG_ROWS / 2 : DG_ROWS);
  const int t0 = blockIdx.y * DG_TOK;

  // buffer windows over this tile's weight rows and token rows (loads past them read zeros)
  const uint32_t kb = 2u * (uint32_t)K;
  const int na = min(GU ? DG_ROWS / 2 : DG_ROWS, rows - row0);
  const int nx = min(DG_TOK, T - t0);
  // the wave's 4 weight loads per chunk (LDS rows 64*wave .. +63): GU waves 0-1 gate, 2-3 up
  const half_t *wsrc = (GU && wave >= 2) ? wb : wa;
  const int wrow0 = GU ? 64 * (wave & 1) : 64 * wave;  // first row of the matrix the wave loads
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wsrc + (size_t)row0 * K, (uint32_t)na * kb);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (size_t)t0 * K, (uint32_t)max(nx, 0) * kb);
  uint32_t oa[4], ox[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = 16 * i + (lane >> 2);  // row within the wave's 64
    oa[i] = (uint32_t)(wrow0 + lr) * kb + 16u * (uint32_t)((lane & 3) ^ dg_swz(lr));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int lr = 16 * (2 * wave + i) + (lane >> 2);
    ox[i] = (uint32_t)lr * kb + 16u * (uint32_t)((lane & 3) ^ dg_swz(lr));
  }
  auto issue = [&](int st, int c) {
    char *sa = ring + st * DG_STAGE_BYTES + wave * 4096;
    char *sx = ring + st * DG_STAGE_BYTES + DG_A_BYTES + wave * 2048;
    const uint32_t k0 = (uint32_t)c * 2u * DG_KC;
#pragma unroll
    for (int i = 0; i < 4; ++i) buf_load_lds16(rw, sa + 1024 * i, oa[i] + k0);
#pragma unroll
    for (int i = 0; i < 2; ++i) buf_load_lds16(rx, sx + 1024 * i, ox[i] + k0);
  };

  // this wave's A fragments: LDS rows of row n-tile i (gate rows 0-127, up rows 128-255)
  int arow_base[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    arow_base[i] = GU ? (i < 4 ? 64 * wr + 16 * i : 128 + 64 * wr + 16 * (i - 4)) : 128 * wr + 16 * i;
  const int fo = 16 * (g ^ dg_swz(r16));  // the lane's chunk in its fragment row

  f4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f4){0.f, 0.f, 0.f, 0.f};

  const int nk = K / DG_KC;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int c = 0; c < nk; ++c) {
    if (c + 1 < nk) wait_vm<6>();  // this wave's loads of chunk c have landed
    else wait_vm<0>();
    __syncthreads();  // ... every wave's; and every wave is done with chunk c-1's stage
    if (c + 2 < nk) issue((c + 2) % DG_STAGES, c + 2);
    const char *sa = ring + (c % DG_STAGES) * DG_STAGE_BYTES;
    const char *sx = sa + DG_A_BYTES;
    h8 bx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bx[j] = *reinterpret_cast<const h8 *>(sx + (64 * wc + 16 * j + r16) * 64 + fo);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const h8 av = *reinterpret_cast<const h8 *>(sa + (arow_base[i] + r16) * 64 + fo);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(av, bx[j], acc[i][j]);
    }
  }

  // epilogue: accumulator (i, j) lane (r16, g) = row n-tile i rows 4g..4g+3, token 16j + r16
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + 64 * wc + 16 * j + r16;
    if (t >= T) continue;
    const int e = xexp[t];  // the token's pre-scale
    if (GU) {
      half_t *hs = reinterpret_cast<half_t *>(out);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = row0 + 64 * wr + 16 * i + 4 * g;
        if (row >= rows) continue;
        half_t hv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) hv[q] = (half_t)swiglu_scaled(acc[i][j][q], acc[4 + i][j][q], e);
        uint2 pk;
        __builtin_memcpy(&pk, hv, 8);
        *reinterpret_cast<uint2 *>(hs + (size_t)t * rows + row) = pk;
      }
    } else {
      float *y = reinterpret_cast<float *>(out);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = row0 + 128 * wr + 16 * i + 4 * g;
        if (row >= rows) continue;
        f4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = scale_2e(acc[i][j][q], e);
        *reinterpret_cast<f4 *>(y + (size_t)t * rows + row) = v;
      }
    }
  }
}

// ------------------------------------------------------------------ launchers
// Prefill: four n-tiles (64 tokens) per workgroup.
// Activations of the wide-tile GEMMs: one buffer window from the activation
// rows to the end of their hi/lo sums (false if it does not fit 2 GiB).
static bool act_window(const void *rows, const void *s_hi, const void *s_lo, const void *xe16, int64_t nrows, int K,
                       GemmAct &xa) {
  const uint8_t *b = (const uint8_t *)rows;
  const int64_t ohi = (const uint8_t *)s_hi - b, olo = (const uint8_t *)s_lo - b;
  const int64_t sbytes = nrows * (int64_t)(K / 16) * 2;
  int64_t end = (ohi > olo ? ohi : olo) + sbytes;
  const int64_t oxe = xe16 ? (const uint8_t *)xe16 - b : -1;
  if (xe16 && oxe + 16 * nrows > end) end = oxe + 16 * nrows;
  if (ohi < nrows * (int64_t)K * 2 || olo < nrows * (int64_t)K * 2 || (xe16 && oxe < nrows * (int64_t)K * 2) ||
      end > (int64_t)0x80000000LL)
    return false;
  xa.o_xe = xe16 ? (uint32_t)oxe : DS4_OOB;
  xa.base = b;
  xa.len = (uint32_t)end;
  xa.o_shi = (uint32_t)ohi;
  xa.o_slo = (uint32_t)olo;
  xa.row_bytes = (uint32_t)K * 2;
  xa.srow_bytes = (uint32_t)(K / 16) * 2;
  return true;
}

template <int B>
static hipError_t gateup_b(const GemmArgs &a, int max_tiles, hipStream_t s, const Timing *tm) {
  if (a.tile_n > 64) {
    GemmAct xa;
    if (a.tile_n > 16 * PT_NTM || !act_window(a.x16, a.xs_hi, a.xs_lo, a.xe16, a.T, a.H, xa)) return hipErrorInvalidValue;
    const int nrb = (a.I + 16 * PT_NW - 1) / (16 * PT_NW);
    DS4_LAUNCH(tm, (k_moe_gemm_wide<2, 1, B>), gemm_grid(nrb, max_tiles), dim3(64 * PT_NW), 0, s, a, xa,
               nrb);
    return hipGetLastError();
  }
  constexpr int R = GEMM_R_GU, NW = GEMM_NW_GU;
  const int rows_per_wg = 16 * R * NW;
  const int nrb = (a.I + rows_per_wg - 1) / rows_per_wg;
  const dim3 grid = gemm_grid(nrb, max_tiles);
  DS4_LAUNCH(tm, (k_moe_gemm<2, R, NW, false, B>), grid, dim3(64 * NW), 0, s, a, nrb);
  return hipGetLastError();
}

hipError_t launch_gateup(const GemmArgs &a, int max_tiles, hipStream_t s, const Timing *tm) {
  if (max_tiles <= 0) return hipSuccess;
  switch (unit_bits(a.bits)) {
    case 2: return gateup_b<2>(a, max_tiles, s, tm);
    case 4: return gateup_b<4>(a, max_tiles, s, tm);
    case 6: return gateup_b<6>(a, max_tiles, s, tm);
    default: return hipErrorInvalidValue;
  }
}

template <int B>
static hipError_t down_b(const GemmArgs &a, int max_tiles, hipStream_t s, const Timing *tm) {
  if (a.tile_n > 64) {
    GemmAct xa;
    if (a.tile_n > 16 * PT_NTM || a.I != a.Ipad ||
        !act_window(a.h, a.hs_hi, a.hs_lo, nullptr, (int64_t)a.T * a.k, a.Ipad, xa))
      return hipErrorInvalidValue;
    const int nrb = (a.H + 32 * PT_NW - 1) / (32 * PT_NW);
    DS4_LAUNCH(tm, (k_moe_gemm_wide<1, 2, B>), gemm_grid(nrb, max_tiles), dim3(64 * PT_NW), 0, s, a, xa,
               nrb);
    return hipGetLastError();
  }
  constexpr int R = GEMM_R_DN, NW = GEMM_NW_DN;
  const int rows_per_wg = 16 * R * NW;
  const int nrb = (a.H + rows_per_wg - 1) / rows_per_wg;
  const dim3 grid = gemm_grid(nrb, max_tiles);
  if (a.I == a.Ipad)
    DS4_LAUNCH(tm, (k_moe_gemm<1, R, NW, false, B>), grid, dim3(64 * NW), 0, s, a, nrb);
  else
    DS4_LAUNCH(tm, (k_moe_gemm<1, R, NW, true, B>), grid, dim3(64 * NW), 0, s, a, nrb);
  return hipGetLastError();
}

hipError_t launch_down(const GemmArgs &a, int max_tiles, hipStream_t s, const Timing *tm) {
  if (max_tiles <= 0) return hipSuccess;
  switch (unit_bits(a.bits_dn)) {
    case 2: return down_b<2>(a, max_tiles, s, tm);
    case 4: return down_b<4>(a, max_tiles, s, tm);
    case 6: return down_b<6>(a, max_tiles, s, tm);
    default: return hipErrorInvalidValue;
  }
}

// Small batches (T <= 16).
template <int NT, int B>
static void gateup_dec_lds(const GemmArgs &a, int n_rt, const DecRoute *rr, dim3 grid, hipStream_t s,
                           const Timing *tm) {
  if (rr)
    DS4_LAUNCH(tm, (k_gateup_dec_lds<GU_LDS_PD, NT, true, B, GU_LDS_KS>), grid, dim3(256), 0, s, a, n_rt, *rr);
  else
    DS4_LAUNCH(tm, (k_gateup_dec_lds<GU_LDS_PD, NT, false, B, GU_LDS_KS>), grid, dim3(256), 0, s, a, n_rt,
               DecRoute{});
}

template <int B>
static hipError_t gateup_dec_b(const GemmArgs &a, int max_tiles, const DecRoute *rr, hipStream_t s,
                               const Timing *tm) {
  const int n_rt = a.I >> 4;
  if (a.T >= GU_SH_MIN_T) {  // activations shared by the workgroup's row tiles
    if (a.T > 4) {
      constexpr int NW = GU_SH_NW;
      const dim3 grid((unsigned)((int64_t)((n_rt + NW - 1) / NW) * max_tiles));
      DS4_LAUNCH(tm, (k_gateup_dec_sh<GU_SH_PD, NW, B, 16, false, true>), grid, dim3(64 * NW), 0, s, a, n_rt,
                 DecRoute{});
    } else {  // four token slots, four waves (the routing takes 256 threads)
      const dim3 grid((unsigned)((int64_t)((n_rt + 3) / 4) * max_tiles));
      // two tokens: scales through registers and a 4-slot ring; three or four:
      // scales through LDS and a 2-slot ring (fewer registers, more workgroups)
      const DecRoute r = rr ? *rr : DecRoute{};
      if (a.T == 2) {
        if (rr) DS4_LAUNCH(tm, (k_gateup_dec_sh<4, 4, B, 4, true, false>), grid, dim3(256), 0, s, a, n_rt, r);
        else DS4_LAUNCH(tm, (k_gateup_dec_sh<4, 4, B, 4, false, false>), grid, dim3(256), 0, s, a, n_rt, r);
      } else {
        if (rr) DS4_LAUNCH(tm, (k_gateup_dec_sh<2, 4, B, 4, true, true>), grid, dim3(256), 0, s, a, n_rt, r);
        else DS4_LAUNCH(tm, (k_gateup_dec_sh<2, 4, B, 4, false, true>), grid, dim3(256), 0, s, a, n_rt, r);
      }
    }
    return hipGetLastError();
  }
  // one token: row tiles split over two waves each, activations per wave
  static_assert(GU_SH_MIN_T == 2, "the per-wave kernel is instantiated for one token");
  const int nrb = (n_rt + 4 / GU_LDS_KS - 1) / (4 / GU_LDS_KS);
  const dim3 grid((unsigned)((int64_t)nrb * max_tiles));
  gateup_dec_lds<1, B>(a, n_rt, rr, grid, s, tm);
  return hipGetLastError();
}

hipError_t launch_gateup_dec(const GemmArgs &a, int max_tiles, const DecRoute *rr, hipStream_t s,
                             const Timing *tm) {
  if (max_tiles <= 0) return hipSuccess;
  if (rr && (a.T > 4 || rr->E > 256 || rr->k > 16)) return hipErrorInvalidValue;
  switch (unit_bits(a.bits)) {
    case 2: return gateup_dec_b<2>(a, max_tiles, rr, s, tm);
    case 4: return gateup_dec_b<4>(a, max_tiles, rr, s, tm);
    case 6: return gateup_dec_b<6>(a, max_tiles, rr, s, tm);
    default: return hipErrorInvalidValue;
  }
}

template <int B>
static hipError_t down_combine_dec_b(const GemmArgs &a, hipStream_t s, const Timing *tm, const Timing *tm_combine) {
  const dim3 grid((unsigned)(a.H >> 4));
  if (a.I == a.Ipad && a.T <= 4) {
    switch (a.T) {
      case 1:  // 16 waves, each tile's reduction split over two (a shorter chain per wave)
        if (a.Ipad % 512 == 0) {
          DS4_LAUNCH(tm, (k_down_dec_lds<2, 1, B, 2>), grid, dim3(1024), 0, s, a);
        } else {
          DS4_LAUNCH(tm, (k_down_dec_lds<DN_LDS_PD, 1, B, 1>), grid, dim3(512), 0, s, a);
        }
        break;
      case 2:
        if (a.Ipad % 512 == 0) DS4_LAUNCH(tm, (k_down_dec_lds<2, 2, B, 2>), grid, dim3(1024), 0, s, a);
        else DS4_LAUNCH(tm, (k_down_dec_lds<DN_LDS_PD, 2, B, 1>), grid, dim3(512), 0, s, a);
        break;
      case 3:
        if (a.Ipad % 512 == 0) DS4_LAUNCH(tm, (k_down_dec_lds<2, 3, B, 2>), grid, dim3(1024), 0, s, a);
        else DS4_LAUNCH(tm, (k_down_dec_lds<DN_LDS_PD, 3, B, 1>), grid, dim3(512), 0, s, a);
        break;
      default:
        if (a.Ipad % 512 == 0) DS4_LAUNCH(tm, (k_down_dec_lds<2, 4, B, 2>), grid, dim3(1024), 0, s, a);
        else DS4_LAUNCH(tm, (k_down_dec_lds<DN_LDS_PD, 4, B, 1>), grid, dim3(512), 0, s, a);
    }
    return hipGetLastError();
  }
  if (a.I == a.Ipad && a.dpart) {  // two row tiles per wave, the tiles in two halves
    static_assert(DN2_NH <= DEC_DOWN_SPLITS, "workspace partials");
    DS4_LAUNCH(tm, (k_down_dec2<DN2_PD, B, DN2_SDL, DN2_R, DN2_NH>), dim3((unsigned)(a.H / (16 * DN2_R)), DN2_NH),
               dim3(512), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    DS4_LAUNCH(tm_combine, k_down_reduce<DN2_NH>, dim3((unsigned)((a.T * a.H / 4 + 255) / 256)), dim3(256), 0, s,
               a.dpart, a.ysh, a.y, a.T, a.H);
    return hipGetLastError();
  }
  // I below 256 (padded reduction)
  DS4_LAUNCH(tm, (k_down_dec<DN_DEC_PD, true, B>), grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_combine_dec(const GemmArgs &a, hipStream_t s, const Timing *tm, const Timing *tm_combine) {
  switch (unit_bits(a.bits_dn)) {
    case 2: return down_combine_dec_b<2>(a, s, tm, tm_combine);
    case 4: return down_combine_dec_b<4>(a, s, tm, tm_combine);
    case 6: return down_combine_dec_b<6>(a, s, tm, tm_combine);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(const float *yp, const int32_t *pos, const float *w, const int32_t *xexp, const float *ysh,
                          float *y, int T, int k, int H, hipStream_t s, const Timing *tm) {
  if (T <= 0) return hipSuccess;
  DS4_LAUNCH(tm, k_combine, dim3(T, (H + 1023) / 1024), dim3(256), 0, s, yp, pos, w, xexp, ysh, y, T, k, H);
  return hipGetLastError();
}

hipError_t launch_shared_convert(const uint16_t *wg, const uint16_t *wu, const uint16_t *wd, _Float16 *dst, int H,
                                 int Is, hipStream_t s, const Timing *tm) {
  const uint64_t n8 = (uint64_t)H * Is / 8;
  const uint64_t groups = (3 * n8 + 255) / 256;
  DS4_LAUNCH(tm, k_bf16_to_f16, dim3((unsigned)(groups < 8192 ? groups : 8192)), dim3(256), 0, s, wg, wu, wd, dst, n8);
  return hipGetLastError();
}

hipError_t launch_shared_gateup(const uint16_t *wg, const uint16_t *wu, const _Float16 *w16, const _Float16 *x16,
                                const int32_t *xexp, _Float16 *hs, int T, int H, int Is, hipStream_t s,
                                const Timing *tm) {
  if (T <= 0) return hipSuccess;
  if (T >= SHARED_DENSE_MIN_T) {  // fp16 copies: gate at w16, up after it
    if (!w16) return hipErrorInvalidValue;
    const dim3 grid((Is + DG_ROWS / 2 - 1) / (DG_ROWS / 2), (T + DG_TOK - 1) / DG_TOK);
    DS4_LAUNCH(tm, (k_dense_gemm<true>), grid, dim3(256), 0, s, w16, w16 + (size_t)Is * H, x16, xexp, hs, T, H, Is);
    return hipGetLastError();
  }
  constexpr int R = 1, NT = 4;
  const dim3 grid((Is + 16 * R * WAVES - 1) / (16 * R * WAVES), (T + 16 * NT - 1) / (16 * NT));
  DS4_LAUNCH(tm, (k_shared_gateup<R, NT>), grid, dim3(256), 0, s, wg, wu, x16, xexp, hs, T, H, Is);
  return hipGetLastError();
}

hipError_t launch_shared_down(const uint16_t *wd, const _Float16 *w16, const _Float16 *hs, const int32_t *xexp,
                              float *ysh, int T, int H, int Is, hipStream_t s, const Timing *tm) {
  if (T <= 0) return hipSuccess;
  if (T >= SHARED_DENSE_MIN_T) {  // fp16 copies: down after gate and up
    if (!w16) return hipErrorInvalidValue;
    const dim3 grid((H + DG_ROWS - 1) / DG_ROWS, (T + DG_TOK - 1) / DG_TOK);
    DS4_LAUNCH(tm, (k_dense_gemm<false>), grid, dim3(256), 0, s, w16 + 2 * (size_t)Is * H, nullptr, hs, xexp, ysh,
               T, Is, H);
    return hipGetLastError();
  }
  constexpr int R = 1, NT = 4;
  const dim3 grid((H + 16 * R * WAVES - 1) / (16 * R * WAVES), (T + 16 * NT - 1) / (16 * NT));
  DS4_LAUNCH(tm, (k_shared_down<R, NT>), grid, dim3(256), 0, s, wd, hs, xexp, ysh, T, H, Is);
  return hipGetLastError();
}

}  // namespace ds4
