/*
 * Seeded synthetic inputs for the routed 2-bit MoE layer.
 *
 * This module produces INPUTS only: Gaussian activations, router weights,
 * router bias, shared-expert weights, and routed-expert weights already
 * quantized into the canonical 84-byte super-block.  It contains none of the
 * layer's arithmetic (no dequantization, no routing, no FFN): both the CPU
 * oracle and the GPU library consume the bytes it writes.
 *
 * Random numbers: Philox4x32-10, the counter-based generator of Salmon,
 * Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3"
 * (SC'11), written here from that paper's definition (two 32x32->64-bit
 * multiplies per round, Weyl key schedule, 10 rounds).  Each tensor has its own
 * key (master seed, stream id), so any one expert can be regenerated alone.
 * Normals come from the Box-Muller transform in double precision.
 *
 * Canonical block (84 bytes per 256 consecutive weights of the row-major
 * flattened tensor): scales[16] at byte 0 (low nibble = sub-block scale,
 * high nibble = sub-block min), qs[64] at byte 16 (weight i of the block in
 * byte i/4, bits 2*(i%4)..2*(i%4)+1), d at byte 80 and dmin at byte 82, both
 * IEEE binary16 little-endian.  The value a block encodes for weight i in
 * sub-block j = i/16 is d*sc_j*q_i - dmin*m_j.
 *
 * The quantizer is plain round-to-nearest min/max per 16-weight sub-block;
 * it only has to produce valid, realistic blocks (it is not under test).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void mulhilo(uint32_t a, uint32_t b, uint32_t *hi, uint32_t *lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

/* One Philox4x32-10 evaluation: counter c[4], key k[2] -> out[4]. */
void synth_philox4x32_10(const uint32_t c_in[4], const uint32_t k_in[2], uint32_t out[4]) {
  uint32_t c0 = c_in[0], c1 = c_in[1], c2 = c_in[2], c3 = c_in[3];
  uint32_t k0 = k_in[0], k1 = k_in[1];
  for (int r = 0; r < 10; ++r) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo(PHILOX_M0, c0, &hi0, &lo0);
    mulhilo(PHILOX_M1, c2, &hi1, &lo1);
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += PHILOX_W0;
    k1 += PHILOX_W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Uniform in the open interval (0,1) from a 32-bit word. */
static inline double u01(uint32_t r) { return ((double)r + 0.5) * (1.0 / 4294967296.0); }

/* Four standard normals from counter index `ctr` of stream (seed, stream). */
static inline void normals4(uint64_t seed, uint32_t stream, uint64_t ctr, double z[4]) {
  uint32_t c[4] = {(uint32_t)ctr, (uint32_t)(ctr >> 32), stream, 0x5EED5EEDu};
  uint32_t k[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t r[4];
  synth_philox4x32_10(c, k, r);
  const double two_pi = 6.283185307179586476925286766559;
  double rad0 = sqrt(-2.0 * log(u01(r[0])));
  double rad1 = sqrt(-2.0 * log(u01(r[2])));
  z[0] = rad0 * cos(two_pi * u01(r[1]));
  z[1] = rad0 * sin(two_pi * u01(r[1]));
  z[2] = rad1 * cos(two_pi * u01(r[3]));
  z[3] = rad1 * sin(two_pi * u01(r[3]));
}

/* n normals N(0, sigma) as fp32, element i of the stream = normal number i. */
void synth_normal_f32(uint64_t seed, uint32_t stream, double sigma, int64_t n, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t blk = 0; blk < (n + 3) / 4; ++blk) {
    double z[4];
    normals4(seed, stream, (uint64_t)blk, z);
    for (int j = 0; j < 4; ++j) {
      int64_t i = blk * 4 + j;
      if (i < n) out[i] = (float)(sigma * z[j]);
    }
  }
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs). */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

void synth_f32_to_bf16(const float *in, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}

/* fp32 -> binary16 bits, round to nearest even, with subnormals; |f| is
 * assumed below the binary16 overflow threshold (scales of small weights). */
static uint16_t f32_to_f16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x47800000u) return (uint16_t)(sign | 0x7C00u); /* overflow -> inf */
  if (a < 0x33000000u) return (uint16_t)sign;              /* < 2^-25 -> 0 */
  int e = (int)(a >> 23) - 127;
  uint32_t mant = (a & 0x7FFFFFu) | 0x800000u;
  int shift;
  uint32_t h_exp;
  if (e >= -14) { shift = 13; h_exp = (uint32_t)(e + 15); }
  else { shift = 13 + (-14 - e); h_exp = 0; }
  uint32_t q = mant >> shift;
  uint32_t rem = mant & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1;
  uint32_t bits;
  if (h_exp == 0) bits = q; /* subnormal (q may carry into the exponent: fine) */
  else bits = (h_exp << 10) + (q - 0x400u); /* q in [0x400, 0x800] */
  return (uint16_t)(sign | bits);
}

static float f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  float v;
  if (e == 0) v = ldexpf((float)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexpf((float)(m | 0x400u), (int)e - 25);
  uint32_t u;
  memcpy(&u, &v, 4);
  u |= sign;
  memcpy(&v, &u, 4);
  return v;
}

static inline int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* Bytes of one canonical block of 256 weights with `bits`-bit codes (2, 4, 5
 * or 6): scales[16], codes (256*bits/8 bytes), d, dmin. */
static inline int block_bytes(int bits) { return 16 + 32 * bits + 4; }

/* Quantize 256 fp32 weights into one canonical block (RTN), `bits`-bit
 * codes: per sub-block of 16 the range [min(0, min w), max w] is split into
 * 2^bits - 1 steps of d*sc, the offset is dmin*m; the codes form one bit
 * stream from byte 16, lowest bits first (code i at bits bits*i ..
 * bits*i + bits - 1; for 2 and 4 bits: byte 16 + i*bits/8). */
void synth_quantize_block_bits(const float *w, uint8_t *blk, int bits) {
  const int levels = (1 << bits) - 1, nb = block_bytes(bits);
  float scf[16], mnv[16];
  float max_scf = 0.f, max_mn = 0.f;
  for (int j = 0; j < 16; ++j) {
    float mn = 0.f, mx = -INFINITY;
    for (int i = 0; i < 16; ++i) {
      float v = w[16 * j + i];
      if (v < mn) mn = v;
      if (v > mx) mx = v;
    }
    scf[j] = (mx - mn) / (float)levels;
    mnv[j] = -mn; /* >= 0 */
    if (scf[j] > max_scf) max_scf = scf[j];
    if (mnv[j] > max_mn) max_mn = mnv[j];
  }
  uint16_t d_bits = f32_to_f16(max_scf / 15.0f);
  uint16_t dmin_bits = f32_to_f16(max_mn / 15.0f);
  float d = f16_to_f32(d_bits), dmin = f16_to_f32(dmin_bits);
  memset(blk, 0, (size_t)nb);
  for (int j = 0; j < 16; ++j) {
    int sc = d > 0.f ? clampi((int)lrintf(scf[j] / d), 0, 15) : 0;
    int m = dmin > 0.f ? clampi((int)lrintf(mnv[j] / dmin), 0, 15) : 0;
    blk[j] = (uint8_t)(sc | (m << 4));
    float step = d * (float)sc, off = dmin * (float)m;
    for (int i = 0; i < 16; ++i) {
      int q = step > 0.f ? clampi((int)lrintf((w[16 * j + i] + off) / step), 0, levels) : 0;
      const int bit = bits * (16 * j + i);
      const unsigned v = (unsigned)q << (bit & 7);
      blk[16 + (bit >> 3)] |= (uint8_t)(v & 0xFFu);
      if ((bit & 7) + bits > 8) blk[16 + (bit >> 3) + 1] |= (uint8_t)(v >> 8);
    }
  }
  blk[nb - 4] = (uint8_t)(d_bits & 0xFF);
  blk[nb - 3] = (uint8_t)(d_bits >> 8);
  blk[nb - 2] = (uint8_t)(dmin_bits & 0xFF);
  blk[nb - 1] = (uint8_t)(dmin_bits >> 8);
}

/* Quantize 256 fp32 weights into one canonical 84-byte 2-bit block (RTN). */
void synth_quantize_block(const float *w, uint8_t *blk) { synth_quantize_block_bits(w, blk, 2); }

/* Quantize n_blocks*256 fp32 weights (row-major flattened) to blocks. */
void synth_quantize_bits(const float *w, int64_t n_blocks, int bits, uint8_t *out) {
  const int nb = block_bytes(bits);
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < n_blocks; ++b) synth_quantize_block_bits(w + 256 * b, out + nb * b, bits);
}

void synth_quantize(const float *w, int64_t n_blocks, uint8_t *out) { synth_quantize_bits(w, n_blocks, 2, out); }

/*
 * Generate and quantize `n_mats` matrices of rows*cols weights N(0, sigma)
 * to `bits`-bit blocks.  Matrix e (e = 0..n_mats-1) uses stream
 * (stream_base + e); the whole matrix is one stream, so (seed, stream) fixes
 * its bytes regardless of how many matrices are generated together.
 */
void synth_qk_matrices(uint64_t seed, uint32_t stream_base, int64_t n_mats, int64_t rows, int64_t cols,
                       double sigma, int bits, uint8_t *out) {
  int64_t per = rows * cols;      /* weights per matrix, multiple of 256 */
  int64_t nblk = per / 256;
  const int nb = block_bytes(bits);
  const int64_t CH = 64;          /* blocks per work item */
  int64_t chunks = (nblk + CH - 1) / CH;
#pragma omp parallel
  {
    float buf[CH * 256];
#pragma omp for schedule(static) collapse(2)
    for (int64_t e = 0; e < n_mats; ++e) {
      for (int64_t c = 0; c < chunks; ++c) {
        int64_t b0 = c * CH, b1 = b0 + CH < nblk ? b0 + CH : nblk;
        int64_t i0 = b0 * 256, i1 = b1 * 256;
        for (int64_t i = i0; i < i1; i += 4) {
          double z[4];
          normals4(seed, (uint32_t)(stream_base + e), (uint64_t)(i / 4), z);
          for (int j = 0; j < 4; ++j) buf[i - i0 + j] = (float)(sigma * z[j]);
        }
        for (int64_t b = b0; b < b1; ++b)
          synth_quantize_block_bits(buf + (b - b0) * 256, out + (e * nblk + b) * nb, bits);
      }
    }
  }
}

void synth_q2k_matrices(uint64_t seed, uint32_t stream_base, int64_t n_mats, int64_t rows, int64_t cols,
                        double sigma, uint8_t *out) {
  synth_qk_matrices(seed, stream_base, n_mats, rows, cols, sigma, 2, out);
}

void synth_u32(uint64_t seed, uint32_t stream, int64_t n, uint32_t *out) {
  for (int64_t blk = 0; blk < (n + 3) / 4; ++blk) {
    uint32_t c[4] = {(uint32_t)blk, (uint32_t)((uint64_t)blk >> 32), stream, 0xC0FFEE00u};
    uint32_t k[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t r[4];
    synth_philox4x32_10(c, k, r);
    for (int j = 0; j < 4; ++j)
      if (blk * 4 + j < n) out[blk * 4 + j] = r[j];
  }
}

int synth_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
