/*
 * CPU oracle for the routed 2-bit MoE layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package's smoke check and the benchmark's CPU
 * baseline leg may call this code.  The GPU library never links, loads or
 * calls it, and it includes nothing from the GPU library (its only headers are
 * the C standard library's).
 *
 * Everything is plain and sequential per output, in double precision, written
 * from the definitions.  Sources (titles of the web pages describing the ds4 /
 * DwarfStar engine; no code is printed on any of them):
 *   [models]   molayo1419.me translation of the ds4 README, "Models" section:
 *              only the routed MoE experts are quantized to 2 bits, down uses
 *              Q2_K; shared experts, projections and routing stay unquantized.
 *   [faq1]     opensource-hub.com "antirez/ds4" library page, FAQ #1 (router
 *              numeric test): the router score is sqrt(softplus(x)); evaluating
 *              softplus as log(1+exp(x)) in fp32 loses precision near logit -12;
 *              the exact reference uses log1p.
 *   [workload] the five layer workloads the method is measured on: 256-weight
 *              super-blocks of 16 sub-blocks, 4-bit scale (low nibble) and 4-bit
 *              min (high nibble) per sub-block, 2-bit codes four to a byte lowest
 *              bits first, fp16 d and dmin, w = d*scale*q - dmin*min; top-k
 *              with ties to the lower expert index and weights normalised to sum
 *              to one; SwiGLU experts; weighted combine plus an optional shared
 *              expert.
 *
 * Readings taken where those sources are silent (each is listed with its
 * reason in the design notes):
 *   - block byte order: scales[16] @0, qs[64] @16, d @80, dmin @82 (84 bytes);
 *   - code order: weight i of a block -> byte 16+i/4, bits 2*(i%4);
 *   - the 4-bit variant of the routed experts (the q2/q4 mix on the [models]
 *     page keeps some layers at 4 bits; no page gives a 4-bit block): the same
 *     block with 4-bit codes, weight i -> byte 16+i/2, bits 4*(i%2), d @144,
 *     dmin @146 (148 bytes), w = d*scale*q - dmin*min with q in 0..15;
 *   - blocks tile the row-major flattened tensor (a block may span rows);
 *   - router logit = round-to-fp32 of the fp64 sum over h of x*W plus bias;
 *   - selection ranks logits (sqrt(softplus) is strictly increasing), ties
 *     to the lower expert index, NaN ranks below every number;
 *   - weights w_j = s_j / sum_{i<k} s_i, no further scaling;
 *   - SwiGLU h = silu(gate) * up, silu(z) = z / (1 + exp(-z));
 *   - y = sum_j w_j * down(h_j) in rank order, plus the ungated shared expert,
 *     rounded once to fp32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* IEEE binary16 (little-endian bits) -> double, exact. */
static double half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int m = h & 0x3FF;
  double v;
  if (e == 0) v = ldexp((double)m, -24);                 /* zero / subnormal */
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m + 1024), e - 25);           /* 1.m * 2^(e-15) */
  return sign ? -v : v;
}

/* Bytes of one block of 256 weights with `bits`-bit codes (2 or 4). */
static int64_t block_bytes(int bits) { return 16 + 32 * bits + 4; }

/* Value of weight i (0..255) of one canonical block with `bits`-bit codes,
 * exact in double: every product has at most 19 significant bits and the
 * difference of two such numbers of the binary16 range fits in 53 bits.
 * [workload] */
static double block_weight(const uint8_t *blk, int i, int bits) {
  const int per_byte = 8 / bits, nb = (int)block_bytes(bits);
  int j = i / 16;                                  /* sub-block */
  int sc = blk[j] & 0x0F;                          /* low nibble: scale */
  int mn = blk[j] >> 4;                            /* high nibble: min  */
  int q = (blk[16 + i / per_byte] >> (bits * (i % per_byte))) & ((1 << bits) - 1);
  double d = half_to_double((uint16_t)(blk[nb - 4] | (blk[nb - 3] << 8)));
  double dmin = half_to_double((uint16_t)(blk[nb - 2] | (blk[nb - 1] << 8)));
  return d * sc * q - dmin * mn;
}

/* Dequantize n blocks (256 weights each) to doubles. */
void oracle_dequant_f64_bits(const uint8_t *blocks, int64_t nblocks, int bits, double *out) {
  const int64_t nb = block_bytes(bits);
  for (int64_t b = 0; b < nblocks; ++b)
    for (int i = 0; i < 256; ++i) out[b * 256 + i] = block_weight(blocks + nb * b, i, bits);
}

/* Dequantize n blocks to fp32: the exact value rounded once to nearest. */
void oracle_dequant_f32_bits(const uint8_t *blocks, int64_t nblocks, int bits, float *out) {
  const int64_t nb = block_bytes(bits);
  for (int64_t b = 0; b < nblocks; ++b)
    for (int i = 0; i < 256; ++i) out[b * 256 + i] = (float)block_weight(blocks + nb * b, i, bits);
}

void oracle_dequant_f64(const uint8_t *blocks, int64_t nblocks, double *out) {
  oracle_dequant_f64_bits(blocks, nblocks, 2, out);
}

void oracle_dequant_f32(const uint8_t *blocks, int64_t nblocks, float *out) {
  oracle_dequant_f32_bits(blocks, nblocks, 2, out);
}

/* Router logits, l[t,e] = fp32( sum_h x[t,h]*W[e,h] + b[e] ), the sum
 * accumulated in double from h = 0 upward, the bias added last. */
void oracle_logits(const float *x, const float *wr, const float *bias, int64_t T, int64_t E, int64_t H,
                   float *logits) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t h = 0; h < H; ++h) acc += (double)x[t * H + h] * (double)wr[e * H + h];
      if (bias) acc += (double)bias[e];
      logits[t * E + e] = (float)acc;
    }
}

/* Router score sqrt(softplus(l)) in double, softplus written in the form that
 * never forms 1 + exp(l) for very negative l: max(l,0) + log1p(exp(-|l|)).
 * [faq1] */
double oracle_score(double l) {
  double a = fabs(l);
  double sp = (l > 0 ? l : 0.0) + log1p(exp(-a));
  return sqrt(sp);
}

void oracle_scores(const float *logits, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_score((double)logits[i]);
}

/* Ranking: does expert a come before expert b for logits la, lb? */
static int ranks_before(float la, int a, float lb, int b) {
  int na = isnan(la), nb = isnan(lb);
  if (na || nb) {
    if (na && nb) return a < b;
    return nb;                     /* a number beats NaN */
  }
  if (la != lb) return la > lb;
  return a < b;
}

static const float *g_sort_row;   /* comparator context (used by one thread) */
static int cmp_experts(const void *pa, const void *pb) {
  int a = *(const int *)pa, b = *(const int *)pb;
  if (a == b) return 0;
  return ranks_before(g_sort_row[a], a, g_sort_row[b], b) ? -1 : 1;
}

/* Top-k by a full sort of all E experts; w_j = s_j / sum of the k scores.
 * idx and w are [T,k] in rank order; wd (nullable) receives the weights in
 * double. */
void oracle_topk(const float *logits, int64_t T, int64_t E, int64_t k, int32_t *idx, float *w, double *wd) {
  int *order = (int *)malloc(sizeof(int) * (size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) order[e] = e;
    g_sort_row = logits + t * E;
    qsort(order, (size_t)E, sizeof(int), cmp_experts);   /* total order: unique result */
    double s[64], S = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      s[j] = oracle_score((double)logits[t * E + order[j]]);
      S += s[j];
    }
    for (int64_t j = 0; j < k; ++j) {
      idx[t * k + j] = order[j];
      double wj = s[j] / S;
      w[t * k + j] = (float)wj;
      if (wd) wd[t * k + j] = wj;
    }
  }
  free(order);
}

/* Counting sort of assignments a = t*k + j by expert, stable in a (hence in
 * t): counts[e], offsets[e] = exclusive prefix sum (offsets[E] = T*k), and
 * perm[offsets[e] + r] = the r-th assignment to expert e. */
void oracle_permute(const int32_t *idx, int64_t T, int64_t k, int64_t E, int32_t *counts, int32_t *offsets,
                    int32_t *perm) {
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t a = 0; a < T * k; ++a) counts[idx[a]]++;
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
  for (int64_t e = 0; e < E; ++e) fill[e] = offsets[e];
  for (int64_t a = 0; a < T * k; ++a) perm[fill[idx[a]]++] = (int32_t)a;
  free(fill);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Dense SwiGLU FFN on one token: y = Wd * (silu(Wg x) * (Wu x)).
 * Wg, Wu [I,H], Wd [H,I] row-major doubles; every dot product sequential. */
static void swiglu_ffn(const double *Wg, const double *Wu, const double *Wd, const double *x, int64_t H,
                       int64_t I, double *hbuf, double *y) {
  for (int64_t i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    for (int64_t c = 0; c < H; ++c) {
      g += Wg[i * H + c] * x[c];
      u += Wu[i * H + c] * x[c];
    }
    hbuf[i] = silu(g) * u;
  }
  for (int64_t r = 0; r < H; ++r) {
    double acc = 0.0;
    for (int64_t i = 0; i < I; ++i) acc += Wd[r * I + i] * hbuf[i];
    y[r] = acc;
  }
}

/*
 * The whole layer for T tokens.
 *   x [T,H] fp32 values (bf16 inputs widened exactly by the caller);
 *   wr [E,H] fp32 values; bias [E] or NULL;
 *   gate, up: E canonical-block matrices W[I,H]; down: E matrices W[H,I];
 *   sh_gate, sh_up [Is,H], sh_down [H,Is] fp32 values or NULL (Is = 0);
 * Outputs: y [T,H] fp32; idx/w [T,k] (nullable).
 * Each routed expert is dequantized once and applied to each of its tokens
 * separately; every token's FFN is computed densely and independently.
 */
int oracle_layer_bits(const float *x, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, const float *wr,
                      const float *bias, const uint8_t *gate, const uint8_t *up, const uint8_t *down, int bits,
                      int64_t Is, const float *sh_gate, const float *sh_up, const float *sh_down, float *y,
                      int32_t *idx_out, float *w_out) {
  if (T <= 0) return 0;
  float *logits = (float *)malloc(sizeof(float) * (size_t)(T * E));
  int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * k));
  float *w = (float *)malloc(sizeof(float) * (size_t)(T * k));
  double *wd = (double *)malloc(sizeof(double) * (size_t)(T * k));
  double *Y = (double *)calloc((size_t)(T * k * H), sizeof(double));
  if (!logits || !idx || !w || !wd || !Y) return 1;
  oracle_logits(x, wr, bias, T, E, H, logits);
  oracle_topk(logits, T, E, k, idx, w, wd);
  int64_t mat_blocks = I * H / 256;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t e = 0; e < E; ++e) {
    int64_t n = 0;
    for (int64_t a = 0; a < T * k; ++a) n += idx[a] == e;
    if (!n) continue;
    double *Wg = (double *)malloc(sizeof(double) * (size_t)(I * H));
    double *Wu = (double *)malloc(sizeof(double) * (size_t)(I * H));
    double *Wd = (double *)malloc(sizeof(double) * (size_t)(H * I));
    double *xt = (double *)malloc(sizeof(double) * (size_t)H);
    double *hb = (double *)malloc(sizeof(double) * (size_t)I);
    const int64_t mat_bytes = mat_blocks * block_bytes(bits);
    oracle_dequant_f64_bits(gate + e * mat_bytes, mat_blocks, bits, Wg);
    oracle_dequant_f64_bits(up + e * mat_bytes, mat_blocks, bits, Wu);
    oracle_dequant_f64_bits(down + e * mat_bytes, mat_blocks, bits, Wd);
    for (int64_t a = 0; a < T * k; ++a) {
      if (idx[a] != e) continue;
      int64_t t = a / k;
      for (int64_t c = 0; c < H; ++c) xt[c] = (double)x[t * H + c];
      swiglu_ffn(Wg, Wu, Wd, xt, H, I, hb, Y + a * H);
    }
    free(Wg); free(Wu); free(Wd); free(xt); free(hb);
  }

  double *Sg = NULL, *Su = NULL, *Sd = NULL;
  if (Is > 0) {
    Sg = (double *)malloc(sizeof(double) * (size_t)(Is * H));
    Su = (double *)malloc(sizeof(double) * (size_t)(Is * H));
    Sd = (double *)malloc(sizeof(double) * (size_t)(H * Is));
    for (int64_t i = 0; i < Is * H; ++i) { Sg[i] = sh_gate[i]; Su[i] = sh_up[i]; Sd[i] = sh_down[i]; }
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double *acc = (double *)calloc((size_t)H, sizeof(double));
    for (int64_t j = 0; j < k; ++j)              /* rank order */
      for (int64_t c = 0; c < H; ++c) acc[c] += wd[t * k + j] * Y[(t * k + j) * H + c];
    if (Is > 0) {
      double *xt = (double *)malloc(sizeof(double) * (size_t)H);
      double *hb = (double *)malloc(sizeof(double) * (size_t)Is);
      double *ys = (double *)malloc(sizeof(double) * (size_t)H);
      for (int64_t c = 0; c < H; ++c) xt[c] = (double)x[t * H + c];
      swiglu_ffn(Sg, Su, Sd, xt, H, Is, hb, ys);
      for (int64_t c = 0; c < H; ++c) acc[c] += ys[c];
      free(xt); free(hb); free(ys);
    }
    for (int64_t c = 0; c < H; ++c) y[t * H + c] = (float)acc[c];
    free(acc);
  }
  if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)(T * k));
  if (w_out) memcpy(w_out, w, sizeof(float) * (size_t)(T * k));
  free(Sg); free(Su); free(Sd);
  free(logits); free(idx); free(w); free(wd); free(Y);
  return 0;
}

int oracle_layer(const float *x, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, const float *wr,
                 const float *bias, const uint8_t *gate, const uint8_t *up, const uint8_t *down, int64_t Is,
                 const float *sh_gate, const float *sh_up, const float *sh_down, float *y, int32_t *idx_out,
                 float *w_out) {
  return oracle_layer_bits(x, T, H, I, E, k, wr, bias, gate, up, down, 2, Is, sh_gate, sh_up, sh_down, y, idx_out,
                           w_out);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
