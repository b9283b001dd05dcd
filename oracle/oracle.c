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
 *   - 5- and 6-bit variants (the [models] page's GLM notes name 5-bit gate/up
 *     and down up to 6 bits; no page gives their blocks): the same block with
 *     5- or 6-bit codes as one bit stream from byte 16, lowest bits first
 *     (weight i at bits b*i .. b*i+b-1, which is the 2- and 4-bit order
 *     above), d @16+32b, dmin @18+32b (180 and 212 bytes), q in 0..2^b-1;
 *   - the down matrices may use a code width of their own (the [models] page
 *     gives routed gate/up and routed down different block types);
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

/* Bytes of one block of 256 weights with `bits`-bit codes (2, 4, 5 or 6). */
static int64_t block_bytes(int bits) { return 16 + 32 * bits + 4; }

/* Value of weight i (0..255) of one canonical block with `bits`-bit codes,
 * given the block's d and dmin; exact in double: every product has at most
 * 21 significant bits and the difference of two such numbers of the binary16
 * range fits in 53 bits.  [workload] */
static double block_weight_dm(const uint8_t *blk, int i, int bits, double d, double dmin) {
  int j = i / 16;                                  /* sub-block */
  int sc = blk[j] & 0x0F;                          /* low nibble: scale */
  int mn = blk[j] >> 4;                            /* high nibble: min  */
  /* code i: bits bits*i .. bits*i+bits-1 of the stream from byte 16 (the
   * byte after the last code byte is d's, inside the block) */
  const int bit = bits * i;
  const unsigned two = blk[16 + (bit >> 3)] | ((unsigned)blk[16 + (bit >> 3) + 1] << 8);
  int q = (int)((two >> (bit & 7)) & ((1u << bits) - 1u));
  return d * sc * q - dmin * mn;
}

/* d (bytes nb-4, nb-3) and dmin (bytes nb-2, nb-1) of one block. */
static void block_d_dmin(const uint8_t *blk, int bits, double *d, double *dmin) {
  const int nb = (int)block_bytes(bits);
  *d = half_to_double((uint16_t)(blk[nb - 4] | (blk[nb - 3] << 8)));
  *dmin = half_to_double((uint16_t)(blk[nb - 2] | (blk[nb - 1] << 8)));
}

/* Dequantize n blocks (256 weights each) to doubles. */
void oracle_dequant_f64_bits(const uint8_t *blocks, int64_t nblocks, int bits, double *out) {
  const int64_t nb = block_bytes(bits);
#pragma omp parallel for schedule(static) if (nblocks >= 4096)
  for (int64_t b = 0; b < nblocks; ++b) {
    double d, dmin;
    block_d_dmin(blocks + nb * b, bits, &d, &dmin);
    for (int i = 0; i < 256; ++i) out[b * 256 + i] = block_weight_dm(blocks + nb * b, i, bits, d, dmin);
  }
}

/* Dequantize n blocks to fp32: the exact value rounded once to nearest. */
void oracle_dequant_f32_bits(const uint8_t *blocks, int64_t nblocks, int bits, float *out) {
  const int64_t nb = block_bytes(bits);
  for (int64_t b = 0; b < nblocks; ++b) {
    double d, dmin;
    block_d_dmin(blocks + nb * b, bits, &d, &dmin);
    for (int i = 0; i < 256; ++i) out[b * 256 + i] = (float)block_weight_dm(blocks + nb * b, i, bits, d, dmin);
  }
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

/* Outputs computed side by side: 4 rows of W by 8 tokens.  Lane j of a
 * 4-wide vector below belongs to one token, so every output keeps its own
 * accumulator and its arithmetic is that of a lone dot product. */
#define TB 8
#define RB 4
typedef double dvec4 __attribute__((vector_size(32)));

/* out[t][r] = sum_{c=0}^{K-1} W[r][c] * v[t][c] for the n rows v[t] of
 * vT, stored transposed in blocks of TB tokens: vT[blk][c][j] is
 * v[TB*blk + j][c] (rows beyond n are zero and their outputs are dropped).
 * W [R,K] row-major; out [n,R].  Every sum is taken in order c = 0, 1, ...,
 * product first, then the addition, both rounded in double. */
static void rows_times_tokens(const double *W, int64_t R, int64_t K, const double *vT, int64_t n, double *out) {
  const int64_t nblk = (n + TB - 1) / TB;
  for (int64_t b0 = 0; b0 < nblk; b0 += 16)      /* 128 tokens at a time, so that they stay in cache */
#pragma omp parallel for schedule(static)
  for (int64_t r0 = 0; r0 < R; r0 += RB)
    for (int64_t b = b0; b < nblk && b < b0 + 16; ++b) {
      const double *w[RB];
      for (int i = 0; i < RB; ++i) w[i] = W + (r0 + i < R ? r0 + i : R - 1) * K;   /* rows past R: dropped */
      dvec4 lo[RB] = {{0}}, hi[RB] = {{0}};          /* tokens 0-3 and 4-7 of the block */
      const double *v = vT + b * K * TB;
      for (int64_t c = 0; c < K; ++c) {
        dvec4 v_lo, v_hi;
        memcpy(&v_lo, v + c * TB, sizeof v_lo);
        memcpy(&v_hi, v + c * TB + 4, sizeof v_hi);
        for (int i = 0; i < RB; ++i) {
          lo[i] += w[i][c] * v_lo;
          hi[i] += w[i][c] * v_hi;
        }
      }
      for (int i = 0; i < RB && r0 + i < R; ++i)
        for (int j = 0; j < TB && TB * b + j < n; ++j)
          out[(TB * b + j) * R + r0 + i] = j < 4 ? lo[i][j] : hi[i][j - 4];
    }
}

/* v [n,K] row-major -> the transposed token blocks read by rows_times_tokens. */
static double *token_blocks(const double *v, int64_t n, int64_t K) {
  const int64_t nblk = (n + TB - 1) / TB;
  double *vT = (double *)calloc((size_t)(nblk * K * TB), sizeof(double));
  if (!vT) return NULL;
  for (int64_t t = 0; t < n; ++t)
    for (int64_t c = 0; c < K; ++c) vT[(t / TB) * K * TB + c * TB + t % TB] = v[t * K + c];
  return vT;
}

/* Dense SwiGLU FFN on n tokens: y_t = Wd * (silu(Wg x_t) * (Wu x_t)).
 * Wg, Wu [I,H], Wd [H,I] row-major doubles; xs [n,H]; y [n,H].  Each token's
 * FFN is computed on its own (rows_times_tokens).  Returns 0, or 1 when out
 * of memory. */
static int swiglu_ffn(const double *Wg, const double *Wu, const double *Wd, const double *xs, int64_t n, int64_t H,
                      int64_t I, double *y) {
  double *xT = token_blocks(xs, n, H);
  double *g = (double *)malloc(sizeof(double) * (size_t)(n * I));
  double *u = (double *)malloc(sizeof(double) * (size_t)(n * I));
  if (!xT || !g || !u) { free(xT); free(g); free(u); return 1; }
  rows_times_tokens(Wg, I, H, xT, n, g);
  rows_times_tokens(Wu, I, H, xT, n, u);
  free(xT);
  for (int64_t i = 0; i < n * I; ++i) g[i] = silu(g[i]) * u[i];   /* h */
  free(u);
  double *hT = token_blocks(g, n, I);
  free(g);
  if (!hT) return 1;
  rows_times_tokens(Wd, H, I, hT, n, y);
  free(hT);
  return 0;
}

/*
 * The whole layer for T tokens.
 *   x [T,H] fp32 values (bf16 inputs widened exactly by the caller);
 *   wr [E,H] fp32 values; bias [E] or NULL;
 *   gate, up: E canonical-block matrices W[I,H]; down: E matrices W[H,I];
 *   sh_gate, sh_up [Is,H], sh_down [H,Is] fp32 values or NULL (Is = 0);
 * Outputs: y [T,H] fp32; idx/w [T,k] (nullable).
 * Each routed expert is dequantized once and applied to each of its tokens;
 * every token's FFN is computed densely and independently.
 */
int oracle_layer_bits2(const float *x, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, const float *wr,
                       const float *bias, const uint8_t *gate, const uint8_t *up, const uint8_t *down, int bits,
                       int bits_down, int64_t Is, const float *sh_gate, const float *sh_up, const float *sh_down,
                       float *y, int32_t *idx_out, float *w_out) {
  if (T <= 0) return 0;
  int rc = 0;
  float *logits = (float *)malloc(sizeof(float) * (size_t)(T * E));
  int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * k));
  float *w = (float *)malloc(sizeof(float) * (size_t)(T * k));
  double *wd = (double *)malloc(sizeof(double) * (size_t)(T * k));
  double *Y = (double *)calloc((size_t)(T * k * H), sizeof(double));   /* per assignment a = t*k + j */
  double *xd = (double *)malloc(sizeof(double) * (size_t)(T * H));
  int64_t *as = (int64_t *)malloc(sizeof(int64_t) * (size_t)(T * k));
  double *Wg = (double *)malloc(sizeof(double) * (size_t)(I * H));
  double *Wu = (double *)malloc(sizeof(double) * (size_t)(I * H));
  double *Wd = (double *)malloc(sizeof(double) * (size_t)(H * I));
  double *xs = (double *)malloc(sizeof(double) * (size_t)(T * H));
  double *ys = (double *)malloc(sizeof(double) * (size_t)(T * H));
  if (!logits || !idx || !w || !wd || !Y || !xd || !as || !Wg || !Wu || !Wd || !xs || !ys) { rc = 1; goto done; }
  oracle_logits(x, wr, bias, T, E, H, logits);
  oracle_topk(logits, T, E, k, idx, w, wd);
  for (int64_t i = 0; i < T * H; ++i) xd[i] = (double)x[i];

  const int64_t mat_blocks = I * H / 256, mat_bytes = mat_blocks * block_bytes(bits);
  const int64_t down_bytes = mat_blocks * block_bytes(bits_down);   /* down in its own code width */
  for (int64_t e = 0; e < E; ++e) {
    int64_t n = 0;                                   /* the expert's assignments, a ascending */
    for (int64_t a = 0; a < T * k; ++a)
      if (idx[a] == e) as[n++] = a;
    if (!n) continue;
    oracle_dequant_f64_bits(gate + e * mat_bytes, mat_blocks, bits, Wg);
    oracle_dequant_f64_bits(up + e * mat_bytes, mat_blocks, bits, Wu);
    oracle_dequant_f64_bits(down + e * down_bytes, mat_blocks, bits_down, Wd);
    for (int64_t j = 0; j < n; ++j) memcpy(xs + j * H, xd + (as[j] / k) * H, sizeof(double) * (size_t)H);
    if (swiglu_ffn(Wg, Wu, Wd, xs, n, H, I, ys)) { rc = 1; goto done; }
    for (int64_t j = 0; j < n; ++j) memcpy(Y + as[j] * H, ys + j * H, sizeof(double) * (size_t)H);
  }

  if (Is > 0) {                                      /* the shared expert on every token */
    free(Wg); free(Wu); free(Wd);
    Wg = (double *)malloc(sizeof(double) * (size_t)(Is * H));
    Wu = (double *)malloc(sizeof(double) * (size_t)(Is * H));
    Wd = (double *)malloc(sizeof(double) * (size_t)(H * Is));
    if (!Wg || !Wu || !Wd) { rc = 1; goto done; }
    for (int64_t i = 0; i < Is * H; ++i) { Wg[i] = sh_gate[i]; Wu[i] = sh_up[i]; Wd[i] = sh_down[i]; }
    if (swiglu_ffn(Wg, Wu, Wd, xd, T, H, Is, ys)) { rc = 1; goto done; }
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int64_t j = 0; j < k; ++j) acc += wd[t * k + j] * Y[(t * k + j) * H + c];   /* rank order */
      if (Is > 0) acc += ys[t * H + c];
      y[t * H + c] = (float)acc;
    }
  if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)(T * k));
  if (w_out) memcpy(w_out, w, sizeof(float) * (size_t)(T * k));
done:
  free(logits); free(idx); free(w); free(wd); free(Y); free(xd); free(as);
  free(Wg); free(Wu); free(Wd); free(xs); free(ys);
  return rc;
}

int oracle_layer_bits(const float *x, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, const float *wr,
                      const float *bias, const uint8_t *gate, const uint8_t *up, const uint8_t *down, int bits,
                      int64_t Is, const float *sh_gate, const float *sh_up, const float *sh_down, float *y,
                      int32_t *idx_out, float *w_out) {
  return oracle_layer_bits2(x, T, H, I, E, k, wr, bias, gate, up, down, bits, bits, Is, sh_gate, sh_up, sh_down, y,
                            idx_out, w_out);
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
