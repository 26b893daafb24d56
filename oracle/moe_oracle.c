/*
 * moe_oracle.c -- CPU oracle for the fused MoE expert layer.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain reference that the
 * GPU path is checked against. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it. The product library never
 * links, loads or calls it, and it shares no code with the HIP kernels.
 *
 * What it computes (one MoE expert layer, no token dropping):
 *   router  : logits[t,e] = sum_h x[t,h] * W_r[e,h] (the gating scores the
 *             routing starts from; the pages do not spell this projection
 *             out, see router_logits below).
 *   route   : per token, the k largest router logits (ties -> lower expert
 *             index), in descending order, and a softmax over those k logits.
 *   permute : a stable counting sort of the T*k (token, slot) assignments by
 *             expert id into per-expert contiguous row blocks.
 *   gate/up : per expert, G = X W_gate, U = X W_up, h = silu(G) * U.
 *   down    : y = h W_down.
 *   combine : out[t] = sum_j w[t,j] * y[row of (t,j)]  (+ s_t * shared(x[t])).
 *   fp8     : weights as OCP E4M3 codes with one power-of-two scale per
 *             output column; the layer is then computed on the dequantized
 *             weights (see the fp8 section below).
 *   mxfp4   : weights as E2M1 codes with one power-of-two scale per 32
 *             K-values of a column (OCP MX); likewise (mxfp4 section).
 *   mxfp8   : weights as E4M3 codes with one power-of-two scale per 32
 *             K-values of a column (OCP MX); likewise (mxfp8 section).
 *   backward: the chain rule through the routed layer for a fixed routing,
 *             through the softmax over the k selected logits, and through
 *             the shared expert and its gate (backward section).
 *
 * Sources (restated, not quoted):
 *   - "Triton-MoE-Dispatch-Kernel erreicht 131 % von Megablocks" (lumeric.app),
 *     summary paragraph: the gate and up projections are computed together and
 *     feed SwiGLU; the layer is dispatch -> fused gate/up -> down -> combine.
 *   - "DeepGEMM ..." article (itsolotime.com), section 1.1: the MoE layer runs
 *     dispatch -> linear1 -> SwiGLU -> linear2 -> combine; section 3.1: the
 *     activations of an m-grouped GEMM are stored contiguously per expert.
 *   - HPC-Ops article (ntfzh.com), FusedMoE paragraph: data re-arrangement
 *     before the grouped GEMM, then a weighted-average reduce afterwards.
 *   - Triton MoE page (setupai.cc), key points: block-scheduled grouped GEMM
 *     over variable expert batch sizes.
 *   The pages fix neither routing details nor precision. Readings taken here:
 *   softmax over the k selected logits; ties to the lower expert index with
 *   -0 == +0; rows inside an expert block in ascending token order; all
 *   floating-point arithmetic in IEEE double (fp64) with sums taken in
 *   ascending index order; SwiGLU h = silu(x W_gate) * (x W_up) with
 *   silu(z) = z / (1 + exp(-z)) (Shazeer, "GLU Variants Improve Transformer").
 *
 * Data: bf16 tensors are passed as uint16 bit patterns; floats as fp32; all
 * results of arithmetic are fp64. Row-major, contiguous. Weights are
 * W_gate/W_up [E,H,F] and W_down [E,F,H].
 *
 * Pins (in tests/): a numpy fp64 dense brute force (every expert run on every
 * token, masked and weighted), the E=1,k=1 reduction to a textbook SwiGLU FFN,
 * closed-form routing weights, brute-force routing and permutation by full
 * sort, hand-worked fixtures, exact scaling and zero invariants.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_NONFINITE (-2)
#define ORC_ERR_ID (-3)
#define ORC_ERR_NOMEM (-4)

static inline double bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads of the later parallel loops (the CPU baseline's single-thread
 * figure); no effect on any result, rows being independent. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ----------------------------------------------------------------- router */

/* Router projection: logits[t,e] = sum_h x[t,h] * W_r[e,h], h ascending, in
 * fp64 (each bf16 product is exact in fp64, so only the sum rounds). The
 * routing is done on the device from such gating scores in the Triton MoE
 * page (setupai.cc), technical deep-dive; the pages do not state how the
 * scores are produced. Reading taken: one bias-free linear map of the token
 * row, W_r stored [E,H] (row e = expert e's router vector). */
int oracle_router_logits(const uint16_t* x, int64_t T, int H, int E,
                         const uint16_t* wr, double* logits) {
  if (T < 0 || H < 1 || E < 1) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      const uint16_t* xr = x + t * H;
      const uint16_t* wrow = wr + (int64_t)e * H;
      double s = 0.0;
      for (int h = 0; h < H; ++h) s += bf16_to_f64(xr[h]) * bf16_to_f64(wrow[h]);
      logits[t * E + e] = s;
    }
  return ORC_OK;
}

/* -------------------------------------------------------------------- fp8 */

/* Weights in 8-bit floating point. The DeepGEMM article (itsolotime.com),
 * sections 1.1 and 5.3, runs the Mega MoE's two expert GEMMs in low
 * precision (FP8 and FP4 operands) but gives no format details. Readings
 * taken: the weights are stored as E4M3 codes of the OCP 8-bit floating
 * point specification (1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent field 0 is subnormal, m/8 * 2^-6; S.1111.111 is NaN; no
 * infinities; largest finite value 448), each output column n of each
 * matrix g with one scale 2^e[g,n]; the activations stay bf16. Every
 * dequantized weight code * 2^e is then exactly a bf16 value (8 exponent
 * bits cover the range), so the layer on fp8 weights is the bf16 layer on
 * the dequantized weights. */

/* Value of one E4M3 code (NaN for the two NaN codes). */
double oracle_e4m3_value(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Per column: e = the smallest integer with max_k |w[g,k,n]| <= 448 * 2^e
 * (0 for an all-zero column), so nothing saturates; then each weight's code
 * is the E4M3 value nearest to w / 2^e, found by scanning all 127
 * non-negative finite codes, a tie going to the code with an even mantissa
 * (round to nearest, ties to even, on the code grid); the sign is the
 * weight's. w bf16 [G,K,N] -> codes [G,K,N], scales[g*N+n] = 2^e. */
int oracle_quantize_e4m3(const uint16_t* w, int64_t G, int K, int N, uint8_t* codes,
                         double* scales) {
  if (G < 0 || K < 1 || N < 1) return ORC_ERR_ARG;
  double mag[127];
  for (int c = 0; c < 127; ++c) mag[c] = oracle_e4m3_value((uint8_t)c);
#pragma omp parallel for schedule(static)
  for (int64_t gn = 0; gn < G * N; ++gn) {
    const int64_t g = gn / N;
    const int n = (int)(gn % N);
    const uint16_t* wg = w + g * (int64_t)K * N;
    double amax = 0.0;
    for (int k = 0; k < K; ++k) {
      const double a = fabs(bf16_to_f64(wg[(int64_t)k * N + n]));
      if (a > amax) amax = a;
    }
    int e = 0;
    if (amax > 0.0) {
      e = -200;
      while (amax > ldexp(448.0, e)) ++e;
    }
    scales[gn] = ldexp(1.0, e);
    for (int k = 0; k < K; ++k) {
      const double x = bf16_to_f64(wg[(int64_t)k * N + n]);
      const double v = fabs(ldexp(x, -e));
      int best = 0;
      for (int c = 1; c < 127; ++c) {
        const double dc = fabs(mag[c] - v), db = fabs(mag[best] - v);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
      }
      codes[g * (int64_t)K * N + (int64_t)k * N + n] =
          (uint8_t)(best | (signbit(x) ? 0x80 : 0));
    }
  }
  return ORC_OK;
}

/* w[g,k,n] = value(codes[g,k,n]) * scales[g*N+n]. */
void oracle_dequant_e4m3(const uint8_t* codes, const double* scales, int64_t G, int K, int N,
                         double* w) {
  for (int64_t g = 0; g < G; ++g)
    for (int k = 0; k < K; ++k)
      for (int n = 0; n < N; ++n) {
        const int64_t i = g * (int64_t)K * N + (int64_t)k * N + n;
        w[i] = oracle_e4m3_value(codes[i]) * scales[g * N + n];
      }
}

/* ------------------------------------------------------------------ mxfp4 */

/* Weights in 4-bit floating point with block scales. The DeepGEMM article
 * (itsolotime.com), sections 1.1 and 5.3, pairs FP8 activations with FP4
 * expert weights in the Mega MoE but gives no format. Readings taken: the
 * OCP Microscaling (MX) format MXFP4. Each weight is an E2M1 code (1 sign
 * bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent field 0 is
 * subnormal, m * 0.5; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities
 * or NaN), and every block of 32 consecutive K-values of one output column
 * shares one E8M0 scale 2^X (scale byte X + 127). The activations stay
 * bf16. Every dequantized weight code * 2^X is exactly a bf16 value, so the
 * layer on MXFP4 weights is the bf16 layer on the dequantized weights. */

/* Value of one E2M1 code (the low 4 bits of c). */
double oracle_e2m1_value(uint8_t c) {
  const int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  const double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* Value of one E8M0 scale byte (0xFF, NaN in the format, is never made). */
double oracle_e8m0_value(uint8_t s) { return s == 0xFF ? NAN : ldexp(1.0, (int)s - 127); }

/* Per column n and K-block b (K-values 32b .. 32b+31, the last block of a
 * K that is not a multiple of 32 shorter): with amax the block's largest
 * |w|, X = floor(log2(amax)) - 2 (2 = the exponent of the largest E2M1
 * value, 1.5 * 2^2), the MX rule, raised to -125 where it is smaller (so
 * that every nonzero dequantized weight is a normal bf16 value; it only
 * matters for blocks whose largest weight is below 2^-123); an all-zero
 * block takes X = 0. Each weight's code is the E2M1 value nearest to
 * w / 2^X found by scanning the 8 magnitudes, a tie going to the code with
 * mantissa bit 0 (round to nearest, ties to even), so magnitudes above 6
 * become 6 (the MX rule saturates); the sign is the weight's (also for
 * zeros). w bf16 [G,K,N] -> codes [G,K,N] (one per byte, values 0..15),
 * scale bytes [G, ceil(K/32), N]. */
int oracle_quantize_mxfp4(const uint16_t* w, int64_t G, int K, int N, uint8_t* codes,
                          uint8_t* scale_bytes) {
  if (G < 0 || K < 1 || N < 1) return ORC_ERR_ARG;
  const int KB = (K + 31) / 32;
  double mag[8];
  for (int c = 0; c < 8; ++c) mag[c] = oracle_e2m1_value((uint8_t)c);
#pragma omp parallel for schedule(static)
  for (int64_t gbn = 0; gbn < G * KB * (int64_t)N; ++gbn) {
    const int64_t g = gbn / ((int64_t)KB * N);
    const int b = (int)((gbn / N) % KB);
    const int n = (int)(gbn % N);
    const uint16_t* wg = w + g * (int64_t)K * N;
    const int k_end = 32 * b + 32 < K ? 32 * b + 32 : K;
    double amax = 0.0;
    for (int k = 32 * b; k < k_end; ++k) {
      const double a = fabs(bf16_to_f64(wg[(int64_t)k * N + n]));
      if (a > amax) amax = a;
    }
    int X = 0;
    if (amax > 0.0) {
      int E;
      frexp(amax, &E);  /* amax = f * 2^E, f in [0.5, 1): floor(log2(amax)) = E - 1 */
      X = E - 1 - 2;
      if (X < -125) X = -125;
    }
    scale_bytes[gbn] = (uint8_t)(X + 127);
    for (int k = 32 * b; k < k_end; ++k) {
      const double x = bf16_to_f64(wg[(int64_t)k * N + n]);
      const double v = fabs(ldexp(x, -X));
      int best = 0;
      for (int c = 1; c < 8; ++c) {
        const double dc = fabs(mag[c] - v), db = fabs(mag[best] - v);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
      }
      codes[g * (int64_t)K * N + (int64_t)k * N + n] = (uint8_t)(best | (signbit(x) ? 8 : 0));
    }
  }
  return ORC_OK;
}

/* w[g,k,n] = value(codes[g,k,n]) * value(scale_bytes[g, k/32, n]). */
void oracle_dequant_mxfp4(const uint8_t* codes, const uint8_t* scale_bytes, int64_t G, int K,
                          int N, double* w) {
  const int KB = (K + 31) / 32;
  for (int64_t g = 0; g < G; ++g)
    for (int k = 0; k < K; ++k)
      for (int n = 0; n < N; ++n) {
        const int64_t i = g * (int64_t)K * N + (int64_t)k * N + n;
        w[i] = oracle_e2m1_value(codes[i]) *
               oracle_e8m0_value(scale_bytes[(g * KB + k / 32) * (int64_t)N + n]);
      }
}

/* ------------------------------------------------------------------ mxfp8 */

/* Weights in 8-bit floating point with block scales: the FP8 expert GEMM
 * "with block scales" of the DeepGEMM article (itsolotime.com), sections 1.1
 * and 5.3, which fixes no format. Reading taken: the OCP Microscaling (MX)
 * format MXFP8 with E4M3 elements. Every block of 32 consecutive K-values of
 * one output column shares one E8M0 scale 2^X (scale byte X + 127), and each
 * weight is an E4M3 code (see the fp8 section) of w / 2^X. The activations
 * stay bf16; every dequantized weight code * 2^X is exactly a bf16 value, so
 * the layer on MXFP8 weights is the bf16 layer on the dequantized weights. */

/* Per column n and K-block b (K-values 32b .. 32b+31, the last block of a
 * K that is not a multiple of 32 shorter): with amax the block's largest
 * |w|, X = floor(log2(amax)) - 8 (8 = the exponent of the largest E4M3
 * value, 1.75 * 2^8), the MX rule, raised to -117 where it is smaller (the
 * smallest nonzero code, 2^-9, times 2^-117 is the least normal bf16 value;
 * it only matters for blocks whose largest weight is below 2^-109); an
 * all-zero block takes X = 0. Each weight's code is the finite E4M3 value
 * nearest to w / 2^X, found by scanning the 127 non-negative finite codes, a
 * tie going to the code with an even mantissa (round to nearest, ties to
 * even), so magnitudes above 448 become 448 (the MX rule saturates); the
 * sign is the weight's (also for zeros). w bf16 [G,K,N] -> codes [G,K,N],
 * scale bytes [G, ceil(K/32), N]. */
int oracle_quantize_mxfp8(const uint16_t* w, int64_t G, int K, int N, uint8_t* codes,
                          uint8_t* scale_bytes) {
  if (G < 0 || K < 1 || N < 1) return ORC_ERR_ARG;
  const int KB = (K + 31) / 32;
  double mag[127];
  for (int c = 0; c < 127; ++c) mag[c] = oracle_e4m3_value((uint8_t)c);
#pragma omp parallel for schedule(static)
  for (int64_t gbn = 0; gbn < G * KB * (int64_t)N; ++gbn) {
    const int64_t g = gbn / ((int64_t)KB * N);
    const int b = (int)((gbn / N) % KB);
    const int n = (int)(gbn % N);
    const uint16_t* wg = w + g * (int64_t)K * N;
    const int k_end = 32 * b + 32 < K ? 32 * b + 32 : K;
    double amax = 0.0;
    for (int k = 32 * b; k < k_end; ++k) {
      const double a = fabs(bf16_to_f64(wg[(int64_t)k * N + n]));
      if (a > amax) amax = a;
    }
    int X = 0;
    if (amax > 0.0) {
      int E;
      frexp(amax, &E);  /* amax = f * 2^E, f in [0.5, 1): floor(log2(amax)) = E - 1 */
      X = E - 1 - 8;
      if (X < -117) X = -117;
    }
    scale_bytes[gbn] = (uint8_t)(X + 127);
    for (int k = 32 * b; k < k_end; ++k) {
      const double x = bf16_to_f64(wg[(int64_t)k * N + n]);
      const double v = fabs(ldexp(x, -X));
      int best = 0;
      for (int c = 1; c < 127; ++c) {
        const double dc = fabs(mag[c] - v), db = fabs(mag[best] - v);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
      }
      codes[g * (int64_t)K * N + (int64_t)k * N + n] =
          (uint8_t)(best | (signbit(x) ? 0x80 : 0));
    }
  }
  return ORC_OK;
}

/* w[g,k,n] = value(codes[g,k,n]) * value(scale_bytes[g, k/32, n]). */
void oracle_dequant_mxfp8(const uint8_t* codes, const uint8_t* scale_bytes, int64_t G, int K,
                          int N, double* w) {
  const int KB = (K + 31) / 32;
  for (int64_t g = 0; g < G; ++g)
    for (int k = 0; k < K; ++k)
      for (int n = 0; n < N; ++n) {
        const int64_t i = g * (int64_t)K * N + (int64_t)k * N + n;
        w[i] = oracle_e4m3_value(codes[i]) *
               oracle_e8m0_value(scale_bytes[(g * KB + k / 32) * (int64_t)N + n]);
      }
}

/* ------------------------------------------------------------------ route */

/* One token: the k largest of E logits, larger first, equal logits taken in
 * ascending expert order; then softmax over the chosen logits. `taken` is
 * scratch of E bytes. Returns ORC_ERR_NONFINITE on a NaN/Inf logit. */
static int route_one(const float* l, int E, int k, int32_t* ids, double* w,
                     unsigned char* taken) {
  for (int e = 0; e < E; ++e) {
    if (!isfinite(l[e])) return ORC_ERR_NONFINITE;
    taken[e] = 0;
  }
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      /* strict '>' keeps the earlier (lower) index on a tie; IEEE compare
       * treats -0.0 and +0.0 as equal, so they tie as well */
      if (best < 0 || l[e] > l[best]) best = e;
    }
    taken[best] = 1;
    ids[j] = best;
  }
  /* softmax over the k selected logits; slot 0 holds the largest, which is
   * subtracted before exponentiation */
  double m = (double)l[ids[0]];
  double s = 0.0;
  for (int j = 0; j < k; ++j) {
    w[j] = exp((double)l[ids[j]] - m);
    s += w[j];
  }
  for (int j = 0; j < k; ++j) w[j] = w[j] / s;
  return ORC_OK;
}

int oracle_route(const float* logits, int64_t T, int E, int k, int32_t* ids,
                 double* w) {
  if (T < 0 || E < 1 || k < 1 || k > E) return ORC_ERR_ARG;
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  if (!taken) return ORC_ERR_NOMEM;
  int rc = ORC_OK;
  for (int64_t t = 0; t < T && rc == ORC_OK; ++t)
    rc = route_one(logits + t * E, E, k, ids + t * k, w + t * k, taken);
  free(taken);
  return rc;
}

/* ---------------------------------------------------------------- permute */

/* Stable counting sort of the flat assignments i = t*k + j by expert id.
 * offsets[E+1] = exclusive prefix of the per-expert counts; row p of the
 * permuted layout holds token row_token[p]; row_dest[t*k+j] = p. */
int oracle_permute(const int32_t* ids, int64_t T, int E, int k,
                   int32_t* offsets, int32_t* row_token, int32_t* row_dest) {
  if (T < 0 || E < 1 || k < 1) return ORC_ERR_ARG;
  int64_t A = T * k;
  int64_t* next = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  if (!next) return ORC_ERR_NOMEM;
  for (int64_t i = 0; i < A; ++i) {
    if (ids[i] < 0 || ids[i] >= E) {
      free(next);
      return ORC_ERR_ID;
    }
    next[ids[i]] += 1; /* count */
  }
  int64_t run = 0;
  for (int e = 0; e < E; ++e) {
    offsets[e] = (int32_t)run;
    int64_t c = next[e];
    next[e] = run; /* first free row of expert e */
    run += c;
  }
  offsets[E] = (int32_t)run;
  for (int64_t t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int64_t p = next[ids[t * k + j]]++;
      row_token[p] = (int32_t)t;
      row_dest[t * k + j] = (int32_t)p;
    }
  free(next);
  return ORC_OK;
}

/* x_perm[p,:] = x[row_token[p],:] (a bit copy). */
void oracle_gather(const uint16_t* x, const int32_t* row_token, int64_t A,
                   int H, uint16_t* x_perm) {
  for (int64_t p = 0; p < A; ++p)
    memcpy(x_perm + p * H, x + (int64_t)row_token[p] * H,
           (size_t)H * sizeof(uint16_t));
}

/* ------------------------------------------------------------ expert FFN */

static inline double silu(double z) { return z / (1.0 + exp(-z)); }

/* One row through gate/up + SwiGLU: G[f] = sum_h x[h] Wg[h,f] (h ascending),
 * likewise U; h[f] = silu(G[f]) * U[f]. G and U are scratch of F doubles. */
static void gateup_row(const uint16_t* x, int H, int F, const uint16_t* wg,
                       const uint16_t* wu, double* hrow, double* G, double* U) {
  for (int f = 0; f < F; ++f) G[f] = 0.0, U[f] = 0.0;
  for (int h = 0; h < H; ++h) {
    double xv = bf16_to_f64(x[h]);
    const uint16_t* rg = wg + (int64_t)h * F;
    const uint16_t* ru = wu + (int64_t)h * F;
    for (int f = 0; f < F; ++f) {
      G[f] += xv * bf16_to_f64(rg[f]);
      U[f] += xv * bf16_to_f64(ru[f]);
    }
  }
  for (int f = 0; f < F; ++f) hrow[f] = silu(G[f]) * U[f];
}

/* One row through the down projection: y[c] = sum_f h[f] Wd[f,c] (f asc). */
static void down_row(const double* hrow, int F, int H, const uint16_t* wd,
                     double* y) {
  for (int c = 0; c < H; ++c) y[c] = 0.0;
  for (int f = 0; f < F; ++f) {
    double hv = hrow[f];
    const uint16_t* rd = wd + (int64_t)f * H;
    for (int c = 0; c < H; ++c) y[c] += hv * bf16_to_f64(rd[c]);
  }
}

/* M rows of x [M,H] through one expert's gate/up + SwiGLU -> h [M,F]. */
int oracle_gateup_rows(const uint16_t* x, int64_t M, int H, int F,
                       const uint16_t* wg, const uint16_t* wu, double* h) {
  int rc = ORC_OK;
#pragma omp parallel
  {
    double* G = (double*)malloc(sizeof(double) * (size_t)F * 2);
    if (!G) {
#pragma omp atomic write
      rc = ORC_ERR_NOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < M; ++r)
        gateup_row(x + r * H, H, F, wg, wu, h + r * F, G, G + F);
      free(G);
    }
  }
  return rc;
}

/* M rows of h [M,F] through one expert's down projection -> y [M,H]. */
int oracle_down_rows(const double* h, int64_t M, int F, int H,
                     const uint16_t* wd, double* y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < M; ++r) down_row(h + r * F, F, H, wd, y + r * H);
  return ORC_OK;
}

/* Expert owning permuted row p: the e with offsets[e] <= p < offsets[e+1]. */
static int expert_of_row(const int32_t* offsets, int E, int64_t p) {
  int e = 0;
  while (e < E && !(p >= offsets[e] && p < offsets[e + 1])) ++e;
  return e;
}

/* Grouped gate/up + SwiGLU over the permuted rows: rows of expert e use
 * W_gate[e], W_up[e]. x_perm [A,H], h [A,F], A = offsets[E]. */
int oracle_grouped_gateup(const uint16_t* x_perm, const int32_t* offsets,
                          int E, int H, int F, const uint16_t* wg,
                          const uint16_t* wu, double* h) {
  int64_t A = offsets[E];
  int rc = ORC_OK;
#pragma omp parallel
  {
    double* G = (double*)malloc(sizeof(double) * (size_t)F * 2);
    if (!G) {
#pragma omp atomic write
      rc = ORC_ERR_NOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t p = 0; p < A; ++p) {
        int e = expert_of_row(offsets, E, p);
        int64_t wo = (int64_t)e * H * F;
        gateup_row(x_perm + p * H, H, F, wg + wo, wu + wo, h + p * F, G,
                   G + F);
      }
      free(G);
    }
  }
  return rc;
}

/* Grouped down projection: rows of expert e use W_down[e]. y [A,H]. */
int oracle_grouped_down(const double* h, const int32_t* offsets, int E, int F,
                        int H, const uint16_t* wd, double* y) {
  int64_t A = offsets[E];
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < A; ++p) {
    int e = expert_of_row(offsets, E, p);
    down_row(h + p * F, F, H, wd + (int64_t)e * F * H, y + p * H);
  }
  return ORC_OK;
}

/* ---------------------------------------------------------------- combine */

/* out[t,c] = sum_j w[t,j] * y[row_dest[t,j], c]  (j ascending), then
 * + s[t] * y_sh[t,c] when a shared expert is present (y_sh, s non-NULL). */
void oracle_combine(const double* y, const int32_t* row_dest, const double* w,
                    int64_t T, int H, int k, const double* y_sh,
                    const double* s, double* out) {
#pragma omp parallel for
  for (int64_t t = 0; t < T; ++t)
    for (int c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j)
        acc += w[t * k + j] * y[(int64_t)row_dest[t * k + j] * H + c];
      if (y_sh) acc += s[t] * y_sh[t * H + c];
      out[t * H + c] = acc;
    }
}

/* Shared-expert gate: s_t = 1 when no gate logits are given, else the
 * logistic sigmoid 1 / (1 + exp(-g_t)). */
void oracle_shared_gate(const float* gate_logits, int64_t T, double* s) {
  for (int64_t t = 0; t < T; ++t)
    s[t] = gate_logits ? 1.0 / (1.0 + exp(-(double)gate_logits[t])) : 1.0;
}

/* -------------------------------------------------------- whole forward */

/* Full layer: route -> permute -> gather -> grouped gate/up -> grouped down
 * -> (shared expert) -> combine. Shared expert is present when Fs > 0.
 * Outputs: out [T,H] fp64, and (each may be NULL) ids [T,k], w [T,k],
 * offsets [E+1], row_token [T*k], row_dest [T*k], h [T*k,F], y [T*k,H]. */
int oracle_forward(const uint16_t* x, const float* logits, int64_t T, int H,
                   int F, int E, int k, const uint16_t* wg, const uint16_t* wu,
                   const uint16_t* wd, int Fs, const uint16_t* wsg,
                   const uint16_t* wsu, const uint16_t* wsd,
                   const float* gate_logits, double* out, int32_t* ids_out,
                   double* w_out, int32_t* offsets_out,
                   int32_t* row_token_out, int32_t* row_dest_out,
                   double* h_out, double* y_out) {
  if (T < 0 || H < 1 || F < 1 || E < 1 || k < 1 || k > E || Fs < 0)
    return ORC_ERR_ARG;
  int64_t A = T * k;
  int rc = ORC_ERR_NOMEM;
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
  double* w = (double*)malloc(sizeof(double) * (size_t)(A + 1));
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* row_token = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
  int32_t* row_dest = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
  uint16_t* x_perm = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(A * H + 1));
  double* h = (double*)malloc(sizeof(double) * (size_t)(A * F + 1));
  double* y = (double*)malloc(sizeof(double) * (size_t)(A * H + 1));
  double* h_sh = Fs > 0 ? (double*)malloc(sizeof(double) * (size_t)(T * Fs + 1)) : NULL;
  double* y_sh = Fs > 0 ? (double*)malloc(sizeof(double) * (size_t)(T * H + 1)) : NULL;
  double* s = Fs > 0 ? (double*)malloc(sizeof(double) * (size_t)(T + 1)) : NULL;
  if (!ids || !w || !offsets || !row_token || !row_dest || !x_perm || !h ||
      !y || (Fs > 0 && (!h_sh || !y_sh || !s)))
    goto done;

  rc = oracle_route(logits, T, E, k, ids, w);
  if (rc) goto done;
  rc = oracle_permute(ids, T, E, k, offsets, row_token, row_dest);
  if (rc) goto done;
  oracle_gather(x, row_token, A, H, x_perm);
  rc = oracle_grouped_gateup(x_perm, offsets, E, H, F, wg, wu, h);
  if (rc) goto done;
  oracle_grouped_down(h, offsets, E, F, H, wd, y);
  if (Fs > 0) {
    rc = oracle_gateup_rows(x, T, H, Fs, wsg, wsu, h_sh);
    if (rc) goto done;
    oracle_down_rows(h_sh, T, Fs, H, wsd, y_sh);
    oracle_shared_gate(gate_logits, T, s);
  }
  oracle_combine(y, row_dest, w, T, H, k, y_sh, s, out);

  if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)A);
  if (w_out) memcpy(w_out, w, sizeof(double) * (size_t)A);
  if (offsets_out) memcpy(offsets_out, offsets, sizeof(int32_t) * (size_t)(E + 1));
  if (row_token_out) memcpy(row_token_out, row_token, sizeof(int32_t) * (size_t)A);
  if (row_dest_out) memcpy(row_dest_out, row_dest, sizeof(int32_t) * (size_t)A);
  if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)(A * F));
  if (y_out) memcpy(y_out, y, sizeof(double) * (size_t)(A * H));
  rc = ORC_OK;
done:
  free(ids); free(w); free(offsets); free(row_token); free(row_dest);
  free(x_perm); free(h); free(y); free(h_sh); free(y_sh); free(s);
  return rc;
}

/* ---------------------------------------------------------------- backward */

/* Training backward of the routed layer (the grouped-GEMM news page says the
 * kernel serves training as well as inference; the pages give no backward,
 * so this is the derivative of the forward above, by the chain rule). With
 * the routing (ids, w) fixed and out[t] = sum_j w[t,j] y(t,j),
 * y = h W_down[e], h = silu(G) * U, G = x W_gate[e], U = x W_up[e]:
 *   dw[t,j]   = <dout[t], y(t,j)>
 *   dy        = w[t,j] dout[t]
 *   dh[f]     = sum_c dy[c] W_down[e][f][c]
 *   dG        = dh U silu'(G),  silu'(z) = s(z) (1 + z (1 - s(z))), s the logistic
 *   dU        = dh silu(G)
 *   dx[t]     = sum_j (dG W_gate[e]^T + dU W_up[e]^T)          (j ascending)
 *   dW_gate[e] = sum over e's rows of x^T dG, dW_up[e] likewise with dU,
 *   dW_down[e] = sum over e's rows of h^T dy                      (rows ascending)
 * x, weights and dout bf16, w fp32, everything else fp64. */
int oracle_backward(const uint16_t* x, const int32_t* ids, const float* w, int64_t T, int H,
                    int F, int E, int k, const uint16_t* wg, const uint16_t* wu,
                    const uint16_t* wd, const uint16_t* dout, double* dx, double* dw,
                    double* dwg, double* dwu, double* dwd) {
  if (T < 0 || H < 1 || F < 1 || E < 1 || k < 1 || k > E) return ORC_ERR_ARG;
  const int64_t A = T * k;
  int rc = ORC_ERR_NOMEM;
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* row_token = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
  int32_t* row_dest = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
  int32_t* row_slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
  double* hr = (double*)malloc(sizeof(double) * (size_t)(A * F + 1));
  double* dGr = (double*)malloc(sizeof(double) * (size_t)(A * F + 1));
  double* dUr = (double*)malloc(sizeof(double) * (size_t)(A * F + 1));
  double* dyr = (double*)malloc(sizeof(double) * (size_t)(A * H + 1));
  double* dxr = (double*)malloc(sizeof(double) * (size_t)(A * H + 1));
  if (!offsets || !row_token || !row_dest || !row_slot || !hr || !dGr || !dUr || !dyr || !dxr)
    goto done;
  for (int64_t i = 0; i < A; ++i)
    if (ids[i] < 0 || ids[i] >= E) { rc = ORC_ERR_ARG; goto done; }
  rc = oracle_permute(ids, T, E, k, offsets, row_token, row_dest);
  if (rc) goto done;
  for (int64_t i = 0; i < A; ++i) row_slot[row_dest[i]] = (int32_t)(i % k);
  rc = ORC_OK;
  /* per assignment row: forward, then the row's backward */
#pragma omp parallel
  {
    double* G = (double*)malloc(sizeof(double) * (size_t)F * 2);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    double* dh = (double*)malloc(sizeof(double) * (size_t)F);
    if (!G || !y || !dh) {
#pragma omp atomic write
      rc = ORC_ERR_NOMEM;
    } else {
      double* U = G + F;
#pragma omp for schedule(static)
      for (int64_t p = 0; p < A; ++p) {
        const int64_t t = row_token[p];
        const int j = row_slot[p];
        int e = 0;
        while (offsets[e + 1] <= p) ++e;
        const uint16_t* xt = x + t * H;
        const uint16_t* wge = wg + (int64_t)e * H * F;
        const uint16_t* wue = wu + (int64_t)e * H * F;
        const uint16_t* wde = wd + (int64_t)e * F * H;
        double* h = hr + p * F;
        gateup_row(xt, H, F, wge, wue, h, G, U);
        down_row(h, F, H, wde, y);
        const double wj = (double)w[t * k + j];
        double d = 0.0;
        for (int c = 0; c < H; ++c) d += bf16_to_f64(dout[t * H + c]) * y[c];
        dw[t * k + j] = d;
        double* dy = dyr + p * H;
        for (int c = 0; c < H; ++c) dy[c] = wj * bf16_to_f64(dout[t * H + c]);
        for (int f = 0; f < F; ++f) {
          double a = 0.0;
          const uint16_t* rd = wde + (int64_t)f * H;
          for (int c = 0; c < H; ++c) a += dy[c] * bf16_to_f64(rd[c]);
          dh[f] = a;
        }
        double* dG = dGr + p * F;
        double* dU = dUr + p * F;
        for (int f = 0; f < F; ++f) {
          const double z = G[f], sg = 1.0 / (1.0 + exp(-z));
          dG[f] = dh[f] * U[f] * sg * (1.0 + z * (1.0 - sg));
          dU[f] = dh[f] * silu(z);
        }
        double* dxp = dxr + p * H;
        for (int i = 0; i < H; ++i) {
          double a = 0.0;
          const uint16_t* rg = wge + (int64_t)i * F;
          const uint16_t* ru = wue + (int64_t)i * F;
          for (int f = 0; f < F; ++f) a += dG[f] * bf16_to_f64(rg[f]) + dU[f] * bf16_to_f64(ru[f]);
          dxp[i] = a;
        }
      }
    }
    free(G); free(y); free(dh);
  }
  if (rc) goto done;
  /* dx: the k rows of each token, slots ascending */
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int i = 0; i < H; ++i) {
      double a = 0.0;
      for (int j = 0; j < k; ++j) a += dxr[(int64_t)row_dest[t * k + j] * H + i];
      dx[t * H + i] = a;
    }
  /* weight gradients: each expert's rows in ascending order */
#pragma omp parallel for schedule(dynamic)
  for (int e = 0; e < E; ++e) {
    double* gg = dwg + (int64_t)e * H * F;
    double* gu = dwu + (int64_t)e * H * F;
    double* gd = dwd + (int64_t)e * F * H;
    for (int64_t i = 0; i < (int64_t)H * F; ++i) gg[i] = 0.0, gu[i] = 0.0, gd[i] = 0.0;
    for (int64_t p = offsets[e]; p < offsets[e + 1]; ++p) {
      const uint16_t* xp = x + (int64_t)row_token[p] * H;
      const double* dG = dGr + p * F;
      const double* dU = dUr + p * F;
      const double* h = hr + p * F;
      const double* dy = dyr + p * H;
      for (int i = 0; i < H; ++i) {
        const double xv = bf16_to_f64(xp[i]);
        for (int f = 0; f < F; ++f) {
          gg[(int64_t)i * F + f] += xv * dG[f];
          gu[(int64_t)i * F + f] += xv * dU[f];
        }
      }
      for (int f = 0; f < F; ++f)
        for (int c = 0; c < H; ++c) gd[(int64_t)f * H + c] += h[f] * dy[c];
    }
  }
done:
  free(offsets); free(row_token); free(row_dest); free(row_slot);
  free(hr); free(dGr); free(dUr); free(dyr); free(dxr);
  return rc;
}

/* Backward of the shared expert (the always-on FFN of the DeepSeek-V3- and
 * Qwen2-MoE-shaped layers; the pages give no backward, so this is the chain
 * rule through the forward's shared term). With out[t] += s_t y_sh[t],
 * s_t = 1 without gate logits, else the logistic sigmoid of g_t (as
 * oracle_shared_gate), and y_sh[t] = (silu(x_t W_sg) * (x_t W_su)) W_sd:
 *   d g_t   = <dout[t], y_sh[t]> s_t (1 - s_t)        (with gate logits only)
 *   dy      = s_t dout[t]
 *   dh, dG, dU as for a routed row (oracle_backward)
 *   dx[t]   = dG W_sg^T + dU W_su^T                     (the shared part only)
 *   dW_sg = sum_t x_t^T dG_t, dW_su likewise with dU, dW_sd = sum_t h_t^T dy_t
 *   (t ascending).
 * x, weights and dout bf16, gate logits fp32, everything else fp64.
 * dx [T,H], dg [T] (written only with gate logits), dwsg, dwsu [H,Fs],
 * dwsd [Fs,H]. */
int oracle_shared_backward(const uint16_t* x, int64_t T, int H, int Fs, const uint16_t* wsg,
                           const uint16_t* wsu, const uint16_t* wsd, const float* gate_logits,
                           const uint16_t* dout, double* dx, double* dg, double* dwsg,
                           double* dwsu, double* dwsd) {
  if (T < 0 || H < 1 || Fs < 1) return ORC_ERR_ARG;
  int rc = ORC_ERR_NOMEM;
  double* s = (double*)malloc(sizeof(double) * (size_t)(T + 1));
  double* hr = (double*)malloc(sizeof(double) * (size_t)(T * Fs + 1));
  double* dGr = (double*)malloc(sizeof(double) * (size_t)(T * Fs + 1));
  double* dUr = (double*)malloc(sizeof(double) * (size_t)(T * Fs + 1));
  double* dyr = (double*)malloc(sizeof(double) * (size_t)(T * H + 1));
  if (!s || !hr || !dGr || !dUr || !dyr) goto done;
  oracle_shared_gate(gate_logits, T, s);
  rc = ORC_OK;
#pragma omp parallel
  {
    double* G = (double*)malloc(sizeof(double) * (size_t)Fs * 2);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    double* dh = (double*)malloc(sizeof(double) * (size_t)Fs);
    if (!G || !y || !dh) {
#pragma omp atomic write
      rc = ORC_ERR_NOMEM;
    } else {
      double* U = G + Fs;
#pragma omp for schedule(static)
      for (int64_t t = 0; t < T; ++t) {
        const uint16_t* xt = x + t * H;
        double* h = hr + t * Fs;
        gateup_row(xt, H, Fs, wsg, wsu, h, G, U);
        down_row(h, Fs, H, wsd, y);
        if (gate_logits) {
          double d = 0.0;
          for (int c = 0; c < H; ++c) d += bf16_to_f64(dout[t * H + c]) * y[c];
          dg[t] = d * s[t] * (1.0 - s[t]);
        }
        double* dy = dyr + t * H;
        for (int c = 0; c < H; ++c) dy[c] = s[t] * bf16_to_f64(dout[t * H + c]);
        for (int f = 0; f < Fs; ++f) {
          double a = 0.0;
          const uint16_t* rd = wsd + (int64_t)f * H;
          for (int c = 0; c < H; ++c) a += dy[c] * bf16_to_f64(rd[c]);
          dh[f] = a;
        }
        double* dG = dGr + t * Fs;
        double* dU = dUr + t * Fs;
        for (int f = 0; f < Fs; ++f) {
          const double z = G[f], sg = 1.0 / (1.0 + exp(-z));
          dG[f] = dh[f] * U[f] * sg * (1.0 + z * (1.0 - sg));
          dU[f] = dh[f] * silu(z);
        }
        for (int i = 0; i < H; ++i) {
          double a = 0.0;
          const uint16_t* rg = wsg + (int64_t)i * Fs;
          const uint16_t* ru = wsu + (int64_t)i * Fs;
          for (int f = 0; f < Fs; ++f)
            a += dG[f] * bf16_to_f64(rg[f]) + dU[f] * bf16_to_f64(ru[f]);
          dx[t * H + i] = a;
        }
      }
    }
    free(G); free(y); free(dh);
  }
  if (rc) goto done;
  /* weight gradients over the tokens in ascending order (one output row of
   * each matrix per iteration, so the rows can run in parallel) */
#pragma omp parallel for schedule(static)
  for (int i = 0; i < H; ++i) {
    double* gg = dwsg + (int64_t)i * Fs;
    double* gu = dwsu + (int64_t)i * Fs;
    for (int f = 0; f < Fs; ++f) gg[f] = 0.0, gu[f] = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      const double xv = bf16_to_f64(x[t * H + i]);
      const double* dG = dGr + t * Fs;
      const double* dU = dUr + t * Fs;
      for (int f = 0; f < Fs; ++f) {
        gg[f] += xv * dG[f];
        gu[f] += xv * dU[f];
      }
    }
  }
#pragma omp parallel for schedule(static)
  for (int f = 0; f < Fs; ++f) {
    double* gd = dwsd + (int64_t)f * H;
    for (int c = 0; c < H; ++c) gd[c] = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      const double hv = hr[t * Fs + f];
      const double* dy = dyr + t * H;
      for (int c = 0; c < H; ++c) gd[c] += hv * dy[c];
    }
  }
done:
  free(s); free(hr); free(dGr); free(dUr); free(dyr);
  return rc;
}

/* Backward of the routing weights: w = softmax over the k selected logits,
 * so dl[t, ids[t,j]] = w_j (dw_j - sum_i w_i dw_i) (i ascending) and 0 for
 * the experts not selected. dl [T,E] fp64. */
void oracle_route_backward(const int32_t* ids, const float* w, const double* dw, int64_t T,
                           int E, int k, double* dl) {
  for (int64_t t = 0; t < T; ++t) {
    double s = 0.0;
    for (int j = 0; j < k; ++j) s += (double)w[t * k + j] * dw[t * k + j];
    for (int e = 0; e < E; ++e) dl[t * E + e] = 0.0;
    for (int j = 0; j < k; ++j)
      dl[t * E + ids[t * k + j]] = (double)w[t * k + j] * (dw[t * k + j] - s);
  }
}

/* Backward for selected tokens only: dx[i] and dw[i] (the routing-weight
 * gradient) of token tokens[i]. A token's input and routing-weight
 * gradients depend on that token alone, so they equal rows tokens[i] of
 * oracle_backward's dx and dw: the same per-row arithmetic in the same
 * order (its k rows in slot order), one token at a time. */
int oracle_backward_tokens(const uint16_t* x, const int32_t* ids, const float* w, int64_t T,
                           int H, int F, int E, int k, const uint16_t* wg, const uint16_t* wu,
                           const uint16_t* wd, const uint16_t* dout, const int64_t* tokens,
                           int64_t n, double* dx, double* dw) {
  if (T < 0 || H < 1 || F < 1 || E < 1 || k < 1 || k > E) return ORC_ERR_ARG;
  for (int64_t i = 0; i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= T) return ORC_ERR_ARG;
  for (int64_t i = 0; i < n * k; ++i) {
    const int32_t e = ids[tokens[i / k] * k + i % k];
    if (e < 0 || e >= E) return ORC_ERR_ARG;
  }
  int rc = ORC_OK;
#pragma omp parallel
  {
    double* buf = (double*)malloc(sizeof(double) * ((size_t)F * 5 + (size_t)H * 3));
    if (!buf) {
#pragma omp atomic write
      rc = ORC_ERR_NOMEM;
    } else {
      double *G = buf, *U = G + F, *hrow = U + F, *dG = hrow + F, *dU = dG + F;
      double *y = dU + F, *dy = y + H, *dxp = dy + H;
#pragma omp for schedule(dynamic, 1)
      for (int64_t s = 0; s < n; ++s) {
        const int64_t t = tokens[s];
        const uint16_t* xt = x + t * H;
        for (int i = 0; i < H; ++i) dx[s * H + i] = 0.0;
        for (int j = 0; j < k; ++j) {
          const int e = ids[t * k + j];
          const uint16_t* wge = wg + (int64_t)e * H * F;
          const uint16_t* wue = wu + (int64_t)e * H * F;
          const uint16_t* wde = wd + (int64_t)e * F * H;
          gateup_row(xt, H, F, wge, wue, hrow, G, U);
          down_row(hrow, F, H, wde, y);
          const double wj = (double)w[t * k + j];
          double d = 0.0;
          for (int c = 0; c < H; ++c) d += bf16_to_f64(dout[t * H + c]) * y[c];
          dw[s * k + j] = d;
          for (int c = 0; c < H; ++c) dy[c] = wj * bf16_to_f64(dout[t * H + c]);
          for (int f = 0; f < F; ++f) {
            double a = 0.0;
            const uint16_t* rd = wde + (int64_t)f * H;
            for (int c = 0; c < H; ++c) a += dy[c] * bf16_to_f64(rd[c]);
            const double z = G[f], sg = 1.0 / (1.0 + exp(-z));
            dG[f] = a * U[f] * sg * (1.0 + z * (1.0 - sg));
            dU[f] = a * silu(z);
          }
          for (int i = 0; i < H; ++i) {
            double a = 0.0;
            const uint16_t* rg = wge + (int64_t)i * F;
            const uint16_t* ru = wue + (int64_t)i * F;
            for (int f = 0; f < F; ++f)
              a += dG[f] * bf16_to_f64(rg[f]) + dU[f] * bf16_to_f64(ru[f]);
            dxp[i] = a;
          }
          /* slots in ascending order, as oracle_backward adds them */
          for (int i = 0; i < H; ++i) dx[s * H + i] += dxp[i];
        }
      }
      free(buf);
    }
  }
  return rc;
}

/* Selected columns of the weight gradients: for each pair (ecol[i],
 * fcol[i]) = (e, f), column f of dW_gate[e] and dW_up[e] ([H] each) and row
 * f of dW_down[e] ([H]). Each is a sum over expert e's rows in ascending
 * permuted order (oracle_permute) of the same per-row quantities as in
 * oracle_backward, restricted to column f: G, U and dh at f are the same
 * dot products in the same order, so the results equal oracle_backward's
 * elements. */
int oracle_backward_wcols(const uint16_t* x, const int32_t* ids, const float* w, int64_t T,
                          int H, int F, int E, int k, const uint16_t* wg, const uint16_t* wu,
                          const uint16_t* wd, const uint16_t* dout, const int32_t* ecol,
                          const int32_t* fcol, int64_t n, double* dwg, double* dwu,
                          double* dwd) {
  if (T < 0 || H < 1 || F < 1 || E < 1 || k < 1 || k > E) return ORC_ERR_ARG;
  for (int64_t i = 0; i < n; ++i)
    if (ecol[i] < 0 || ecol[i] >= E || fcol[i] < 0 || fcol[i] >= F) return ORC_ERR_ARG;
  const int64_t A = T * k;
  for (int64_t i = 0; i < A; ++i)
    if (ids[i] < 0 || ids[i] >= E) return ORC_ERR_ARG;
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* row_token = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
  int32_t* row_dest = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
  int32_t* row_slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)(A + 1));
  int rc = ORC_ERR_NOMEM;
  if (!offsets || !row_token || !row_dest || !row_slot) goto done;
  rc = oracle_permute(ids, T, E, k, offsets, row_token, row_dest);
  if (rc) goto done;
  for (int64_t i = 0; i < A; ++i) row_slot[row_dest[i]] = (int32_t)(i % k);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t s = 0; s < n; ++s) {
    const int e = ecol[s], f = fcol[s];
    const uint16_t* wge = wg + (int64_t)e * H * F;
    const uint16_t* wue = wu + (int64_t)e * H * F;
    const uint16_t* rd = wd + ((int64_t)e * F + f) * H;
    double* gg = dwg + s * H;
    double* gu = dwu + s * H;
    double* gd = dwd + s * H;
    for (int i = 0; i < H; ++i) gg[i] = 0.0, gu[i] = 0.0, gd[i] = 0.0;
    for (int64_t p = offsets[e]; p < offsets[e + 1]; ++p) {
      const int64_t t = row_token[p];
      const uint16_t* xt = x + t * H;
      double G = 0.0, U = 0.0;
      for (int h = 0; h < H; ++h) {
        const double xv = bf16_to_f64(xt[h]);
        G += xv * bf16_to_f64(wge[(int64_t)h * F + f]);
        U += xv * bf16_to_f64(wue[(int64_t)h * F + f]);
      }
      const double wj = (double)w[t * k + row_slot[p]];
      double a = 0.0;
      for (int c = 0; c < H; ++c) a += wj * bf16_to_f64(dout[t * H + c]) * bf16_to_f64(rd[c]);
      const double sg = 1.0 / (1.0 + exp(-G));
      const double dG = a * U * sg * (1.0 + G * (1.0 - sg));
      const double dU = a * silu(G);
      const double hv = silu(G) * U;
      for (int i = 0; i < H; ++i) {
        const double xv = bf16_to_f64(xt[i]);
        gg[i] += xv * dG;
        gu[i] += xv * dU;
        gd[i] += hv * (wj * bf16_to_f64(dout[t * H + i]));
      }
    }
  }
  rc = ORC_OK;
done:
  free(offsets); free(row_token); free(row_dest); free(row_slot);
  return rc;
}

/* Output rows of selected tokens only. Every token's output depends on that
 * token alone, so out[i] for token tokens[i] equals row tokens[i] of
 * oracle_forward; it is computed here with the same per-row functions, one
 * token at a time (route that token, run its k experts, combine). */
int oracle_forward_tokens(const uint16_t* x, const float* logits, int64_t T,
                          int H, int F, int E, int k, const uint16_t* wg,
                          const uint16_t* wu, const uint16_t* wd, int Fs,
                          const uint16_t* wsg, const uint16_t* wsu,
                          const uint16_t* wsd, const float* gate_logits,
                          const int64_t* tokens, int64_t n, double* out,
                          int32_t* ids_out, double* w_out) {
  if (T < 0 || H < 1 || F < 1 || E < 1 || k < 1 || k > E || Fs < 0)
    return ORC_ERR_ARG;
  for (int64_t i = 0; i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= T) return ORC_ERR_ARG;
  int rc = ORC_OK;
#pragma omp parallel
  {
    int Fmax = F > Fs ? F : Fs;
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    int32_t* dest = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    double* w = (double*)malloc(sizeof(double) * (size_t)k);
    double* GU = (double*)malloc(sizeof(double) * (size_t)Fmax * 2);
    double* hrow = (double*)malloc(sizeof(double) * (size_t)Fmax);
    double* y = (double*)malloc(sizeof(double) * (size_t)k * H);
    double* ysh = (double*)malloc(sizeof(double) * (size_t)H);
    if (!taken || !ids || !dest || !w || !GU || !hrow || !y || !ysh) {
#pragma omp atomic write
      rc = ORC_ERR_NOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < n; ++i) {
        int64_t t = tokens[i];
        const uint16_t* xt = x + t * H;
        int r = route_one(logits + t * E, E, k, ids, w, taken);
        if (r) {
#pragma omp atomic write
          rc = r;
          continue;
        }
        for (int j = 0; j < k; ++j) {
          int64_t wo = (int64_t)ids[j] * H * F;
          gateup_row(xt, H, F, wg + wo, wu + wo, hrow, GU, GU + F);
          down_row(hrow, F, H, wd + (int64_t)ids[j] * F * H, y + (int64_t)j * H);
          dest[j] = j;
        }
        double s = 0.0;
        if (Fs > 0) {
          gateup_row(xt, H, Fs, wsg, wsu, hrow, GU, GU + Fs);
          down_row(hrow, Fs, H, wsd, ysh);
          oracle_shared_gate(gate_logits ? gate_logits + t : NULL, 1, &s);
        }
        oracle_combine(y, dest, w, 1, H, k, Fs > 0 ? ysh : NULL, &s,
                       out + i * H);
        if (ids_out) memcpy(ids_out + i * k, ids, sizeof(int32_t) * (size_t)k);
        if (w_out) memcpy(w_out + i * k, w, sizeof(double) * (size_t)k);
      }
    }
    free(taken); free(ids); free(dest); free(w); free(GU); free(hrow);
    free(y); free(ysh);
  }
  return rc;
}
