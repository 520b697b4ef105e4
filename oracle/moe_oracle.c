/*
 * CPU oracle for the frozen low-precision MoE expert forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the HIP library; it is written to be read against the method's
 * description, not to be fast.
 *
 * What it computes (Orbit announcement, "技术细节" section, the paragraph on
 * active-expert-chunked dequantization): every token activates only the
 * experts its router selects; the selected experts are grouped into
 * fixed-size batches, each batch is dequantized temporarily to high
 * precision, a grouped GEMM runs on it, and the high-precision weights are
 * released before the next batch.  Chunking only reorders when each expert is
 * dequantized, so the result is the plain dense definition:
 *
 *   ids_t   = top-k experts of logits_t (descending logit, ties -> smaller id)
 *   w_t     = softmax of the k selected logits (= full softmax renormalised)
 *   x~      = Q_A(x_t R_e)                          (R_e = OFT rotation, else I)
 *   g, u    = x~ D(W_gate,e)^T, x~ D(W_up,e)^T      (D = exact dequantizer)
 *   h       = Q_A(silu(g) * u)
 *   y_j     = h D(W_down,e)^T
 *   out_t   = sum_j w_tj y_j
 *
 * Q_A is the activation format fed to the expert GEMMs: identity for INT4
 * weights; FP8 E4M3 with an fp32 scale per [1,128] block (NeMo RL FP8 post,
 * Table 1 "Input activations"); MXFP8 (E4M3 + E8M0 per 32) for MXFP4 weights.
 * Precision: dequantized weights are fp32, dot products accumulate in fp64,
 * stored results are fp32.  Quantizer decisions are taken in fp32.
 *
 * Materialized numerics (layer flag `materialized`): the same announcement
 * paragraph read literally -- each chunk's experts are dequantized into a
 * temporary BF16 copy and an ordinary BF16 grouped GEMM runs on it.  Then
 * every dequantized weight is rounded once to bf16 (nearest, ties to even),
 * the GEMM inputs are bf16 (the token row; after the OFT rotation x R_e
 * rounded to bf16), there is no activation quantizer, and h = silu(g) * u is
 * rounded to bf16 before the down projection.  Accumulation stays fp64.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math: IEEE fp32 division
 * and rounding are relied on).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_INT4 = 1, OR_FP8 = 2, OR_MXFP4 = 3, OR_FP8_POW2 = 4, OR_NVFP4 = 5 };

/* ------------------------------------------------------------------ codecs */

/* v rounded to the nearest value with 8 significant bits (bf16), ties to
 * even, for v in bf16's normal range (or 0): v = m 2^e with 0.5 <= |m| < 1,
 * so m 2^8 is rounded to an integer in the default rounding mode. */
static double bf16_round(double v) {
  int e;
  double m;
  if (v == 0.0 || !isfinite(v)) return v;
  m = frexp(v, &e);
  return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

/* bf16 bit pattern -> float: the upper 16 bits of an IEEE binary32. */
static float bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* OCP E4M3FN: sign | 4-bit exponent (bias 7) | 3-bit mantissa.  Exponent
 * field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; there is no infinity. */
static double e4m3_value(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(8.0 + m, e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

/* OCP E2M1: sign | 2-bit exponent (bias 1) | 1-bit mantissa; exponent 0 is
 * subnormal (m * 0.5). */
static double e2m1_value(uint8_t nib) {
  int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(2.0 + m, e - 2); /* (1 + m/2) 2^(e-1) */
  return s ? -v : v;
}

/* OCP E8M0 scale: 2^(c-127); 0xFF is NaN. */
static double e8m0_value(uint8_t c) { return c == 255 ? NAN : ldexp(1.0, (int)c - 127); }

/* Two's-complement 4-bit integer. */
static int int4_value(uint8_t nib) { return (nib & 8) ? (int)(nib & 15) - 16 : (int)(nib & 15); }

/* Nibble i of a packed array: element 2j in the low nibble of byte j. */
static uint8_t nibble_at(const uint8_t* p, int64_t i) {
  uint8_t b = p[i >> 1];
  return (i & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
}

/* Nearest E4M3FN code to v, ties to the even code, magnitudes above the
 * largest finite value (448) saturate to it.  NaN -> 0x7F.  Uses the sorted
 * table of the 127 non-negative finite codes: find the two neighbours of |v|
 * by bisection and take the closer. */
static uint8_t e4m3_encode(float vf) {
  double v = (double)vf, a;
  uint8_t sign, lo, hi, mid;
  if (isnan(vf)) return 0x7F;
  sign = signbit(vf) ? 0x80 : 0;
  a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  /* codes 0x00..0x7E are increasing in value; find lo with value(lo) <= a < value(lo+1) */
  lo = 0;
  hi = 0x7E;
  while (hi - lo > 1) {
    mid = (uint8_t)((lo + hi) / 2);
    if (e4m3_value(mid) <= a) lo = mid; else hi = mid;
  }
  if (e4m3_value(hi) <= a) lo = hi;
  if (lo == 0x7E) return sign | lo;
  {
    double dl = a - e4m3_value(lo), dh = e4m3_value((uint8_t)(lo + 1)) - a;
    uint8_t c = lo;
    if (dh < dl || (dh == dl && (lo & 1))) c = (uint8_t)(lo + 1);
    return sign | c;
  }
}

/* ------------------------------------------------------ activation quantizers */

/* FP8 [1,128]: per row and per 128 consecutive elements, amax = max |v|,
 * s = amax / 448 (fp32, correctly rounded; s = 1 when amax = 0), and
 * q = E4M3(fl32(v / s)).  Dequantized value: e4m3(q) * s.
 * (NeMo RL FP8 post, Table 1: input activations FP8 E4M3, [1,128], FP32 scale.) */
static void quant_fp8_row(int K, const float* v, uint8_t* q, float* s) {
  for (int b = 0; b < K / 128; ++b) {
    float amax = 0.0f, sc;
    for (int i = 0; i < 128; ++i) {
      float a = fabsf(v[b * 128 + i]);
      if (a > amax) amax = a;
    }
    sc = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    s[b] = sc;
    for (int i = 0; i < 128; ++i) {
      volatile float r = v[b * 128 + i] / sc; /* fp32 division */
      q[b * 128 + i] = e4m3_encode(r);
    }
  }
}

/* FP8 [1,128] with power-of-two scales (NeMo RL FP8 post, recipe switches
 * for power-of-two weight and activation scaling factors): as above, but
 * the scale is the smallest power of two >= fl32(amax / 448), so no element
 * saturates and v / s is exact scaling.  s = 1 when amax = 0.  The scale is
 * kept within the E8M0 range: at least 2^-127 (an amax below 448 * 2^-127,
 * i.e. a block of bf16 subnormals, takes 2^-127). */
static float pow2_at_least(float x) {
  int e;
  const float m = frexpf(x, &e); /* x = m * 2^e, m in [0.5, 1) */
  return m == 0.5f ? x : ldexpf(1.0f, e);
}
static void quant_fp8_row_pow2(int K, const float* v, uint8_t* q, float* s) {
  for (int b = 0; b < K / 128; ++b) {
    float amax = 0.0f, sc;
    for (int i = 0; i < 128; ++i) {
      float a = fabsf(v[b * 128 + i]);
      if (a > amax) amax = a;
    }
    sc = (amax == 0.0f) ? 1.0f : pow2_at_least(amax / 448.0f);
    if (sc < ldexpf(1.0f, -127)) sc = ldexpf(1.0f, -127);
    s[b] = sc;
    for (int i = 0; i < 128; ++i) {
      volatile float r = v[b * 128 + i] / sc; /* exact: sc is a power of two */
      q[b * 128 + i] = e4m3_encode(r);
    }
  }
}

/* MXFP8: per row and per 32 consecutive elements, the shared exponent is
 * X = floor(log2(amax)) - 8 (8 = exponent of E4M3's largest power of two),
 * clamped to the E8M0 range [-127, 127]; X = 0 when amax = 0.  Elements are
 * E4M3(v * 2^-X) with saturation; the scale byte is X + 127. */
static void quant_mxfp8_row(int K, const float* v, uint8_t* q, uint8_t* e8) {
  for (int b = 0; b < K / 32; ++b) {
    float amax = 0.0f;
    int X = 0;
    for (int i = 0; i < 32; ++i) {
      float a = fabsf(v[b * 32 + i]);
      if (a > amax) amax = a;
    }
    if (amax > 0.0f) {
      int p;
      frexp((double)amax, &p); /* amax = f 2^p, f in [0.5, 1) -> floor(log2) = p - 1 */
      X = (p - 1) - 8;
      if (X < -127) X = -127;
      if (X > 127) X = 127;
    }
    e8[b] = (uint8_t)(X + 127);
    for (int i = 0; i < 32; ++i) q[b * 32 + i] = e4m3_encode((float)ldexp((double)v[b * 32 + i], -X));
  }
}

/* ---------------------------------------------------------------- routing */

typedef struct {
  float val;
  int id;
} or_key;

static int key_cmp(const void* a, const void* b) {
  const or_key *x = (const or_key*)a, *y = (const or_key*)b;
  if (x->val > y->val) return -1; /* descending value; -0 == +0 */
  if (x->val < y->val) return 1;
  return x->id - y->id; /* ties -> smaller expert id first */
}

/* Router: for every token sort all E logits (descending, ties by id), keep the
 * first k, and weight them by the softmax over those k logits (fp64, stored
 * fp32).  Same as full softmax -> top-k -> renormalise. */
int oracle_route(int T, int E, int k, const float* logits, int32_t* ids, float* w) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return 1;
#pragma omp parallel
  {
    or_key* keys = (or_key*)malloc(sizeof(or_key) * (size_t)E);
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t) {
      double z = 0.0;
      for (int e = 0; e < E; ++e) {
        keys[e].val = logits[(int64_t)t * E + e];
        keys[e].id = e;
      }
      qsort(keys, (size_t)E, sizeof(or_key), key_cmp);
      for (int j = 0; j < k; ++j) z += exp((double)keys[j].val - (double)keys[0].val);
      for (int j = 0; j < k; ++j) {
        ids[(int64_t)t * k + j] = keys[j].id;
        w[(int64_t)t * k + j] = (float)(exp((double)keys[j].val - (double)keys[0].val) / z);
      }
    }
    free(keys);
  }
  return 0;
}

/* Permutation by expert: a stable counting sort of the flat (token, slot)
 * pairs p = t*k + j by expert id.  counts[e]; offsets = exclusive scan
 * (offsets[E] = T*k); sorted_rows[row] = p; row_of[p] = row; active = experts
 * with count > 0 in ascending id. */
int oracle_permute(int T, int E, int k, const int32_t* ids, int32_t* counts, int32_t* offsets,
                   int32_t* sorted_rows, int32_t* row_of, int32_t* active, int32_t* num_active) {
  int64_t R = (int64_t)T * k;
  int32_t* fill;
  int na = 0;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < R; ++p) {
    if (ids[p] < 0 || ids[p] >= E) return 1;
    counts[ids[p]]++;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int64_t p = 0; p < R; ++p) { /* pairs visited in (t, j) order: stable */
    int e = ids[p];
    int32_t row = offsets[e] + fill[e]++;
    sorted_rows[row] = (int32_t)p;
    row_of[p] = row;
  }
  free(fill);
  for (int e = 0; e < E; ++e)
    if (counts[e] > 0) active[na++] = e;
  *num_active = na;
  return 0;
}

/* ----------------------------------------------------------- dequantizers */

/* Dequantize the N x K weight matrix of one expert to fp32 (w = q * s).
 *   INT4 : q two's-complement nibble, s bf16 per (n, 32 along K), stored
 *          group-major: s[(k/32) * N + n]
 *   FP8  : q E4M3FN, s fp32 per [128,128] block (n/128, k/128)
 *   MXFP4: q E2M1 nibble, s E8M0 per (n, 32 along K), group-major as INT4
 *   NVFP4: q E2M1 nibble, s E4M3 per (n, 16 along K), group-major
 *          s[(k/16) * N + n], times g, the matrix's fp32 second-level scale
 *          (the format's public definition; the pages only name it)
 * g is 1 for the other formats. */
static void dequant_matrix(int fmt, int N, int K, const uint8_t* q, const void* s, double g, int to_bf16,
                           float* out) {
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n) {
    for (int kk = 0; kk < K; ++kk) {
      double v;
      if (fmt == OR_INT4) {
        v = (double)int4_value(nibble_at(q, (int64_t)n * K + kk)) *
            (double)bf16_value(((const uint16_t*)s)[(int64_t)(kk / 32) * N + n]);
      } else if (fmt == OR_FP8 || fmt == OR_FP8_POW2) {
        v = e4m3_value(q[(int64_t)n * K + kk]) *
            (double)((const float*)s)[(int64_t)(n / 128) * (K / 128) + kk / 128];
      } else if (fmt == OR_NVFP4) {
        v = e2m1_value(nibble_at(q, (int64_t)n * K + kk)) *
            e4m3_value(((const uint8_t*)s)[(int64_t)(kk / 16) * N + n]) * g;
      } else {
        v = e2m1_value(nibble_at(q, (int64_t)n * K + kk)) *
            e8m0_value(((const uint8_t*)s)[(int64_t)(kk / 32) * N + n]);
      }
      out[(int64_t)n * K + kk] = (float)(to_bf16 ? bf16_round(v) : v);
    }
  }
}

/* Activation quantizer of a weight format applied to one fp32 row: returns
 * the dequantized values (exact in double).  INT4 and NVFP4 weights take the
 * activations as they are. */
static void act_quant_row(int fmt, int K, const float* v, double* out, uint8_t* qtmp, float* stmp,
                          uint8_t* etmp) {
  if (fmt == OR_FP8 || fmt == OR_FP8_POW2) {
    if (fmt == OR_FP8) quant_fp8_row(K, v, qtmp, stmp);
    else quant_fp8_row_pow2(K, v, qtmp, stmp);
    for (int i = 0; i < K; ++i) out[i] = e4m3_value(qtmp[i]) * (double)stmp[i / 128];
  } else if (fmt == OR_MXFP4) {
    quant_mxfp8_row(K, v, qtmp, etmp);
    for (int i = 0; i < K; ++i) out[i] = e4m3_value(qtmp[i]) * e8m0_value(etmp[i / 32]);
  } else {
    for (int i = 0; i < K; ++i) out[i] = (double)v[i];
  }
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

typedef struct {
  int32_t T, H, I, E, k, fmt;
  int32_t oft_block;             /* 0: no adapter; 32: block-diagonal 32x32 R */
  int64_t adapter_expert_stride; /* elements between experts' R; 0 = shared */
  int32_t materialized;          /* 1: BF16 temporary weights (see the header) */
  const float* g13;              /* NVFP4: per-expert second-level scales of W13 and W2 */
  const float* g2;
} oracle_layer;

static double gscale(const float* g, int e) { return g != NULL ? (double)g[e] : 1.0; }

/* One expert FFN row: x (bf16 token row) -> y (fp32, length H).
 * W13 = [2I][H] fp32 dequantized (gate rows then up rows), W2 = [H][I]. */
static void expert_row(const oracle_layer* L, const uint16_t* xrow, const uint16_t* R_e,
                       const float* W13, const float* W2, float* y, float* fbuf, double* dbuf,
                       uint8_t* qtmp, float* stmp, uint8_t* etmp) {
  const int H = L->H, I = L->I;
  float* xr = fbuf;        /* H: rotated input, stored fp32 */
  float* hf = fbuf + H;    /* I: SwiGLU output, stored fp32 */
  double* xq = dbuf;       /* H: quantized input values */
  double* hq = dbuf + H;   /* I: quantized SwiGLU values */
  /* 1. OFT: x' = x R_e with R_e block-diagonal (block b acts on dims 32b..32b+31) */
  if (R_e != NULL) {
    int B = L->oft_block;
    for (int b = 0; b < H / B; ++b)
      for (int j = 0; j < B; ++j) {
        double acc = 0.0;
        for (int i = 0; i < B; ++i)
          acc += (double)bf16_value(xrow[b * B + i]) * (double)bf16_value(R_e[(int64_t)b * B * B + i * B + j]);
        xr[b * B + j] = (float)(L->materialized ? bf16_round(acc) : acc);
      }
  } else {
    for (int i = 0; i < H; ++i) xr[i] = bf16_value(xrow[i]);
  }
  /* 2. input activation format (BF16 temporaries: the bf16 row as it is) */
  if (L->materialized)
    for (int i = 0; i < H; ++i) xq[i] = (double)xr[i];
  else
    act_quant_row(L->fmt, H, xr, xq, qtmp, stmp, etmp);
  /* 3. gate and up projections, SwiGLU */
  for (int n = 0; n < I; ++n) {
    double g = 0.0, u = 0.0;
    const float* wg = W13 + (int64_t)n * H;
    const float* wu = W13 + (int64_t)(I + n) * H;
    for (int kk = 0; kk < H; ++kk) {
      g += xq[kk] * (double)wg[kk];
      u += xq[kk] * (double)wu[kk];
    }
    const double hv = silu((double)(float)g) * (double)(float)u;
    hf[n] = (float)(L->materialized ? bf16_round(hv) : hv);
  }
  /* 4. down-projection input format, then the down projection */
  if (L->materialized)
    for (int i = 0; i < I; ++i) hq[i] = (double)hf[i];
  else
    act_quant_row(L->fmt, I, hf, hq, qtmp, stmp, etmp);
  for (int n = 0; n < H; ++n) {
    double acc = 0.0;
    const float* wd = W2 + (int64_t)n * I;
    for (int kk = 0; kk < I; ++kk) acc += hq[kk] * (double)wd[kk];
    y[n] = (float)acc;
  }
}

static int64_t packed_bytes(int fmt, int64_t n) { return (fmt == OR_FP8 || fmt == OR_FP8_POW2) ? n : n / 2; }
static int64_t scale_bytes(int fmt, int N, int K) {
  if (fmt == OR_INT4) return (int64_t)N * (K / 32) * 2;
  if (fmt == OR_NVFP4) return (int64_t)N * (K / 16);
  if (fmt == OR_FP8 || fmt == OR_FP8_POW2) return (int64_t)(N / 128) * (K / 128) * 4;
  return (int64_t)N * (K / 32);
}

/* Full forward.  Tokens to output: `tokens[0..n_tokens)` (NULL: all tokens,
 * in order).  out: [n_tokens][H] fp32.  y_out (optional): [n_tokens][k][H] fp32,
 * each selected expert's output before weighting.  topk_ids/topk_w (optional):
 * [T][k] routing of every token.
 * Steps: route all tokens; permute; walk the active experts chunk by chunk
 * (chunk_experts per chunk); dequantize the chunk's experts to fp32, compute
 * the rows of those experts that belong to the requested tokens, release the
 * chunk; finally combine each token's k expert outputs with its weights. */
int oracle_forward(const oracle_layer* L, const uint16_t* x, const float* logits, const uint8_t* w13,
                   const uint8_t* w2, const void* s13, const void* s2, const uint16_t* oft,
                   int chunk_experts, const int32_t* tokens, int n_tokens, float* out, float* y_out,
                   int32_t* topk_ids_out, float* topk_w_out) {
  const int T = L->T, H = L->H, I = L->I, E = L->E, k = L->k, fmt = L->fmt;
  const int64_t R = (int64_t)T * k;
  int32_t *ids, *counts, *offsets, *sorted_rows, *row_of, *active, *slot, num_active = 0;
  float *wts, *ybuf;
  int rc = 0;
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || k > E || chunk_experts < 1) return 1;
  if (H % 32 || I % 32 || ((fmt == OR_FP8 || fmt == OR_FP8_POW2) && (H % 128 || I % 128))) return 1;
  if (oft != NULL && (L->oft_block != 32 || H % 32)) return 1;
  if (tokens == NULL) n_tokens = T;
  if (T == 0 || n_tokens == 0) return 0;

  ids = (int32_t*)malloc(sizeof(int32_t) * R);
  wts = (float*)malloc(sizeof(float) * R);
  counts = (int32_t*)malloc(sizeof(int32_t) * E);
  offsets = (int32_t*)malloc(sizeof(int32_t) * (E + 1));
  sorted_rows = (int32_t*)malloc(sizeof(int32_t) * R);
  row_of = (int32_t*)malloc(sizeof(int32_t) * R);
  active = (int32_t*)malloc(sizeof(int32_t) * E);
  slot = (int32_t*)malloc(sizeof(int32_t) * T);
  ybuf = (float*)malloc(sizeof(float) * (size_t)n_tokens * k * H);

  oracle_route(T, E, k, logits, ids, wts);
  oracle_permute(T, E, k, ids, counts, offsets, sorted_rows, row_of, active, &num_active);
  if (topk_ids_out) memcpy(topk_ids_out, ids, sizeof(int32_t) * R);
  if (topk_w_out) memcpy(topk_w_out, wts, sizeof(float) * R);
  for (int t = 0; t < T; ++t) slot[t] = -1;
  for (int i = 0; i < n_tokens; ++i) {
    int t = tokens ? tokens[i] : i;
    if (t < 0 || t >= T) { rc = 1; goto done; }
    slot[t] = i;
  }

  for (int c0 = 0; c0 < num_active; c0 += chunk_experts) {
    int nc = num_active - c0 < chunk_experts ? num_active - c0 : chunk_experts;
    float** W13c = (float**)calloc((size_t)nc, sizeof(float*));
    float** W2c = (float**)calloc((size_t)nc, sizeof(float*));
    int64_t nrows = 0;
    int64_t* rows;
    /* temporary high-precision weights of this chunk's experts (only experts
     * that own a requested row are touched) */
    for (int a = 0; a < nc; ++a) {
      int e = active[c0 + a], need = 0;
      for (int32_t r = offsets[e]; r < offsets[e + 1] && !need; ++r) need = slot[sorted_rows[r] / k] >= 0;
      if (!need) continue;
      W13c[a] = (float*)malloc(sizeof(float) * (size_t)2 * I * H);
      W2c[a] = (float*)malloc(sizeof(float) * (size_t)H * I);
      dequant_matrix(fmt, 2 * I, H, w13 + packed_bytes(fmt, (int64_t)e * 2 * I * H),
                     (const uint8_t*)s13 + (int64_t)e * scale_bytes(fmt, 2 * I, H), gscale(L->g13, e),
                     L->materialized, W13c[a]);
      dequant_matrix(fmt, H, I, w2 + packed_bytes(fmt, (int64_t)e * H * I),
                     (const uint8_t*)s2 + (int64_t)e * scale_bytes(fmt, H, I), gscale(L->g2, e),
                     L->materialized, W2c[a]);
    }
    /* the chunk's grouped GEMM, row by row */
    rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(offsets[active[c0 + nc - 1] + 1] - offsets[active[c0]] + 1));
    for (int a = 0; a < nc; ++a) {
      int e = active[c0 + a];
      for (int32_t r = offsets[e]; r < offsets[e + 1]; ++r)
        if (slot[sorted_rows[r] / k] >= 0) rows[nrows++] = ((int64_t)a << 32) | (uint32_t)r;
    }
#pragma omp parallel
    {
      float* fbuf = (float*)malloc(sizeof(float) * (size_t)(H + I));
      double* dbuf = (double*)malloc(sizeof(double) * (size_t)(H + I));
      uint8_t* qtmp = (uint8_t*)malloc((size_t)(H > I ? H : I));
      float* stmp = (float*)malloc(sizeof(float) * (size_t)((H > I ? H : I) / 32 + 1));
      uint8_t* etmp = (uint8_t*)malloc((size_t)((H > I ? H : I) / 32 + 1));
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < nrows; ++i) {
        int a = (int)(rows[i] >> 32);
        int32_t r = (int32_t)(rows[i] & 0xffffffff);
        int e = active[c0 + a];
        int32_t p = sorted_rows[r];
        int t = p / k, j = p % k;
        const uint16_t* R_e = oft ? oft + (int64_t)e * L->adapter_expert_stride : NULL;
        expert_row(L, x + (int64_t)t * H, R_e, W13c[a], W2c[a], ybuf + ((int64_t)slot[t] * k + j) * H, fbuf, dbuf,
                   qtmp, stmp, etmp);
      }
      free(fbuf); free(dbuf); free(qtmp); free(stmp); free(etmp);
    }
    free(rows);
    for (int a = 0; a < nc; ++a) { free(W13c[a]); free(W2c[a]); } /* release */
    free(W13c); free(W2c);
  }

  /* combine: out_t = sum_j w_tj y_tj, slots in ascending j */
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n_tokens; ++i) {
    int t = tokens ? tokens[i] : i;
    for (int n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) acc += (double)wts[(int64_t)t * k + j] * (double)ybuf[((int64_t)i * k + j) * H + n];
      out[(int64_t)i * H + n] = (float)acc;
    }
  }
  if (y_out) memcpy(y_out, ybuf, sizeof(float) * (size_t)n_tokens * k * H);
done:
  free(ids); free(wts); free(counts); free(offsets); free(sorted_rows); free(row_of); free(active);
  free(slot); free(ybuf);
  return rc;
}

/* ---------------------------------------------------------------- backward
 *
 * Frozen-base backward (Orbit announcement, 技术细节: the GEMM backward that
 * bypasses the base weight gradient, so nothing is computed for the frozen
 * base; Orbit analysis page, 机制拆解: the base takes part in the forward but
 * carries no backward update, the adapter's parameters get the gradients).
 * Given dL/dout, it returns dL/dx, dL/dlogits and, with an adapter, dL/dR;
 * no gradient for W13 or W2.  The forward is the oracle's own (exactly
 * dequantized weights; activation quantizers of the FP8 / MXFP4 formats are
 * passed straight through in the backward).  All arithmetic in fp64.
 *
 *   per selected (t, j), expert e = ids_tj, w = w_tj:
 *     x' = x_t R_e;  a = Q(x') Wg^T;  b = Q(x') Wu^T;  h = silu(a) b
 *     u  = dout_t W2                 (the gradient reaching Q(h), before w)
 *     g_tj = <u, Q(h)> = <dout_t, y_tj>
 *     dh = w u;  da = dh b silu'(a);  db = dh silu(a)
 *     dx' = da Wg + db Wu
 *     dR_e += x_t^T dx'  on each 32x32 diagonal block
 *     dx_tj = dx' R_e^T
 *   dx_t = sum_j dx_tj
 *   dlogits[t][ids_tj] = w_tj (g_tj - sum_i w_ti g_ti)  (softmax over the k
 *   selected logits); 0 for experts not selected.
 *
 * silu'(a) = s (1 + a (1 - s)) with s = 1 / (1 + e^-a). */
static void expert_row_backward(const oracle_layer* L, const uint16_t* xrow, const uint16_t* R_e, const float* W13,
                                const float* W2, const float* dout, double w, double* dx, double* dR_e, double* g,
                                double* buf, uint8_t* qtmp, float* stmp, uint8_t* etmp) {
  const int H = L->H, I = L->I;
  float* xr = (float*)buf;                 /* H floats (in the first H/2 doubles) */
  double* xq = buf + H;                    /* H */
  double* a = xq + H;                      /* I */
  double* b = a + I;                       /* I */
  double* hq = b + I;                      /* I */
  double* u = hq + I;                      /* I */
  double* dxr = u + I;                     /* H: dL/dx' */
  float* hf = (float*)(dxr + H);           /* I floats */
  int B = L->oft_block;
  /* forward of this row, as the oracle's forward computes it */
  if (R_e != NULL) {
    for (int bb = 0; bb < H / B; ++bb)
      for (int j = 0; j < B; ++j) {
        double acc = 0.0;
        for (int i = 0; i < B; ++i)
          acc += (double)bf16_value(xrow[bb * B + i]) * (double)bf16_value(R_e[(int64_t)bb * B * B + i * B + j]);
        xr[bb * B + j] = (float)acc;
      }
  } else {
    for (int i = 0; i < H; ++i) xr[i] = bf16_value(xrow[i]);
  }
  act_quant_row(L->fmt, H, xr, xq, qtmp, stmp, etmp);
  for (int n = 0; n < I; ++n) {
    double ga = 0.0, ub = 0.0;
    const float* wg = W13 + (int64_t)n * H;
    const float* wu = W13 + (int64_t)(I + n) * H;
    for (int kk = 0; kk < H; ++kk) {
      ga += xq[kk] * (double)wg[kk];
      ub += xq[kk] * (double)wu[kk];
    }
    a[n] = ga;
    b[n] = ub;
    hf[n] = (float)(silu((double)(float)ga) * (double)(float)ub);
  }
  act_quant_row(L->fmt, I, hf, hq, qtmp, stmp, etmp);
  /* u = dout W2 (W2 is [H][I]) and g = <u, Q(h)> */
  for (int i = 0; i < I; ++i) u[i] = 0.0;
  for (int n = 0; n < H; ++n) {
    const double d = (double)dout[n];
    const float* wd = W2 + (int64_t)n * I;
    for (int i = 0; i < I; ++i) u[i] += d * (double)wd[i];
  }
  double gg = 0.0;
  for (int i = 0; i < I; ++i) gg += u[i] * hq[i];
  *g = gg;
  /* SwiGLU backward, then dx' = da Wg + db Wu */
  for (int kk = 0; kk < H; ++kk) dxr[kk] = 0.0;
  for (int n = 0; n < I; ++n) {
    const double sg = 1.0 / (1.0 + exp(-a[n]));
    const double dh = w * u[n];
    const double da = dh * b[n] * sg * (1.0 + a[n] * (1.0 - sg));
    const double db = dh * a[n] * sg;
    const float* wg = W13 + (int64_t)n * H;
    const float* wu = W13 + (int64_t)(I + n) * H;
    for (int kk = 0; kk < H; ++kk) dxr[kk] += da * (double)wg[kk] + db * (double)wu[kk];
  }
  /* adapter: dR_e += x^T dx' per diagonal block; dx = dx' R_e^T */
  if (R_e != NULL) {
    for (int bb = 0; bb < H / B; ++bb)
      for (int i = 0; i < B; ++i) {
        const double xi = (double)bf16_value(xrow[bb * B + i]);
        double acc = 0.0;
        for (int j = 0; j < B; ++j) {
          dR_e[(int64_t)bb * B * B + i * B + j] += xi * dxr[bb * B + j];
          acc += dxr[bb * B + j] * (double)bf16_value(R_e[(int64_t)bb * B * B + i * B + j]);
        }
        dx[bb * B + i] = acc;
      }
  } else {
    for (int kk = 0; kk < H; ++kk) dx[kk] = dxr[kk];
  }
}

/* dout: [n_tokens][H] fp32 (rows of the requested tokens, in request order).
 * Outputs for the requested tokens: dx [n][H] fp32, dlogits [n][E] fp32;
 * doft (optional, with an adapter): fp64, shaped like the adapter (per-expert
 * blocks at adapter_expert_stride, or one shared block set), accumulated over
 * the rows of the requested tokens only (zeroed first); g (optional): [n][k]
 * fp64, g_tj = <dout_t, y_tj> per selected slot. */
int oracle_backward(const oracle_layer* L, const uint16_t* x, const float* logits, const uint8_t* w13,
                    const uint8_t* w2, const void* s13, const void* s2, const uint16_t* oft, const float* dout,
                    int chunk_experts, const int32_t* tokens, int n_tokens, float* dx_out, float* dlogits_out,
                    double* doft_out, double* g_out) {
  const int T = L->T, H = L->H, I = L->I, E = L->E, k = L->k, fmt = L->fmt;
  const int64_t R = (int64_t)T * k;
  int32_t *ids, *counts, *offsets, *sorted_rows, *row_of, *active, *slot, num_active = 0;
  float* wts;
  double *dxbuf, *gbuf;
  int rc = 0;
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || k > E || chunk_experts < 1 || L->materialized) return 1;
  if (H % 32 || I % 32 || ((fmt == OR_FP8 || fmt == OR_FP8_POW2) && (H % 128 || I % 128))) return 1;
  if (oft != NULL && (L->oft_block != 32 || H % 32)) return 1;
  if (tokens == NULL) n_tokens = T;
  if (T == 0 || n_tokens == 0) return 0;
  const int64_t n_oft = oft ? (L->adapter_expert_stride ? (int64_t)E * L->adapter_expert_stride : (int64_t)H * 32) : 0;
  if (doft_out && oft) memset(doft_out, 0, sizeof(double) * (size_t)n_oft);

  ids = (int32_t*)malloc(sizeof(int32_t) * R);
  wts = (float*)malloc(sizeof(float) * R);
  counts = (int32_t*)malloc(sizeof(int32_t) * E);
  offsets = (int32_t*)malloc(sizeof(int32_t) * (E + 1));
  sorted_rows = (int32_t*)malloc(sizeof(int32_t) * R);
  row_of = (int32_t*)malloc(sizeof(int32_t) * R);
  active = (int32_t*)malloc(sizeof(int32_t) * E);
  slot = (int32_t*)malloc(sizeof(int32_t) * T);
  dxbuf = (double*)malloc(sizeof(double) * (size_t)n_tokens * k * H);
  gbuf = (double*)malloc(sizeof(double) * (size_t)n_tokens * k);

  oracle_route(T, E, k, logits, ids, wts);
  oracle_permute(T, E, k, ids, counts, offsets, sorted_rows, row_of, active, &num_active);
  for (int t = 0; t < T; ++t) slot[t] = -1;
  for (int i = 0; i < n_tokens; ++i) {
    int t = tokens ? tokens[i] : i;
    if (t < 0 || t >= T) { rc = 1; goto done; }
    slot[t] = i;
  }

  for (int c0 = 0; c0 < num_active; c0 += chunk_experts) {
    int nc = num_active - c0 < chunk_experts ? num_active - c0 : chunk_experts;
    for (int a = 0; a < nc; ++a) {
      int e = active[c0 + a], need = 0;
      for (int32_t r = offsets[e]; r < offsets[e + 1] && !need; ++r) need = slot[sorted_rows[r] / k] >= 0;
      if (!need) continue;
      float* W13 = (float*)malloc(sizeof(float) * (size_t)2 * I * H);
      float* W2 = (float*)malloc(sizeof(float) * (size_t)H * I);
      dequant_matrix(fmt, 2 * I, H, w13 + packed_bytes(fmt, (int64_t)e * 2 * I * H),
                     (const uint8_t*)s13 + (int64_t)e * scale_bytes(fmt, 2 * I, H), gscale(L->g13, e), 0, W13);
      dequant_matrix(fmt, H, I, w2 + packed_bytes(fmt, (int64_t)e * H * I),
                     (const uint8_t*)s2 + (int64_t)e * scale_bytes(fmt, H, I), gscale(L->g2, e), 0, W2);
      const uint16_t* R_e = oft ? oft + (int64_t)e * L->adapter_expert_stride : NULL;
      double* dR_e = (oft && doft_out) ? doft_out + (int64_t)e * L->adapter_expert_stride : NULL;
      const int32_t r0 = offsets[e], r1 = offsets[e + 1];
#pragma omp parallel
      {
        double* buf = (double*)malloc(sizeof(double) * (size_t)(4 * H + 5 * I));
        double* dRl = R_e ? (double*)calloc((size_t)H * 32, sizeof(double)) : NULL;
        uint8_t* qtmp = (uint8_t*)malloc((size_t)(H > I ? H : I));
        float* stmp = (float*)malloc(sizeof(float) * (size_t)((H > I ? H : I) / 32 + 1));
        uint8_t* etmp = (uint8_t*)malloc((size_t)((H > I ? H : I) / 32 + 1));
#pragma omp for schedule(dynamic, 1)
        for (int32_t r = r0; r < r1; ++r) {
          int32_t p = sorted_rows[r];
          int t = p / k, j = p % k;
          if (slot[t] < 0) continue;
          const int64_t q = (int64_t)slot[t] * k + j;
          expert_row_backward(L, x + (int64_t)t * H, R_e, W13, W2, dout + (int64_t)slot[t] * H, (double)wts[p],
                              dxbuf + q * H, dRl, gbuf + q, buf, qtmp, stmp, etmp);
        }
        if (dRl && dR_e) {
#pragma omp critical
          for (int64_t i = 0; i < (int64_t)H * 32; ++i) dR_e[i] += dRl[i];
        }
        free(buf); free(dRl); free(qtmp); free(stmp); free(etmp);
      }
      free(W13); free(W2); /* release */
    }
  }

  for (int i = 0; i < n_tokens; ++i) {
    int t = tokens ? tokens[i] : i;
    for (int n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) acc += dxbuf[((int64_t)i * k + j) * H + n];
      dx_out[(int64_t)i * H + n] = (float)acc;
    }
    double mean = 0.0;
    for (int j = 0; j < k; ++j) mean += (double)wts[(int64_t)t * k + j] * gbuf[(int64_t)i * k + j];
    for (int e = 0; e < E; ++e) dlogits_out[(int64_t)i * E + e] = 0.0f;
    if (g_out)
      for (int j = 0; j < k; ++j) g_out[(int64_t)i * k + j] = gbuf[(int64_t)i * k + j];
    for (int j = 0; j < k; ++j)
      dlogits_out[(int64_t)i * E + ids[(int64_t)t * k + j]] =
          (float)((double)wts[(int64_t)t * k + j] * (gbuf[(int64_t)i * k + j] - mean));
  }
done:
  free(ids); free(wts); free(counts); free(offsets); free(sorted_rows); free(row_of); free(active);
  free(slot); free(dxbuf); free(gbuf);
  return rc;
}

/* Combine on its own: out[t] = sum_j w[t][j] * y_perm[row_of[t*k+j]], with
 * y_perm given as bf16 rows; fp64 sum, fp32 result. */
int oracle_combine(int T, int k, int H, const uint16_t* y_perm, const float* w, const int32_t* row_of, float* out) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t)
    for (int n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j)
        acc += (double)w[(int64_t)t * k + j] * (double)bf16_value(y_perm[(int64_t)row_of[(int64_t)t * k + j] * H + n]);
      out[(int64_t)t * H + n] = (float)acc;
    }
  return 0;
}

/* LM head log-prob of a target token (a final parameter-free RMSNorm, then
 * logits = z W_lm^T, then log-softmax at the target):
 *   z = h / sqrt(mean(h^2) + 1e-6);  lp_t = logit_t[y_t] - logsumexp_v logit_t[v]
 * fp64 throughout, fp32 result.  W_lm is [V][H] bf16. */
int oracle_lm_head_logprob(int T, int H, int V, const float* h, const uint16_t* wlm, const int32_t* targets,
                           float* lp) {
  double* logit = (double*)malloc(sizeof(double) * (size_t)V);
  double* z = (double*)malloc(sizeof(double) * (size_t)H);
  for (int t = 0; t < T; ++t) {
    double ms = 0.0, mx = -INFINITY, se = 0.0;
    for (int i = 0; i < H; ++i) ms += (double)h[(int64_t)t * H + i] * (double)h[(int64_t)t * H + i];
    ms = 1.0 / sqrt(ms / H + 1e-6);
    for (int i = 0; i < H; ++i) z[i] = (double)h[(int64_t)t * H + i] * ms;
#pragma omp parallel for schedule(static)
    for (int v = 0; v < V; ++v) {
      double acc = 0.0;
      for (int i = 0; i < H; ++i) acc += z[i] * (double)bf16_value(wlm[(int64_t)v * H + i]);
      logit[v] = acc;
    }
    for (int v = 0; v < V; ++v) if (logit[v] > mx) mx = logit[v];
    for (int v = 0; v < V; ++v) se += exp(logit[v] - mx);
    if (targets[t] < 0 || targets[t] >= V) { free(logit); free(z); return 1; }
    lp[t] = (float)(logit[targets[t]] - (mx + log(se)));
  }
  free(logit); free(z);
  return 0;
}

/* ------------------------------------------------- exported codec helpers */

/* Decode n codes of a format into doubles: fmt 0 = bf16 (uint16 input),
 * 1 = int4 nibble, 2 = E4M3FN, 3 = E2M1 nibble, 4 = E8M0 (uint8 input). */
void oracle_decode(int fmt, int64_t n, const void* codes, double* out) {
  for (int64_t i = 0; i < n; ++i) {
    if (fmt == 0) out[i] = bf16_value(((const uint16_t*)codes)[i]);
    else {
      uint8_t c = ((const uint8_t*)codes)[i];
      out[i] = fmt == 1 ? int4_value(c) : fmt == 2 ? e4m3_value(c) : fmt == 3 ? e2m1_value(c) : e8m0_value(c);
    }
  }
}

void oracle_encode_e4m3(int64_t n, const float* v, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(v[i]);
}

/* Row-wise activation quantizers on an [R][K] fp32 array. */
void oracle_quant_fp8(int R, int K, const float* v, uint8_t* q, float* s) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < R; ++r) quant_fp8_row(K, v + (int64_t)r * K, q + (int64_t)r * K, s + (int64_t)r * (K / 128));
}
void oracle_quant_fp8_pow2(int R, int K, const float* v, uint8_t* q, float* s) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < R; ++r)
    quant_fp8_row_pow2(K, v + (int64_t)r * K, q + (int64_t)r * K, s + (int64_t)r * (K / 128));
}
void oracle_quant_mxfp8(int R, int K, const float* v, uint8_t* q, uint8_t* e8) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < R; ++r) quant_mxfp8_row(K, v + (int64_t)r * K, q + (int64_t)r * K, e8 + (int64_t)r * (K / 32));
}

/* One expert's N x K weights dequantized to fp32 (format codes as above). */
void oracle_dequant(int fmt, int N, int K, const uint8_t* q, const void* s, double g, float* out) {
  dequant_matrix(fmt, N, K, q, s, g, 0, out);
}

/* One expert's weights as the BF16 temporary copy holds them. */
void oracle_dequant_bf16(int fmt, int N, int K, const uint8_t* q, const void* s, double g, float* out) {
  dequant_matrix(fmt, N, K, q, s, g, 1, out);
}

void oracle_round_bf16(int64_t n, const double* v, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(v[i]);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
