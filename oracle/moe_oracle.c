/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU oracle of the fused
 * Mixture-of-Experts forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The GPU product
 * path neither links nor calls it, and this file shares no code, header or
 * table with the GPU path.
 *
 * What it computes, and where the pages say so (pages cited by title):
 *  - "flashinfer.fused_moe.cute_dsl_fused_moe" (FlashInfer API reference),
 *    Parameters x / x_sf / w1_alpha / w2_alpha / fc2_input_scale /
 *    num_local_experts / local_expert_offset / use_fused_finalize /
 *    swiglu_alpha, swiglu_beta, swiglu_limit, activation_type, situ_beta,
 *    situ_linear_beta and the signature's defaults: the three quantisation
 *    modes, the per-expert fp32 scales, the local expert share, the SwiGLU
 *    parameters and the gated GeGLU-tanh / SiTU activations.
 *  - "flashinfer.fused_moe.alphamoe_nvfp4_routed_moe", summary and
 *    Parameters: packed E2M1 with linear E4M3 block-16 scales, route-order
 *    finalize seeded from the existing output, `accumulate`,
 *    `routed_scaling_factor`.
 *  - "vllm.models.flint.ops.moe_cute", module docstring and grouped_moe: the
 *    weights decoded exactly (E2M1 x E4M3), fp32 accumulation, the
 *    per-expert scale applied to the accumulator, gate/up kept in fp32 and
 *    silu(g)*u rounded once to bf16; the routing plan (tile tables,
 *    expanded<->permuted maps), GEMM1, GEMM2 writing unweighted bf16 rows in
 *    permuted order and the caller-side weighted top-k reduction.
 *  - "feat(moe): MXFP8 x MXFP4 CuTe-DSL fused MoE for SM100, plus large-batch
 *    routing locality" (FlashInfer pull request 4440), description: MXFP8
 *    (E4M3 + block-32 E8M0) activations, MXFP4 (E2M1 + block-32 E8M0)
 *    weights, an MXFP8 FC1 intermediate, a bf16 output.
 * The number formats are the ones the OCP Microscaling Formats v1.0 and OCP
 * 8-bit floating point specifications define; the pages name them only.
 *
 * Precision.  Dot products are summed in fp64 in index order.  Every product
 * of two decoded 4/8-bit values is exact in fp64.  Where the pages state an
 * fp32 step (the per-expert scale on the fp32 accumulator, the finalize
 * accumulator) it is taken in fp32.  Quantisation decisions (scale and
 * element codes) are taken in fp32: the pages give every global scale as an
 * fp32 tensor (w1_alpha, w2_alpha, fc2_input_scale of
 * "flashinfer.fused_moe.cute_dsl_fused_moe", Parameters), so a block scale
 * blockamax / (6 * scale) and an element quotient v / (block scale * scale)
 * are fp32 expressions of fp32 operands, and the OCP conversions (round to
 * nearest even, saturation) are defined on that fp32 value.
 * Readings of passages the pages leave open are listed where they are used.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_W4A16 = 0, ORC_W4A4 = 1, ORC_MXFP8_MXFP4 = 2 };
enum { ORC_ELEM_E4M3 = 0, ORC_ELEM_E2M1 = 1 };
enum { ORC_ACT_SWIGLU = 0, ORC_ACT_GEGLU_TANH = 1, ORC_ACT_RELU2 = 2 };

/* ------------------------------------------------------------------------ */
/* Number formats (OCP MX v1.0 / OCP FP8, as named by the pages)            */
/* ------------------------------------------------------------------------ */

/* E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN. */
double orc_e2m1_value(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* E4M3 ("fn"): bias 7, subnormals m/8 * 2^-6, S.1111.111 is NaN, no inf. */
double orc_e4m3_value(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* E8M0: 2^(code - 127); code 255 is NaN. */
double orc_e8m0_value(int code) {
  code &= 255;
  if (code == 255) return NAN;
  return ldexp(1.0, code - 127);
}

float orc_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round an exact value to bf16, nearest-even, once.  bf16 keeps 8
 * significant bits; its subnormal quantum is 2^-133. */
uint16_t orc_bf16_round(double v) {
  if (isnan(v)) return 0x7fc0;
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  uint32_t bits = 0;
  if (a != 0.0) {
    int e;
    frexp(a, &e);
    int ex = e - 1; /* floor(log2 a) */
    if (ex < -126) ex = -126;
    double quantum = ldexp(1.0, ex - 7);
    double r = nearbyint(a / quantum) * quantum; /* exact; may reach 2^(ex+1) */
    float rf = (float)r;                          /* exact, or inf past the top */
    memcpy(&bits, &rf, 4);
    bits >>= 16;
  }
  return (uint16_t)(bits | (neg ? 0x8000u : 0u));
}

/* fp32 -> E4M3, nearest-even, saturating to +-448 (reading: "satfinite";
 * the sign of a zero result follows the input). NaN -> 0x7f. */
int orc_e4m3_encode(float v) {
  if (isnan(v)) return 0x7f;
  int s = signbit(v) ? 0x80 : 0;
  double a = fabs((double)v);
  if (a >= 448.0) return s | 0x7e;
  int code;
  if (a < 0x1p-6) {
    code = (int)nearbyint(a / 0x1p-9); /* subnormal grid; 8 lands on 2^-6 */
  } else {
    int e;
    frexp(a, &e);
    int ex = e - 1;
    int q = (int)nearbyint(a / ldexp(1.0, ex - 3)); /* 8..16 */
    code = (ex + 6) * 8 + q;                         /* q == 16 carries */
  }
  if (code > 0x7e) code = 0x7e;
  return s | code;
}

/* fp32 -> E2M1, nearest-even, saturating to +-6; the sign of a zero result
 * follows the input.  NaN -> +6 (never produced by valid inputs). */
int orc_e2m1_encode(float v) {
  if (isnan(v)) return 7;
  int s = signbit(v) ? 8 : 0;
  double a = fabs((double)v);
  if (a >= 6.0) return s | 7;
  int code;
  if (a < 1.0) {
    code = (int)nearbyint(a / 0.5); /* 0, 0.5, 1.0 */
  } else {
    int e;
    frexp(a, &e);
    int ex = e - 1;                                   /* 0..2 */
    int q = (int)nearbyint(a / ldexp(1.0, ex - 1));   /* 2..4 */
    code = 2 * ex + q;
  }
  if (code > 7) code = 7;
  return s | code;
}

void orc_bf16_round_array(const double* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_bf16_round(v[i]);
}
void orc_e4m3_encode_array(const float* v, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)orc_e4m3_encode(v[i]);
}
void orc_e2m1_encode_array(const float* v, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)orc_e2m1_encode(v[i]);
}

static inline int nibble(const uint8_t* q, int64_t i) {
  return (i & 1) ? (q[i >> 1] >> 4) & 15 : q[i >> 1] & 15;
}
static inline void set_nibble(uint8_t* q, int64_t i, int c) {
  if (i & 1) q[i >> 1] = (uint8_t)((q[i >> 1] & 0x0f) | (c << 4));
  else q[i >> 1] = (uint8_t)((q[i >> 1] & 0xf0) | (c & 15));
}

/* ------------------------------------------------------------------------ */
/* Quantisers                                                                */
/* ------------------------------------------------------------------------ */

/* Per-tensor NVFP4 global scale: amax / (6 * 448), so that the largest
 * block scale lands on E4M3's largest value (reading of the pages' "global
 * scale"; the workload recipe states this formula). */
float orc_nvfp4_global_scale(float amax) { return amax / 2688.0f; }

/* NVFP4 quantisation of rows x cols (cols % 16 == 0), blocks of 16 along a
 * row.  Block scale code s = E4M3(blockamax / (6 * gscale)); element code
 * q = E2M1(v / (decode(s) * gscale)), all decided in fp32.  A block whose
 * decoded scale times gscale is 0 gets all-zero codes.  Packed output: two
 * codes per byte, element 2i in the low nibble. */
void orc_nvfp4_quantize(const float* v, int64_t rows, int64_t cols, int64_t ld,
                        float gscale, uint8_t* q, uint8_t* sf) {
  int64_t nb = cols / 16;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    const float* row = v + r * ld;
    for (int64_t b = 0; b < nb; b++) {
      float bamax = 0.0f;
      for (int i = 0; i < 16; i++) {
        float a = fabsf(row[b * 16 + i]);
        if (a > bamax) bamax = a;
      }
      int scode = 0;
      if (gscale > 0.0f && bamax > 0.0f) {
        float t = 6.0f * gscale;
        float s = bamax / t;
        scode = orc_e4m3_encode(s);
      }
      sf[r * nb + b] = (uint8_t)scode;
      float denom = (float)orc_e4m3_value(scode) * gscale;
      for (int i = 0; i < 16; i++) {
        int64_t col = b * 16 + i;
        int c = 0;
        if (denom > 0.0f) c = orc_e2m1_encode(row[col] / denom);
        set_nibble(q + r * (cols / 2), col, c);
      }
    }
  }
}

/* MX quantisation (OCP MX v1.0 rule) of rows x cols, blocks of 32 along a
 * row: shared exponent floor(log2 blockamax) - emax (emax 8 for E4M3, 2 for
 * E2M1), stored as E8M0 code clamp(that + 127, 0, 254); a zero block gets
 * code 0.  Elements are v / 2^(code-127), rounded nearest-even and
 * saturated.  E4M3 output is one byte per element, E2M1 is packed. */
void orc_mx_quantize(const float* v, int64_t rows, int64_t cols, int64_t ld,
                     int elem, uint8_t* q, uint8_t* sf) {
  int64_t nb = cols / 32;
  int emax = (elem == ORC_ELEM_E4M3) ? 8 : 2;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    const float* row = v + r * ld;
    for (int64_t b = 0; b < nb; b++) {
      float amax = 0.0f;
      for (int i = 0; i < 32; i++) {
        float a = fabsf(row[b * 32 + i]);
        if (a > amax) amax = a;
      }
      int code = 0;
      if (amax > 0.0f && isfinite(amax)) {
        int e;
        frexpf(amax, &e);
        code = (e - 1) - emax + 127;
        if (code < 0) code = 0;
        if (code > 254) code = 254;
      }
      sf[r * nb + b] = (uint8_t)code;
      double X = ldexp(1.0, code - 127);
      for (int i = 0; i < 32; i++) {
        int64_t col = b * 32 + i;
        float s = (float)((double)row[col] / X); /* exact: X is a power of two */
        if (elem == ORC_ELEM_E4M3) q[r * cols + col] = (uint8_t)orc_e4m3_encode(s);
        else set_nibble(q + r * (cols / 2), col, orc_e2m1_encode(s));
      }
    }
  }
}

/* bf16 -> fp32 helper for quantising bf16 tensors. */
static float* bf16_rows_to_f32(const uint16_t* v, int64_t n) {
  float* f = (float*)malloc((size_t)n * sizeof(float));
  for (int64_t i = 0; i < n; i++) f[i] = orc_bf16_value(v[i]);
  return f;
}

float orc_amax_bf16(const uint16_t* v, int64_t n) {
  float m = 0.0f;
  for (int64_t i = 0; i < n; i++) {
    float a = fabsf(orc_bf16_value(v[i]));
    if (a > m) m = a;
  }
  return m;
}

/* Quantise a bf16 tensor to NVFP4 with a per-tensor global scale computed
 * from its amax; returns the global scale. */
float orc_nvfp4_quantize_bf16(const uint16_t* v, int64_t rows, int64_t cols,
                              uint8_t* q, uint8_t* sf) {
  float* f = bf16_rows_to_f32(v, rows * cols);
  float gs = orc_nvfp4_global_scale(orc_amax_bf16(v, rows * cols));
  orc_nvfp4_quantize(f, rows, cols, cols, gs, q, sf);
  free(f);
  return gs;
}

void orc_mx_quantize_bf16(const uint16_t* v, int64_t rows, int64_t cols, int elem,
                          uint8_t* q, uint8_t* sf) {
  float* f = bf16_rows_to_f32(v, rows * cols);
  orc_mx_quantize(f, rows, cols, cols, elem, q, sf);
  free(f);
}

/* ------------------------------------------------------------------------ */
/* Routing plan: the outputs moe_sort hands to the grouped GEMMs in          */
/* "vllm.models.flint.ops.moe_cute" grouped_moe.                             */
/* Readings: a route r = t*top_k + j is local iff offset <= id < offset+E_l; */
/* inside an expert the slots follow ascending r (stable); each expert's     */
/* range is padded to a multiple of the tile; tile tables list the local     */
/* expert index and the exclusive end of the valid rows; unused entries -1.  */
/* ------------------------------------------------------------------------ */

int64_t orc_route_slots(int64_t M, int top_k, int num_local_experts, int tile) {
  int64_t routes = M * top_k;
  int64_t busy = routes < num_local_experts ? routes : num_local_experts;
  int64_t need = routes + busy * (tile - 1);
  return (need + tile - 1) / tile * tile;
}

void orc_sort(const int32_t* topk_ids, int64_t M, int top_k, int num_local_experts,
              int local_expert_offset, int tile, int32_t* e2p, int32_t* p2e,
              int32_t* tile_expert, int32_t* tile_limit, int32_t* num_tiles,
              int32_t* expert_offsets, int32_t* expert_counts) {
  int64_t R = M * top_k;
  int E = num_local_experts;
  int64_t slots = orc_route_slots(M, top_k, E, tile);
  int64_t max_tiles = slots / tile;
  int64_t* count = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
  for (int64_t r = 0; r < R; r++) {
    int le = topk_ids[r] - local_expert_offset;
    if (topk_ids[r] >= local_expert_offset && le < E) count[le]++;
  }
  int64_t* base = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
  for (int le = 0; le < E; le++) {
    int64_t padded = (count[le] + tile - 1) / tile * tile;
    base[le + 1] = base[le] + padded;
  }
  for (int64_t s = 0; s < slots; s++) p2e[s] = -1;
  for (int64_t i = 0; i < max_tiles; i++) { tile_expert[i] = -1; tile_limit[i] = -1; }
  int64_t* fill = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
  for (int64_t r = 0; r < R; r++) {
    int le = topk_ids[r] - local_expert_offset;
    if (topk_ids[r] >= local_expert_offset && le < E) {
      int64_t slot = base[le] + fill[le]++;
      e2p[r] = (int32_t)slot;
      p2e[slot] = (int32_t)r;
    } else {
      e2p[r] = -1;
    }
  }
  int64_t nt = 0;
  for (int le = 0; le < E; le++) {
    int64_t tiles = (count[le] + tile - 1) / tile;
    for (int64_t i = 0; i < tiles; i++) {
      int64_t end = base[le] + (i + 1) * tile;
      int64_t lim = base[le] + count[le];
      tile_expert[nt] = le;
      tile_limit[nt] = (int32_t)(end < lim ? end : lim);
      nt++;
    }
    expert_offsets[le] = (int32_t)base[le];
    expert_counts[le] = (int32_t)count[le];
  }
  expert_offsets[E] = (int32_t)base[E];
  *num_tiles = (int32_t)nt;
  free(count);
  free(base);
  free(fill);
}

/* ------------------------------------------------------------------------ */
/* The problem and the expert FFN                                            */
/* ------------------------------------------------------------------------ */

typedef struct {
  int mode; /* ORC_W4A16, ORC_W4A4, ORC_MXFP8_MXFP4 */
  int M, H, I, top_k, num_experts, num_local_experts, local_expert_offset;
  const void* x;        /* bf16 [M,H] | packed E2M1 [M,H/2] | E4M3 [M,H]      */
  const uint8_t* x_sf;  /* NULL | E4M3 [M,H/16] | E8M0 [M,H/32], contiguous   */
  int64_t x_row_stride; /* row stride of x in its storage units (2-byte or 1) */
  const int32_t* topk_ids;
  const float* topk_weights;
  const uint8_t* w1;    /* packed E2M1 [E_l, 2I, H/2]; rows [0,I) gate, [I,2I) up */
  const uint8_t* w1_sf; /* E4M3 [E_l, 2I, H/16] | E8M0 [E_l, 2I, H/32]        */
  const float* w1_alpha;
  const uint8_t* w2;    /* packed E2M1 [E_l, H, I/2] */
  const uint8_t* w2_sf; /* E4M3 [E_l, H, I/16] | E8M0 [E_l, H, I/32] */
  const float* w2_alpha;
  float swiglu_alpha, swiglu_beta, swiglu_limit;
  float fc2_input_scale; /* W4A4: global scale of the FC1-output requantisation */
  float routed_scaling_factor;
  int activation;         /* ORC_ACT_SWIGLU (SwiGLU, or SiTU when situ_beta > 0) | ORC_ACT_GEGLU_TANH |
                             ORC_ACT_RELU2 (non-gated: W1 has I rows) */
  float situ_beta;        /* > 0 selects SiTU; 0 = unset */
  float situ_linear_beta; /* > 0: SiTU tanh clamp of the up branch; 0 = unset */
  const float* w1_alpha_up;     /* NULL, or fp32 [E_l]: the up half's own scale */
  const float* per_token_scale; /* NULL, or fp32 [M] (W4A4): GEMM1 input row scale */
  const float* fc1_bias;        /* NULL, or fp32 [E_l, 2I]: GEMM1 bias, gate then up ([E_l, I] for ReLU^2) */
  const float* fc2_bias;        /* NULL, or fp32 [E_l, H]: GEMM2 bias */
} orc_moe_t;

static int sf_block(int mode) { return mode == ORC_MXFP8_MXFP4 ? 32 : 16; }

/* Decode tables filled once from the closed forms above (speed only). */
static double T_E2M1[16], T_E4M3[256], T_E8M0[256];
__attribute__((constructor)) static void init_tables(void) {
  for (int c = 0; c < 16; c++) T_E2M1[c] = orc_e2m1_value(c);
  for (int c = 0; c < 256; c++) T_E4M3[c] = orc_e4m3_value(c);
  for (int c = 0; c < 256; c++) T_E8M0[c] = orc_e8m0_value(c);
}

/* Decoded activation row of token t (its block scale included; in W4A4 the
 * activation's global scale is part of w1_alpha). */
static void dequant_x_row(const orc_moe_t* p, int64_t t, double* a) {
  int H = p->H;
  if (p->mode == ORC_W4A16) {
    const uint16_t* x = (const uint16_t*)p->x + t * p->x_row_stride;
    for (int h = 0; h < H; h++) a[h] = orc_bf16_value(x[h]);
  } else if (p->mode == ORC_W4A4) {
    const uint8_t* x = (const uint8_t*)p->x + t * p->x_row_stride;
    const uint8_t* s = p->x_sf + t * (int64_t)(H / 16);
    for (int h = 0; h < H; h++) a[h] = T_E2M1[nibble(x, h)] * T_E4M3[s[h / 16]];
  } else {
    const uint8_t* x = (const uint8_t*)p->x + t * p->x_row_stride;
    const uint8_t* s = p->x_sf + t * (int64_t)(H / 32);
    for (int h = 0; h < H; h++) a[h] = T_E4M3[x[h]] * T_E8M0[s[h / 32]];
  }
}

/* Decoded weight row: packed E2M1 codes times their block scale (E4M3 for
 * NVFP4, E8M0 for MXFP4); the per-expert global scale is not included. */
static void dequant_w_row(int mode, const uint8_t* q, const uint8_t* sf, int K, double* w) {
  if (mode == ORC_MXFP8_MXFP4) {
    for (int k = 0; k < K; k++) w[k] = T_E2M1[nibble(q, k)] * T_E8M0[sf[k / 32]];
  } else {
    for (int k = 0; k < K; k++) w[k] = T_E2M1[nibble(q, k)] * T_E4M3[sf[k / 16]];
  }
}

/* W1 rows per expert: gate and up (2I), or I for the non-gated ReLU^2. */
static int w1_rows(const orc_moe_t* p) { return p->activation == ORC_ACT_RELU2 ? p->I : 2 * p->I; }

static const uint8_t* w1_row(const orc_moe_t* p, int le, int n, const uint8_t** sf) {
  int64_t row = (int64_t)le * w1_rows(p) + n;
  *sf = p->w1_sf + row * (p->H / sf_block(p->mode));
  return p->w1 + row * (p->H / 2);
}
static const uint8_t* w2_row(const orc_moe_t* p, int le, int c, const uint8_t** sf) {
  int64_t row = (int64_t)le * p->H + c;
  *sf = p->w2_sf + row * (p->I / sf_block(p->mode));
  return p->w2 + row * (p->I / 2);
}

static double dot(const double* a, const double* b, int n) {
  double s = 0.0;
  for (int i = 0; i < n; i++) s += a[i] * b[i];
  return s;
}

/* SwiGLU with alpha / beta / limit (reading of the pages' parameter names,
 * defaults 1 / 0 / FLT_MAX): g' = min(g, limit), u' = clamp(u, -limit,
 * limit), y = g' * sigmoid(alpha * g') * (u' + beta); exactly silu(g) * u at
 * the defaults.  Evaluated in fp64. */
double orc_swiglu(float g, float u, float alpha, float beta, float limit) {
  double gc = (double)g < (double)limit ? (double)g : (double)limit;
  double uc = u;
  if (uc > limit) uc = limit;
  if (uc < -(double)limit) uc = -(double)limit;
  double sig = 1.0 / (1.0 + exp(-(double)alpha * gc));
  return gc * sig * (uc + (double)beta);
}

/* GeGLU with the tanh approximation of GELU ("flashinfer.fused_moe.
 * cute_dsl_fused_moe", Parameters, activation_type GegluTanh):
 * y = gelu_tanh(g) * u, gelu_tanh(x) = x/2 * (1 + tanh(sqrt(2/pi) *
 * (x + 0.044715 x^3))), the published tanh form of GELU (Hendrycks and
 * Gimpel).  Evaluated in fp64. */
double orc_geglu_tanh(float g, float u) {
  double x = g;
  double z = sqrt(2.0 / 3.14159265358979323846) * (x + 0.044715 * x * x * x);
  return 0.5 * x * (1.0 + tanh(z)) * (double)u;
}

/* SiTU (same Parameters, situ_beta and situ_linear_beta): the gate
 * beta * tanh(g / beta) * sigmoid(g) in place of SiLU's g * sigmoid(g), and
 * when linear_beta > 0 the up branch clamped the same way,
 * linear_beta * tanh(u / linear_beta).  Evaluated in fp64. */
double orc_situ(float g, float u, float beta, float linear_beta) {
  double b = beta;
  double gate = b * tanh((double)g / b) / (1.0 + exp(-(double)g));
  double up = u;
  if (linear_beta > 0.0f) up = (double)linear_beta * tanh((double)u / (double)linear_beta);
  return gate * up;
}

/* The FC1 activation of one gate/up pair, as the problem selects it. */
static double gated_act(const orc_moe_t* p, float g, float u) {
  if (p->activation == ORC_ACT_GEGLU_TANH) return orc_geglu_tanh(g, u);
  if (p->situ_beta > 0.0f) return orc_situ(g, u, p->situ_beta, p->situ_linear_beta);
  return orc_swiglu(g, u, p->swiglu_alpha, p->swiglu_beta, p->swiglu_limit);
}

/* fp32 accumulator value times the per-expert fp32 scale, in fp32. */
static float scale_acc(double acc, float alpha) {
  float a = (float)acc;
  float r = a * alpha;
  return r;
}

/* Gate and up values of token t through local expert le from their fp64
 * sums: the accumulator in fp32 times the expert's gate scale (w1_alpha) or
 * up scale (w1_alpha_up when given, "flashinfer.fused_moe.
 * alphamoe_nvfp4_routed_moe", Parameters output1_scale_gate_scalar /
 * output1_scale_scalar), then times the token's per_token_scale when given
 * ("flashinfer.fused_moe.cute_dsl_fused_moe", Parameters per_token_scale):
 * separate fp32 multiplies in that order. */
static void gate_up(const orc_moe_t* p, int le, int64_t t, int j, double G, double U, float* g, float* u) {
  float gv = scale_acc(G, p->w1_alpha[le]);
  float uv = scale_acc(U, p->w1_alpha_up ? p->w1_alpha_up[le] : p->w1_alpha[le]);
  if (p->per_token_scale) {
    float s = p->per_token_scale[t];
    gv = gv * s;
    uv = uv * s;
  }
  if (p->fc1_bias) {
    const float* b = p->fc1_bias + (int64_t)le * 2 * p->I;
    gv = gv + b[j];
    uv = uv + b[p->I + j];
  }
  *g = gv;
  *u = uv;
}

/* FC1 output j of token t through local expert le, before its bf16
 * rounding, from the fp64 sums of its W1 rows: the gated activation of the
 * gate / up pair (G from row j, U from row I + j), or for ReLU^2
 * ("flashinfer.fused_moe.cute_dsl_fused_moe", Parameters activation_type:
 * non-gated Relu2) max(h, 0)^2 of the single row j, h scaled like the gate
 * (expert scale, per-token scale, bias) in fp32. */
static double fc1_out(const orc_moe_t* p, int le, int64_t t, int j, double G, double U) {
  if (p->activation == ORC_ACT_RELU2) {
    float h = scale_acc(G, p->w1_alpha[le]);
    if (p->per_token_scale) h = h * p->per_token_scale[t];
    if (p->fc1_bias) h = h + p->fc1_bias[(int64_t)le * p->I + j];
    double r = h > 0.0f ? (double)h : 0.0;
    return r * r;
  }
  float g, u;
  gate_up(p, le, t, j, G, U, &g, &u);
  return gated_act(p, g, u);
}

/* GEMM2 output of column c through local expert le before its bf16
 * rounding: the fp32 accumulator times w2_alpha, plus the expert's fc2 bias
 * when given ("flashinfer.fused_moe.cutlass_fused_moe", Parameters
 * fc1_expert_biases / fc2_expert_biases: per-expert GEMM biases). */
static float gemm2_value(const orc_moe_t* p, int le, int c, double acc) {
  float v = scale_acc(acc, p->w2_alpha[le]);
  if (p->fc2_bias) v = v + p->fc2_bias[(int64_t)le * p->H + c];
  return v;
}

/* FC1 output of one row: y1 (bf16, rounded once), then the GEMM2 input as
 * the mode stores it (bf16 | NVFP4 with fc2_input_scale | MXFP8) and its
 * decoded values a2 (for W4A4 without the global scale, which is part of
 * w2_alpha). */
static void swiglu_row_and_requant(const orc_moe_t* p, int le, int64_t t, const double* G, const double* U,
                                   uint16_t* y1_bf16, uint8_t* y1q, uint8_t* y1sf, double* a2) {
  int I = p->I;
  float* y = (float*)malloc((size_t)I * sizeof(float));
  for (int j = 0; j < I; j++) {
    uint16_t b = orc_bf16_round(fc1_out(p, le, t, j, G[j], U[j]));
    if (y1_bf16) y1_bf16[j] = b;
    y[j] = orc_bf16_value(b);
  }
  if (p->mode == ORC_W4A16) {
    for (int j = 0; j < I; j++) a2[j] = y[j];
  } else if (p->mode == ORC_W4A4) {
    uint8_t* q = (uint8_t*)calloc((size_t)I / 2, 1);
    uint8_t* s = (uint8_t*)calloc((size_t)I / 16, 1);
    orc_nvfp4_quantize(y, 1, I, I, p->fc2_input_scale, q, s);
    for (int j = 0; j < I; j++) a2[j] = orc_e2m1_value(nibble(q, j)) * orc_e4m3_value(s[j / 16]);
    if (y1q) memcpy(y1q, q, (size_t)I / 2);
    if (y1sf) memcpy(y1sf, s, (size_t)I / 16);
    free(q);
    free(s);
  } else {
    uint8_t* q = (uint8_t*)calloc((size_t)I, 1);
    uint8_t* s = (uint8_t*)calloc((size_t)I / 32, 1);
    orc_mx_quantize(y, 1, I, I, ORC_ELEM_E4M3, q, s);
    for (int j = 0; j < I; j++) a2[j] = orc_e4m3_value(q[j]) * orc_e8m0_value(s[j / 32]);
    if (y1q) memcpy(y1q, q, (size_t)I);
    if (y1sf) memcpy(y1sf, s, (size_t)I / 32);
    free(q);
    free(s);
  }
  free(y);
}

/* GEMM1 + SwiGLU (+ requantisation) of token t through local expert le,
 * decoding the weight rows on the fly.  Outputs may be NULL. */
void orc_gemm1_route(const orc_moe_t* p, int64_t t, int le, uint16_t* y1_bf16, uint8_t* y1q,
                     uint8_t* y1sf, double* a2) {
  int H = p->H, I = p->I;
  double* a = (double*)malloc((size_t)H * sizeof(double));
  double* G = (double*)malloc((size_t)I * sizeof(double));
  double* U = (double*)calloc((size_t)I, sizeof(double));
  dequant_x_row(p, t, a);
#pragma omp parallel
  {
    double* w = (double*)malloc((size_t)H * sizeof(double));
#pragma omp for schedule(static)
    for (int n = 0; n < w1_rows(p); n++) {
      const uint8_t* sf;
      const uint8_t* q = w1_row(p, le, n, &sf);
      dequant_w_row(p->mode, q, sf, H, w);
      double acc = dot(a, w, H);
      if (n < I) G[n] = acc;
      else U[n - I] = acc;
    }
    free(w);
  }
  swiglu_row_and_requant(p, le, t, G, U, y1_bf16, y1q, y1sf, a2);
  free(a);
  free(G);
  free(U);
}

/* GEMM2 of one route: y2[c] = bf16(fp32(sum_i a2[i] * w2[c][i]) * w2_alpha [+ fc2_bias]). */
void orc_gemm2_route(const orc_moe_t* p, int le, const double* a2, uint16_t* y2) {
  int H = p->H, I = p->I;
#pragma omp parallel
  {
    double* w = (double*)malloc((size_t)I * sizeof(double));
#pragma omp for schedule(static)
    for (int c = 0; c < H; c++) {
      const uint8_t* sf;
      const uint8_t* q = w2_row(p, le, c, &sf);
      dequant_w_row(p->mode, q, sf, I, w);
      y2[c] = orc_bf16_round(gemm2_value(p, le, c, dot(a2, w, I)));
    }
    free(w);
  }
}

/* Weighted top-k finalize in route order ("alphamoe_nvfp4_routed_moe"
 * summary; the caller-side reduction of "grouped_moe"):
 *   acc = accumulate ? out_prev : 0  (fp32)
 *   for j = 0..top_k-1, local routes only: acc = acc + fp32(w*rsf) * y2
 *   out = bf16(acc)
 * Separate fp32 multiplies and adds (no fused multiply-add). */
void orc_finalize(const uint16_t* y2, const int32_t* e2p, const float* topk_weights, int64_t M,
                  int top_k, int H, float rsf, int accumulate, const uint16_t* out_prev,
                  uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < M; t++) {
    for (int h = 0; h < H; h++) {
      float acc = accumulate ? orc_bf16_value(out_prev[t * H + h]) : 0.0f;
      for (int j = 0; j < top_k; j++) {
        int32_t s = e2p[t * top_k + j];
        if (s < 0) continue;
        float wf = topk_weights[t * top_k + j] * rsf;
        float prod = wf * orc_bf16_value(y2[(int64_t)s * H + h]);
        acc = acc + prod;
      }
      out[t * H + h] = orc_bf16_round(acc);
    }
  }
}

/* Per-token brute force: out[i] for token tokens[i], each local route's FFN
 * computed directly (no plan), then the same route-order finalize.
 * out_prev (used when accumulate) and out are [ntok, H]. */
void orc_forward_tokens(const orc_moe_t* p, const int32_t* tokens, int ntok, int accumulate,
                        const uint16_t* out_prev, uint16_t* out) {
  int H = p->H, I = p->I, k = p->top_k;
  double* a2 = (double*)malloc((size_t)I * sizeof(double));
  uint16_t* y2 = (uint16_t*)malloc((size_t)H * sizeof(uint16_t));
  float* acc = (float*)malloc((size_t)H * sizeof(float));
  for (int i = 0; i < ntok; i++) {
    int64_t t = tokens[i];
    for (int h = 0; h < H; h++)
      acc[h] = accumulate ? orc_bf16_value(out_prev[(int64_t)i * H + h]) : 0.0f;
    for (int j = 0; j < k; j++) {
      int32_t id = p->topk_ids[t * k + j];
      int le = id - p->local_expert_offset;
      if (id < p->local_expert_offset || le >= p->num_local_experts) continue;
      orc_gemm1_route(p, t, le, NULL, NULL, NULL, a2);
      orc_gemm2_route(p, le, a2, y2);
      float wf = p->topk_weights[t * k + j] * p->routed_scaling_factor;
      for (int h = 0; h < H; h++) {
        float prod = wf * orc_bf16_value(y2[h]);
        acc[h] = acc[h] + prod;
      }
    }
    for (int h = 0; h < H; h++) out[(int64_t)i * H + h] = orc_bf16_round(acc[h]);
  }
  free(a2);
  free(y2);
  free(acc);
}

/* Decoded weights of one expert: W1 [2I (or I), H] and W2 [H, I] in fp64. */
static void dequant_expert(const orc_moe_t* p, int le, double* wd1, double* wd2) {
  int H = p->H, I = p->I;
  if (wd1) {
#pragma omp parallel for schedule(static)
    for (int n = 0; n < w1_rows(p); n++) {
      const uint8_t* sf;
      const uint8_t* q = w1_row(p, le, n, &sf);
      dequant_w_row(p->mode, q, sf, H, wd1 + (int64_t)n * H);
    }
  }
  if (wd2) {
#pragma omp parallel for schedule(static)
    for (int c = 0; c < H; c++) {
      const uint8_t* sf;
      const uint8_t* q = w2_row(p, le, c, &sf);
      dequant_w_row(p->mode, q, sf, I, wd2 + (int64_t)c * I);
    }
  }
}

/* Plan-based forward: the routing plan, then expert by expert GEMM1 +
 * SwiGLU (+ requant) into y1 and GEMM2 into y2, both in permuted slot
 * order, then the finalize.  y1 is bf16 [slots, I] (W4A16), packed NVFP4
 * [slots, I/2] + E4M3 [slots, I/16] (W4A4) or E4M3 [slots, I] + E8M0
 * [slots, I/32] (MXFP8); y2 is bf16 [slots, H].  Padding rows are left as
 * they were.  Plan arrays as in orc_sort. */
void orc_forward_plan(const orc_moe_t* p, int tile, int32_t* e2p, int32_t* p2e,
                      int32_t* tile_expert, int32_t* tile_limit, int32_t* num_tiles,
                      int32_t* expert_offsets, int32_t* expert_counts, void* y1, uint8_t* y1_sf,
                      uint16_t* y2, int accumulate, const uint16_t* out_prev, uint16_t* out) {
  int H = p->H, I = p->I, E = p->num_local_experts;
  orc_sort(p->topk_ids, p->M, p->top_k, E, p->local_expert_offset, tile, e2p, p2e, tile_expert,
           tile_limit, num_tiles, expert_offsets, expert_counts);
  double* wd1 = (double*)malloc((size_t)2 * I * H * sizeof(double));
  double* wd2 = (double*)malloc((size_t)H * I * sizeof(double));
  for (int le = 0; le < E; le++) {
    int cnt = expert_counts[le];
    if (cnt == 0) continue;
    dequant_expert(p, le, wd1, wd2);
    int64_t base = expert_offsets[le];
#pragma omp parallel
    {
      double* a = (double*)malloc((size_t)H * sizeof(double));
      double* G = (double*)malloc((size_t)I * sizeof(double));
      double* U = (double*)malloc((size_t)I * sizeof(double));
      double* a2 = (double*)malloc((size_t)I * sizeof(double));
#pragma omp for schedule(dynamic, 1)
      for (int i = 0; i < cnt; i++) {
        int64_t slot = base + i;
        int64_t t = p2e[slot] / p->top_k;
        dequant_x_row(p, t, a);
        for (int n = 0; n < I; n++) G[n] = dot(a, wd1 + (int64_t)n * H, H);
        for (int n = 0; n < I; n++) U[n] = w1_rows(p) > I ? dot(a, wd1 + (int64_t)(I + n) * H, H) : 0.0;
        uint16_t* yb = NULL;
        uint8_t *yq = NULL, *ys = NULL;
        if (p->mode == ORC_W4A16) {
          yb = (uint16_t*)y1 + slot * I;
        } else if (p->mode == ORC_W4A4) {
          yq = (uint8_t*)y1 + slot * (I / 2);
          ys = y1_sf + slot * (I / 16);
        } else {
          yq = (uint8_t*)y1 + slot * I;
          ys = y1_sf + slot * (I / 32);
        }
        swiglu_row_and_requant(p, le, t, G, U, yb, yq, ys, a2);
        for (int c = 0; c < H; c++)
          y2[slot * H + c] = orc_bf16_round(gemm2_value(p, le, c, dot(a2, wd2 + (int64_t)c * I, I)));
      }
      free(a);
      free(G);
      free(U);
      free(a2);
    }
  }
  free(wd1);
  free(wd2);
  orc_finalize(y2, e2p, p->topk_weights, p->M, p->top_k, H, p->routed_scaling_factor, accumulate,
               out_prev, out);
}

/* Calibration pass for the W4A4 FC1-output requantisation: the largest
 * |y1| over every local route, over 6 * 448 (the workload recipe's
 * fc2_input_scale).  y1 does not depend on fc2_input_scale. */
float orc_fc2_input_scale(const orc_moe_t* p) {
  int H = p->H, I = p->I, E = p->num_local_experts, k = p->top_k;
  double* wd1 = (double*)malloc((size_t)2 * I * H * sizeof(double));
  int64_t R = (int64_t)p->M * k;
  float amax = 0.0f;
  for (int le = 0; le < E; le++) {
    int any = 0;
    for (int64_t r = 0; r < R && !any; r++) any = (p->topk_ids[r] - p->local_expert_offset == le);
    if (!any) continue;
    dequant_expert(p, le, wd1, NULL);
#pragma omp parallel
    {
      double* a = (double*)malloc((size_t)H * sizeof(double));
      float local = 0.0f;
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < R; r++) {
        if (p->topk_ids[r] - p->local_expert_offset != le) continue;
        dequant_x_row(p, r / k, a);
        for (int n = 0; n < I; n++) {
          const double U = w1_rows(p) > I ? dot(a, wd1 + (int64_t)(I + n) * H, H) : 0.0;
          uint16_t b = orc_bf16_round(fc1_out(p, le, r / k, n, dot(a, wd1 + (int64_t)n * H, H), U));
          float v = fabsf(orc_bf16_value(b));
          if (v > local) local = v;
        }
      }
#pragma omp critical
      if (local > amax) amax = local;
      free(a);
    }
  }
  free(wd1);
  return orc_nvfp4_global_scale(amax);
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
