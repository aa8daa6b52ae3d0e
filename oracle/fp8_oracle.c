/*
 * fp8_oracle.c -- CPU oracle for block-scaled FP8 quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow reference that the GPU kernels are
 * checked against.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load it.  The product library never links, calls or includes it, and it
 * shares no code, header, table or constant generator with the HIP sources.
 *
 * What it follows (the pages are quoted by title and section; nothing is copied):
 *  [P1] "Infraestructura de Entrenamiento FP8: Precisión Numérica de Nueva Generación"
 *       (introl.com blog), section "El panorama de la precisión numérica": E4M3 has 4 exponent
 *       and 3 mantissa bits and reaches +-448; E5M2 has 5 exponent and 2 mantissa bits.
 *  [P1] section "Transformer Engine: la base de software": the DelayedScaling recipe (margin 0,
 *       HYBRID format = E4M3 forward / E5M2 backward, amax history of 16, reduction "max"),
 *       and the rule that the scale comes from the largest magnitudes of earlier iterations.
 *  [P1] section "Estrategias de escalado y estabilidad": per-tensor, block and delayed scaling.
 *  [P3] "NVIDIA NeMo RL logra una aceleración del 48% con entrenamiento de precisión FP8 de
 *       extremo a extremo" (hotbookzone.com), section "El avance técnico": block-quantized E4M3
 *       with 128x128 weight tiles and 1x128 activation blocks.
 *  [P3] section "Por qué esto es importante para la economía de la IA": the option of
 *       power-of-2 scale factors.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  - E4M3 is the variant with bias 7, no infinities and NaN only at S.1111.111: it is the only
 *    4/3-bit layout whose largest finite value is 448.  E5M2 is the IEEE-like layout (bias 15,
 *    infinities at exponent 31 / mantissa 0, NaN otherwise), largest finite 57344.
 *  - Encoding is round-to-nearest with ties to the even code, computed once from the fp32
 *    value; magnitudes above the largest finite value (infinity included) saturate to it,
 *    for both formats; NaN maps to 0x7F with the input's sign; subnormals are kept.
 *  - Scale s multiplies before the cast: s = fl32(FMAX / amax); the stored dequantization
 *    factor is fl32(1 / s).  amax == 0 or non-finite -> s = 1.  s == +inf -> FLT_MAX.
 *    Power-of-2 mode rounds s down to 2^floor(log2 s).
 *  - Blocks at the tensor edge are clipped to the tensor.
 *  - Delayed state starts as history = 0, s = 1.  Each call quantizes with the current s,
 *    then pushes the new amax at history[0] (newest first), then recomputes s from
 *    max(history) if that is positive and finite; otherwise s is kept.
 *
 * All floating-point work below is IEEE binary32 / binary64 with round-to-nearest and no
 * flush-to-zero; every worker thread resets the FP environment before it starts.
 */
#include <float.h>
#include <fenv.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { O_E4M3 = 0, O_E5M2 = 1 };
enum { O_BLOCK_1x128 = 0, O_BLOCK_128x128 = 1, O_BLOCK_1x32 = 3 };
enum { O_SCALE_FP32 = 0, O_SCALE_POW2 = 1 };

/* Format parameters, from the bit splits named in [P1] and the readings above. */
typedef struct {
  int ebits;      /* exponent field width */
  int mbits;      /* mantissa field width */
  int bias;       /* exponent bias */
  int has_inf;    /* exponent all-ones with mantissa 0 means infinity */
  double fmax;    /* largest finite magnitude */
  int max_code;   /* code of +fmax */
} o_format;

static const o_format O_FORMATS[2] = {
    {4, 3, 7, 0, 448.0, 0x7E},
    {5, 2, 15, 1, 57344.0, 0x7B},
};

static int o_fmt_ok(int fmt) { return fmt == O_E4M3 || fmt == O_E5M2; }

/* Value of one code: (-1)^s * 2^(e-bias) * (1 + m/2^M) for normal codes,
 * (-1)^s * 2^(1-bias) * (m/2^M) for exponent field 0.  Returns NaN for NaN codes. */
double o_decode(int fmt, int code) {
  if (!o_fmt_ok(fmt)) return NAN;
  const o_format* f = &O_FORMATS[fmt];
  int sign = (code >> 7) & 1;
  int e = (code >> f->mbits) & ((1 << f->ebits) - 1);
  int m = code & ((1 << f->mbits) - 1);
  int emax_field = (1 << f->ebits) - 1;
  double v;
  if (f->has_inf) {
    if (e == emax_field) {
      if (m != 0) return NAN;
      return sign ? -INFINITY : INFINITY;
    }
  } else if (e == emax_field && m == (1 << f->mbits) - 1) {
    return NAN;
  }
  if (e == 0)
    v = ldexp((double)m, 1 - f->bias - f->mbits);
  else
    v = ldexp((double)((1 << f->mbits) + m), e - f->bias - f->mbits);
  return sign ? -v : v;
}

/* Nearest integer, ties to even (the FP environment is round-to-nearest, which is the mode
 * nearbyint uses). */
static double o_round_half_even(double r) { return nearbyint(r); }

/* Nearest representable value with ties to the even code, saturating, NaN -> 0x7F|sign. */
uint8_t o_encode(int fmt, float v) {
  const o_format* f = &O_FORMATS[fmt];
  int sign = signbit(v) ? 1 : 0;
  if (isnan(v)) return (uint8_t)(0x7F | (sign << 7));
  double a = fabs((double)v);
  if (a > f->fmax) return (uint8_t)(f->max_code | (sign << 7));
  if (a == 0.0) return (uint8_t)(sign << 7);
  int e2;
  frexp(a, &e2);                 /* a = frac * 2^e2 with frac in [0.5, 1) */
  int ex = e2 - 1;               /* floor(log2 a) */
  int emin = 1 - f->bias;        /* exponent of the smallest normal */
  if (ex < emin) ex = emin;      /* subnormal range shares the spacing of the first binade */
  double quantum = ldexp(1.0, ex - f->mbits);   /* spacing of representable values here */
  /* a / quantum is exact: a is an fp32 value and quantum a power of two well inside the
   * double range, so the only rounding is the one to an integer count of quanta. */
  double n = o_round_half_even(a / quantum);
  if (n == 0.0) return (uint8_t)(sign << 7);
  long ni = (long)n;
  int efield, mfield;
  long implicit = 1L << f->mbits;
  if (ex == emin && ni < implicit) {
    efield = 0;                  /* subnormal */
    mfield = (int)ni;
  } else {
    if (ni == 2 * implicit) {    /* rounding carried into the next binade */
      ni = implicit;
      ex += 1;
    }
    efield = ex + f->bias;
    mfield = (int)(ni - implicit);
  }
  return (uint8_t)((sign << 7) | (efield << f->mbits) | mfield);
}

/* bf16 bit pattern -> fp32 (exact: bf16 is the top half of an fp32). */
static float o_bf16_to_f32(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float x;
  memcpy(&x, &u, sizeof x);
  return x;
}

/* Scale from a block's largest magnitude (readings listed in the header). */
float o_scale_from_amax(int fmt, int mode, float amax, int finite) {
  const o_format* f = &O_FORMATS[fmt];
  if (!finite || amax == 0.0f) return 1.0f;
  float fmax = (float)f->fmax;
  float s = fmax / amax;                 /* binary32 division, round to nearest even */
  if (isinf(s)) s = FLT_MAX;
  if (mode == O_SCALE_POW2) {
    int e;
    frexpf(s, &e);                       /* s = frac * 2^e, frac in [0.5, 1) */
    s = ldexpf(1.0f, e - 1);             /* 2^floor(log2 s) */
  }
  return s;
}

/* ---------------------------------------------------------------- threads */
typedef void (*o_task_fn)(void* ctx, int64_t begin, int64_t end);
typedef struct {
  o_task_fn fn;
  void* ctx;
  int64_t begin, end;
} o_task;

static void* o_task_run(void* p) {
  o_task* t = (o_task*)p;
  fesetenv(FE_DFL_ENV);
  t->fn(t->ctx, t->begin, t->end);
  return NULL;
}

/* Run fn over [0, n) split into nthreads contiguous ranges (nthreads <= 1: calling thread). */
static void o_parallel(o_task_fn fn, void* ctx, int64_t n, int nthreads) {
  if (nthreads > 256) nthreads = 256;
  if (nthreads <= 1 || n < 2) {
    fenv_t saved;
    fegetenv(&saved);
    fesetenv(FE_DFL_ENV);
    fn(ctx, 0, n);
    fesetenv(&saved);
    return;
  }
  if ((int64_t)nthreads > n) nthreads = (int)n;
  pthread_t th[256];
  o_task tasks[256];
  int started[256];
  for (int i = 0; i < nthreads; ++i) {
    tasks[i].fn = fn;
    tasks[i].ctx = ctx;
    tasks[i].begin = n * i / nthreads;
    tasks[i].end = n * (i + 1) / nthreads;
    started[i] = pthread_create(&th[i], NULL, o_task_run, &tasks[i]) == 0;
    if (!started[i]) o_task_run(&tasks[i]);
  }
  for (int i = 0; i < nthreads; ++i)
    if (started[i]) pthread_join(th[i], NULL);
}

/* ---------------------------------------------------------------- encode a range */
typedef struct {
  int fmt;
  const float* in;
  uint32_t first_bits;
  uint8_t* out;
} o_enc_ctx;

static void o_enc_task(void* p, int64_t b, int64_t e) {
  o_enc_ctx* c = (o_enc_ctx*)p;
  for (int64_t i = b; i < e; ++i) {
    float v;
    if (c->in) {
      v = c->in[i];
    } else {
      uint32_t u = c->first_bits + (uint32_t)i;
      memcpy(&v, &u, sizeof v);
    }
    c->out[i] = o_encode(c->fmt, v);
  }
}

/* Encode n fp32 values. */
int o_encode_array(int fmt, const float* in, int64_t n, uint8_t* out, int nthreads) {
  if (!o_fmt_ok(fmt) || n < 0 || (n > 0 && (!in || !out))) return -1;
  o_enc_ctx c = {fmt, in, 0, out};
  o_parallel(o_enc_task, &c, n, nthreads);
  return 0;
}

/* Encode the fp32 values whose bit patterns are first_bits, first_bits+1, ... (count values). */
int o_encode_bit_range(int fmt, uint32_t first_bits, int64_t count, uint8_t* out, int nthreads) {
  if (!o_fmt_ok(fmt) || count < 0 || count > ((int64_t)1 << 32) || (count > 0 && !out)) return -1;
  o_enc_ctx c = {fmt, NULL, first_bits, out};
  o_parallel(o_enc_task, &c, count, nthreads);
  return 0;
}

/* ---------------------------------------------------------------- blockwise quantization */
typedef struct {
  const uint16_t* x;
  int64_t rows, cols;
  int fmt, mode;
  int64_t bh;          /* block height: 1 or 128 */
  int64_t bw;          /* block width: 128, or 32 (one row by 32 columns) */
  int64_t nbc;         /* blocks per row of blocks */
  uint8_t* q;
  float* scale_inv;    /* logical [ceil(rows/bh)][nbc] */
} o_bw_ctx;

static void o_bw_task(void* p, int64_t b, int64_t e) {
  o_bw_ctx* c = (o_bw_ctx*)p;
  for (int64_t bi = b; bi < e; ++bi) {
    int64_t r0 = bi * c->bh;
    int64_t r1 = r0 + c->bh < c->rows ? r0 + c->bh : c->rows;
    for (int64_t bj = 0; bj < c->nbc; ++bj) {
      int64_t c0 = bj * c->bw;
      int64_t c1 = c0 + c->bw < c->cols ? c0 + c->bw : c->cols;
      /* step 1: largest magnitude in the block (finite flag for NaN / Inf) */
      float amax = 0.0f;
      int finite = 1;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t cc = c0; cc < c1; ++cc) {
          float v = o_bf16_to_f32(c->x[r * c->cols + cc]);
          if (!isfinite(v)) {
            finite = 0;
          } else if (fabsf(v) > amax) {
            amax = fabsf(v);
          }
        }
      /* step 2: scale; step 3: multiply in fp32 and encode */
      float s = o_scale_from_amax(c->fmt, c->mode, amax, finite);
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t cc = c0; cc < c1; ++cc) {
          float v = o_bf16_to_f32(c->x[r * c->cols + cc]);
          float y = v * s;
          c->q[r * c->cols + cc] = o_encode(c->fmt, y);
        }
      /* step 4: dequantization factor */
      c->scale_inv[bi * c->nbc + bj] = 1.0f / s;
    }
  }
}

/*
 * Blockwise quantization of a contiguous row-major bf16 matrix x[rows][cols].
 * gran O_BLOCK_1x128: a block is one row by 128 consecutive columns;
 * gran O_BLOCK_128x128: a block is a 128x128 tile;
 * gran O_BLOCK_1x32: a block is one row by 32 consecutive columns (the microscaling blocks).
 * Edge blocks are clipped.
 * q[rows][cols] receives the codes; scale_inv receives one fp32 per block in the logical
 * order [block row][block column].  Returns 0, or -1 on a bad argument.
 */
int o_quantize_blockwise(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int gran,
                         int mode, uint8_t* q, float* scale_inv, int nthreads) {
  if (!o_fmt_ok(fmt) || (gran != O_BLOCK_1x128 && gran != O_BLOCK_128x128 && gran != O_BLOCK_1x32) ||
      (mode != O_SCALE_FP32 && mode != O_SCALE_POW2) || rows < 0 || cols < 0)
    return -1;
  if (rows == 0 || cols == 0) return 0;
  if (!x || !q || !scale_inv) return -1;
  o_bw_ctx c;
  c.x = x;
  c.rows = rows;
  c.cols = cols;
  c.fmt = fmt;
  c.mode = mode;
  c.bh = gran == O_BLOCK_128x128 ? 128 : 1;
  c.bw = gran == O_BLOCK_1x32 ? 32 : 128;
  c.nbc = (cols + c.bw - 1) / c.bw;
  c.q = q;
  c.scale_inv = scale_inv;
  int64_t nbr = (rows + c.bh - 1) / c.bh;
  o_parallel(o_bw_task, &c, nbr, nthreads);
  return 0;
}

/* ---------------------------------------------------------------- delayed per-tensor scaling */
typedef struct {
  const uint16_t* x;
  int fmt;
  float s;
  uint8_t* q;
} o_dl_ctx;

static void o_dl_task(void* p, int64_t b, int64_t e) {
  o_dl_ctx* c = (o_dl_ctx*)p;
  for (int64_t i = b; i < e; ++i) {
    float v = o_bf16_to_f32(c->x[i]);
    float y = v * c->s;
    c->q[i] = o_encode(c->fmt, y);
  }
}

/*
 * One step of per-tensor delayed scaling on x[n] (bf16), state (history[hist_len], *scale).
 * Quantizes with the scale held in the state (derived from earlier steps only), records this
 * tensor's amax, and advances the state for the next step.
 * Outputs: q[n]; *scale_inv_used = fl32(1 / scale used); history and *scale updated.
 */
int o_delayed_step(const uint16_t* x, int64_t n, int fmt, int mode, int margin, int hist_len,
                   float* history, float* scale, uint8_t* q, float* scale_inv_used,
                   int nthreads) {
  if (!o_fmt_ok(fmt) || (mode != O_SCALE_FP32 && mode != O_SCALE_POW2) || n < 0 ||
      hist_len < 1 || hist_len > 1024 || margin < 0 || margin > 64 || !history || !scale ||
      !scale_inv_used || (n > 0 && (!x || !q)))
    return -1;
  fenv_t saved;
  fegetenv(&saved);
  fesetenv(FE_DFL_ENV);
  const o_format* f = &O_FORMATS[fmt];
  float s = *scale;

  /* quantize with the scale from earlier steps */
  o_dl_ctx c = {x, fmt, s, q};
  o_parallel(o_dl_task, &c, n, nthreads);
  *scale_inv_used = 1.0f / s;

  /* amax of this tensor; NaN anywhere makes it NaN */
  float a = 0.0f;
  int has_nan = 0;
  for (int64_t i = 0; i < n; ++i) {
    float v = o_bf16_to_f32(x[i]);
    if (isnan(v))
      has_nan = 1;
    else if (fabsf(v) > a)
      a = fabsf(v);
  }
  if (has_nan) a = NAN;

  /* push, newest first */
  for (int i = hist_len - 1; i >= 1; --i) history[i] = history[i - 1];
  history[0] = a;

  /* reduce the history with "max" */
  float ref = 0.0f;
  int ref_nan = 0;
  for (int i = 0; i < hist_len; ++i) {
    if (isnan(history[i]))
      ref_nan = 1;
    else if (history[i] > ref)
      ref = history[i];
  }
  if (!ref_nan && ref > 0.0f && isfinite(ref)) {
    float fmax = (float)f->fmax;
    float ns = fmax / ref;
    ns = ns / ldexpf(1.0f, margin);
    if (isinf(ns)) ns = FLT_MAX;
    if (mode == O_SCALE_POW2) {
      int e;
      frexpf(ns, &e);
      ns = ldexpf(1.0f, e - 1);
    }
    *scale = ns;
  }
  fesetenv(&saved);
  return 0;
}

/* ---------------------------------------------------------------- dequantization to fp64 */
typedef struct {
  const uint8_t* q;
  int64_t rows, cols;
  int fmt;
  int64_t bh, bw;       /* block shape; bh = rows and bw = cols for one per-tensor scale */
  int64_t nbc;
  const float* scale_inv;
  double* out;
  double table[256];
} o_dq_ctx;

static void o_dq_task(void* p, int64_t b, int64_t e) {
  o_dq_ctx* c = (o_dq_ctx*)p;
  for (int64_t r = b; r < e; ++r)
    for (int64_t cc = 0; cc < c->cols; ++cc) {
      double si = (double)c->scale_inv[(r / c->bh) * c->nbc + cc / c->bw];
      c->out[r * c->cols + cc] = c->table[c->q[r * c->cols + cc]] * si;
    }
}

/*
 * value = decode(code) * scale_inv[block], in fp64 (exact: a <= 4-bit significand times an
 * fp32).  bh x bw is the block shape (1x128, 128x128, or rows x cols for one scale); scale_inv
 * is in the logical order [block row][block column].
 */
int o_dequantize(const uint8_t* q, int64_t rows, int64_t cols, int fmt, int64_t bh, int64_t bw,
                 const float* scale_inv, double* out, int nthreads) {
  if (!o_fmt_ok(fmt) || rows < 0 || cols < 0 || bh < 1 || bw < 1) return -1;
  if (rows == 0 || cols == 0) return 0;
  if (!q || !scale_inv || !out) return -1;
  o_dq_ctx* c = (o_dq_ctx*)malloc(sizeof(o_dq_ctx));
  if (!c) return -1;
  c->q = q;
  c->rows = rows;
  c->cols = cols;
  c->fmt = fmt;
  c->bh = bh;
  c->bw = bw;
  c->nbc = (cols + bw - 1) / bw;
  c->scale_inv = scale_inv;
  c->out = out;
  for (int i = 0; i < 256; ++i) c->table[i] = o_decode(fmt, i);
  o_parallel(o_dq_task, c, rows, nthreads);
  free(c);
  return 0;
}
