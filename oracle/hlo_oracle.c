/*
 * hlo_oracle.c -- plain, slow, single-threaded CPU interpreter of the op
 * semantics of one HLO fusion.  TEST INFRASTRUCTURE ONLY: it is used by the
 * tests, by the smoke check and by the CPU-baseline leg of the benchmark.  The
 * product library never links, loads or calls it, and it shares no code with
 * the product (no headers, helpers, tables or constants).
 *
 * How it computes (deliberately naive):
 *   - Every element value is carried as a long double that holds exactly the
 *     value of the node's declared element type (f32, bf16, f16 values and the
 *     integer storage values of quantized types are all exact in it).
 *   - A node's value at a logical multi-index is computed by its defining
 *     formula, recursively, straight from the op definitions ("point
 *     evaluation"): nothing is fused, tiled, vectorised or reordered.
 *   - Each op rounds its exact (or long-double) result once to its declared
 *     element type, with round-to-nearest-even.  Long double keeps 64
 *     significand bits, which is at least 2p+2 for p = 24 (f32), 11 (f16) and
 *     8 (bf16), so rounding a long-double add, multiply or divide to the
 *     target type gives the correctly rounded result of the exact operation.
 *   - exp, log and tanh use expl, logl and tanhl and round once.
 *   - Sums in reduce are accumulated in long double and rounded once.
 *   - Physical buffers are decoded and encoded with the minor_to_major layout
 *     formula, computed here by its own naive loop.
 *
 * Sources (page title, then section):
 *   Shapes and layout: "Minor-to-major dimension ordering", "Default
 *     minor-to-major ordering", "Array indexing".
 *   StableHLO Specification: "Types" (quantized element types and their
 *     constraints), Ops add, broadcast_in_dim, convert, dot_general,
 *     dynamic_slice, exponential, log, maximum, minimum, multiply, reduce,
 *     reshape, reduce_precision, round_nearest_even, tanh; "Programs" (the
 *     start_indices and limit_indices attributes of slice).
 *   Operation semantics: Reduce, BroadcastInDim, ConvertElementType, Collapse,
 *     DynamicSlice.
 *   StableHLO Quantization: "Per-tensor quantization", "Per-axis quantization".
 *   XLA:GPU Emitters: "Indexing transforms" (transpose as an output-to-input
 *     index map).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define OR_MAX_RANK 8
#define OR_MAX_OPERANDS 9 /* dynamic_slice: the operand and one start index per dim */
#define OR_MAX_ATTR 24

/* element types */
/* si4/ui4 (Specification, "Types": 4-bit integers): the pages give no memory
   packing.  Reading taken here: two elements per byte in physical (linear)
   order, the element with the even linear index in the low four bits. */
enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2, OR_S8 = 3, OR_S32 = 4, OR_U8 = 5, OR_S4 = 6, OR_U4 = 7 };

/* ops */
enum {
  OR_PARAM = 0, OR_CONSTANT = 1, OR_LOG = 2, OR_EXP = 3, OR_TANH = 4,
  OR_ADD = 5, OR_SUBTRACT = 6, OR_MULTIPLY = 7, OR_DIVIDE = 8,
  OR_MAXIMUM = 9, OR_MINIMUM = 10, OR_NEGATE = 11, OR_ABS = 12,
  OR_CONVERT = 13, OR_BROADCAST_IN_DIM = 14, OR_RESHAPE = 15,
  OR_TRANSPOSE = 16, OR_DEQUANTIZE = 17, OR_QUANTIZE = 18, OR_REDUCE = 19,
  OR_DOT = 20, OR_REVERSE = 21, OR_IOTA = 22, OR_PAD = 23, OR_CONCATENATE = 24,
  OR_SLICE = 25, OR_DYNAMIC_SLICE = 26
};

enum { OR_RED_ADD = 0, OR_RED_MAX = 1, OR_RED_MIN = 2, OR_RED_ARGMAX = 3 };

typedef struct {
  int32_t dtype;               /* element (storage) type */
  int32_t rank;
  int64_t dims[OR_MAX_RANK];
  int32_t m2m[OR_MAX_RANK];    /* minor_to_major; meaningful for params/root */
  int32_t quantized;           /* 1: a quantized element type, expressed f32 */
  int32_t qdim;                /* quantization_dimension, -1 = per-tensor */
  int64_t nq;                  /* number of (scale, zero_point) pairs */
  const double *scales;        /* nq values (f32-representable) */
  const int64_t *zero_points;  /* nq values */
  int64_t storage_min, storage_max;
} or_type;

typedef struct {
  int32_t op;
  int32_t n_operands;
  int32_t operands[OR_MAX_OPERANDS];
  or_type type;
  int32_t param_index;         /* OR_PARAM */
  double constant;             /* OR_CONSTANT: scalar, broadcast over type */
  int32_t n_attr;              /* permutation | broadcast dims | reduce dims |
                                  reverse dims | iota dim | pad low, high,
                                  interior | concatenate dim | slice start,
                                  limit, strides | dynamic_slice sizes */
  int64_t attr[OR_MAX_ATTR];
  int32_t reducer;             /* OR_REDUCE */
  double init;                 /* OR_REDUCE */
} or_node;

typedef struct {
  const or_node *nodes;
  int32_t n_nodes;
  const void *const *params;
  int32_t n_params;
} graph;

static char g_err[512];
static void set_err(const char *m, int node) {
  snprintf(g_err, sizeof g_err, "node %d: %s", node, m);
}
const char *or_last_error(void) { return g_err; }
int or_version(void) { return 1; }

/* ------------------------------------------------------------------------ */
/* Rounding to a binary floating-point format.                               */
/* p = significand bits including the hidden bit, emin/emax = exponent range */
/* of normal numbers.  Round to nearest, ties to even; subnormals kept;      */
/* overflow goes to the signed infinity.                                     */
/* ------------------------------------------------------------------------ */
long double or_round_format(long double v, int p, int emin, int emax) {
  if (isnan(v)) return v;
  if (isinf(v) || v == 0.0L) return v;
  int e = ilogbl(v); /* floor(log2|v|) */
  if (e < emin) e = emin;
  long double quantum = ldexpl(1.0L, e - (p - 1));
  long double r = nearbyintl(v / quantum) * quantum; /* scaling is exact */
  long double maxf = ldexpl(2.0L - ldexpl(1.0L, 1 - p), emax);
  if (fabsl(r) > maxf) return v > 0 ? (long double)INFINITY : -(long double)INFINITY;
  if (r == 0.0L) return signbit(v) ? -0.0L : 0.0L;
  return r;
}
double or_round_format_d(double v, int p, int emin, int emax) {
  return (double)or_round_format((long double)v, p, emin, emax);
}

static int is_float_type(int dt) { return dt == OR_F32 || dt == OR_BF16 || dt == OR_F16; }

static long double round_to(int dtype, long double v) {
  switch (dtype) {
    case OR_F32: return or_round_format(v, 24, -126, 127);
    case OR_BF16: return or_round_format(v, 8, -126, 127);
    case OR_F16: return or_round_format(v, 11, -14, 15);
    default: return v; /* integers are produced exactly by their ops */
  }
}

/* ------------------------------------------------------------------------ */
/* Layout: linear index of a logical multi-index.                           */
/* linear = sum_k idx[m2m[k]] * stride_k, stride_0 = 1,                     */
/* stride_{k+1} = stride_k * dims[m2m[k]]  (Shapes and layout: minor_to_major) */
/* ------------------------------------------------------------------------ */
int64_t or_linear_index(int32_t rank, const int64_t *dims, const int32_t *m2m,
                        const int64_t *idx) {
  int64_t lin = 0, stride = 1;
  for (int k = 0; k < rank; ++k) {
    int d = m2m[k];
    lin += idx[d] * stride;
    stride *= dims[d];
  }
  return lin;
}

static int64_t num_elements(const or_type *t) {
  int64_t n = 1;
  for (int d = 0; d < t->rank; ++d) n *= t->dims[d];
  return n;
}

/* ------------------------------------------------------------------------ */
/* Element decode / encode                                                   */
/* ------------------------------------------------------------------------ */
static long double decode_f16(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  long double v;
  if (e == 31) v = m ? (long double)NAN : (long double)INFINITY;
  else if (e == 0) v = ldexpl((long double)m, -24);
  else v = ldexpl((long double)(1024 + m), e - 25);
  return s ? -v : v;
}
static uint16_t encode_f16(long double v) {
  uint16_t s = signbit(v) ? 0x8000 : 0;
  if (isnan(v)) return 0x7E00;
  long double a = fabsl(v);
  if (isinf(a)) return s | 0x7C00;
  if (a == 0) return s;
  int e = ilogbl(a);
  if (e < -14) return s | (uint16_t)(a / ldexpl(1.0L, -24)); /* subnormal, exact */
  uint16_t m = (uint16_t)(a / ldexpl(1.0L, e - 10)) - 1024;
  return s | (uint16_t)((e + 15) << 10) | m;
}

static long double load_elem(int dtype, const void *buf, int64_t lin) {
  switch (dtype) {
    case OR_F32: return (long double)((const float *)buf)[lin];
    case OR_BF16: {
      uint32_t bits = (uint32_t)((const uint16_t *)buf)[lin] << 16;
      float f;
      memcpy(&f, &bits, 4);
      return (long double)f;
    }
    case OR_F16: return decode_f16(((const uint16_t *)buf)[lin]);
    case OR_S8: return (long double)((const int8_t *)buf)[lin];
    case OR_U8: return (long double)((const uint8_t *)buf)[lin];
    case OR_S32: return (long double)((const int32_t *)buf)[lin];
    case OR_S4: case OR_U4: {
      const unsigned byte = ((const uint8_t *)buf)[lin / 2];
      const int nib = (int)((lin % 2) ? (byte >> 4) : (byte & 0xFu));
      return (long double)(dtype == OR_S4 && nib >= 8 ? nib - 16 : nib);
    }
  }
  return NAN;
}

static void store_elem(int dtype, void *buf, int64_t lin, long double v) {
  switch (dtype) {
    case OR_F32: ((float *)buf)[lin] = (float)v; break; /* v is f32-exact */
    case OR_BF16: {
      uint16_t h;
      if (isnan(v)) h = signbit(v) ? 0xFFC0 : 0x7FC0;
      else {
        float f = (float)v; /* exact: v is a bf16 value */
        uint32_t bits;
        memcpy(&bits, &f, 4);
        h = (uint16_t)(bits >> 16);
      }
      ((uint16_t *)buf)[lin] = h;
      break;
    }
    case OR_F16: ((uint16_t *)buf)[lin] = encode_f16(v); break;
    case OR_S8: ((int8_t *)buf)[lin] = (int8_t)v; break;
    case OR_U8: ((uint8_t *)buf)[lin] = (uint8_t)v; break;
    case OR_S32: ((int32_t *)buf)[lin] = (int32_t)v; break;
    case OR_S4: case OR_U4: {
      /* v is in [-8, 7] (si4) or [0, 15] (ui4); its low four bits are the
         two's-complement nibble.  The other nibble of the byte is kept. */
      uint8_t *b = (uint8_t *)buf + lin / 2;
      const unsigned nib = (unsigned)((int)v & 0xF);
      *b = (lin % 2) ? (uint8_t)((*b & 0x0Fu) | (nib << 4)) : (uint8_t)((*b & 0xF0u) | nib);
      break;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* IEEE 754-2019 maximum / minimum: NaN if either operand is NaN, and        */
/* -0 < +0 (StableHLO Specification: maximum, minimum).                      */
/* ------------------------------------------------------------------------ */
static long double ieee_maximum(long double a, long double b) {
  if (isnan(a) || isnan(b)) return (long double)NAN;
  if (a == 0 && b == 0) return (signbit(a) && signbit(b)) ? -0.0L : 0.0L;
  return a > b ? a : b;
}
static long double ieee_minimum(long double a, long double b) {
  if (isnan(a) || isnan(b)) return (long double)NAN;
  if (a == 0 && b == 0) return (signbit(a) || signbit(b)) ? -0.0L : 0.0L;
  return a < b ? a : b;
}

/* ------------------------------------------------------------------------ */
/* Uniform quantization (StableHLO Specification "Types": f = (i - zero_point)*scale; */
/* StableHLO Quantization: real_value = scale * (quantized_value - zero_point)) */
/* ------------------------------------------------------------------------ */
static int64_t qslice(const or_type *t, const int64_t *idx) {
  return t->qdim < 0 ? 0 : idx[t->qdim];
}

static long double dequantize(const or_type *qt, long double q, const int64_t *idx,
                              int result_dtype) {
  int64_t s = qslice(qt, idx);
  long double scale = round_to(OR_F32, (long double)qt->scales[s]);
  long double diff = q - (long double)qt->zero_points[s]; /* exact integer */
  return round_to(result_dtype, scale * diff);
}

/* Quantize: t = expressed-type(y / scale) by IEEE division; round t to the
 * nearest integer, ties to even; add the zero point as an integer; clamp to
 * [storage_min, storage_max].  Non-finite input is rejected. */
static int quantize(const or_type *qt, long double y, const int64_t *idx, long double *out) {
  if (!isfinite(y)) return -1;
  int64_t s = qslice(qt, idx);
  long double scale = round_to(OR_F32, (long double)qt->scales[s]);
  long double t = round_to(OR_F32, y / scale);
  long double r = nearbyintl(t); /* default rounding mode: ties to even */
  long double q = r + (long double)qt->zero_points[s];
  if (q < (long double)qt->storage_min) q = (long double)qt->storage_min;
  if (q > (long double)qt->storage_max) q = (long double)qt->storage_max;
  *out = q;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Point evaluation                                                          */
/* ------------------------------------------------------------------------ */
typedef struct {
  long double abs_sum;  /* reduce-add root: sum of |operand| over the slice */
  long double raw;      /* reduce root: the accumulator before rounding */
} aux_t;

static int eval(const graph *g, int n, const int64_t *idx, long double *out, aux_t *aux);

static int eval_reduce(const graph *g, int n, const int64_t *ridx, long double *out,
                       aux_t *aux) {
  const or_node *nd = &g->nodes[n];
  const or_node *in = &g->nodes[nd->operands[0]];
  int rank = in->type.rank;
  int is_red[OR_MAX_RANK] = {0};
  for (int k = 0; k < nd->n_attr; ++k) is_red[nd->attr[k]] = 1;
  /* operand index: kept dims take the result index in order */
  int64_t oidx[OR_MAX_RANK];
  int rd[OR_MAX_RANK], nrd = 0;
  for (int d = 0, r = 0; d < rank; ++d) {
    if (is_red[d]) { oidx[d] = 0; rd[nrd++] = d; }
    else oidx[d] = ridx[r++];
  }
  long double acc = (long double)nd->init;
  long double arg = (long double)nd->constant; /* argmax: the index part of the tuple */
  long double abs_sum = 0;
  int64_t count = 1;
  for (int k = 0; k < nrd; ++k) count *= in->type.dims[rd[k]];
  /* lexicographic walk over the reduced dims */
  for (int64_t it = 0; it < count; ++it) {
    long double x;
    int rc = eval(g, nd->operands[0], oidx, &x, NULL);
    if (rc) return rc;
    if (nd->reducer == OR_RED_ADD) { acc += x; abs_sum += fabsl(x); }
    else if (nd->reducer == OR_RED_MAX) acc = ieee_maximum(acc, x);
    else if (nd->reducer == OR_RED_MIN) acc = ieee_minimum(acc, x);
    else {
      /* Operation semantics, "Variadic Reduce": f(max, argmax, value, index)
       * = value >= max ? (value, index) : (max, argmax), applied in order */
      long double k;
      rc = eval(g, nd->operands[1], oidx, &k, NULL);
      if (rc) return rc;
      if (x >= acc) { acc = x; arg = k; }
    }
    for (int k = nrd - 1; k >= 0; --k) {
      if (++oidx[rd[k]] < in->type.dims[rd[k]]) break;
      oidx[rd[k]] = 0;
    }
  }
  if (aux) { aux->abs_sum = abs_sum; aux->raw = acc; }
  *out = nd->reducer == OR_RED_ARGMAX ? arg : round_to(nd->type.dtype, acc);
  return 0;
}

static int eval(const graph *g, int n, const int64_t *idx, long double *out, aux_t *aux) {
  const or_node *nd = &g->nodes[n];
  const or_type *t = &nd->type;
  long double a = 0, b = 0;
  int64_t oidx[OR_MAX_RANK];
  int rc;
  switch (nd->op) {
    case OR_PARAM: {
      if (nd->param_index < 0 || nd->param_index >= g->n_params) { set_err("bad param", n); return -2; }
      int64_t lin = or_linear_index(t->rank, t->dims, t->m2m, idx);
      *out = load_elem(t->dtype, g->params[nd->param_index], lin);
      return 0;
    }
    case OR_CONSTANT:
      *out = round_to(t->dtype, (long double)nd->constant);
      return 0;
    case OR_LOG: case OR_EXP: case OR_TANH: case OR_NEGATE: case OR_ABS:
    case OR_ADD: case OR_SUBTRACT: case OR_MULTIPLY: case OR_DIVIDE:
    case OR_MAXIMUM: case OR_MINIMUM: {
      /* A quantized op (StableHLO Specification, each op's semantics for
       * quantized types: dequantize_op_quantize): its quantized operands are
       * dequantized, the op runs on the expressed (f32) values, and the f32
       * result is quantized to the result type. */
      const int dt = t->quantized ? OR_F32 : t->dtype;
      const int binary = nd->op != OR_LOG && nd->op != OR_EXP && nd->op != OR_TANH &&
                         nd->op != OR_NEGATE && nd->op != OR_ABS;
      long double r;
      if ((rc = eval(g, nd->operands[0], idx, &a, NULL))) return rc;
      if (g->nodes[nd->operands[0]].type.quantized) a = dequantize(&g->nodes[nd->operands[0]].type, a, idx, OR_F32);
      if (binary) {
        if ((rc = eval(g, nd->operands[1], idx, &b, NULL))) return rc;
        if (g->nodes[nd->operands[1]].type.quantized) b = dequantize(&g->nodes[nd->operands[1]].type, b, idx, OR_F32);
      }
      switch (nd->op) {
        case OR_LOG: r = round_to(dt, logl(a)); break;
        case OR_EXP: r = round_to(dt, expl(a)); break;
        case OR_TANH: r = round_to(dt, tanhl(a)); break;
        case OR_NEGATE: r = -a; break;
        case OR_ABS: r = fabsl(a); break;
        case OR_ADD: r = round_to(dt, a + b); break;
        case OR_SUBTRACT: r = round_to(dt, a - b); break;
        case OR_MULTIPLY: r = round_to(dt, a * b); break;
        case OR_DIVIDE: r = round_to(dt, a / b); break;
        case OR_MAXIMUM: r = ieee_maximum(a, b); break;
        default: r = ieee_minimum(a, b); break;
      }
      if (!t->quantized) {
        *out = r;
        return 0;
      }
      if (quantize(t, r, idx, out)) { set_err("quantize of a non-finite value", n); return -3; }
      return 0;
    }
    case OR_CONVERT: {
      if ((rc = eval(g, nd->operands[0], idx, &a, NULL))) return rc;
      if (is_float_type(t->dtype)) *out = round_to(t->dtype, a); /* int->float RNE; float->float RNE */
      else *out = truncl(a); /* float->integer truncates; ints pass */
      return 0;
    }
    case OR_BROADCAST_IN_DIM: {
      /* operand_index[d] = 0 if dim(operand, d) = 1 else result_index[bdims[d]] */
      const or_type *ot = &g->nodes[nd->operands[0]].type;
      for (int d = 0; d < ot->rank; ++d)
        oidx[d] = ot->dims[d] == 1 ? 0 : idx[nd->attr[d]];
      return eval(g, nd->operands[0], oidx, out, NULL);
    }
    case OR_TRANSPOSE: {
      /* result dim d is operand dim perm[d]: operand_index[perm[d]] = result_index[d] */
      for (int d = 0; d < t->rank; ++d) oidx[nd->attr[d]] = idx[d];
      return eval(g, nd->operands[0], oidx, out, NULL);
    }
    case OR_RESHAPE: {
      /* same position in the lexicographic order of both index spaces */
      const or_type *ot = &g->nodes[nd->operands[0]].type;
      int64_t pos = 0;
      for (int d = 0; d < t->rank; ++d) pos = pos * t->dims[d] + idx[d];
      for (int d = ot->rank - 1; d >= 0; --d) {
        oidx[d] = pos % ot->dims[d];
        pos /= ot->dims[d];
      }
      return eval(g, nd->operands[0], oidx, out, NULL);
    }
    case OR_REVERSE: {
      /* operand_index[d] = dim(result, d) - result_index[d] - 1 for d in
       * dimensions, result_index[d] otherwise */
      for (int d = 0; d < t->rank; ++d) oidx[d] = idx[d];
      for (int k = 0; k < nd->n_attr; ++k) {
        const int d = (int)nd->attr[k];
        oidx[d] = t->dims[d] - idx[d] - 1;
      }
      return eval(g, nd->operands[0], oidx, out, NULL);
    }
    case OR_IOTA:
      /* the index along iota_dimension, in the element type */
      *out = round_to(t->dtype, (long double)idx[nd->attr[0]]);
      return 0;
    case OR_PAD: {
      /* result[i] = operand[j] where i = edge_padding_low + j * (interior_padding + 1)
       * for an operand index j; padding_value elsewhere */
      const or_type *ot = &g->nodes[nd->operands[0]].type;
      const int r = ot->rank;
      int inside = 1;
      for (int d = 0; d < r && inside; ++d) {
        const int64_t lo = nd->attr[d], step = nd->attr[2 * r + d] + 1;
        const int64_t k = idx[d] - lo;
        if (k < 0 || k % step != 0 || k / step >= ot->dims[d]) inside = 0;
        else oidx[d] = k / step;
      }
      if (inside) return eval(g, nd->operands[0], oidx, out, NULL);
      return eval(g, nd->operands[1], oidx, out, NULL); /* rank 0: no index */
    }
    case OR_CONCATENATE: {
      /* result[.., i_d, ..] = inputs[k][.., i_d - (d_0 + ... + d_{k-1}), ..] */
      const int cd = (int)nd->attr[0];
      int64_t off = 0;
      for (int k = 0; k < nd->n_operands; ++k) {
        const int64_t dk = g->nodes[nd->operands[k]].type.dims[cd];
        if (idx[cd] < off + dk) {
          for (int d = 0; d < t->rank; ++d) oidx[d] = idx[d];
          oidx[cd] = idx[cd] - off;
          return eval(g, nd->operands[k], oidx, out, NULL);
        }
        off += dk;
      }
      set_err("concatenate index out of range", n);
      return -2;
    }
    case OR_SLICE: {
      /* result[i] = operand[start_indices + i * strides]; attr holds
       * start_indices[rank], limit_indices[rank], strides[rank] */
      const int r = t->rank;
      for (int d = 0; d < r; ++d) oidx[d] = nd->attr[d] + idx[d] * nd->attr[2 * r + d];
      return eval(g, nd->operands[0], oidx, out, NULL);
    }
    case OR_DYNAMIC_SLICE: {
      /* adjusted_start_indices = clamp(0, start_indices, shape(operand) -
       * slice_sizes); operand_index = adjusted_start_indices + result_index.
       * Operand 1 + d is the rank-0 start index of dim d; attr holds
       * slice_sizes[rank]. */
      const or_type *ot = &g->nodes[nd->operands[0]].type;
      const int64_t none[OR_MAX_RANK] = {0};
      for (int d = 0; d < ot->rank; ++d) {
        long double sv;
        if ((rc = eval(g, nd->operands[1 + d], none, &sv, NULL))) return rc;
        int64_t start = (int64_t)sv;
        const int64_t hi = ot->dims[d] - nd->attr[d];
        if (start < 0) start = 0;
        if (start > hi) start = hi;
        oidx[d] = start + idx[d];
      }
      return eval(g, nd->operands[0], oidx, out, NULL);
    }
    case OR_DEQUANTIZE: {
      const or_type *qt = &g->nodes[nd->operands[0]].type;
      if ((rc = eval(g, nd->operands[0], idx, &a, NULL))) return rc;
      *out = dequantize(qt, a, idx, t->dtype);
      return 0;
    }
    case OR_QUANTIZE: {
      const or_type *it = &g->nodes[nd->operands[0]].type;
      if ((rc = eval(g, nd->operands[0], idx, &a, NULL))) return rc;
      if (it->quantized) a = dequantize(it, a, idx, OR_F32); /* requantize */
      if (quantize(t, a, idx, out)) { set_err("quantize of a non-finite value", n); return -3; }
      return 0;
    }
    case OR_REDUCE:
      return eval_reduce(g, n, idx, out, aux);
    case OR_DOT: {
      /* [m,k] x [k,n] -> [m,n]: sum over k of lhs[i,k]*rhs[k,j], long double, one rounding */
      const or_type *lt = &g->nodes[nd->operands[0]].type;
      long double acc = 0;
      for (int64_t k = 0; k < lt->dims[1]; ++k) {
        int64_t li[2] = {idx[0], k}, ri[2] = {k, idx[1]};
        if ((rc = eval(g, nd->operands[0], li, &a, NULL))) return rc;
        if ((rc = eval(g, nd->operands[1], ri, &b, NULL))) return rc;
        acc += a * b;
      }
      *out = round_to(t->dtype, acc);
      return 0;
    }
  }
  set_err("unknown op", n);
  return -1;
}

/* ------------------------------------------------------------------------ */
/* Shape checks: just enough to refuse a malformed graph.                    */
/* ------------------------------------------------------------------------ */
static int check(const graph *g, int root) {
  if (root < 0 || root >= g->n_nodes) { set_err("bad root", root); return -1; }
  for (int n = 0; n < g->n_nodes; ++n) {
    const or_node *nd = &g->nodes[n];
    if (nd->type.rank < 0 || nd->type.rank > OR_MAX_RANK) { set_err("bad rank", n); return -1; }
    for (int k = 0; k < nd->n_operands; ++k)
      if (nd->operands[k] < 0 || nd->operands[k] >= n) { set_err("operand not earlier", n); return -1; }
    if (nd->op == OR_TRANSPOSE) {
      const or_type *ot = &g->nodes[nd->operands[0]].type;
      int seen[OR_MAX_RANK] = {0};
      if (nd->n_attr != nd->type.rank || ot->rank != nd->type.rank) { set_err("transpose rank", n); return -1; }
      for (int d = 0; d < nd->n_attr; ++d) {
        if (nd->attr[d] < 0 || nd->attr[d] >= ot->rank || seen[nd->attr[d]]++) { set_err("not a permutation", n); return -1; }
        if (nd->type.dims[d] != ot->dims[nd->attr[d]]) { set_err("transpose dims", n); return -1; }
      }
    }
    if (nd->op == OR_BROADCAST_IN_DIM) {
      const or_type *ot = &g->nodes[nd->operands[0]].type;
      if (nd->n_attr != ot->rank) { set_err("broadcast dims count", n); return -1; }
      for (int d = 0; d < ot->rank; ++d) {
        int64_t rd = nd->attr[d];
        if (rd < 0 || rd >= nd->type.rank) { set_err("broadcast dim range", n); return -1; }
        if (ot->dims[d] != 1 && ot->dims[d] != nd->type.dims[rd]) { set_err("broadcast dim size", n); return -1; }
      }
    }
    if (nd->op == OR_SLICE) {
      const or_type *ot = &g->nodes[nd->operands[0]].type;
      const int r = ot->rank;
      if (nd->n_attr != 3 * r || nd->type.rank != r) { set_err("slice attributes", n); return -1; }
      for (int d = 0; d < r; ++d) {
        const int64_t st = nd->attr[d], lim = nd->attr[r + d], step = nd->attr[2 * r + d];
        if (st < 0 || st > lim || lim > ot->dims[d] || step < 1) { set_err("slice bounds", n); return -1; }
        if (nd->type.dims[d] != (lim - st + step - 1) / step) { set_err("slice result dims", n); return -1; }
      }
    }
    if (nd->op == OR_DYNAMIC_SLICE) {
      const or_type *ot = &g->nodes[nd->operands[0]].type;
      if (nd->n_operands != 1 + ot->rank || nd->n_attr != ot->rank || nd->type.rank != ot->rank) {
        set_err("dynamic_slice operands", n);
        return -1;
      }
      for (int d = 0; d < ot->rank; ++d) {
        if (g->nodes[nd->operands[1 + d]].type.rank != 0) { set_err("start index not rank 0", n); return -1; }
        if (nd->attr[d] < 0 || nd->attr[d] > ot->dims[d] || nd->type.dims[d] != nd->attr[d]) {
          set_err("dynamic_slice sizes", n);
          return -1;
        }
      }
    }
    if (nd->op == OR_RESHAPE && num_elements(&nd->type) != num_elements(&g->nodes[nd->operands[0]].type)) {
      set_err("reshape size", n);
      return -1;
    }
  }
  return 0;
}

/* Evaluate the whole root and encode it into `out` in the root's layout. */
int or_eval(const or_node *nodes, int32_t n_nodes, int32_t root, const void *const *params,
            int32_t n_params, void *out) {
  graph g = {nodes, n_nodes, params, n_params};
  if (check(&g, root)) return -1;
  const or_type *t = &nodes[root].type;
  int64_t idx[OR_MAX_RANK] = {0};
  int64_t total = num_elements(t);
  for (int64_t it = 0; it < total; ++it) {
    long double v;
    int rc = eval(&g, root, idx, &v, NULL);
    if (rc) return rc;
    store_elem(t->dtype, out, or_linear_index(t->rank, t->dims, t->m2m, idx), v);
    for (int d = t->rank - 1; d >= 0; --d) {
      if (++idx[d] < t->dims[d]) break;
      idx[d] = 0;
    }
  }
  return 0;
}

/* Evaluate the root at n_points logical indices (n_points x rank, row-major).
 * values[i] receives the value; if aux is non-NULL, aux[2i] = sum of |x| and
 * aux[2i+1] = the unrounded accumulator when the root is a reduce. */
int or_eval_points(const or_node *nodes, int32_t n_nodes, int32_t root,
                   const void *const *params, int32_t n_params, int64_t n_points,
                   const int64_t *points, double *values, double *aux) {
  graph g = {nodes, n_nodes, params, n_params};
  if (check(&g, root)) return -1;
  int rank = nodes[root].type.rank;
  for (int64_t i = 0; i < n_points; ++i) {
    long double v;
    aux_t ax = {0, 0};
    const int64_t *p = points + i * rank;
    for (int d = 0; d < rank; ++d)
      if (p[d] < 0 || p[d] >= nodes[root].type.dims[d]) { set_err("point out of range", root); return -4; }
    int rc = eval(&g, root, p, &v, &ax);
    if (rc) return rc;
    values[i] = (double)v;
    if (aux) { aux[2 * i] = (double)ax.abs_sum; aux[2 * i + 1] = (double)ax.raw; }
  }
  return 0;
}

/* Batch form of or_linear_index: idx is n x rank (row-major), out gets n values. */
void or_linear_indices(int32_t rank, const int64_t *dims, const int32_t *m2m, int64_t n,
                       const int64_t *idx, int64_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_linear_index(rank, dims, m2m, idx + i * rank);
}
