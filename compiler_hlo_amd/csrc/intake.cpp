// intake.cpp -- descriptor intake and validation.
//
// Each check below is a constraint of the op as the StableHLO Specification
// ("Ops", the Constraints list of each op) or the "Types" section states it;
// a broken constraint is HF_ERR_INVALID.  Valid fusions outside what the
// library implements are HF_ERR_UNSUPPORTED.  All of it runs on the host.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <sstream>

#include "ir.h"

namespace hf {

void fail(hf_status st, const std::string &msg) { throw Error{st, msg}; }

int dtype_bits(hf_dtype dt) {
  switch (dt) {
    case HF_F32: case HF_S32: return 32;
    case HF_BF16: case HF_F16: return 16;
    case HF_S8: case HF_U8: return 8;
    case HF_S4: case HF_U4: return 4;
  }
  return 0;
}

// Whole bytes of one element (4-bit types count as one: callers that size
// buffers use storage_bytes).
int dtype_bytes(hf_dtype dt) { return dtype_bits(dt) >= 8 ? dtype_bits(dt) / 8 : 1; }

// Bytes that hold n elements: 4-bit types pack two per byte.
int64_t storage_bytes(hf_dtype dt, int64_t n) { return (n * dtype_bits(dt) + 7) / 8; }

bool is_nibble(hf_dtype dt) { return dt == HF_S4 || dt == HF_U4; }

bool is_float(hf_dtype dt) { return dt == HF_F32 || dt == HF_BF16 || dt == HF_F16; }

const char *dtype_name(hf_dtype dt) {
  switch (dt) {
    case HF_F32: return "f32";
    case HF_BF16: return "bf16";
    case HF_F16: return "f16";
    case HF_S8: return "s8";
    case HF_U8: return "u8";
    case HF_S32: return "s32";
    case HF_S4: return "s4";
    case HF_U4: return "u4";
  }
  return "?";
}

const char *op_name(hf_op op) {
  switch (op) {
    case HF_PARAMETER: return "parameter";
    case HF_CONSTANT: return "constant";
    case HF_ADD: return "add";
    case HF_SUBTRACT: return "subtract";
    case HF_MULTIPLY: return "multiply";
    case HF_DIVIDE: return "divide";
    case HF_MAXIMUM: return "maximum";
    case HF_MINIMUM: return "minimum";
    case HF_LOG: return "log";
    case HF_EXP: return "exponential";
    case HF_TANH: return "tanh";
    case HF_NEGATE: return "negate";
    case HF_ABS: return "abs";
    case HF_CONVERT: return "convert";
    case HF_BROADCAST_IN_DIM: return "broadcast_in_dim";
    case HF_RESHAPE: return "reshape";
    case HF_TRANSPOSE: return "transpose";
    case HF_UNIFORM_DEQUANTIZE: return "uniform_dequantize";
    case HF_UNIFORM_QUANTIZE: return "uniform_quantize";
    case HF_REDUCE: return "reduce";
    case HF_REVERSE: return "reverse";
    case HF_IOTA: return "iota";
    case HF_PAD: return "pad";
    case HF_CONCATENATE: return "concatenate";
    case HF_SLICE: return "slice";
    case HF_DYNAMIC_SLICE: return "dynamic_slice";
  }
  return "?";
}

namespace {

struct Ctx {
  int node;
  hf_op op;
  std::string where() const {
    std::ostringstream s;
    s << "node " << node << " (" << op_name(op) << "): ";
    return s.str();
  }
  [[noreturn]] void invalid(const std::string &m) const { fail(HF_ERR_INVALID, where() + m); }
  [[noreturn]] void unsupported(const std::string &m) const { fail(HF_ERR_UNSUPPORTED, where() + m); }
};

bool valid_dtype(int dt) { return dt >= HF_F32 && dt <= HF_U4; }

std::string dims_str(const Type &t) {
  std::ostringstream s;
  s << dtype_name(t.dt) << "[";
  for (int d = 0; d < t.rank; ++d) s << (d ? "," : "") << t.dims[d];
  s << "]";
  return s.str();
}

// Type intake: shape, layout (a permutation of [0, rank)), quantization
// constraints C1-C13 of quantized element types.
Type take_type(const hf_type &src, Graph &g, const Ctx &c) {
  Type t;
  if (!valid_dtype(src.dtype)) c.invalid("unknown element type");
  t.dt = (hf_dtype)src.dtype;
  if (src.rank < 0 || src.rank > HF_MAX_RANK) c.invalid("rank out of range [0, 8]");
  t.rank = src.rank;
  for (int d = 0; d < t.rank; ++d) {
    if (src.dims[d] < 0) c.invalid("negative dimension size");
    t.dims[d] = src.dims[d];
  }
  if (src.has_layout) {
    bool seen[HF_MAX_RANK] = {false};
    for (int k = 0; k < t.rank; ++k) {
      int d = src.minor_to_major[k];
      if (d < 0 || d >= t.rank || seen[d]) {
        std::ostringstream s;
        s << "minor_to_major is not a permutation of [0," << t.rank << ")";
        c.invalid(s.str());
      }
      seen[d] = true;
      t.m2m[k] = d;
    }
  } else {
    for (int k = 0; k < t.rank; ++k) t.m2m[k] = t.rank - 1 - k;  // default: major to minor
  }
  // kernels index with 32-bit offsets
  int64_t n = 1;
  for (int d = 0; d < t.rank; ++d) {
    if (t.dims[d] > 0 && n > (int64_t(1) << 40) / t.dims[d]) c.unsupported("array too large");
    n *= t.dims[d];
  }
  // element indices of every array, byte offsets of the ones in memory (the
  // parameters and the result: checked in intake)
  if (n >= (int64_t(1) << 31)) c.unsupported("array of 2^31 elements or more");
  if (src.quant) {
    const hf_quant &q = *src.quant;
    if (t.dt != HF_S8 && t.dt != HF_U8 && t.dt != HF_S4 && t.dt != HF_U4)
      c.unsupported("quantized storage type must be s8, u8, s4 or u4");
    Quant qq;
    qq.storage = t.dt;
    int32_t tmin = 0, tmax = 255;
    if (t.dt == HF_S8) tmin = -128, tmax = 127;
    else if (t.dt == HF_S4) tmin = -8, tmax = 7;
    else if (t.dt == HF_U4) tmin = 0, tmax = 15;
    qq.smin = q.has_storage_range ? q.storage_min : tmin;
    qq.smax = q.has_storage_range ? q.storage_max : tmax;
    if (!(tmin <= qq.smin && qq.smin < qq.smax && qq.smax <= tmax))
      c.invalid("storage_min/storage_max break min(storage) <= storage_min < storage_max <= max(storage) (C4)");
    if (q.n < 1 || !q.scales || !q.zero_points) c.invalid("quantization parameters missing");
    if (q.quantization_dimension < 0) {
      if (q.quantization_dimension != -1) c.invalid("quantization_dimension must be >= 0 (C12) or -1");
      if (q.n != 1) c.invalid("per-tensor quantization needs exactly one scale (C11)");
    } else {
      if (q.quantization_dimension >= t.rank) c.invalid("quantization_dimension < rank violated (C12)");
      if (q.n != t.dims[q.quantization_dimension])
        c.invalid("dim(quantization_dimension) = size(scales) violated (C13)");
    }
    qq.qdim = q.quantization_dimension;
    for (int i = 0; i < q.n; ++i) {
      float s = q.scales[i];
      if (!std::isfinite(s)) c.invalid("scales must be finite (C7)");
      if (!(s > 0.0f)) c.invalid("scales must be > 0 (C6)");
      if (q.zero_points[i] < qq.smin || q.zero_points[i] > qq.smax)
        c.invalid("storage_min <= zero_points <= storage_max violated (C8)");
      qq.scales.push_back(s);
      qq.zero_points.push_back(q.zero_points[i]);
    }
    t.quant = (int)g.quants.size();
    g.quants.push_back(std::move(qq));
  }
  return t;
}

void need_operands(const hf_node &n, int k, const Ctx &c) {
  if (n.n_operands != k) {
    std::ostringstream s;
    s << "expects " << k << " operand(s), got " << n.n_operands;
    c.invalid(s.str());
  }
}

}  // namespace

// Rewrites each elementwise op on quantized values into dequantize, the op
// on f32 values, and quantize to the op's result type
// (dequantize_op_quantize), so that the rest of the library sees only float
// arithmetic between uniform_dequantize and uniform_quantize.
void expand_quantized_ops(Graph &g) {
  auto elementwise = [](hf_op op) {
    switch (op) {
      case HF_ADD: case HF_SUBTRACT: case HF_MULTIPLY: case HF_DIVIDE: case HF_MAXIMUM: case HF_MINIMUM:
      case HF_LOG: case HF_EXP: case HF_TANH: case HF_NEGATE: case HF_ABS:
        return true;
      default:
        return false;
    }
  };
  bool any = false;
  for (const Node &nd : g.nodes) any |= elementwise(nd.op) && nd.t.quant >= 0;
  if (!any) return;
  auto f32_of = [](const Type &q) {
    Type t = q;
    t.dt = HF_F32;
    t.quant = -1;
    for (int d = 0; d < t.rank; ++d) t.m2m[d] = t.rank - 1 - d;
    return t;
  };
  std::vector<Node> out;
  std::vector<int> map(g.nodes.size(), -1);
  for (size_t i = 0; i < g.nodes.size(); ++i) {
    Node nd = g.nodes[i];
    for (int &o : nd.opd) o = map[o];
    if (elementwise(nd.op) && nd.t.quant >= 0) {
      for (int &o : nd.opd) {
        Node d;
        d.op = HF_UNIFORM_DEQUANTIZE;
        d.opd = {o};
        d.t = f32_of(out[o].t);
        out.push_back(d);
        o = (int)out.size() - 1;
      }
      const Type qt = nd.t;
      nd.t = f32_of(qt);
      out.push_back(nd);
      Node q;
      q.op = HF_UNIFORM_QUANTIZE;
      q.opd = {(int)out.size() - 1};
      q.t = qt;
      out.push_back(q);
    } else {
      out.push_back(nd);
    }
    map[i] = (int)out.size() - 1;
  }
  for (int &p : g.param_node)
    if (p >= 0) p = map[p];
  g.root = map[g.root];
  g.nodes = std::move(out);
}

Graph intake(const hf_fusion_desc *desc) {
  if (!desc) fail(HF_ERR_INVALID, "descriptor is NULL");
  if (desc->abi_version != HF_ABI_VERSION) fail(HF_ERR_INVALID, "abi_version mismatch");
  if (desc->n_nodes < 1 || desc->n_nodes > HF_MAX_NODES || !desc->nodes)
    fail(HF_ERR_INVALID, "n_nodes out of range [1, 256] or nodes NULL");
  if (desc->n_params < 0 || desc->n_params > HF_MAX_PARAMS)
    fail(HF_ERR_INVALID, "n_params out of range [0, 16]");
  if (desc->root < 0 || desc->root >= desc->n_nodes) fail(HF_ERR_INVALID, "root out of range");

  Graph g;
  g.n_params = desc->n_params;
  g.root = desc->root;
  g.param_node.assign(g.n_params, -1);
  g.nodes.resize(desc->n_nodes);

  for (int i = 0; i < desc->n_nodes; ++i) {
    const hf_node &src = desc->nodes[i];
    // the enum-valued fields are plain integers at the boundary: each is
    // range-checked before it becomes an enum
    if (src.op < HF_PARAMETER || src.op > HF_DYNAMIC_SLICE)
      fail(HF_ERR_INVALID, "node " + std::to_string(i) + ": unknown op");
    Ctx c{i, (hf_op)src.op};
    Node &n = g.nodes[i];
    n.op = (hf_op)src.op;
    if (src.n_operands < 0 || src.n_operands > HF_MAX_OPERANDS) c.invalid("n_operands out of range");
    for (int k = 0; k < src.n_operands; ++k) {
      int o = src.operands[k];
      if (o < 0 || o >= i) c.invalid("operand must be an earlier node");
      n.opd.push_back(o);
    }
    n.t = take_type(src.type, g, c);
    if ((src.op == HF_PARAMETER || i == desc->root) && storage_bytes(n.t.dt, n.t.numel()) >= (int64_t(1) << 31))
      c.unsupported("array of 2 GiB or more");
    if (src.n_attr < 0 || src.n_attr > HF_MAX_ATTR) c.invalid("n_attr out of range");
    for (int k = 0; k < src.n_attr; ++k) n.attr.push_back(src.attr[k]);
    n.param = src.parameter_number;
    n.cst = src.constant;
    n.reducer = src.reducer >= HF_REDUCER_ADD && src.reducer <= HF_REDUCER_ARGMAX ? (hf_reducer)src.reducer
                                                                                  : HF_REDUCER_ADD;  // checked if HF_REDUCE
    n.init = src.init_value;

    const Type &t = n.t;
    auto opt = [&](int k) -> const Type & { return g.nodes[n.opd[k]].t; };
    bool quantized = t.quant >= 0;
    // An elementwise op on quantized values (StableHLO Specification: each
    // op's semantics for quantized types, dequantize_op_quantize): operands
    // and result per-tensor quantized with one baseline type (storage type
    // and range; the scales and zero points may differ).
    auto check_quantized = [&]() {
      for (size_t k = 0; k < n.opd.size(); ++k)
        if (opt((int)k).quant < 0 || !quantized)
          c.invalid("baseline types differ (C1): quantized and non-quantized element types mixed");
      for (size_t k = 0; k <= n.opd.size(); ++k) {
        const Quant &q = g.quants[k < n.opd.size() ? opt((int)k).quant : t.quant];
        const Quant &r = g.quants[t.quant];
        if (q.qdim >= 0) c.invalid("operands and result must be per-tensor quantized tensors (I1)");
        if (q.smin != r.smin || q.smax != r.smax || q.storage != r.storage)
          c.invalid("baseline types differ (C1): storage types or ranges differ");
      }
    };

    switch (src.op) {
      case HF_PARAMETER:
        need_operands(src, 0, c);
        if (n.param < 0 || n.param >= g.n_params) c.invalid("parameter_number out of range [0, n_params)");
        if (g.param_node[n.param] >= 0) c.invalid("parameter_number used twice");
        g.param_node[n.param] = i;
        break;
      case HF_CONSTANT:
        need_operands(src, 0, c);
        if (quantized) c.unsupported("quantized constants");
        if (!is_float(t.dt)) {
          // integer constants serve as dynamic_slice start indices (checked
          // against their users below)
          if (t.rank != 0) c.unsupported("integer constants must be rank 0 (dynamic_slice start indices)");
          const double lo = t.dt == HF_S32 ? INT32_MIN : t.dt == HF_S8 ? -128 : t.dt == HF_S4 ? -8 : 0;
          const double hi = t.dt == HF_S32 ? INT32_MAX : t.dt == HF_S8 ? 127 : t.dt == HF_U8 ? 255
                          : t.dt == HF_S4 ? 7 : 15;
          if (n.cst != std::floor(n.cst) || n.cst < lo || n.cst > hi)
            c.invalid("the constant is not a value of its integer element type");
        }
        break;
      case HF_LOG: case HF_EXP: case HF_TANH: case HF_NEGATE: case HF_ABS:
        need_operands(src, 1, c);
        if (!t.same_shape(opt(0)) || t.dt != opt(0).dt)
          c.invalid("baseline_type(operand) = baseline_type(result) violated (C1): " +
                    dims_str(opt(0)) + " vs " + dims_str(t));
        if (quantized || opt(0).quant >= 0) check_quantized();
        else if (!is_float(t.dt)) c.unsupported("only floating-point element types are supported");
        break;
      case HF_ADD: case HF_SUBTRACT: case HF_MULTIPLY: case HF_DIVIDE:
      case HF_MAXIMUM: case HF_MINIMUM:
        need_operands(src, 2, c);
        if (!t.same_shape(opt(0)) || !t.same_shape(opt(1)) || t.dt != opt(0).dt || t.dt != opt(1).dt)
          c.invalid("baseline_type(lhs) = baseline_type(rhs) = baseline_type(result) violated (C1): " +
                    dims_str(opt(0)) + ", " + dims_str(opt(1)) + " -> " + dims_str(t));
        if (quantized || opt(0).quant >= 0 || opt(1).quant >= 0) check_quantized();
        else if (!is_float(t.dt)) c.unsupported("only floating-point element types are supported");
        break;
      case HF_CONVERT:
        need_operands(src, 1, c);
        if (!t.same_shape(opt(0))) c.invalid("shape(operand) = shape(result) violated (C1)");
        if (quantized || opt(0).quant >= 0)
          c.unsupported("convert of quantized types: use uniform_quantize/uniform_dequantize");
        if (!is_float(t.dt)) c.unsupported("conversion to an integer type is not supported");
        if (opt(0).dt == HF_S32 && t.dt != HF_F32)
          c.unsupported("s32 converts to f32 only");
        break;
      case HF_BROADCAST_IN_DIM: {
        need_operands(src, 1, c);
        const Type &o = opt(0);
        if (t.dt != o.dt) c.invalid("element_type(operand) = element_type(result) violated (C1)");
        if (quantized || o.quant >= 0) c.unsupported("broadcast of quantized values");
        if ((int)n.attr.size() != o.rank) c.invalid("size(broadcast_dimensions) = rank(operand) violated (C2)");
        bool seen[HF_MAX_RANK] = {false};
        for (int d = 0; d < o.rank; ++d) {
          int64_t bd = n.attr[d];
          if (bd < 0 || bd >= t.rank) c.invalid("0 <= broadcast_dimensions < rank(result) violated (C3)");
          if (seen[bd]) c.invalid("is_unique(broadcast_dimensions) violated (C4)");
          seen[bd] = true;
          if (o.dims[d] != 1 && o.dims[d] != t.dims[bd])
            c.invalid("dim(operand, d) = 1 or dim(result, broadcast_dimensions[d]) violated (C5)");
        }
        break;
      }
      case HF_RESHAPE:
        need_operands(src, 1, c);
        if (t.dt != opt(0).dt) c.invalid("element types differ (C1)");
        if (t.numel() != opt(0).numel()) c.invalid("size(operand) = size(result) violated (C2)");
        if (quantized || opt(0).quant >= 0) c.unsupported("reshape of quantized values");
        break;
      case HF_TRANSPOSE: {
        need_operands(src, 1, c);
        const Type &o = opt(0);
        if (t.dt != o.dt) c.invalid("element types differ");
        if (quantized || o.quant >= 0) c.unsupported("transpose of quantized values");
        if ((int)n.attr.size() != t.rank || o.rank != t.rank) c.invalid("permutation length must equal rank");
        bool seen[HF_MAX_RANK] = {false};
        for (int d = 0; d < t.rank; ++d) {
          int64_t p = n.attr[d];
          if (p < 0 || p >= t.rank || seen[p]) {
            std::ostringstream s;
            s << "attr is not a permutation of [0," << t.rank << ")";
            c.invalid(s.str());
          }
          seen[p] = true;
          if (t.dims[d] != o.dims[p]) c.invalid("dim(result, d) = dim(operand, permutation[d]) violated");
        }
        break;
      }
      case HF_REVERSE: {
        need_operands(src, 1, c);
        const Type &o = opt(0);
        if (!t.same_shape(o) || t.dt != o.dt) c.invalid("type(operand) = type(result) violated (C1)");
        if (quantized || o.quant >= 0) c.unsupported("reverse of quantized values");
        bool seen[HF_MAX_RANK] = {false};
        for (int64_t d : n.attr) {
          if (d < 0 || d >= t.rank) c.invalid("0 <= dimensions < rank(result) violated (C3)");
          if (seen[d]) c.invalid("is_unique(dimensions) violated (C2)");
          seen[d] = true;
        }
        break;
      }
      case HF_IOTA:
        need_operands(src, 0, c);
        if (n.attr.size() != 1 || n.attr[0] < 0 || n.attr[0] >= t.rank)
          c.invalid("0 <= iota_dimension < rank(output) violated (C1)");
        if (quantized) c.unsupported("quantized iota");
        if (!is_float(t.dt) && t.dt != HF_S32) c.unsupported("iota of an 8-bit or 4-bit integer type");
        // the index converts to f32 first: one rounding only while it is exact there
        if ((t.dt == HF_BF16 || t.dt == HF_F16) && !n.attr.empty() && t.dims[n.attr[0]] > (int64_t(1) << 24))
          c.unsupported("16-bit float iota longer than 2^24");
        break;
      case HF_PAD: {
        need_operands(src, 2, c);
        const Type &o = opt(0), &pv = opt(1);
        if (t.dt != o.dt || pv.dt != o.dt)
          c.invalid("element_type(operand) = element_type(padding_value) = element_type(result) violated (C1)");
        if (quantized || o.quant >= 0 || pv.quant >= 0) c.unsupported("pad of quantized values");
        if (pv.rank != 0) c.invalid("padding_value must be a 0-dimensional tensor (I2)");
        if ((int)n.attr.size() != 3 * o.rank || o.rank != t.rank)
          c.invalid("size(edge_padding_low) = size(edge_padding_high) = size(interior_padding) = rank(operand) "
                    "violated (C2)");
        for (int d = 0; d < o.rank; ++d) {
          const int64_t lo = n.attr[d], hi = n.attr[o.rank + d], in = n.attr[2 * o.rank + d];
          if (in < 0) c.invalid("0 <= interior_padding violated (C3)");
          if (t.dims[d] != o.dims[d] + lo + std::max<int64_t>(o.dims[d] - 1, 0) * in + hi)
            c.invalid("shape(result) = shape(operand) + edge_padding_low + max(shape(operand) - 1, 0) * "
                      "interior_padding + edge_padding_high violated (C4)");
        }
        break;
      }
      case HF_CONCATENATE: {
        if (n.opd.empty()) c.invalid("0 < size(inputs) violated (C3)");
        if (n.attr.size() != 1 || n.attr[0] < 0 || n.attr[0] >= opt(0).rank)
          c.invalid("0 <= dimension < rank(inputs[0]) violated (C4)");
        const int cd = n.attr.empty() ? 0 : (int)n.attr[0];
        int64_t total = 0;
        for (size_t k = 0; k < n.opd.size(); ++k) {
          const Type &o = opt((int)k);
          if (o.dt != opt(0).dt) c.invalid("same(element_type(inputs...)) violated (C1)");
          if (o.quant >= 0) c.unsupported("concatenate of quantized values");
          if (o.rank != t.rank) c.invalid("same(shape(inputs...)) except dim(inputs..., dimension) violated (C2)");
          for (int d = 0; d < t.rank; ++d)
            if (d != cd && o.dims[d] != t.dims[d])
              c.invalid("same(shape(inputs...)) except dim(inputs..., dimension) violated (C2)");
          total += o.dims[cd];
        }
        if (t.dt != opt(0).dt) c.invalid("element_type(result) = element_type(inputs[0]) violated (C5)");
        if (quantized) c.unsupported("concatenate of quantized values");
        if (t.dims[cd] != total) c.invalid("dim(result, dimension) = sum of dim(inputs..., dimension) violated (C6)");
        break;
      }
      case HF_SLICE: {
        // start_indices, limit_indices (the attributes "Programs" names) and
        // strides; the op's own section lies in the part of the pages that
        // is cut off, so the constraints are those of its definition:
        // result[i] = operand[start + i * strides].
        need_operands(src, 1, c);
        const Type &o = opt(0);
        if (t.dt != o.dt) c.invalid("element_type(operand) = element_type(result) violated");
        if (quantized || o.quant >= 0) c.unsupported("slice of quantized values");
        if ((int)n.attr.size() != 3 * o.rank || o.rank != t.rank)
          c.invalid("size(start_indices) = size(limit_indices) = size(strides) = rank(operand) violated");
        for (int d = 0; d < o.rank; ++d) {
          const int64_t st = n.attr[d], lim = n.attr[o.rank + d], step = n.attr[2 * o.rank + d];
          if (!(0 <= st && st <= lim && lim <= o.dims[d])) c.invalid("0 <= start_indices <= limit_indices <= shape(operand) violated");
          if (step < 1) c.invalid("0 < strides violated");
          if (t.dims[d] != (lim - st + step - 1) / step)
            c.invalid("shape(result) = ceil((limit_indices - start_indices) / strides) violated");
        }
        break;
      }
      case HF_DYNAMIC_SLICE: {
        // StableHLO Specification, "dynamic_slice", constraints C1-C5
        if (n.opd.empty()) c.invalid("expects the operand and one start index per dimension (C2)");
        const Type &o = opt(0);
        if (t.dt != o.dt) c.invalid("element_type(operand) = element_type(result) violated (C1)");
        if (quantized || o.quant >= 0) c.unsupported("dynamic_slice of quantized values");
        if ((int)n.opd.size() != 1 + o.rank || (int)n.attr.size() != o.rank)
          c.invalid("size(start_indices) = size(slice_sizes) = rank(operand) violated (C2)");
        if (t.rank != o.rank) c.invalid("shape(result) = slice_sizes violated (C5)");
        for (int d = 0; d < o.rank; ++d) {
          const Node &si = g.nodes[n.opd[1 + d]];
          if (si.t.rank != 0 || is_float(si.t.dt) || si.t.quant >= 0)
            c.invalid("start_indices must be 0-dimensional tensors of integer type (I2)");
          if (si.t.dt != opt(1).dt) c.invalid("same(type(start_indices...)) violated (C3)");
          if (si.op != HF_PARAMETER && si.op != HF_CONSTANT)
            c.unsupported("start indices must be parameters or constants");
          if (n.attr[d] < 0 || n.attr[d] > o.dims[d]) c.invalid("0 <= slice_sizes <= shape(operand) violated (C4)");
          if (t.dims[d] != n.attr[d]) c.invalid("shape(result) = slice_sizes violated (C5)");
        }
        break;
      }
      case HF_UNIFORM_DEQUANTIZE:
        need_operands(src, 1, c);
        if (opt(0).quant < 0) c.invalid("operand must have a quantized element type");
        if (quantized || t.dt != HF_F32) c.unsupported("the expressed type must be f32");
        if (!t.same_shape(opt(0))) c.invalid("shape(operand) = shape(result) violated");
        break;
      case HF_UNIFORM_QUANTIZE:
        need_operands(src, 1, c);
        if (!quantized) c.invalid("result must have a quantized element type");
        if (!t.same_shape(opt(0))) c.invalid("shape(operand) = shape(result) violated");
        if (opt(0).quant < 0 && opt(0).dt != HF_F32) c.unsupported("operand must be f32 or quantized");
        break;
      case HF_REDUCE: {
        if (src.reducer < HF_REDUCER_ADD || src.reducer > HF_REDUCER_ARGMAX) c.invalid("unknown reducer");
        need_operands(src, src.reducer == HF_REDUCER_ARGMAX ? 2 : 1, c);
        const Type &o = opt(0);
        if (src.reducer == HF_REDUCER_ARGMAX) {
          // variadic max/argmax: {values, indices} -> the index of the maximum
          const Node &ix = g.nodes[n.opd[1]];
          if (!is_float(o.dt) || o.quant >= 0) c.unsupported("argmax values must be floating point");
          if (!ix.t.same_shape(o)) c.invalid("all inputs must have the same dimensions");
          if (t.dt != HF_S32 || ix.t.dt != HF_S32) c.invalid("the argmax result and the indices must be s32");
          if (n.attr.size() != 1) c.unsupported("argmax over more than one dimension");
          if (ix.op != HF_IOTA || n.attr.empty() || ix.attr[0] != n.attr[0])
            c.unsupported("argmax indices must be an iota along the reduced dimension");
          if (n.cst != std::floor(n.cst) || n.cst < INT32_MIN || n.cst > INT32_MAX)
            c.invalid("the index init value must be an s32 value");
        } else {
          if (t.dt != o.dt)
            c.invalid("element_type(inputs) = element_type(init_values) = result type violated (C2, C8)");
          if (!is_float(t.dt) || o.quant >= 0) c.unsupported("only floating-point reductions are supported");
        }
        bool red[HF_MAX_RANK] = {false};
        for (int64_t d : n.attr) {
          if (d < 0 || d >= o.rank) c.invalid("0 <= dimensions < rank(inputs[0]) violated (C4)");
          if (red[d]) c.invalid("is_unique(dimensions) violated (C5)");
          red[d] = true;
        }
        int r = 0;
        for (int d = 0; d < o.rank; ++d) {
          if (red[d]) continue;
          if (r >= t.rank || t.dims[r] != o.dims[d])
            c.invalid("shape(results) = shape(inputs) without dimensions violated (C7)");
          ++r;
        }
        if (r != t.rank) c.invalid("shape(results) = shape(inputs) without dimensions violated (C7)");
        if (std::isnan(n.init)) c.unsupported("NaN init value");
        break;
      }
    }
  }

  expand_quantized_ops(g);

  // reachability from the root and user lists
  std::vector<int> stack{g.root};
  g.nodes[g.root].live = true;
  while (!stack.empty()) {
    int i = stack.back();
    stack.pop_back();
    for (int o : g.nodes[i].opd)
      if (!g.nodes[o].live) {
        g.nodes[o].live = true;
        stack.push_back(o);
      }
  }
  for (int i = 0; i < (int)g.nodes.size(); ++i) {
    if (!g.nodes[i].live) continue;
    for (int o : g.nodes[i].opd) g.nodes[o].users.push_back(i);
    if (g.nodes[i].op == HF_REDUCE) {
      if (g.reduce >= 0)
        fail(HF_ERR_UNSUPPORTED, "node " + std::to_string(i) + " (reduce): a fusion holds at most one reduce (its hero)");
      g.reduce = i;
    }
  }
  // An integer constant is only ever a dynamic_slice start index.
  for (int i = 0; i < (int)g.nodes.size(); ++i) {
    const Node &nd = g.nodes[i];
    if (!nd.live || nd.op != HF_CONSTANT || is_float(nd.t.dt)) continue;
    if (i == g.root) fail(HF_ERR_UNSUPPORTED, "node " + std::to_string(i) + " (constant): an integer constant as the root");
    for (int u : nd.users) {
      const Node &un = g.nodes[u];
      bool start = un.op == HF_DYNAMIC_SLICE;
      if (start && un.opd[0] == i) start = false;
      if (!start)
        fail(HF_ERR_UNSUPPORTED, "node " + std::to_string(i) +
                                     " (constant): integer constants are supported as dynamic_slice start indices only");
    }
  }
  // Everything that depends on the reduce is its epilogue, evaluated once per
  // reduce output: elementwise ops on the reduce's output space only.
  if (g.reduce >= 0 && g.reduce != g.root) {
    std::vector<char> dep(g.nodes.size(), 0);
    for (int i = 0; i < (int)g.nodes.size(); ++i) {
      if (!g.nodes[i].live) continue;
      dep[i] = i == g.reduce;
      for (int o : g.nodes[i].opd) dep[i] |= dep[o];
      if (!dep[i] || i == g.reduce) continue;
      switch (g.nodes[i].op) {
        case HF_ADD: case HF_SUBTRACT: case HF_MULTIPLY: case HF_DIVIDE: case HF_MAXIMUM: case HF_MINIMUM:
        case HF_LOG: case HF_EXP: case HF_TANH: case HF_NEGATE: case HF_ABS: case HF_CONVERT:
        case HF_UNIFORM_DEQUANTIZE: case HF_UNIFORM_QUANTIZE:
          break;
        default:
          fail(HF_ERR_UNSUPPORTED, "node " + std::to_string(i) + " (" + op_name(g.nodes[i].op) +
                                       "): only elementwise ops may follow the reduce");
      }
    }
  }
  return g;
}

}  // namespace hf
