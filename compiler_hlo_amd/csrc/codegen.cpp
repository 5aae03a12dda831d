// codegen.cpp -- HIP source for one planned fusion.
//
// Each partition becomes one __device__ function of its root node's index
// (XLA:GPU Emitters, "Subgraph functions": one index argument per dimension,
// one result), computing HF_V lanes that advance along the function's lane
// dimension.  Parameters are read through the composed output-to-input index
// maps ("Indexing transforms"); a read that is contiguous along the lane
// becomes one vector load, a read that does not move with the lane one scalar
// load, anything else one load per lane.  Functions of other partitions are
// called with the mapped index.  The hero glue (hf_loop_eval, hf_tr_load, ...)
// turns the hero's physical coordinates into logical indices and is followed
// by the hand-written hero template.
#include <cmath>
#include <cstdio>
#include <map>
#include <sstream>

#include "plan.h"

namespace hf {
namespace {

std::string flit(double v) {
  if (std::isnan(v)) return "__builtin_nanf(\"\")";
  if (std::isinf(v)) return v > 0 ? "__builtin_inff()" : "(-__builtin_inff())";
  char buf[64];
  std::snprintf(buf, sizeof buf, "%af", (double)(float)v);
  return std::string("(") + buf + ")";
}

const char *ctype(hf_dtype dt) {
  switch (dt) {
    case HF_F32: return "float";
    case HF_BF16: case HF_F16: return "hf_u16";
    case HF_S8: return "signed char";
    case HF_U8: return "unsigned char";
    case HF_S32: return "int";
  }
  return "void";
}

bool reg_is_float(const Type &t) { return is_float(t.dt) && t.quant < 0; }
const char *rtype(const Type &t) { return reg_is_float(t) ? "float" : "int"; }

std::string rnd(hf_dtype dt, const std::string &x) {
  if (dt == HF_BF16) return "hf_rnd_bf16(" + x + ")";
  if (dt == HF_F16) return "hf_rnd_f16(" + x + ")";
  return x;
}

struct Body {
  std::ostringstream os;
  std::map<std::string, std::string> memo;
  int root = -1;
  int lane = -1;
  int V = 1;
  int tmp = 0;
  bool tile = false;
};

class Gen {
 public:
  Gen(const Graph &g, Plan &P) : g_(g), P_(P) {}

  std::string fn(int ci, int node, int lane) {
    std::string name = "hf_c" + std::to_string(ci) + "_n" + std::to_string(node) + "_l" + std::to_string(lane + 1);
    if (done_.count(name)) return name;
    done_[name] = true;
    const Ctx &c = P_.ctx[ci];
    const Type &t = g_.nodes[node].t;
    Body b;
    b.root = node;
    b.lane = lane;
    b.V = c.V;
    b.tile = c.leaf >= 0;
    std::string v = val(ci, b, node, identity_index(t.rank));
    std::ostringstream f;
    f << "// partition of node " << node << " (" << op_name(g_.nodes[node].op) << "), lanes along "
      << (lane >= 0 ? "i" + std::to_string(lane) : std::string("nothing")) << "\n";
    f << "__device__ __forceinline__ void " << name << "(const HfArgs &A";
    if (b.tile) f << ", const " << tile_type() << " *__restrict__ hf_tile, int hf_w0, int hf_u0";
    for (int d = 0; d < t.rank; ++d) f << ", int i" << d;
    f << ", " << rtype(t) << " (&hf_out)[" << c.V << "]) {\n";
    f << b.os.str();
    f << "#pragma unroll\n  for (int l = 0; l < " << c.V << "; ++l) hf_out[l] = " << v << "[l];\n}\n\n";
    defs_ << f.str();
    return name;
  }

  std::string tile_type() const {
    if (P_.staged < 0) return "float";
    return rtype(g_.nodes[P_.staged].t);
  }

  std::string defs() const { return defs_.str(); }

 private:
  std::string fresh(Body &b, int n) { return "v" + std::to_string(n) + "_" + std::to_string(b.tmp++); }

  std::string offset(const Type &t, const Index &E) {
    std::vector<long long> st = phys_strides(t);
    std::string s;
    for (int d = 0; d < t.rank; ++d) {
      if (E[d].k == Term::ZERO || t.dims[d] <= 1 || st[d] == 0) continue;
      if (!s.empty()) s += " + ";
      s += term_str(E[d]);
      if (st[d] != 1) s += " * " + std::to_string(st[d]);
    }
    return s.empty() ? "0" : s;
  }

  // dim of E that is the lane variable (or -1)
  static int lane_dim(const Index &E, int lane) {
    if (lane < 0) return -1;
    for (size_t d = 0; d < E.size(); ++d)
      if (E[d].k == Term::VAR && E[d].var == lane) return (int)d;
    return -1;
  }

  std::string scalar_load(hf_dtype dt, const std::string &ptr, const std::string &off) {
    std::string x = ptr + "[" + off + "]";
    switch (dt) {
      case HF_F32: return x;
      case HF_BF16: return "hf_bf16_bits(" + x + ")";
      case HF_F16: return "(float)__builtin_bit_cast(_Float16, " + x + ")";
      default: return "(int)" + x;
    }
  }

  std::string vector_load(hf_dtype dt, const std::string &ptr, const std::string &off, int V,
                          const std::string &dst) {
    switch (dt) {
      case HF_F32: return "hf_ld_f32<" + std::to_string(V) + ">(" + ptr + ", " + off + ", " + dst + ");";
      case HF_BF16: return "hf_ld_h<" + std::to_string(V) + ", false>(" + ptr + ", " + off + ", " + dst + ");";
      case HF_F16: return "hf_ld_h<" + std::to_string(V) + ", true>(" + ptr + ", " + off + ", " + dst + ");";
      case HF_S8: return "hf_ld_b<" + std::to_string(V) + ", true>(" + ptr + ", " + off + ", " + dst + ");";
      case HF_U8: return "hf_ld_b<" + std::to_string(V) + ", false>(" + ptr + ", " + off + ", " + dst + ");";
      case HF_S32: return "hf_ld_i32<" + std::to_string(V) + ">(" + ptr + ", " + off + ", " + dst + ");";
    }
    return "";
  }

  // Load of an array (parameter or per-axis quantization array) of type
  // (dt, t) at index E into a new V-lane register array.
  std::string load(Body &b, int tag, const char *reg, hf_dtype dt, const Type &t, const std::string &ptr,
                   const Index &E) {
    std::string v = "v" + std::to_string(tag) + "_" + std::to_string(b.tmp++);
    std::string off = offset(t, E);
    int ld = b.V > 1 ? lane_dim(E, b.lane) : -1;
    std::vector<long long> st = phys_strides(t);
    b.os << "  " << reg << " " << v << "[" << b.V << "];\n";
    if (ld < 0 || t.dims[ld] <= 1) {
      b.os << "  { const " << reg << " s = " << scalar_load(dt, ptr, off) << ";\n";
      b.os << "#pragma unroll\n    for (int l = 0; l < " << b.V << "; ++l) " << v << "[l] = s; }\n";
    } else if (st[ld] == 1 && t.dims[ld] % b.V == 0) {
      b.os << "  " << vector_load(dt, ptr, off, b.V, v) << "\n";
    } else {
      b.os << "  { const int o = " << off << ";\n";
      b.os << "#pragma unroll\n    for (int l = 0; l < " << b.V << "; ++l) " << v << "[l] = "
           << scalar_load(dt, ptr, "o + l * " + std::to_string(st[ld])) << "; }\n";
    }
    return v;
  }

  // per-axis / per-tensor quantization parameters at index E: names of a
  // scale array and a zero-point array (V lanes each)
  void quant_params(Body &b, int q, const Index &E, std::string *sc, std::string *zp) {
    const Quant &Q = g_.quants[q];
    if (Q.qdim < 0) {
      *sc = "hf_qs" + std::to_string(b.tmp++);
      *zp = "hf_qz" + std::to_string(b.tmp++);
      b.os << "  float " << *sc << "[" << b.V << "]; int " << *zp << "[" << b.V << "];\n";
      b.os << "#pragma unroll\n  for (int l = 0; l < " << b.V << "; ++l) { " << *sc << "[l] = " << flit(Q.scales[0])
           << "; " << *zp << "[l] = " << Q.zero_points[0] << "; }\n";
      return;
    }
    Type vt;
    vt.rank = 1;
    vt.dims[0] = (int64_t)Q.scales.size();
    vt.m2m[0] = 0;
    Index e1{E[Q.qdim]};
    vt.dt = HF_F32;
    *sc = load(b, 9000 + q, "float", HF_F32, vt, "A.qs" + std::to_string(q), e1);
    vt.dt = Q.storage;
    *zp = load(b, 9100 + q, "int", Q.storage, vt, "A.qz" + std::to_string(q), e1);
  }

  void lanes(Body &b, const std::string &dst, const char *reg, const std::string &expr) {
    b.os << "  " << reg << " " << dst << "[" << b.V << "];\n";
    b.os << "#pragma unroll\n  for (int l = 0; l < " << b.V << "; ++l) " << dst << "[l] = " << expr << ";\n";
  }

  std::string val(int ci, Body &b, int n, const Index &E) {
    std::string key = std::to_string(n) + "@" + index_key(E);
    auto it = b.memo.find(key);
    if (it != b.memo.end()) return it->second;
    const Ctx &c = P_.ctx[ci];
    const Node &nd = g_.nodes[n];
    const Type &t = nd.t;
    std::string v;
    bool other_partition = n != b.root && c.part[n] >= 0 && c.part_root[c.part[n]] == n;
    if (n == c.leaf) {
      // staged value from the LDS tile: [w][u] with u along the lane
      v = fresh(b, n);
      const Term &tw = E[P_.lane_in], &tu = E[P_.lane_out];
      b.os << "  " << rtype(t) << " " << v << "[" << b.V << "];\n";
      b.os << "  { const int o = (" << term_str(tw) << " - hf_w0) * HF_PITCH + (" << term_str(tu) << " - hf_u0);\n";
      b.os << "#pragma unroll\n    for (int l = 0; l < " << b.V << "; ++l) " << v << "[l] = hf_tile[o + l]; }\n";
    } else if (nd.op == HF_PARAMETER) {
      v = load(b, n, rtype(t), t.dt, t, "A.p" + std::to_string(nd.param), E);
    } else if (nd.op == HF_CONSTANT) {
      v = fresh(b, n);
      lanes(b, v, "float", flit(round_to_dtype(nd.cst, t.dt)));
    } else if (other_partition) {
      int ld = lane_dim(E, b.lane);
      std::string f = fn(ci, n, ld);
      v = fresh(b, n);
      b.os << "  " << rtype(t) << " " << v << "[" << b.V << "];\n  " << f << "(A";
      if (b.tile) b.os << ", hf_tile, hf_w0, hf_u0";
      for (int d = 0; d < t.rank; ++d) b.os << ", " << term_str(E[d]);
      b.os << ", " << v << ");\n";
    } else {
      std::vector<std::string> a;
      for (int o : nd.opd) {
        bool general = false;
        a.push_back(val(ci, b, o, operand_index(g_, n, E, &general)));
      }
      auto A0 = [&](const char *f) { return std::string(f) + "(" + a[0] + "[l])"; };
      const std::string x = a.empty() ? "" : a[0] + "[l]";
      const std::string y = a.size() > 1 ? a[1] + "[l]" : "";
      switch (nd.op) {
        case HF_TRANSPOSE: case HF_BROADCAST_IN_DIM: case HF_RESHAPE:
          v = a[0];  // pure index transforms
          break;
        case HF_ADD: v = fresh(b, n); lanes(b, v, "float", rnd(t.dt, x + " + " + y)); break;
        case HF_SUBTRACT: v = fresh(b, n); lanes(b, v, "float", rnd(t.dt, x + " - " + y)); break;
        case HF_MULTIPLY: v = fresh(b, n); lanes(b, v, "float", rnd(t.dt, x + " * " + y)); break;
        case HF_DIVIDE: v = fresh(b, n); lanes(b, v, "float", rnd(t.dt, x + " / " + y)); break;
        case HF_MAXIMUM: v = fresh(b, n); lanes(b, v, "float", "hf_max(" + x + ", " + y + ")"); break;
        case HF_MINIMUM: v = fresh(b, n); lanes(b, v, "float", "hf_min(" + x + ", " + y + ")"); break;
        case HF_NEGATE: v = fresh(b, n); lanes(b, v, "float", "-" + x); break;
        case HF_ABS: v = fresh(b, n); lanes(b, v, "float", "__builtin_fabsf(" + x + ")"); break;
        case HF_LOG: v = fresh(b, n); lanes(b, v, "float", rnd(t.dt, A0("logf"))); break;
        case HF_TANH: v = fresh(b, n); lanes(b, v, "float", rnd(t.dt, A0("tanhf"))); break;
        case HF_EXP:
          v = fresh(b, n);
          lanes(b, v, "float", t.dt == HF_BF16 ? rnd(t.dt, A0("hf_exp_for_bf16")) : rnd(t.dt, A0("expf")));
          break;
        case HF_CONVERT: {
          const Type &ot = g_.nodes[nd.opd[0]].t;
          v = fresh(b, n);
          std::string src = reg_is_float(ot) ? x : "(float)" + x;
          // f32 target: exact from bf16/f16/8-bit ints; s32 -> f32 rounds in v_cvt_f32_i32
          lanes(b, v, "float", t.dt == HF_F32 ? src : rnd(t.dt, src));
          break;
        }
        case HF_UNIFORM_DEQUANTIZE: {
          const Type &ot = g_.nodes[nd.opd[0]].t;
          std::string sc, zp;
          quant_params(b, ot.quant, E, &sc, &zp);
          v = fresh(b, n);
          lanes(b, v, "float", sc + "[l] * (float)(" + x + " - " + zp + "[l])");
          break;
        }
        case HF_UNIFORM_QUANTIZE: {
          const Type &ot = g_.nodes[nd.opd[0]].t;
          std::string y0 = a[0];
          if (ot.quant >= 0) {  // requantize: dequantize with the operand's parameters first
            std::string sc, zp;
            quant_params(b, ot.quant, E, &sc, &zp);
            y0 = fresh(b, n);
            lanes(b, y0, "float", sc + "[l] * (float)(" + x + " - " + zp + "[l])");
          }
          const Quant &Q = g_.quants[t.quant];
          std::string sc, zp;
          quant_params(b, t.quant, E, &sc, &zp);
          v = fresh(b, n);
          lanes(b, v, "int", "hf_quantize(" + y0 + "[l], " + sc + "[l], " + zp + "[l], " + std::to_string(Q.smin) +
                                 ", " + std::to_string(Q.smax) + ")");
          break;
        }
        default:
          fail(HF_ERR_UNSUPPORTED, std::string("codegen: op ") + op_name(nd.op) + " inside a prologue");
      }
    }
    b.memo[key] = v;
    return v;
  }

  const Graph &g_;
  Plan &P_;
  std::ostringstream defs_;
  std::map<std::string, bool> done_;
};

// "i<d> = t % D; t /= D" over dims (minor -> major), size-1 dims set to 0
void delinearize(std::ostringstream &os, const Type &t, const std::vector<int> &dims, const std::string &from,
                 const char *tmp) {
  os << "  int " << tmp << " = " << from << ";\n";
  for (size_t k = 0; k < dims.size(); ++k) {
    int d = dims[k];
    if (k + 1 < dims.size())
      os << "  const int i" << d << " = " << tmp << " % " << t.dims[d] << "; " << tmp << " /= " << t.dims[d] << ";\n";
    else
      os << "  const int i" << d << " = " << tmp << ";\n";
  }
  os << "  (void)" << tmp << ";\n";
}

void zero_dims(std::ostringstream &os, const Type &t, const std::vector<char> &set) {
  for (int d = 0; d < t.rank; ++d)
    if (!set[d]) os << "  const int i" << d << " = 0;\n";
}

std::string call_args(const Type &t) {
  std::string s;
  for (int d = 0; d < t.rank; ++d) s += ", i" + std::to_string(d);
  return s;
}

std::string store_call(hf_dtype dt, int V, const std::string &off, const std::string &r) {
  std::string v = std::to_string(V);
  switch (dt) {
    case HF_F32: return "hf_st_f32<" + v + ">(A.out, " + off + ", " + r + ");";
    case HF_BF16: return "hf_st_h<" + v + ", false>(A.out, " + off + ", " + r + ");";
    case HF_F16: return "hf_st_h<" + v + ", true>(A.out, " + off + ", " + r + ");";
    case HF_S8: case HF_U8: return "hf_st_b<" + v + ">(A.out, " + off + ", " + r + ");";
    case HF_S32: return "hf_st_i32<" + v + ">(A.out, " + off + ", " + r + ");";
  }
  return "";
}

std::string out_offset(const Type &t) {
  std::vector<long long> st = phys_strides(t);
  std::string s;
  for (int d = 0; d < t.rank; ++d) {
    if (t.dims[d] <= 1) continue;
    if (!s.empty()) s += " + ";
    s += "i" + std::to_string(d);
    if (st[d] != 1) s += " * " + std::to_string(st[d]);
  }
  return s.empty() ? "0" : s;
}

}  // namespace

std::string generate_source(const Graph &g, Plan &P, const std::string &prelude, const std::string &hero_text) {
  Gen gen(g, P);
  std::ostringstream glue;
  const Node &R = g.nodes[g.root];
  const Type &rt = R.t;

  switch (P.hero) {
    case HF_HERO_LOOP: {
      const Ctx &c = P.ctx[0];
      std::string f = gen.fn(0, c.root, c.lane);
      std::vector<int> rows;
      std::vector<char> set(rt.rank, 0);
      for (int k = 0; k < rt.rank; ++k) {
        int d = rt.m2m[k];
        if (rt.dims[d] > 1 && d != c.lane) {
          rows.push_back(d);
          set[d] = 1;
        }
      }
      long long DL = c.lane >= 0 ? rt.dims[c.lane] : 1;
      glue << "__device__ __forceinline__ void hf_loop_eval(const HfArgs &A, int row, int colv, hf_val_t (&r)[HF_V]) {\n";
      if (!rows.empty()) delinearize(glue, rt, rows, "row", "hf_t");
      else glue << "  (void)row;\n";
      if (c.lane >= 0) {
        set[c.lane] = 1;
        glue << "  const int i" << c.lane << " = colv * HF_V;\n";
      } else {
        glue << "  (void)colv;\n";
      }
      zero_dims(glue, rt, set);
      glue << "  " << f << "(A" << call_args(rt) << ", r);\n}\n";
      glue << "__device__ __forceinline__ void hf_loop_store(const HfArgs &A, int row, int colv, const hf_val_t (&r)[HF_V]) {\n";
      glue << "  " << store_call(rt.dt, c.V, "row * " + std::to_string(DL) + " + colv * HF_V", "r") << "\n}\n";
      break;
    }
    case HF_HERO_TRANSPOSE: {
      const Ctx &ld = P.ctx[0], &st = P.ctx[1];
      std::string fl = gen.fn(0, ld.root, ld.lane);
      std::string fs = P.staged == g.root ? "" : gen.fn(1, st.root, st.lane);
      std::vector<int> batch;
      std::vector<char> set(rt.rank, 0);
      for (int k = 0; k < rt.rank; ++k) {
        int d = rt.m2m[k];
        if (rt.dims[d] > 1 && d != P.lane_in && d != P.lane_out) {
          batch.push_back(d);
          set[d] = 1;
        }
      }
      set[P.lane_in] = set[P.lane_out] = 1;
      auto indices = [&](std::ostringstream &os) {
        if (!batch.empty()) delinearize(os, rt, batch, "b", "hf_t");
        else os << "  (void)b;\n";
        os << "  const int i" << P.lane_in << " = w;\n  const int i" << P.lane_out << " = u;\n";
        zero_dims(os, rt, set);
      };
      glue << "__device__ __forceinline__ void hf_tr_load(const HfArgs &A, int b, int w, int u, hf_tile_t (&r)[HF_VIN]) {\n";
      indices(glue);
      glue << "  " << fl << "(A" << call_args(rt) << ", r);\n}\n";
      glue << "__device__ __forceinline__ void hf_tr_eval(const HfArgs &A, const hf_tile_t *__restrict__ hf_tile, int hf_w0, int hf_u0, int b, int w, int u, hf_val_t (&r)[HF_VOUT]) {\n";
      if (P.staged == g.root) {
        glue << "  (void)A; (void)b;\n  const int o = (w - hf_w0) * HF_PITCH + (u - hf_u0);\n";
        glue << "#pragma unroll\n  for (int l = 0; l < HF_VOUT; ++l) r[l] = hf_tile[o + l];\n}\n";
      } else {
        indices(glue);
        glue << "  " << fs << "(A, hf_tile, hf_w0, hf_u0" << call_args(rt) << ", r);\n}\n";
      }
      glue << "__device__ __forceinline__ void hf_tr_store(const HfArgs &A, int b, int w, int u, const hf_val_t (&r)[HF_VOUT]) {\n";
      indices(glue);
      glue << "  " << store_call(rt.dt, st.V, out_offset(rt), "r") << "\n}\n";
      break;
    }
    case HF_HERO_ROW_REDUCE: case HF_HERO_COLUMN_REDUCE: {
      const Ctx &c = P.ctx[0];
      const Type &it = g.nodes[P.rin].t;
      std::string f = gen.fn(0, c.root, c.lane);
      std::vector<char> red(it.rank, 0);
      for (int64_t d : R.attr) red[d] = 1;
      std::vector<int> kept, reduced;
      for (int d : P.order) (red[d] ? reduced : kept).push_back(d);
      std::vector<char> set(it.rank, 0);
      for (int d : P.order) set[d] = 1;
      // output index r of the reduce result = r-th kept input dim (increasing)
      std::vector<int> kept_inc;
      for (int d = 0; d < it.rank; ++d)
        if (!red[d]) kept_inc.push_back(d);
      std::ostringstream outoff;
      {
        std::vector<long long> ost = phys_strides(rt);
        std::string s;
        for (int r = 0; r < rt.rank; ++r) {
          if (rt.dims[r] <= 1) continue;
          if (!s.empty()) s += " + ";
          s += "i" + std::to_string(kept_inc[r]);
          if (ost[r] != 1) s += " * " + std::to_string(ost[r]);
        }
        outoff << (s.empty() ? "0" : s);
      }
      std::string fin = "hf_red<HF_OP>(" + flit(round_to_dtype(R.init, rt.dt)) + ", acc)";
      fin = rnd(rt.dt, fin);
      std::string store = rt.dt == HF_F32 ? "  A.out[" + outoff.str() + "] = v;\n"
                                          : "  { float s1[1] = {v}; " + store_call(rt.dt, 1, outoff.str(), "s1") + " }\n";
      bool is_row = P.hero == HF_HERO_ROW_REDUCE;
      const char *ev = is_row ? "hf_rr_eval" : "hf_cr_eval";
      glue << "__device__ __forceinline__ void " << ev << "(const HfArgs &A, int " << (is_row ? "row, int kv" : "r, int c")
           << ", float (&x)[HF_V]) {\n";
      std::vector<char> kset(it.rank, 0);
      if (is_row) {
        if (!kept.empty()) delinearize(glue, it, kept, "row", "hf_t");
        else glue << "  (void)row;\n";
        if (!reduced.empty()) delinearize(glue, it, reduced, "kv * HF_V", "hf_k");
        else glue << "  (void)kv;\n";
      } else {
        if (!kept.empty()) delinearize(glue, it, kept, "c", "hf_t");
        else glue << "  (void)c;\n";
        if (!reduced.empty()) delinearize(glue, it, reduced, "r", "hf_k");
        else glue << "  (void)r;\n";
      }
      zero_dims(glue, it, set);
      glue << "  " << f << "(A" << call_args(it) << ", x);\n}\n";
      const char *stn = is_row ? "hf_rr_store" : "hf_cr_store";
      glue << "__device__ __forceinline__ void " << stn << "(const HfArgs &A, int " << (is_row ? "row" : "c")
           << ", float acc) {\n";
      if (!kept.empty()) delinearize(glue, it, kept, is_row ? "row" : "c", "hf_t");
      else glue << "  (void)" << (is_row ? "row" : "c") << ";\n";
      std::vector<char> kset2(it.rank, 0);
      for (int d : kept) kset2[d] = 1;
      for (int d : kept_inc)
        if (!kset2[d]) glue << "  const int i" << d << " = 0;\n";
      glue << "  const float v = " << fin << ";\n" << store << "}\n";
      (void)kset;
      break;
    }
  }

  std::ostringstream src;
  src << prelude << "\n";
  // kernel parameters and the argument bundle
  std::ostringstream params, fields, init;
  auto add = [&](const std::string &type, const std::string &name) {
    if (!params.str().empty()) {
      params << ", ";
      init << ", ";
    }
    params << type << " __restrict__ hf_a_" << name;
    fields << "  " << type << " __restrict__ " << name << ";\n";
    init << "hf_a_" << name;
  };
  for (int k = 0; k < g.n_params; ++k) {
    int pn = g.param_node[k];
    hf_dtype dt = pn >= 0 ? g.nodes[pn].t.dt : HF_F32;
    add(std::string("const ") + ctype(dt) + " *", "p" + std::to_string(k));
  }
  add(std::string(ctype(rt.dt)) + " *", "out");
  for (int q : P.quant_args) {
    add("const float *", "qs" + std::to_string(q));
    add(std::string("const ") + ctype(g.quants[q].storage) + " *", "qz" + std::to_string(q));
  }
  add("void *", "ws");
  src << "struct HfArgs {\n" << fields.str() << "};\n";
  src << "#define HF_KERNEL_PARAMS " << params.str() << "\n";
  src << "#define HF_ARGS_INIT {" << init.str() << "}\n";
  for (auto &m : P.macros) src << "#define " << m.first << " " << m.second << "\n";
  if (P.hero == HF_HERO_TRANSPOSE) {
    src << "typedef " << gen.tile_type() << " hf_tile_t;\n";
  }
  src << "typedef " << rtype(rt) << " hf_val_t;\n\n";
  src << gen.defs() << glue.str() << "\n" << hero_text;
  return src.str();
}

}  // namespace hf
