// codegen.cpp -- HIP source for one planned fusion.
//
// Each partition becomes one __device__ function of its root node's index
// (XLA:GPU Emitters, "Subgraph functions": one index argument per dimension,
// one result), computing V lanes that advance along the function's lane
// dimension.  Parameters are read through the composed output-to-input index
// maps ("Indexing transforms"); a read that is contiguous along the lane
// becomes one raw vector load, a read that does not move with the lane one
// scalar load, anything else one load per lane.
//
// Loads are split from compute: every partition function F comes with a
// register struct hf_R_F and a fetch function F_fetch that issues all of F's
// global loads (and those of the partitions F calls) into that struct.  The
// hero templates call the fetch functions of a whole step (several rows,
// tile rows or row chunks) before any compute, so all of the step's loads
// are in flight together; the compute function F only unpacks registers.
//
// The pipelined loop hero (HF_PIPE) splits the loads once more: those whose
// index does not move with the row (per-axis quantization arrays, a bias
// broadcast along the rows, scalars) go to a second struct hf_I_F, loaded
// once per thread by F_inv before any row is fetched, so that the compute of
// the first row waits for its own row only and not for rows fetched ahead.
#include <cmath>
#include <cstdio>
#include <cstdlib>
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
    case HF_S4: case HF_U4: return "unsigned char";  // two elements per byte
    case HF_S32: return "int";
  }
  return "void";
}

bool reg_is_float(const Type &t) { return is_float(t.dt) && t.quant < 0; }

// Per-axis zero points live on the device one byte per entry, also for 4-bit
// storage types (as the 8-bit type of the same signedness).
hf_dtype zp_dtype(hf_dtype storage) {
  return storage == HF_S4 ? HF_S8 : storage == HF_U4 ? HF_U8 : storage;
}
const char *rtype(const Type &t) { return reg_is_float(t) ? "float" : "int"; }

std::string rnd(hf_dtype dt, const std::string &x) {
  if (dt == HF_BF16) return "hf_rnd_bf16(" + x + ")";
  if (dt == HF_F16) return "hf_rnd_f16(" + x + ")";
  return x;
}

// register value of one stored element
std::string elem_value(hf_dtype dt, const std::string &x) {
  switch (dt) {
    case HF_F32: return x;
    case HF_BF16: return "hf_bf16_bits(" + x + ")";
    case HF_F16: return "hf_f16_bits(" + x + ")";
    default: return "(int)" + x;
  }
}

struct Body {
  std::ostringstream os;     // compute
  std::ostringstream fetch;  // loads into R
  std::ostringstream members;
  std::ostringstream inv_fetch;    // row-invariant loads into I (pipelined loop)
  std::ostringstream inv_members;
  std::ostringstream inv_pin;
  std::map<std::string, std::string> memo;
  int root = -1;
  int lane = -1;
  int V = 1;
  int tmp = 0;
  int nmem = 0;
  int ninv = 0;
  bool tile = false;
  bool rleaf = false;     // the context's leaf is a reduced value passed in (hf_rv)
};

class Gen {
 public:
  Gen(const Graph &g, Plan &P) : g_(g), P_(P) {
    const char *nt = std::getenv("HF_NT");  // tuning knob: bit 0 loads, bit 1 stores
    nt_loads_ = nt ? (std::atoi(nt) & 1) : true;
    // A hero that keeps the next step's loads in flight while it computes
    // needs every load of a step in its fetch phase, small arrays included.
    for (auto &m : P.macros) {
      if (m.first == "HF_RR_PIPE" && m.second) fetch_all_ = true;
      // The pipelined loop fetches every row-dependent load of a row ahead
      // of its compute and loads the row-invariant ones once (hf_I_F).
      if (m.first == "HF_PIPE" && m.second) inv_split_ = true;
    }
  }

  // Emits (once) the struct, fetch and compute functions of the partition
  // rooted at `node` with lanes along `lane`; returns the function name.
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
    b.tile = c.leaf >= 0 && P_.hero == HF_HERO_TRANSPOSE;
    b.rleaf = c.leaf >= 0 && P_.hero != HF_HERO_TRANSPOSE;
    std::string v = val(ci, b, node, identity_index(t.rank));
    std::string idx;
    for (int d = 0; d < t.rank; ++d) idx += ", int i" + std::to_string(d);
    std::string tile = b.tile ? ", const " + tile_type() + " *__restrict__ hf_tile, int hf_w0, int hf_u0" : "";
    if (b.rleaf) tile += ", float hf_rv";
    std::ostringstream f;
    f << "// partition of node " << node << " (" << op_name(g_.nodes[node].op) << "), lanes along "
      << (lane >= 0 ? "i" + std::to_string(lane) : std::string("nothing")) << "\n";
    f << "struct hf_R_" << name << " {\n" << b.members.str() << "  char hf_pad;\n};\n";
    f << "__device__ __forceinline__ void " << name << "_fetch(const HfArgs &A" << idx << ", hf_R_" << name
      << " &R) {\n" << b.fetch.str() << "  (void)A; (void)R;\n}\n";
    std::string inv;
    if (inv_split_) {
      // row-invariant loads, and a pin that keeps them in registers: after
      // it the compiler cannot re-issue them (as rematerialized loads) behind
      // rows already in flight
      f << "struct hf_I_" << name << " {\n" << b.inv_members.str() << "  char hf_pad;\n};\n";
      f << "__device__ __forceinline__ void " << name << "_inv(const HfArgs &A" << idx << ", hf_I_" << name
        << " &I) {\n" << b.inv_fetch.str() << "  (void)A; (void)I;\n}\n";
      f << "__device__ __forceinline__ void " << name << "_pin(hf_I_" << name << " &I) {\n" << b.inv_pin.str()
        << "  (void)I;\n}\n";
      inv = ", const hf_I_" + name + " &I";
    }
    f << "__device__ __forceinline__ void " << name << "(const HfArgs &A" << tile << idx << ", const hf_R_" << name
      << " &R" << inv << ", " << rtype(t) << " (&hf_out)[" << c.V << "]) {\n";
    f << b.os.str();
    f << "#pragma unroll\n  for (int l = 0; l < " << c.V << "; ++l) hf_out[l] = " << v << "[l];\n  (void)A; (void)R;"
      << (inv_split_ ? " (void)I;" : "") << "\n}\n\n";
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
  std::string member(Body &b) { return "s" + std::to_string(b.nmem++); }

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

  // The condition under which a value read at index E is used.  pad and
  // concatenate read their operands at a clamped index (hf_clampi(x, lo, hi),
  // always in range) and select the operand's value only where the clamp
  // leaves x unchanged: elsewhere the result is the padding value or another
  // operand.  So a load whose index holds clamps is needed only where every
  // one of them is the identity; this returns that conjunction ("" when the
  // index holds no clamp).
  static std::string clamp_guard(const Index &E) {
    static const std::string key = "hf_clampi(";
    std::string g;
    for (const Term &t : E) {
      if (t.k != Term::EXPR) continue;
      for (size_t p = t.e.find(key); p != std::string::npos; p = t.e.find(key, p + 1)) {
        // the three arguments, split at the commas of depth one
        std::vector<std::string> arg(1);
        int depth = 1;
        size_t q = p + key.size();
        for (; q < t.e.size() && depth > 0; ++q) {
          const char ch = t.e[q];
          if (ch == '(') ++depth;
          if (ch == ')' && --depth == 0) break;
          if (ch == ',' && depth == 1) arg.emplace_back();
          else arg.back() += ch;
        }
        if (depth != 0 || arg.size() != 3) fail(HF_ERR_UNSUPPORTED, "codegen: unreadable clamp in an index");
        for (std::string &a : arg) {
          const size_t b0 = a.find_first_not_of(' '), b1 = a.find_last_not_of(' ');
          a = b0 == std::string::npos ? a : a.substr(b0, b1 - b0 + 1);
        }
        if (!g.empty()) g += " && ";
        g += "(" + arg[0] + ") >= (" + arg[1] + ") && (" + arg[0] + ") <= (" + arg[2] + ")";
      }
    }
    return g;
  }

  // Where a load goes: the fetch struct R (streaming operands; every load of
  // a hero that fetches whole steps ahead), the row-invariant struct I
  // (pipelined loop), or the compute function itself (small arrays, hoisted
  // out of the hero's row loop by the compiler).
  struct Dest {
    int kind;  // 0 compute, 1 R, 2 I
    std::string name;
    std::ostringstream &os;
  };
  Dest dest(Body &b, const Index &E, bool stream) {
    if (inv_split_ && !stream && row_invariant(E, b.lane)) return {2, "I.i" + std::to_string(b.ninv++), b.inv_fetch};
    if (stream || fetch_all_ || inv_split_) return {1, "R." + member(b), b.fetch};
    return {0, "w" + std::to_string(b.tmp++), b.os};
  }
  void declare(Body &b, const Dest &d, const std::string &type, int count) {
    const std::string dims = count ? "[" + std::to_string(count) + "]" : "";
    if (d.kind == 0) {
      b.os << "  " << type << " " << d.name << dims << ";\n";
      return;
    }
    (d.kind == 1 ? b.members : b.inv_members) << "  " << type << " " << d.name.substr(2) << dims << ";\n";
    // 32- and 64-bit values are pinned in registers (narrower ones are left)
    if (d.kind == 2 && (type == "hf_u32" || type == "float" || type == "int" || type == "double")) {
      if (count)
        b.inv_pin << "#pragma unroll\n  for (int k = 0; k < " << count << "; ++k) asm volatile(\"\" : \"+v\"(" << d.name
                  << "[k]));\n";
      else
        b.inv_pin << "  asm volatile(\"\" : \"+v\"(" << d.name << "));\n";
    }
  }
  // An index whose every term is a constant or the lane variable: the same
  // for every row of the loop hero (the row index feeds the other dims).
  static bool row_invariant(const Index &E, int lane) {
    for (const Term &t : E)
      if (t.k == Term::EXPR || (t.k == Term::VAR && t.var != lane)) return false;
    return true;
  }

  // dim of E that is the lane variable (or -1)
  static int lane_dim(const Index &E, int lane) {
    if (lane < 0) return -1;
    for (size_t d = 0; d < E.size(); ++d)
      if (E[d].k == Term::VAR && E[d].var == lane) return (int)d;
    return -1;
  }

  // s with every occurrence of the lane variable (the token i<lane>) replaced
  // by (i<lane> + l): an index expression evaluated at lane l of a vector.
  static std::string lane_sub(const std::string &s, int lane) {
    if (lane < 0) return s;
    const std::string v = "i" + std::to_string(lane);
    std::string r;
    size_t p = 0;
    for (size_t q = s.find(v); q != std::string::npos; q = s.find(v, q + 1)) {
      const size_t e = q + v.size();
      if ((q > 0 && std::isalnum((unsigned char)s[q - 1])) || (e < s.size() && std::isdigit((unsigned char)s[e]))) continue;
      r += s.substr(p, q - p) + "(" + v + " + l)";
      p = e;
    }
    return r + s.substr(p);
  }
  // Whether an index expression of E uses the lane variable other than as a
  // plain term of its own (then its lanes are read one by one).
  static bool lane_in_expr(const Index &E, int lane) {
    if (lane < 0) return false;
    for (const Term &t : E)
      if (t.k == Term::EXPR && lane_sub(t.e, lane) != t.e) return true;
    return false;
  }

  // Load of an array (parameter or per-axis quantization array) of element
  // type dt and shape t, at index E, into a new V-lane register array.  A
  // streaming operand's raw load goes to the fetch function (and the hero's
  // fetch phase); small, reused arrays are loaded where they are used, so a
  // value that does not change across the hero's steps is loaded once.
  std::string load(Body &b, int tag, const char *reg, hf_dtype dt, const Type &t, const std::string &ptr,
                   const Index &E, bool stream = false) {
    if (is_nibble(dt)) return load_nibbles(b, tag, reg, dt, t, ptr, E, stream);
    std::string v = "v" + std::to_string(tag) + "_" + std::to_string(b.tmp++);
    std::string off = offset(t, E);
    const int V = b.V;
    const int es = dtype_bytes(dt);
    int ld = V > 1 ? lane_dim(E, b.lane) : -1;
    std::vector<long long> st = phys_strides(t);
    b.os << "  " << reg << " " << v << "[" << V << "];\n";
    const Dest dst = dest(b, E, stream);
    std::string m = dst.name;
    std::ostringstream &ld_os = dst.os;
    auto decl = [&](const std::string &type, int count) { declare(b, dst, type, count); };
    const std::string guard = clamp_guard(E);
    if (V > 1 && lane_in_expr(E, b.lane)) {  // each lane's element read on its own
      decl(ctype(dt), V);
      const std::string g = lane_sub(guard, b.lane);
      ld_os << "#pragma unroll\n  for (int l = 0; l < " << V << "; ++l) " << m << "[l] = "
            << (g.empty() ? "" : "(" + g + ") ? ") << ptr << "[" << lane_sub(off, b.lane) << "]"
            << (g.empty() ? "" : " : 0") << ";\n";
      b.os << "#pragma unroll\n  for (int l = 0; l < " << V << "; ++l) " << v << "[l] = "
           << elem_value(dt, m + "[l]") << ";\n";
      return v;
    }
    if (ld < 0 || t.dims[ld] <= 1) {  // does not move with the lane
      decl(ctype(dt), 0);
      if (guard.empty()) ld_os << "  " << m << " = " << ptr << "[" << off << "];\n";
      else ld_os << "  if (" << guard << ") " << m << " = " << ptr << "[" << off << "]; else " << m << " = 0;\n";
      b.os << "  { const " << reg << " s = " << elem_value(dt, m) << ";\n";
      b.os << "#pragma unroll\n    for (int l = 0; l < " << V << "; ++l) " << v << "[l] = s; }\n";
    } else if (st[ld] == 1 && t.dims[ld] % V == 0 && V * es >= 4 && E[ld].add % V == 0 &&
               E[ld].dyn.empty()) {  // contiguous and aligned: raw vector load
      const int nb = V * es;
      decl("hf_u32", nb / 4);
      if (!guard.empty()) ld_os << "  if (" << guard << ")";
      ld_os << "  hf_raw_ld<" << nb << (stream && nt_loads_ ? ", true" : "") << ">(" << ptr << ", (long)(" << off << ") * "
            << es << ", " << m << ");\n";
      if (!guard.empty())
        ld_os << "  else {\n#pragma unroll\n    for (int k = 0; k < " << nb / 4 << "; ++k) " << m << "[k] = 0u;\n  }\n";
      switch (dt) {
        case HF_F32: b.os << "  hf_unpack_f32<" << V << ">(" << m << ", " << v << ");\n"; break;
        case HF_S32: b.os << "  hf_unpack_i32<" << V << ">(" << m << ", " << v << ");\n"; break;
        case HF_BF16: b.os << "  hf_unpack_h<" << V << ", false>(" << m << ", " << v << ");\n"; break;
        case HF_F16: b.os << "  hf_unpack_h<" << V << ", true>(" << m << ", " << v << ");\n"; break;
        case HF_S8: b.os << "  hf_unpack_b<" << V << ", true>(" << m << ", " << v << ");\n"; break;
        case HF_U8: b.os << "  hf_unpack_b<" << V << ", false>(" << m << ", " << v << ");\n"; break;
        case HF_S4: case HF_U4: break;  // 4-bit arrays are loaded by load_nibbles
      }
    } else {  // one load per lane
      decl(ctype(dt), V);
      ld_os << "  { const int o = " << off << ";\n#pragma unroll\n    for (int l = 0; l < " << V << "; ++l) " << m
            << "[l] = " << (guard.empty() ? "" : "(" + guard + ") ? ") << ptr << "[o + l * " << st[ld] << "]"
            << (guard.empty() ? "" : " : 0") << "; }\n";
      b.os << "#pragma unroll\n  for (int l = 0; l < " << V << "; ++l) " << v << "[l] = "
           << elem_value(dt, m + "[l]") << ";\n";
    }
    return v;
  }

  // Load of a 4-bit array (two elements per byte, the even linear index in
  // the low half).  A lane run of V >= 8 elements along the contiguous dim
  // starts at an even element offset (the run start is a multiple of V and
  // every other stride a multiple of that dim's size, itself a multiple of
  // V), so it is one raw load of V/2 bytes.  Otherwise each element is read
  // from its byte and its half picked by the offset's parity.
  std::string load_nibbles(Body &b, int tag, const char *reg, hf_dtype dt, const Type &t, const std::string &ptr,
                           const Index &E, bool stream) {
    std::string v = "v" + std::to_string(tag) + "_" + std::to_string(b.tmp++);
    std::string off = offset(t, E);
    const int V = b.V;
    const char *sgn = dt == HF_S4 ? "true" : "false";
    int ld = V > 1 ? lane_dim(E, b.lane) : -1;
    std::vector<long long> st = phys_strides(t);
    b.os << "  " << reg << " " << v << "[" << V << "];\n";
    const Dest dst = dest(b, E, stream);
    std::string m = dst.name;
    std::ostringstream &ld_os = dst.os;
    auto decl = [&](const std::string &type, int count) { declare(b, dst, type, count); };
    if (V > 1 && lane_in_expr(E, b.lane)) fail(HF_ERR_UNSUPPORTED, "codegen: a 4-bit array read lane by lane");
    const std::string bytes = "((const unsigned char *)" + ptr + ")";
    const std::string guard = clamp_guard(E);
    const std::string gq = guard.empty() ? "" : "(" + guard + ") ? ";
    const std::string gz = guard.empty() ? "" : " : 0";
    if (ld < 0 || t.dims[ld] <= 1) {  // does not move with the lane
      decl("unsigned char", 0);
      ld_os << "  " << m << " = " << gq << bytes << "[(" << off << ") >> 1]" << gz << ";\n";
      b.os << "  { const int s = hf_nibble<" << sgn << ">(" << m << ", (" << off << ") & 1);\n";
      b.os << "#pragma unroll\n    for (int l = 0; l < " << V << "; ++l) " << v << "[l] = s; }\n";
    } else if (st[ld] == 1 && t.dims[ld] % V == 0 && V % 2 == 0 && E[ld].add % V == 0 && E[ld].dyn.empty()) {
      decl("hf_u32", (V + 7) / 8);
      if (V >= 8) {
        if (!guard.empty()) ld_os << "  if (" << guard << ")";
        ld_os << "  hf_raw_ld<" << V / 2 << (stream && nt_loads_ ? ", true" : "") << ">(" << ptr << ", (long)(" << off
              << ") / 2, " << m << ");\n";
        if (!guard.empty())
          ld_os << "  else {\n#pragma unroll\n    for (int k = 0; k < " << (V / 2) / 4 << "; ++k) " << m
                << "[k] = 0u;\n  }\n";
      } else {  // 2 or 4 elements: one byte or one aligned 16-bit word
        const char *w = V == 4 ? "unsigned short" : "unsigned char";
        ld_os << "  " << m << "[0] = " << gq << "(hf_u32)*(const " << w << " *)((const unsigned char *)" << ptr
              << " + (long)(" << off << ") / 2)" << gz << ";\n";
      }
      b.os << "  { int s[" << V << "];\n    hf_unpack_n<" << V << ", " << sgn << ">(" << m << ", s);\n";
      b.os << "#pragma unroll\n    for (int l = 0; l < " << V << "; ++l) " << v << "[l] = s[l]; }\n";
    } else {  // one element per lane
      decl("unsigned char", V);
      ld_os << "  { const int o = " << off << ";\n#pragma unroll\n    for (int l = 0; l < " << V << "; ++l) " << m
            << "[l] = " << gq << bytes << "[(o + l * " << st[ld] << ") >> 1]" << gz << "; }\n";
      b.os << "  { const int o = " << off << ";\n#pragma unroll\n    for (int l = 0; l < " << V << "; ++l) " << v
           << "[l] = hf_nibble<" << sgn << ">(" << m << "[l], (o + l * " << st[ld] << ") & 1); }\n";
    }
    return v;
  }

  // Load of a double array (per-axis reciprocal scales) at index E, in the
  // compute function (a small, reused array).
  std::string load_f64(Body &b, int tag, const Type &t, const std::string &ptr, const Index &E) {
    std::string v = "v" + std::to_string(tag) + "_" + std::to_string(b.tmp++);
    std::string off = offset(t, E);
    const int V = b.V;
    int ld = V > 1 ? lane_dim(E, b.lane) : -1;
    b.os << "  double " << v << "[" << V << "];\n";
    if (inv_split_ && row_invariant(E, b.lane)) {  // loaded once, into I
      const Dest dst = dest(b, E, false);
      const bool scalar = ld < 0 || t.dims[ld] <= 1;
      declare(b, dst, "double", scalar ? 0 : V);
      if (scalar) {
        b.inv_fetch << "  " << dst.name << " = " << ptr << "[" << off << "];\n";
        b.os << "#pragma unroll\n  for (int l = 0; l < " << V << "; ++l) " << v << "[l] = " << dst.name << ";\n";
      } else {
        b.inv_fetch << "  { const int o = " << off << ";\n#pragma unroll\n    for (int l = 0; l < " << V << "; ++l) "
                    << dst.name << "[l] = " << ptr << "[o + l]; }\n";
        b.os << "#pragma unroll\n  for (int l = 0; l < " << V << "; ++l) " << v << "[l] = " << dst.name << "[l];\n";
      }
      return v;
    }
    if (ld < 0 || t.dims[ld] <= 1) {
      b.os << "  { const double s = " << ptr << "[" << off << "];\n#pragma unroll\n    for (int l = 0; l < " << V
           << "; ++l) " << v << "[l] = s; }\n";
    } else {
      b.os << "  { const int o = " << off << ";\n#pragma unroll\n    for (int l = 0; l < " << V << "; ++l) " << v
           << "[l] = " << ptr << "[o + l]; }\n";
    }
    return v;
  }

  // per-axis / per-tensor quantization parameters at index E: names of a
  // scale array, a zero-point array and (if rc) a reciprocal-scale array
  void quant_params(Body &b, int q, const Index &E, std::string *sc, std::string *zp, std::string *rc = nullptr) {
    const Quant &Q = g_.quants[q];
    if (Q.qdim < 0) {
      *sc = "hf_qs" + std::to_string(b.tmp++);
      *zp = "hf_qz" + std::to_string(b.tmp++);
      b.os << "  float " << *sc << "[" << b.V << "]; int " << *zp << "[" << b.V << "];\n";
      b.os << "#pragma unroll\n  for (int l = 0; l < " << b.V << "; ++l) { " << *sc << "[l] = " << flit(Q.scales[0])
           << "; " << *zp << "[l] = " << Q.zero_points[0] << "; }\n";
      if (rc) {
        *rc = "hf_qr" + std::to_string(b.tmp++);
        char buf[64];
        std::snprintf(buf, sizeof buf, "%a", reciprocal(Q.scales[0]));
        b.os << "  double " << *rc << "[" << b.V << "];\n#pragma unroll\n  for (int l = 0; l < " << b.V << "; ++l) "
             << *rc << "[l] = " << buf << ";\n";
      }
      return;
    }
    Type vt;
    vt.rank = 1;
    vt.dims[0] = (int64_t)Q.scales.size();
    vt.m2m[0] = 0;
    Index e1{E[Q.qdim]};
    vt.dt = HF_F32;
    *sc = load(b, 9000 + q, "float", HF_F32, vt, "A.qs" + std::to_string(q), e1);
    if (rc) *rc = load_f64(b, 9200 + q, vt, "A.qr" + std::to_string(q), e1);
    vt.dt = zp_dtype(Q.storage);
    *zp = load(b, 9100 + q, "int", vt.dt, vt, "A.qz" + std::to_string(q), e1);
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
    if (n == c.leaf && b.rleaf) {
      // the reduced value of this output element
      v = fresh(b, n);
      lanes(b, v, "float", "hf_rv");
    } else if (n == c.leaf) {
      // staged value from the LDS tile: [w][u] with u along the lane; u is
      // the tile's flattened U index over the merged dims (minor first)
      v = fresh(b, n);
      const Term &tw = E[P_.lane_in];
      std::string tu = term_str(E[P_.u_dims.back()]);
      for (int k = (int)P_.u_dims.size() - 2; k >= 0; --k)
        tu = "(" + tu + ") * " + std::to_string(t.dims[P_.u_dims[k]]) + " + " + term_str(E[P_.u_dims[k]]);
      b.os << "  " << rtype(t) << " " << v << "[" << b.V << "];\n";
      b.os << "  { const int o = (" << term_str(tw) << " - hf_w0) * HF_PITCH + (" << tu << " - hf_u0);\n";
      b.os << "#pragma unroll\n    for (int l = 0; l < " << b.V << "; ++l) " << v << "[l] = hf_tile[o + l]; }\n";
    } else if (nd.op == HF_PARAMETER) {
      v = load(b, n, rtype(t), t.dt, t, "A.p" + std::to_string(nd.param), E, is_streaming(g_, n));
    } else if (nd.op == HF_CONSTANT) {
      v = fresh(b, n);
      lanes(b, v, "float", flit(round_to_dtype(nd.cst, t.dt)));
    } else if (other_partition) {
      if (inv_split_) fail(HF_ERR_UNSUPPORTED, "codegen: the pipelined loop takes one partition");
      int ld = lane_dim(E, b.lane);
      std::string f = fn(ci, n, ld);
      std::string m = member(b);
      std::string args;
      for (int d = 0; d < t.rank; ++d) args += ", " + term_str(E[d]);
      b.members << "  hf_R_" << f << " " << m << ";\n";
      b.fetch << "  " << f << "_fetch(A" << args << ", R." << m << ");\n";
      v = fresh(b, n);
      b.os << "  " << rtype(t) << " " << v << "[" << b.V << "];\n  " << f << "(A";
      if (b.tile) b.os << ", hf_tile, hf_w0, hf_u0";
      if (b.rleaf) b.os << ", hf_rv";
      b.os << args << ", R." << m << ", " << v << ");\n";
    } else {
      std::vector<std::string> a;
      // a dynamic_slice reads its start indices at launch (HfArgs), so only
      // its operand is evaluated here
      const size_t nk = nd.op == HF_DYNAMIC_SLICE ? 1 : nd.opd.size();
      for (size_t k = 0; k < nk; ++k) {
        bool general = false;
        a.push_back(val(ci, b, nd.opd[k], operand_index(g_, n, (int)k, E, &general)));
      }
      auto A0 = [&](const char *f) { return std::string(f) + "(" + a[0] + "[l])"; };
      auto rnd = [&](hf_dtype dt, const std::string &e) { return hf::rnd(dt, e); };
      const std::string x = a.empty() ? "" : a[0] + "[l]";
      const std::string y = a.size() > 1 ? a[1] + "[l]" : "";
      switch (nd.op) {
        case HF_TRANSPOSE: case HF_BROADCAST_IN_DIM: case HF_RESHAPE: case HF_REVERSE: case HF_SLICE:
        case HF_DYNAMIC_SLICE:
          v = a[0];  // pure index transforms
          break;
        case HF_IOTA: {  // the index along iota_dimension
          const Term &tm = E[nd.attr[0]];
          const std::string i = b.V > 1 ? lane_sub(term_str(tm), b.lane) : term_str(tm);
          v = fresh(b, n);
          if (reg_is_float(t)) lanes(b, v, "float", rnd(t.dt, "(float)(" + i + ")"));
          else lanes(b, v, "int", i);
          break;
        }
        case HF_PAD: {  // an operand element where the index lands on one, else the padding value
          const Type &ot = g_.nodes[nd.opd[0]].t;
          const int r = ot.rank;
          std::string pred;
          for (int d = 0; d < r; ++d) {
            const long long lo = nd.attr[d], hi = nd.attr[r + d], step = nd.attr[2 * r + d] + 1;
            if (lo == 0 && hi == 0 && step == 1) continue;
            const std::string k = "(" + (b.V > 1 ? lane_sub(term_str(E[d]), b.lane) : term_str(E[d])) + " - (" +
                                  std::to_string(lo) + "))";
            pred += std::string(pred.empty() ? "" : " && ") + "(" + k + " >= 0 && " + k + " % " +
                    std::to_string(step) + " == 0 && " + k + " / " + std::to_string(step) + " < " +
                    std::to_string(ot.dims[d]) + ")";
          }
          v = fresh(b, n);
          lanes(b, v, rtype(t), pred.empty() ? x : "(" + pred + ") ? " + x + " : " + y);
          break;
        }
        case HF_CONCATENATE: {  // the input whose range along the dim holds the index
          const int cd = (int)nd.attr[0];
          std::vector<long long> end;
          long long off = 0;
          for (int o : nd.opd) end.push_back(off += g_.nodes[o].t.dims[cd]);
          std::string e = a.back() + "[l]";
          const std::string ic = b.V > 1 ? lane_sub(term_str(E[cd]), b.lane) : term_str(E[cd]);
          for (int k = (int)a.size() - 2; k >= 0; --k)
            e = "(" + ic + " < " + std::to_string(end[k]) + ") ? " + a[k] + "[l] : (" + e + ")";
          v = fresh(b, n);
          lanes(b, v, rtype(t), e);
          break;
        }
        case HF_ADD: v = fresh(b, n); lanes(b, v, "float", rnd(t.dt, x + " + " + y)); break;
        case HF_SUBTRACT: v = fresh(b, n); lanes(b, v, "float", rnd(t.dt, x + " - " + y)); break;
        case HF_MULTIPLY: v = fresh(b, n); lanes(b, v, "float", rnd(t.dt, x + " * " + y)); break;
        case HF_DIVIDE: v = fresh(b, n); lanes(b, v, "float", rnd(t.dt, x + " / " + y)); break;
        case HF_MAXIMUM: v = fresh(b, n); lanes(b, v, "float", "hf_max(" + x + ", " + y + ")"); break;
        case HF_MINIMUM: v = fresh(b, n); lanes(b, v, "float", "hf_min(" + x + ", " + y + ")"); break;
        case HF_NEGATE: v = fresh(b, n); lanes(b, v, "float", "-" + x); break;
        case HF_ABS: v = fresh(b, n); lanes(b, v, "float", "__builtin_fabsf(" + x + ")"); break;
        case HF_LOG: v = fresh(b, n); lanes(b, v, "float", rnd(t.dt, A0("logf"))); break;
        case HF_TANH:
          v = fresh(b, n);
          lanes(b, v, "float", t.dt == HF_BF16 ? rnd(t.dt, A0("hf_tanh_for_bf16")) : rnd(t.dt, A0("tanhf")));
          break;
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
          std::string sc, zp, rc;
          quant_params(b, t.quant, E, &sc, &zp, &rc);
          v = fresh(b, n);
          // the fusion's 8-bit result: only the low byte of each value is stored
          const bool low_byte = n == g_.root && dtype_bytes(t.dt) == 1;
          b.os << "  int " << v << "[" << b.V << "];\n  hf_quantize_v<" << b.V << (low_byte ? ", true" : "") << ">("
               << y0 << ", " << rc << ", " << zp << ", " << Q.smin << ", " << Q.smax << ", " << v << ");\n";
          (void)sc;
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
  bool nt_loads_ = true;
  bool inv_split_ = false;
  bool fetch_all_ = false;
  std::ostringstream defs_;
  std::map<std::string, bool> done_;
};

// "i<d> = t % D; t /= D" over dims (minor -> major)
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
    case HF_S4: case HF_U4: return "hf_st_n<" + v + ">(A.out, " + off + ", " + r + ");";
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

// Glue pair: NAME_fetch(A, <coords>, REGS &R) and NAME(A, <coords>, const REGS &R, out)
// that set up the index variables with `indices` and call the partition.
void glue_pair(std::ostringstream &glue, const std::string &name, const std::string &coords,
               const std::string &regs, const std::string &fn, const std::string &idx_code,
               const std::string &args, const std::string &extra_params, const std::string &extra_args,
               const std::string &out_decl) {
  glue << "__device__ __forceinline__ void " << name << "_fetch(const HfArgs &A, " << coords << ", " << regs
       << " &R) {\n" << idx_code << "  " << fn << "_fetch(A" << args << ", R);\n}\n";
  glue << "__device__ __forceinline__ void " << name << "(const HfArgs &A" << extra_params << ", " << coords
       << ", const " << regs << " &R, " << out_decl << ") {\n" << idx_code << "  " << fn << "(A" << extra_args << args
       << ", R, hf_res);\n}\n";
}

}  // namespace

std::string generate_source(const Graph &g, Plan &P, const std::string &prelude, const std::string &hero_text) {
  Gen gen(g, P);
  std::ostringstream glue, types;
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
      std::ostringstream ix;
      if (!rows.empty()) delinearize(ix, rt, rows, "row", "hf_t");
      else ix << "  (void)row;\n";
      if (c.lane >= 0) {
        set[c.lane] = 1;
        ix << "  const int i" << c.lane << " = colv * HF_V;\n";
      } else {
        ix << "  (void)colv;\n";
      }
      zero_dims(ix, rt, set);
      types << "typedef hf_R_" << f << " hf_regs_t;\n";
      bool pipe = false;
      for (auto &m : P.macros)
        if (m.first == "HF_PIPE" && m.second) pipe = true;
      if (pipe) {
        // the pipelined loop: row-invariant loads once (hf_loop_inv, at any
        // row of the thread), then pinned; the compute takes both structs
        types << "typedef hf_I_" << f << " hf_inv_t;\n";
        const std::string args = call_args(rt);
        glue << "__device__ __forceinline__ void hf_loop_eval_fetch(const HfArgs &A, int row, int colv, hf_regs_t &R) {\n"
             << ix.str() << "  " << f << "_fetch(A" << args << ", R);\n}\n";
        glue << "__device__ __forceinline__ void hf_loop_inv(const HfArgs &A, int row, int colv, hf_inv_t &I) {\n"
             << ix.str() << "  " << f << "_inv(A" << args << ", I);\n}\n";
        glue << "__device__ __forceinline__ void hf_loop_inv_pin(hf_inv_t &I) { " << f << "_pin(I); }\n";
        glue << "__device__ __forceinline__ void hf_loop_eval(const HfArgs &A, int row, int colv, const hf_regs_t &R, "
                "const hf_inv_t &I, hf_val_t (&hf_res)[HF_V]) {\n"
             << ix.str() << "  " << f << "(A" << args << ", R, I, hf_res);\n}\n";
      } else {
        glue_pair(glue, "hf_loop_eval", "int row, int colv", "hf_regs_t", f, ix.str(), call_args(rt), "", "",
                  "hf_val_t (&hf_res)[HF_V]");
      }
      glue << "__device__ __forceinline__ void hf_loop_store(const HfArgs &A, int row, int colv, const hf_val_t (&r)[HF_V]) {\n";
      glue << "  " << store_call(rt.dt, c.V, "row * " + std::to_string(DL) + " + colv * HF_V", "r") << "\n}\n";
      break;
    }
    case HF_HERO_TRANSPOSE: {
      const Ctx &ld = P.ctx[0], &st = P.ctx[1];
      std::string fl = gen.fn(0, ld.root, ld.lane);
      std::string fs = P.staged == g.root ? "" : gen.fn(1, st.root, st.lane);
      std::vector<int> batch;
      std::vector<char> set(rt.rank, 0), in_u(rt.rank, 0);
      for (int d : P.u_dims) in_u[d] = 1;
      for (int k = 0; k < rt.rank; ++k) {
        int d = rt.m2m[k];
        if (rt.dims[d] > 1 && d != P.lane_in && !in_u[d]) {
          batch.push_back(d);
          set[d] = 1;
        }
      }
      set[P.lane_in] = 1;
      for (int d : P.u_dims) set[d] = 1;
      std::ostringstream ix;
      if (!batch.empty()) delinearize(ix, rt, batch, "b", "hf_t");
      else ix << "  (void)b;\n";
      ix << "  const int i" << P.lane_in << " = w;\n";
      if (P.u_dims.size() == 1) ix << "  const int i" << P.lane_out << " = u;\n";
      else delinearize(ix, rt, P.u_dims, "u", "hf_u");  // the tile's U index over the merged dims
      zero_dims(ix, rt, set);
      types << "typedef hf_R_" << fl << " hf_ldregs_t;\n";
      glue_pair(glue, "hf_tr_load", "int b, int w, int u", "hf_ldregs_t", fl, ix.str(), call_args(rt), "", "",
                "hf_tile_t (&hf_res)[HF_VIN]");
      if (P.staged == g.root) {
        types << "struct hf_stregs_t { char hf_pad; };\n";
        glue << "__device__ __forceinline__ void hf_tr_eval_fetch(const HfArgs &A, int b, int w, int u, hf_stregs_t &R) {"
                " (void)A; (void)b; (void)w; (void)u; (void)R; }\n";
        glue << "__device__ __forceinline__ void hf_tr_eval(const HfArgs &A, const hf_tile_t *__restrict__ hf_tile, "
                "int hf_w0, int hf_u0, int b, int w, int u, const hf_stregs_t &R, hf_val_t (&r)[HF_VOUT]) {\n";
        glue << "  (void)A; (void)b; (void)R;\n  const int o = (w - hf_w0) * HF_PITCH + (u - hf_u0);\n";
        glue << "#pragma unroll\n  for (int l = 0; l < HF_VOUT; ++l) r[l] = hf_tile[o + l];\n}\n";
      } else {
        types << "typedef hf_R_" << fs << " hf_stregs_t;\n";
        glue_pair(glue, "hf_tr_eval", "int b, int w, int u", "hf_stregs_t", fs, ix.str(), call_args(rt),
                  ", const hf_tile_t *__restrict__ hf_tile, int hf_w0, int hf_u0", ", hf_tile, hf_w0, hf_u0",
                  "hf_val_t (&hf_res)[HF_VOUT]");
      }
      glue << "__device__ __forceinline__ void hf_tr_store(const HfArgs &A, int b, int w, int u, const hf_val_t (&r)[HF_VOUT]) {\n";
      glue << ix.str();
      glue << "  " << store_call(rt.dt, st.V, out_offset(rt), "r") << "\n}\n";
      break;
    }
    case HF_HERO_ROW_REDUCE: case HF_HERO_COLUMN_REDUCE: {
      const Ctx &c = P.ctx[0];
      const Node &R = g.nodes[g.reduce];  // the hero; the root may be an epilogue after it
      const Type &it = g.nodes[P.rin].t;
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
      std::string outoff;
      {
        std::vector<long long> ost = phys_strides(rt);
        for (int r = 0; r < rt.rank; ++r) {
          if (rt.dims[r] <= 1) continue;
          if (!outoff.empty()) outoff += " + ";
          outoff += "i" + std::to_string(kept_inc[r]);
          if (ost[r] != 1) outoff += " * " + std::to_string(ost[r]);
        }
        if (outoff.empty()) outoff = "0";
      }
      const hf_dtype odt = R.t.dt;
      std::string fin = rnd(odt, "hf_red<HF_OP>(" + flit(round_to_dtype(R.init, odt)) + ", acc)");
      std::string store;
      if (g.reduce != g.root) {
        // epilogue at the output index (root dim r is the input's kept dim kept_inc[r])
        std::string fe = gen.fn(1, g.root, -1);
        std::string args;
        for (int r = 0; r < rt.rank; ++r) args += ", i" + std::to_string(kept_inc[r]);
        store = "  hf_R_" + fe + " Re;\n  " + fe + "_fetch(A" + args + ", Re);\n  hf_val_t s1[1];\n  " + fe + "(A, v" +
                args + ", Re, s1);\n  " + store_call(rt.dt, 1, outoff, "s1") + "\n";
      } else if (rt.dt == HF_F32) {
        store = "  A.out[" + outoff + "] = v;\n";
      } else {
        store = "  { float s1[1] = {v}; " + store_call(rt.dt, 1, outoff, "s1") + " }\n";
      }
      bool is_row = P.hero == HF_HERO_ROW_REDUCE;
      std::ostringstream ix;
      const char *outer = is_row ? "row" : "c";
      if (is_row) {
        if (!kept.empty()) delinearize(ix, it, kept, "row", "hf_t");
        else ix << "  (void)row;\n";
        if (!reduced.empty()) delinearize(ix, it, reduced, "kv * HF_V", "hf_k");
        else ix << "  (void)kv;\n";
      } else {
        if (!kept.empty()) delinearize(ix, it, kept, "c", "hf_t");
        else ix << "  (void)c;\n";
        if (!reduced.empty()) delinearize(ix, it, reduced, "r", "hf_k");
        else ix << "  (void)r;\n";
      }
      zero_dims(ix, it, set);
      {
        std::string f = gen.fn(0, c.root, c.lane);
        types << "typedef hf_R_" << f << " hf_regs_t;\n";
        glue_pair(glue, is_row ? "hf_rr_eval" : "hf_cr_eval", is_row ? "int row, int kv" : "int r, int c", "hf_regs_t",
                  f, ix.str(), call_args(it), "", "", "float (&hf_res)[HF_V]");
      }
      if (R.reducer == HF_REDUCER_ARGMAX) {
        // max/argmax: the folds start from (init_value, HF_ARG_NONE); the
        // result is the index, or the index init where no element replaced
        // the initial pair
        glue << "#define HF_ARG_V0 " << flit(round_to_dtype(R.init, g.nodes[P.rin].t.dt)) << "\n#define HF_ARG_K0 ("
             << (long long)R.cst << ")\n";
        glue << "__device__ __forceinline__ void " << (is_row ? "hf_rr_store_arg" : "hf_cr_store_arg")
             << "(const HfArgs &A, int " << outer << ", int k) {\n";
        if (!kept.empty()) delinearize(glue, it, kept, outer, "hf_t");
        else glue << "  (void)" << outer << ";\n";
        std::vector<char> kset(it.rank, 0);
        for (int d : kept) kset[d] = 1;
        for (int d : kept_inc)
          if (!kset[d]) glue << "  const int i" << d << " = 0;\n";
        glue << "  A.out[" << outoff << "] = k == HF_ARG_NONE ? HF_ARG_K0 : k;\n}\n";
        break;
      }
      glue << "__device__ __forceinline__ void " << (is_row ? "hf_rr_store" : "hf_cr_store") << "(const HfArgs &A, int "
           << outer << ", float acc) {\n";
      if (!kept.empty()) delinearize(glue, it, kept, outer, "hf_t");
      else glue << "  (void)" << outer << ";\n";
      std::vector<char> kset(it.rank, 0);
      for (int d : kept) kset[d] = 1;
      for (int d : kept_inc)
        if (!kset[d]) glue << "  const int i" << d << " = 0;\n";
      glue << "  const float v = " << fin << ";\n" << store << "}\n";
      break;
    }
  }

  std::ostringstream src;
  if (const char *nt = std::getenv("HF_NT"))  // tuning knob: bit 0 loads, bit 1 stores
    src << "#define HF_NT_STORES " << ((std::atoi(nt) >> 1) & 1) << "\n";
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
    add(std::string("const ") + ctype(zp_dtype(g.quants[q].storage)) + " *", "qz" + std::to_string(q));
    add("const double *", "qr" + std::to_string(q));
  }
  add("void *", "ws");
  // dynamic_slice start indices held in parameters: read once per launch and
  // clamped into [0, dim(operand) - slice_size]
  for (int n = 0; n < (int)g.nodes.size(); ++n) {
    const Node &nd = g.nodes[n];
    if (!nd.live || nd.op != HF_DYNAMIC_SLICE) continue;
    const Type &ot = g.nodes[nd.opd[0]].t;
    for (int d = 0; d < ot.rank; ++d) {
      const Node &si = g.nodes[nd.opd[1 + d]];
      const long long hi = ot.dims[d] - nd.attr[d];
      if (si.op != HF_PARAMETER || hi <= 0) continue;
      const std::string p = "hf_a_p" + std::to_string(si.param);
      std::string v;
      switch (si.t.dt) {
        case HF_S4: v = "hf_nibble<true>(" + p + "[0], 0)"; break;
        case HF_U4: v = "hf_nibble<false>(" + p + "[0], 0)"; break;
        default: v = "(int)" + p + "[0]"; break;
      }
      const std::string name = dyn_start_name(n, d).substr(2);  // without "A."
      fields << "  int " << name << ";\n";
      init << ", hf_clampi(" << v << ", 0, " << hi << ")";
    }
  }
  src << "struct HfArgs {\n" << fields.str() << "};\n";
  src << "#define HF_KERNEL_PARAMS " << params.str() << "\n";
  src << "#define HF_ARGS_INIT {" << init.str() << "}\n";
  for (auto &m : P.macros) src << "#define " << m.first << " " << m.second << "\n";

  if (P.hero == HF_HERO_TRANSPOSE) src << "typedef " << gen.tile_type() << " hf_tile_t;\n";
  src << "typedef " << rtype(rt) << " hf_val_t;\n\n";
  src << gen.defs() << types.str() << glue.str() << "\n" << hero_text;
  // kernel name: hero, result type and shape, and a hash of the source, so
  // profiles can tell fusions apart
  std::string body = src.str();
  uint64_t h = 1469598103934665603ull;
  for (unsigned char ch : body) {
    h ^= ch;
    h *= 1099511628211ull;
  }
  std::ostringstream name;
  name << "hf_" << hero_template_name(P.hero) << "_" << dtype_name(rt.dt);
  for (int d = 0; d < rt.rank; ++d) name << (d ? "x" : "_") << rt.dims[d];
  char hx[16];
  std::snprintf(hx, sizeof hx, "_%08x", (unsigned)(h >> 32));
  name << hx;
  P.kernel_name = name.str();
  P.fold_name = P.kernel_name + "_fold";
  return "#define HF_KERNEL_NAME " + P.kernel_name + "\n#define HF_FOLD_NAME " + P.fold_name + "\n" + body;
}

}  // namespace hf
