// plan.cpp -- hero selection, index-map propagation, partitioning, geometry.
#include "plan.h"

#include <cctype>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <sstream>

namespace hf {

// ------------------------------------------------------------ index terms
std::string term_str(const Term &t) {
  switch (t.k) {
    case Term::ZERO: return "0";
    case Term::VAR: {
      if (!t.add && t.dyn.empty()) return "i" + std::to_string(t.var);
      std::string s = "(i" + std::to_string(t.var);
      if (t.add) s += " + " + std::to_string(t.add);
      if (!t.dyn.empty()) s += " + " + t.dyn;
      return s + ")";
    }
    case Term::EXPR: return "(" + t.e + ")";
  }
  return "0";
}

Term shifted(const Term &t, long long c, const std::string &dyn) {
  if (!c && dyn.empty()) return t;
  Term r = t;
  if (t.k == Term::VAR) {
    r.add += c;
    if (!dyn.empty()) r.dyn = r.dyn.empty() ? dyn : r.dyn + " + " + dyn;
    return r;
  }
  r.k = Term::EXPR;
  r.e = (t.k == Term::ZERO ? std::string("0") : term_str(t)) + " + " + std::to_string(c) + (dyn.empty() ? "" : " + " + dyn);
  return r;
}

std::string dyn_start_name(int n, int d) { return "A.ds" + std::to_string(n) + "_" + std::to_string(d); }

std::string index_key(const Index &E) {
  std::string s;
  for (const Term &t : E) {
    s += term_str(t);
    s += ',';
  }
  return s;
}

Index identity_index(int rank) {
  Index E(rank);
  for (int d = 0; d < rank; ++d) {
    E[d].k = Term::VAR;
    E[d].var = d;
  }
  return E;
}

std::vector<long long> phys_strides(const Type &t) {
  std::vector<long long> s(t.rank, 0);
  long long st = 1;
  for (int k = 0; k < t.rank; ++k) {
    s[t.m2m[k]] = st;
    st *= t.dims[t.m2m[k]];
  }
  return s;
}

int phys_minor(const Type &t) {
  for (int k = 0; k < t.rank; ++k)
    if (t.dims[t.m2m[k]] > 1) return t.m2m[k];
  return -1;
}

namespace {
// Whether index term t moves with the lane variable (lane < 0: assume it does).
bool moves_with_lane(const Term &t, int lane) {
  if (lane < 0) return true;
  if (t.k == Term::VAR) return t.var == lane;
  if (t.k != Term::EXPR) return false;
  const std::string v = "i" + std::to_string(lane);
  for (size_t p = t.e.find(v); p != std::string::npos; p = t.e.find(v, p + 1)) {
    const size_t e = p + v.size();
    if ((p == 0 || !std::isalnum((unsigned char)t.e[p - 1])) && (e >= t.e.size() || !std::isdigit((unsigned char)t.e[e])))
      return true;
  }
  return false;
}
}  // namespace

Index operand_index(const Graph &g, int n, int k, const Index &E, bool *general, int lane) {
  const Node &nd = g.nodes[n];
  const Type &ot = g.nodes[nd.opd[k]].t;
  auto expr = [](const std::string &e) {
    Term t;
    t.k = Term::EXPR;
    t.e = e;
    return t;
  };
  switch (nd.op) {
    case HF_REVERSE: {
      // operand_index[d] = dim(result, d) - result_index[d] - 1 along the reversed dims
      Index O = E;
      for (int64_t d : nd.attr)
        if (nd.t.dims[d] > 1) {
          O[d] = expr("(" + std::to_string(nd.t.dims[d] - 1) + " - (" + term_str(E[d]) + "))");
          if (moves_with_lane(E[d], lane)) *general = true;
        }
      return O;
    }
    case HF_PAD: {
      if (k == 1) return Index();  // padding_value: rank 0
      // result_index = low + operand_index * (interior + 1): read the operand
      // at the candidate index, clamped into range (the value is used only
      // where it is an operand element)
      Index O = E;
      const int r = ot.rank;
      for (int d = 0; d < r; ++d) {
        const long long lo = nd.attr[d], hi = nd.attr[r + d], step = nd.attr[2 * r + d] + 1;
        if (lo == 0 && hi == 0 && step == 1) continue;
        O[d] = expr("hf_clampi((" + term_str(E[d]) + " - (" + std::to_string(lo) + ")) / " + std::to_string(step) +
                    ", 0, " + std::to_string(std::max<long long>(ot.dims[d] - 1, 0)) + ")");
        if (moves_with_lane(E[d], lane)) *general = true;
      }
      return O;
    }
    case HF_CONCATENATE: {
      // input k holds result positions [off_k, off_k + dim_k) along the dim,
      // read clamped into range
      const int cd = (int)nd.attr[0];
      long long off = 0;
      for (int j = 0; j < k; ++j) off += g.nodes[nd.opd[j]].t.dims[cd];
      Index O = E;
      O[cd] = expr("hf_clampi(" + term_str(E[cd]) + " - " + std::to_string(off) + ", 0, " +
                   std::to_string(std::max<long long>(ot.dims[cd] - 1, 0)) + ")");
      if (moves_with_lane(E[cd], lane)) *general = true;
      return O;
    }
    case HF_SLICE: {
      // operand_index = start_indices + result_index * strides
      Index O = E;
      const int r = ot.rank;
      for (int d = 0; d < r; ++d) {
        const long long st = nd.attr[d], step = nd.attr[2 * r + d];
        if (step == 1 || nd.t.dims[d] <= 1) {
          O[d] = shifted(E[d], st, "");
          continue;
        }
        O[d] = expr(term_str(E[d]) + " * " + std::to_string(step) + " + " + std::to_string(st));
        if (moves_with_lane(E[d], lane)) *general = true;
      }
      return O;
    }
    case HF_DYNAMIC_SLICE: {
      // operand_index = clamp(0, start_indices, shape(operand) - slice_sizes)
      // + result_index (StableHLO Specification, "dynamic_slice").  A
      // constant start is clamped here; a parameter start is read and clamped
      // by the kernel at launch (dyn_start_name); a dim sliced whole has the
      // start 0 either way.
      if (k > 0) return Index();  // a start index: rank 0
      Index O = E;
      for (int d = 0; d < ot.rank; ++d) {
        const long long hi = ot.dims[d] - nd.attr[d];
        if (hi <= 0) continue;
        const Node &si = g.nodes[nd.opd[1 + d]];
        if (si.op == HF_CONSTANT) O[d] = shifted(E[d], std::min<long long>(std::max<long long>((long long)si.cst, 0), hi), "");
        else O[d] = shifted(E[d], 0, dyn_start_name(n, d));
      }
      return O;
    }
    case HF_TRANSPOSE: {
      // result dim d is operand dim perm[d]
      Index O(ot.rank);
      for (int d = 0; d < nd.t.rank; ++d) O[nd.attr[d]] = E[d];
      return O;
    }
    case HF_BROADCAST_IN_DIM: {
      // operand_index[d] = 0 if dim(operand, d) = 1 else result_index[bdims[d]]
      Index O(ot.rank);
      for (int d = 0; d < ot.rank; ++d)
        if (ot.dims[d] != 1) O[d] = E[nd.attr[d]];
      return O;
    }
    case HF_RESHAPE: {
      // same position in the lexicographic order of both index spaces
      std::vector<int> rn, on;
      for (int d = 0; d < nd.t.rank; ++d)
        if (nd.t.dims[d] != 1) rn.push_back(d);
      for (int d = 0; d < ot.rank; ++d)
        if (ot.dims[d] != 1) on.push_back(d);
      bool same = rn.size() == on.size();
      for (size_t k = 0; same && k < rn.size(); ++k) same = nd.t.dims[rn[k]] == ot.dims[on[k]];
      Index O(ot.rank);
      if (same) {  // only size-1 dims inserted or removed
        for (size_t k = 0; k < on.size(); ++k) O[on[k]] = E[rn[k]];
        return O;
      }
      if (ot.numel() == 0) return O;
      *general = true;
      std::string pos = "0";
      for (int d : rn) pos = "(" + pos + ")*" + std::to_string(nd.t.dims[d]) + "+" + term_str(E[d]);
      long long after = 1;
      for (int k = (int)on.size() - 1; k >= 0; --k) {
        int d = on[k];
        Term t;
        t.k = Term::EXPR;
        t.e = "((" + pos + ")/" + std::to_string(after) + ")%" + std::to_string(ot.dims[d]);
        O[d] = t;
        after *= ot.dims[d];
      }
      return O;
    }
    default:
      return E;  // elementwise ops, convert, quantize, dequantize
  }
}

// ------------------------------------------------------------ analysis
namespace {

void visit(const Graph &g, Ctx &c, int n, const Index &E) {
  if (!c.maps[n].insert(index_key(E)).second) return;
  c.in_ctx[n] = 1;
  if (n == c.leaf) return;
  const Node &nd = g.nodes[n];
  if (nd.op == HF_PARAMETER) {
    c.param_reads.push_back({n, E});
    return;
  }
  if (nd.op == HF_CONSTANT) return;
  // a dynamic_slice's start indices are read once per launch (kernel
  // arguments), not through the prologue
  const size_t nk = nd.op == HF_DYNAMIC_SLICE ? 1 : nd.opd.size();
  for (size_t k = 0; k < nk; ++k)
    visit(g, c, nd.opd[k], operand_index(g, n, (int)k, E, &c.general, c.lane));
}

// Partitioning (XLA:GPU Emitters, "Partitioning").  A node with one user is
// emitted with that user.  A node with several users is emitted with them
// when they all read it at the same indices.  When its users read it at
// different indices it becomes its own function, evaluated once per index,
// and each of those users heads a function of its own (the page splits
// param -> log -> {transpose, add} into three one-instruction functions).
void partition(const Graph &g, Ctx &c) {
  const int N = (int)g.nodes.size();
  c.part.assign(N, -1);
  c.part_root.clear();
  std::vector<std::vector<int>> users(N);
  for (int u = 0; u < N; ++u) {
    if (!c.in_ctx[u] || u == c.leaf) continue;
    if (g.nodes[u].op == HF_PARAMETER || g.nodes[u].op == HF_CONSTANT) continue;
    for (int o : g.nodes[u].opd)
      if (std::find(users[o].begin(), users[o].end(), u) == users[o].end()) users[o].push_back(u);
  }
  std::vector<char> split(N, 0);
  for (int n = 0; n < N; ++n)
    split[n] = c.in_ctx[n] && users[n].size() >= 2 && c.maps[n].size() >= 2;
  for (int n = N - 1; n >= 0; --n) {
    if (!c.in_ctx[n] || n == c.leaf) continue;
    const Node &nd = g.nodes[n];
    if (nd.op == HF_PARAMETER || nd.op == HF_CONSTANT) continue;
    bool head = n == c.root || split[n];
    for (int o : nd.opd)
      if (split[o]) head = true;
    if (!head) {
      int p = -1;
      for (int u : users[n]) {
        if (p < 0) p = c.part[u];
        else if (c.part[u] != p) head = true;
      }
      if (p < 0) head = true;
      if (!head) c.part[n] = p;
    }
    if (head) {
      c.part[n] = (int)c.part_root.size();
      c.part_root.push_back(n);
    }
  }
}

Ctx make_ctx(const Graph &g, int root, int lane, int leaf = -1) {
  Ctx c;
  c.root = root;
  c.lane = lane;
  c.leaf = leaf;
  c.maps.assign(g.nodes.size(), {});
  c.in_ctx.assign(g.nodes.size(), 0);
  visit(g, c, root, identity_index(g.nodes[root].t.rank));
  partition(g, c);
  return c;
}

int pow2_floor(long long x) {
  int p = 1;
  while ((long long)p * 2 <= x && p < (1 << 30)) p *= 2;
  return p;
}
int pow2_ceil(long long x) {
  int p = 1;
  while (p < x && p < (1 << 30)) p *= 2;
  return p;
}
// largest power of two <= cap dividing n (n > 0)
int vec_width(long long n, int cap) {
  int v = 1;
  while (v * 2 <= cap && n % (v * 2) == 0) v *= 2;
  return v;
}
long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

long long env_ll(const char *name, long long dflt) {
  const char *s = std::getenv(name);
  if (!s || !*s) return dflt;
  return std::atoll(s);
}

enum Access { CONTIG, UNIFORM, STRIDED, GATHER };

// How a param read at E moves when the lane variable `lane` advances.
Access classify(const Graph &g, int p, const Index &E, int lane) {
  const Type &t = g.nodes[p].t;
  if (lane < 0) return UNIFORM;
  int at = -1;
  for (int d = 0; d < t.rank; ++d) {
    if (E[d].k == Term::VAR && E[d].var == lane) at = d;
    // an expression index that moves with the lane (a div/mod reshape, a
    // reversed or padded lane dim) reads a gather; one that does not (a
    // reversed row dim) leaves the lane's accesses as they are
    if (E[d].k == Term::EXPR && moves_with_lane(E[d], lane)) return GATHER;
  }
  if (at < 0) return UNIFORM;
  return at == phys_minor(t) ? CONTIG : STRIDED;
}

bool large(const Graph &g, int p) { return is_streaming(g, p); }

// largest element width in bits among large params read contiguously along
// the lane (0 if none)
int stream_elem_bits(const Graph &g, const Ctx &c) {
  int b = 0;
  for (auto &pr : c.param_reads)
    if (large(g, pr.first) && classify(g, pr.first, pr.second, c.lane) == CONTIG)
      b = std::max(b, dtype_bits(g.nodes[pr.first].t.dt));
  return b;
}

// largest element size among large params read contiguously along the lane
int stream_elem_bytes(const Graph &g, const Ctx &c, int dflt) {
  int b = 0;
  for (auto &pr : c.param_reads)
    if (large(g, pr.first) && classify(g, pr.first, pr.second, c.lane) == CONTIG)
      b = std::max(b, dtype_bytes(g.nodes[pr.first].t.dt));
  return b ? b : dflt;
}

// The largest power of two <= V that divides the static offset (a slice
// start) of every parameter read along the lane, so that raw vector loads
// stay aligned.  Reads with a run-time offset along the lane load one
// element per lane whatever V is.
int align_lanes(const Ctx &c, int V) {
  if (c.lane < 0) return V;
  for (auto &pr : c.param_reads)
    for (const Term &t : pr.second)
      if (t.k == Term::VAR && t.var == c.lane)
        while (V > 1 && t.add % V != 0) V /= 2;
  return V;
}

bool all_coalesced(const Graph &g, const Ctx &c) {
  for (auto &pr : c.param_reads) {
    if (!large(g, pr.first)) continue;
    Access a = classify(g, pr.first, pr.second, c.lane);
    if (a == STRIDED || a == GATHER) return false;
  }
  return true;
}

// nodes of n's operand tree, params and constants excluded
void subtree(const Graph &g, int n, std::vector<char> &in) {
  if (in[n]) return;
  const Node &nd = g.nodes[n];
  if (nd.op == HF_PARAMETER || nd.op == HF_CONSTANT) return;
  in[n] = 1;
  for (int o : nd.opd) subtree(g, o, in);
}

bool exclusive(const Graph &g, int s) {
  std::vector<char> in(g.nodes.size(), 0);
  subtree(g, s, in);
  for (int x = 0; x < (int)g.nodes.size(); ++x) {
    if (!in[x] || x == s) continue;
    for (int u : g.nodes[x].users)
      if (!in[u]) return false;
  }
  return true;
}

// Algorithmic bytes: each parameter element the fusion needs read once, the
// result written once.  A parameter read through a slice needs only the
// elements its index maps reach, at most the evaluation space of each map;
// the rest of it is never touched.
void algorithmic(const Graph &g, Plan &P) {
  long long bytes = 0;
  const int N = (int)g.nodes.size();
  std::vector<char> used(N, 0), qused(g.quants.size(), 0), start_param(N, 0);
  std::vector<long long> reach(N, 0);
  for (Ctx &c : P.ctx) {
    for (int n = 0; n < N; ++n)
      if (c.in_ctx[n]) used[n] = 1;
    const long long space = g.nodes[c.root].t.numel();
    for (auto &pr : c.param_reads) reach[pr.first] += space;
  }
  for (int n = 0; n < N; ++n)
    if (used[n] && g.nodes[n].op == HF_DYNAMIC_SLICE)
      for (size_t k = 1; k < g.nodes[n].opd.size(); ++k)
        if (g.nodes[g.nodes[n].opd[k]].op == HF_PARAMETER) start_param[g.nodes[n].opd[k]] = 1;
  for (int n = 0; n < N; ++n) {
    const Node &nd = g.nodes[n];
    if (start_param[n] && !used[n]) bytes += storage_bytes(nd.t.dt, 1);
    if (!used[n]) continue;
    if (nd.op == HF_PARAMETER) bytes += storage_bytes(nd.t.dt, std::min<long long>(nd.t.numel(), reach[n] ? reach[n] : nd.t.numel()));
    if (nd.t.quant >= 0 && (nd.op == HF_UNIFORM_QUANTIZE || nd.op == HF_PARAMETER)) qused[nd.t.quant] = 1;
  }
  for (size_t q = 0; q < g.quants.size(); ++q)
    if (qused[q] && g.quants[q].qdim >= 0)
      bytes += (long long)g.quants[q].scales.size() * (4 + dtype_bytes(g.quants[q].storage));
  const Type &rt = g.nodes[g.root].t;
  bytes += storage_bytes(rt.dt, rt.numel());
  P.info.algorithmic_bytes = bytes;
}

void common_info(const Graph &g, Plan &P) {
  P.info.hero = P.hero;
  int np = 0;
  for (Ctx &c : P.ctx) np += (int)c.part_root.size();
  P.info.n_partitions = np;
  P.info.block_threads = P.block;
  P.info.grid_blocks = P.grid;
  P.info.lds_bytes = P.lds_bytes;
  P.info.workspace_bytes = P.ws_bytes;
  algorithmic(g, P);
  for (size_t q = 0; q < g.quants.size(); ++q)
    if (g.quants[q].qdim >= 0) P.quant_args.push_back((int)q);
}

// ------------------------------------------------------------ heroes
Plan plan_loop(const Graph &g, Ctx c) {
  Plan P;
  P.hero = HF_HERO_LOOP;
  const Type &rt = g.nodes[g.root].t;
  long long DL = c.lane >= 0 ? rt.dims[c.lane] : 1;
  // Whether the fusion also reads small arrays along the columns (per-axis
  // quantization parameters, a broadcast bias): every thread then holds V
  // elements of each of them in registers.
  bool small = false, per_axis = false;
  for (auto &pr : c.param_reads)
    if (!is_streaming(g, pr.first)) small = true;
  for (const Quant &q : g.quants)
    if (q.qdim >= 0) small = per_axis = true;
  int V = 1;
  int wbits_all = 0;  // widest of the result and the streaming inputs, in bits
  // An index map that moves with the lane (reverse, pad, concatenate or a
  // strided slice along the minor dim, a reshape that reorders it) still
  // gets vector lanes when the context is one partition of whole-byte types
  // with no per-axis arrays: each lane's element is then read on its own
  // (the index evaluated at lane base + l), and the result is stored as one
  // vector.
  bool gather = c.lane >= 0 && c.general && c.part_root.size() <= 1 && !is_nibble(rt.dt) &&
                env_ll("HF_LOOP_GATHER", 1) > 0;
  for (auto &pr : c.param_reads)
    if (is_nibble(g.nodes[pr.first].t.dt)) gather = false;
  for (const Quant &q : g.quants)
    if (q.qdim >= 0) gather = false;
  c.gather = gather;
  if (c.lane >= 0 && (!c.general || gather)) {
    // 128-bit lanes for the widest of the result and the streaming inputs,
    // except where every stream is 4-bit and column data is read: 32 elements
    // a lane then make few, register-heavy waves for what is mostly VALU work
    // (the per-axis s4 requantize with a bias measured 10.8 us at 32, 8.8 at
    // 16, 8.6 at 8 and 8.3 at 4 elements a lane; a per-tensor s4 requantize
    // keeps 32: 6.7 us against 8.1 at 16).
    const int wbits = std::max(dtype_bits(rt.dt), stream_elem_bits(g, c));
    wbits_all = wbits;
    const int vdef = small && wbits <= 4 ? 4 : 128 / wbits;
    V = vec_width(DL, std::max(1, (int)std::min<long long>(env_ll("HF_LOOP_VMAX", vdef), 128 / wbits)));
    V = align_lanes(c, V);
  }
  c.V = V;
  // A 4-bit result is stored a whole byte at a time: each lane needs an even
  // run along the physically minor dim (then that dim is even as well).
  if (is_nibble(rt.dt) && (c.lane < 0 || V % 2 != 0))
    fail(HF_ERR_UNSUPPORTED,
         std::string("a ") + dtype_name(rt.dt) +
             " result needs an even physically minor dim read without a gather along it (lanes write whole bytes)");
  long long cols_v = DL / V;
  long long rows = DL > 0 ? rt.numel() / DL : 0;
  int block = 256;
  long long tpr, rpb, nch;
  // Each wave takes its own rows of one 64-vector column strip: measured at
  // sustained clocks, 64 lanes per row segment beat whole-workgroup rows on
  // the streaming loops (f32 copy 73% -> 77% of peak, GELU 52% -> 54%, the
  // quantized add 57% -> 58.5%; an i8 copy and pad/reverse/concat tied).  A
  // fusion that also reads small arrays along the columns (per-axis
  // quantization parameters, a broadcast bias) shares that column data among
  // the waves through L1, and each thread keeps it in registers over four
  // rows, whose loads it issues together.
  // (128 lanes for one element a lane: reverse and concatenate along the
  // minor dim of f32[4096,4096] took 27.7 and 55.1 us against 29.4 and 59.2
  // with 64.)
  // (Rows of 2 MiB or more take whole-workgroup row segments again: four
  // waves on four such rows read at equal offsets megabytes apart.  A negate
  // over f32[4,4194304], [8,2097152], [16,1048576] and [32,524288] took
  // 27.2, 25.7, 24.8 and 24.5 us with 64 lanes and 22.7-23.0 with 256, and
  // bf16[16,1048576] 14.0 against 13.1; rows of 1 MiB lost 1-2% with 256
  // lanes: f32[64,262144] 22.6 -> 22.9 us, bf16[32,524288] 12.8 -> 13.0.)
  const bool long_rows = V > 1 && DL * (long long)wbits_all / 8 >= (2LL << 20);
  const long long tpr_cap = env_ll("HF_LOOP_TPR", V == 1 ? 128 : long_rows ? 256 : 64);
  if (cols_v >= tpr_cap) {
    tpr = tpr_cap;
    rpb = block / tpr;
    nch = ceil_div(cols_v, tpr);
  } else {
    tpr = std::max<long long>(1, cols_v);
    rpb = block / tpr;
    nch = 1;
  }
  //
  // Fusions of 8-bit streams with one partition (quantized arithmetic, and
  // the per-axis requantize with its column data) run software-pipelined:
  // each thread loads its column data once, then keeps the loads of the next
  // HF_PIPE rows in flight while it computes and stores the current one,
  // over HF_NR rows (a compile-time count, up to 16), in at least 256
  // workgroups (one wave per SIMD).  Loading every row up front left the
  // VALU idle until most of the data had arrived.  Measured at sustained
  // clocks: the per-axis requantize of i8[4096,4096] took 8.88 us with four
  // rows a thread loaded up front, and 7.47-7.52 us pipelined six rows deep
  // over 16 rows (7.69 four deep, 8.1 with eight rows a thread); the
  // quantized add of i8[4096,4096] went from 10.69 to 9.94 us (four deep,
  // 16 rows).  GELU in bf16 (VALU-bound), the f32 pad/reverse/concatenate
  // and si4 streams (2 bytes a lane) ran 8-12% slower pipelined and keep
  // the loop above.
  const bool pipe_any = c.part_root.size() == 1 && c.lane >= 0 && !c.general;
  const bool pipe = (pipe_any && wbits_all == 8 && V * 8 == 128 && env_ll("HF_LOOP_PIPE", 1) > 0) ||
                    (pipe_any && std::getenv("HF_LOOP_PIPE") && env_ll("HF_LOOP_PIPE", 0) > 0);
  // Rows a thread: four where per-axis quantization data is held over the
  // rows; otherwise (a broadcast bias or other small float arrays) two for
  // 4-byte streams and one for narrower ones.  Four rows a thread left
  // x + bias over f32[4096,4096] at 25.5 us and over bf16[4096,4096] at
  // 13.9 us; two (f32) and one (bf16) took 22.0 and 12.3-12.9 us, as the
  // plain copy-like loop does (f32 over [16,1048576] and [65536,256]:
  // 31.9 -> 25.6 and 26.6 -> 22.5 us).
  long long per = !small ? 1 : per_axis ? 4 : wbits_all >= 32 ? 2 : 1;
  // One element a lane (an index map that moves with the lane: reverse, pad
  // or concatenate along the minor dim, or an odd minor dim): up to eight
  // rows a thread, their loads issued together, while at least 1024
  // workgroups remain.  With one row a thread, reverse, pad and
  // concatenate along the minor dim of f32[4096,4096] ran at 3.1-3.5 TB/s;
  // with eight, 4.6-4.9 TB/s (reverse 38.5 -> 27.7 us, concatenate of two
  // 83.9 -> 55.1 us, with the 128-lane row segments above).
  if (V == 1) per = std::max<long long>(per, std::min<long long>(8, nch * ceil_div(rows, rpb) / 1024));
  long long target = env_ll("HF_LOOP_WGS", nch * ceil_div(ceil_div(rows, rpb), per));
  if (pipe && !std::getenv("HF_LOOP_WGS"))
    target = nch * std::max(ceil_div(256, nch), ceil_div(ceil_div(rows, rpb), 16));
  long long ngroups = std::max<long long>(1, std::min(ceil_div(rows, rpb), std::max<long long>(1, target / nch)));
  const long long rstep = ngroups * rpb;
  const long long nr = ceil_div(rows, rstep);
  const long long pd = pipe && nr <= 16 ? std::min(env_ll("HF_LOOP_PIPE", small ? 6 : 4), nr) : 0;
  P.ctx.push_back(c);
  P.block = block;
  P.grid = nch * ngroups;
  P.empty = rt.numel() == 0;
  P.macros = {{"HF_BLOCK", block}, {"HF_V", V}, {"HF_ROWS", rows}, {"HF_COLS_V", cols_v},
              {"HF_TPR", tpr}, {"HF_RPB", rpb}, {"HF_NCH", nch},
              {"HF_UNROLL", env_ll("HF_LOOP_UNROLL", V == 1 && per > 1 ? per : small ? 4 : 2)},
              {"HF_PIPE", pd}, {"HF_RSTEP", rstep}, {"HF_NR", nr}};
  P.info.vector_elems = V;
  P.info.elements = rt.numel();
  P.info.rows = rows;
  P.info.cols = DL;
  common_info(g, P);
  return P;
}

bool try_transpose(const Graph &g, const Ctx &loop, Plan *out) {
  const Type &rt = g.nodes[g.root].t;
  int lout = loop.lane;
  if (lout < 0 || is_nibble(rt.dt)) return false;
  int lin = -1;
  bool any = false;
  // A large parameter whose contiguous dim is read with a plain variable other
  // than the output's minor one is read transposed.  (Whether the load and
  // store phases can then run 128-bit lanes is checked on their own contexts
  // below.)
  for (auto &pr : loop.param_reads) {
    if (!large(g, pr.first)) continue;
    int pm = phys_minor(g.nodes[pr.first].t);
    if (pm < 0) continue;
    const Term &t = pr.second[pm];
    if (t.k == Term::EXPR) return false;
    if (t.k != Term::VAR || t.var == lout) continue;
    if (lin >= 0 && lin != t.var) return false;  // two different transposed directions
    lin = t.var;
    any = true;
  }
  if (!any || lin < 0 || lin == lout || rt.dims[lin] <= 1) return false;
  // candidate staged nodes: transposes read at identity from the root, then the root
  std::vector<int> cands;
  std::string id = index_key(identity_index(rt.rank));
  for (int n = 0; n < (int)g.nodes.size(); ++n)
    if (g.nodes[n].live && g.nodes[n].op == HF_TRANSPOSE && n != g.root && loop.maps[n].size() == 1 &&
        *loop.maps[n].begin() == id)
      cands.push_back(n);
  cands.push_back(g.root);
  for (int s : cands) {
    if (!exclusive(g, s)) continue;
    Ctx ld = make_ctx(g, s, lin);
    Ctx st = make_ctx(g, g.root, lout, s == g.root ? -1 : s);
    if (s == g.root) {
      // staging the root: the store phase only copies from LDS
      st = Ctx();
      st.root = g.root;
      st.leaf = g.root;
      st.lane = lout;
      st.maps.assign(g.nodes.size(), {});
      st.in_ctx.assign(g.nodes.size(), 0);
      st.in_ctx[g.root] = 1;
      st.part.assign(g.nodes.size(), -1);
    }
    if (ld.general || st.general) continue;
    if (!all_coalesced(g, ld) || !all_coalesced(g, st)) continue;
    Plan P;
    P.hero = HF_HERO_TRANSPOSE;
    P.staged = s;
    P.lane_in = lin;
    P.lane_out = lout;
    // The tile's U dim is the output's physically minor dim together with
    // the output dims that lie physically between it and W: for fixed W and
    // batch those are one contiguous run of the output, so a tile over their
    // flattened index writes whole lines (abs(transpose(exp x, {2,1,0})) on
    // f32[20,160,170]: the output's rows of 20 floats then are stored 3200 at
    // a time instead of 80 bytes per workgroup).  Vectors run along the minor
    // dim alone, so they never cross into the next index of a merged dim.
    std::vector<int> udims{lout};
    {
      int kin = 0, kout = 0;
      for (int k = 0; k < rt.rank; ++k) {
        if (rt.m2m[k] == lin) kin = k;
        if (rt.m2m[k] == lout) kout = k;
      }
      for (int k = kout + 1; k < kin; ++k)
        if (rt.dims[rt.m2m[k]] > 1) udims.push_back(rt.m2m[k]);
    }
    P.u_dims = udims;
    long long DU = 1, DW = rt.dims[lin];
    for (int d : udims) DU *= rt.dims[d];
    int vout = align_lanes(st, vec_width(rt.dims[lout], std::max(1, 16 / dtype_bytes(rt.dt))));
    int vin = align_lanes(ld, vec_width(DW, std::max(1, 16 / stream_elem_bytes(g, ld, dtype_bytes(g.nodes[s].t.dt)))));
    ld.V = vin;
    st.V = vout;
    const long long in_row_bytes = DW * stream_elem_bytes(g, ld, dtype_bytes(g.nodes[s].t.dt));
    // 4-byte elements on both sides whose input rows lie a power of two (at
    // least 8 KiB) apart: the row segments of a 64x64 tile then share their
    // low address bits, and with them their HBM channels.  Tiles 128 elements
    // wide in the load (512-byte row segments) and 32 in the store (128-byte
    // segments, whole cache lines), with one 128-bit vector per thread and
    // phase (1024 threads), measured 68% -> 72% of peak on f32[4096,4096]
    // and 68% -> 71% on f32[8192,2048]; other strides and 2-byte types keep
    // 64x64 (the narrow tile lost 2% on f32[4160,4160] and more on bf16).
    // Shorter power-of-two rows (512 B to 4 KiB) take it too when it makes
    // 2048 workgroups or more of whole 32-wide U extents (the shapes
    // measured): f32[65536,256] 26.6 -> 24.2 us,
    // f32[131072,128] 28.6 -> 24.2, f32[32768,1024] 54.0 -> 46.8; rows of
    // 2 KiB tie or lose a little (f32[32768,512] 23.9 -> 24.0 us,
    // f32[16384,512] 13.0 -> 13.2), and f32[4096,1024], a grid of 1024, ran
    // 7.7 us with 64x64 tiles and 7.9 narrow.
    const long long nb = rt.numel() / (DU * DW);
    const bool pow2_rows = in_row_bytes >= 512 && (in_row_bytes & (in_row_bytes - 1)) == 0;
    const bool narrow = pow2_rows && vin == 4 && vout == 4 &&
                        (in_row_bytes >= 8192 || (DU >= 32 && nb * ceil_div(DU, 32) * ceil_div(DW, 128) >= 2048));
    int tu = (int)std::min<long long>(env_ll("HF_TR_TU", narrow ? 32 : 64), pow2_ceil(DU));
    int tw = (int)std::min<long long>(env_ll("HF_TR_TW", narrow ? 128 : 64), pow2_ceil(DW));
    // A tiling that would leave fewer than two workgroups per CU (256 CUs)
    // takes the pages' 32x32 tile instead: abs(transpose(exp x, {2,1,0})) on
    // f32[20,160,170] ran 4.70 us with 64x64 tiles (150 workgroups) and
    // 3.67 us with 32x32 (600).
    // (The narrow tiles above keep their shape: they are for row strides of
    // a power of two.)
    if (!narrow && !std::getenv("HF_TR_TU") && !std::getenv("HF_TR_TW") &&
        nb * ceil_div(DU, tu) * ceil_div(DW, tw) < 512) {
      tu = std::min(tu, 32);
      tw = std::min(tw, 32);
    }
    tu = std::max(tu, vout);
    tw = std::max(tw, vin);
    long long ntu = ceil_div(DU, tu), ntw = ceil_div(DW, tw);
    int pitch = tu + 1;
    // Tile order.  U-tiles fastest keeps the writes of concurrent workgroups
    // spread over the output.  When the input rows of a tile lie 4 KiB or
    // more apart, the reads of U-consecutive tiles share their low address
    // bits (and so their HBM channels); a diagonal order then spreads both,
    // as long as there are at least half as many U-tiles as W-tiles.  With
    // fewer, the U shift repeats within the W-tiles that run together, and
    // their writes share channels: U fastest again (f32[1024,16384] 27.5 us
    // diagonal, 24.8 U fastest; f32[2048,16384], with twice the U-tiles,
    // 47.6 and 53.2).  (Rows of 4 KiB: bf16[16384,2048] took 28.0 us U
    // fastest and 24.4 diagonal.)  Narrow tiles on 4 KiB rows run W fastest
    // (f32[16384,1024] 24.1 us against 24.4 diagonal).  Input rows that are
    // not whole 128-byte lines share their edge lines between
    // W-neighbouring tiles: those go to one XCD (order 3).
    const long long order = env_ll("HF_TR_ORDER", in_row_bytes % 128 != 0          ? 3
                                                  : narrow && in_row_bytes == 4096 ? 1
                                                  : in_row_bytes >= 4096           ? (ntw <= 2 * ntu ? 2 : 0)
                                                                                   : 0);
    // Threads per tile: one 128-bit vector per thread and phase for the
    // narrow tiles above; otherwise 512 when the larger phase of a full tile
    // divides evenly among them (the other phase may leave some idle), else
    // 256.  The 32x32 tiles of small grids whose phases hold 512 and 256
    // vectors (2- or 1-wide loads, 4-wide stores) ran 9-14% shorter on the
    // GPU with 512 threads than with 256: the pages' 3-D example 3.88 ->
    // 3.36 us, f32[300,334] and f32[1000,333] transposed 3.55 -> 3.22 and
    // 3.77 -> 3.36 us (kernel trace).
    const long long lv = (long long)tu * (tw / vin), sv = (long long)tw * (tu / vout);
    int tb = std::max(lv, sv) % 512 == 0 ? 512 : 256;
    if (narrow && lv == 1024 && sv == 1024) tb = 1024;
    const int tblock = (int)env_ll("HF_TR_BLOCK", tb);
    P.ctx.push_back(ld);
    P.ctx.push_back(st);
    P.block = tblock;
    P.grid = nb * ntu * ntw;
    P.lds_bytes = tw * pitch * 4;
    P.empty = rt.numel() == 0;
    P.macros = {{"HF_BLOCK", tblock}, {"HF_TU", tu}, {"HF_TW", tw}, {"HF_PITCH", pitch},
                {"HF_VIN", vin}, {"HF_VOUT", vout}, {"HF_DU", DU}, {"HF_DW", DW},
                {"HF_NTU", ntu}, {"HF_NTW", ntw}, {"HF_ORDER", order}};
    P.info.vector_elems = vout;
    P.info.elements = rt.numel();
    P.info.rows = DW;
    P.info.cols = DU;
    P.info.tile_rows = tw;
    P.info.tile_cols = tu;
    common_info(g, P);
    *out = P;
    return true;
  }
  return false;
}

Plan plan_reduce(const Graph &g) {
  const Node &R = g.nodes[g.reduce];
  int rin = R.opd[0];
  const Type &it = g.nodes[rin].t;
  if (is_nibble(g.nodes[g.root].t.dt))
    fail(HF_ERR_UNSUPPORTED, "4-bit results of a reduce (one output element per thread would share bytes)");
  Ctx c = make_ctx(g, rin, -1);
  // Physical order of the reduce input: taken from the largest parameter that
  // reads the input space through a pure permutation of its dims.
  std::vector<int> order;
  long long best = -1;
  for (auto &pr : c.param_reads) {
    const Type &pt = g.nodes[pr.first].t;
    std::vector<int> o;
    bool ok = true;
    std::vector<char> seen(it.rank, 0);
    for (int k = 0; k < pt.rank && ok; ++k) {
      int d = pt.m2m[k];
      if (pt.dims[d] <= 1) continue;
      const Term &t = pr.second[d];
      if (t.k != Term::VAR || seen[t.var]) ok = false;
      else {
        seen[t.var] = 1;
        o.push_back(t.var);
      }
    }
    for (int d = 0; d < it.rank && ok; ++d)
      if (it.dims[d] > 1 && !seen[d]) ok = false;
    if (ok && pt.numel() > best) {
      best = pt.numel();
      order = o;
    }
  }
  if (best < 0) {
    order.clear();
    for (int d = it.rank - 1; d >= 0; --d)
      if (it.dims[d] > 1) order.push_back(d);
  }
  std::vector<char> red(it.rank, 0);
  for (int64_t d : R.attr) red[d] = 1;
  size_t nk = 0, nj = 0;
  for (int d : order) (red[d] ? nk : nj)++;
  bool row = true;
  if (nk > 0 && nj > 0) {
    bool minor_red = true, minor_kept = true;
    for (size_t k = 0; k < order.size(); ++k) {
      if (k < nk && !red[order[k]]) minor_red = false;
      if (k < nj && red[order[k]]) minor_kept = false;
    }
    // Kept dims on both sides of one physically contiguous block of reduced
    // dims: a column reduce over the kept dims flattened in physical order
    // (the physically major kept dims act as a batch).  Each lane's vector
    // still lies along the minor kept dim, and the index maps delinearize
    // the flattened column over every kept dim.
    size_t first = order.size(), last = 0;
    for (size_t k = 0; k < order.size(); ++k)
      if (red[order[k]]) first = std::min(first, k), last = k;
    const bool batched_col = !red[order[0]] && last - first + 1 == nk;
    if (minor_red) row = true;
    else if (minor_kept || batched_col) row = false;
    else
      fail(HF_ERR_UNSUPPORTED,
           "node " + std::to_string(g.reduce) +
               " (reduce): reduced dimensions are neither the physically minor ones nor one physically contiguous block "
               "after the minor kept ones");
  }
  // K: elements per output (0 when a reduced dim is empty: every output is
  // init); J: outputs
  long long K = 1, J = 1;
  for (int d = 0; d < it.rank; ++d) (red[d] ? K : J) *= it.dims[d];

  Plan P;
  P.rin = rin;
  P.order = order;
  P.empty = R.t.numel() == 0;
  const int op = (int)R.reducer;
  if (row) {
    P.hero = HF_HERO_ROW_REDUCE;
    c.lane = nk > 0 ? order[0] : -1;
    c = make_ctx(g, rin, c.lane);
    int V = 1;
    if (c.lane >= 0 && !c.general)
      V = align_lanes(c, vec_width(it.dims[c.lane], std::max(1, 16 / stream_elem_bytes(g, c, 4))));
    c.V = V;
    long long kv = K / V;
    int block, tpr;
    const long long wave_rows = env_ll("HF_ROW_WAVE_ROWS", 256);
    if (kv >= wave_rows || (kv >= 64 && std::getenv("HF_ROW_BLOCK"))) {
      // 512 threads per row; 256 for max/argmax, whose per-row finish (a
      // pair reduction and a serial combine over the waves) weighs more
      // (measured 71% -> 80% of peak on bf16[8192,8192]; the float paths
      // lost 1-20% at 256)
      block = (int)std::min<long long>(env_ll("HF_ROW_BLOCK", op == HF_REDUCER_ARGMAX ? 256 : 512), pow2_floor(kv));
      tpr = block;
    } else if (kv >= 64) {
      // rows of 64 to 255 vectors: one wave per row, four rows per
      // workgroup (a row per workgroup of one or two waves left the
      // workgroups too small)
      block = 256;
      tpr = 64;
    } else {
      block = 256;
      tpr = pow2_ceil(std::max<long long>(1, kv));
    }
    long long rpb = tpr == block ? 1 : block / tpr;
    // A few long rows: each row splits into segments of at least eight
    // chunks a thread (one batch of loads), one segment per workgroup, so
    // that about 2048 workgroups run; a fold kernel then combines each row's
    // partials in segment order.  f32[16,1048576] summed in 141 us with one
    // workgroup per row (8 workgroups, two rows each).
    long long segs = 1, segkv = kv;
    if (tpr == block && env_ll("HF_ROW_SEGS", 1) > 0) {
      const long long want = ceil_div(2048, std::max<long long>(J, 1));
      segs = std::min(want, kv / ((long long)block * 8));
      if (segs >= 2) {
        segkv = ceil_div(ceil_div(kv, segs), (long long)block) * block;
        segs = ceil_div(kv, segkv);
      }
      if (segs < 2) {
        segs = 1;
        segkv = kv;
      }
    }
    // Whole-row workgroups whose rows split into equal chunks take several
    // rows per step: their loads go out together, and what the prologue reads
    // along the row (a broadcast bias) is loaded once for all of them.
    // Two rows per step for rows of eight or more chunks per thread (measured
    // faster there; two or four chunks gained nothing or lost: f32[4096,4096]
    // 11.08 -> 11.13 us, f32[2048,8192] 11.07 -> 11.44), and for rows of one
    // chunk per thread, whose single load a thread leaves HBM waiting:
    // f32[8192,2048] 11.95 -> 11.12 us, f32[16384,1024] 11.44 -> 11.04,
    // f32[32768,1024] 20.69 -> 20.34.
    long long rr = 1;
    if (segs == 1 && tpr == block && kv % block == 0 && op != HF_REDUCER_ARGMAX)
      rr = std::max<long long>(
          1, std::min<long long>(env_ll("HF_ROW_RPS", kv / block >= 8 || kv == block ? 2 : 1), 4));
    long long pipe = 0;
    if (rr == 1 && tpr == block && kv % block == 0 && kv / block <= 8 && op != HF_REDUCER_ARGMAX)
      pipe = env_ll("HF_ROW_PIPE", 0) ? 1 : 0;
    // Whole-row workgroups: one per row step, up to 65536 (the sum of
    // exp(x) + bias over bf16[8,1,1280,16384], 10,240 rows, took 56.2 us in
    // 10,240 workgroups against 57.2 us in 8192 that loop over the rows, the
    // f32 row mean of 16,384 rows 38.7 against 39.2 us; 4096 or fewer
    // workgroups lost 5-13% on that sum).  Several rows per
    // workgroup keep a grid-stride loop over 2048 workgroups of 256 threads,
    // one full round of 32 waves on each of the 256 CUs: summing rows of 16
    // to 512 f32 (64 MiB) took 11.4-12.0 us there against 12.9-13.5 with
    // 8192 workgroups and 11.9-12.3 with 4096 (3072: 12.2-13.1 us).
    long long target = env_ll("HF_ROW_WGS", tpr == block ? 65536 : 2048);
    P.grid = std::max<long long>(1, std::min(ceil_div(J, rpb * rr) * segs, target));
    const long long pipe_k = ceil_div(J, P.grid);  // rows per workgroup
    if (pipe_k > 1024 || segs > 1) pipe = 0;
    P.block = block;
    P.lds_bytes = tpr == block ? (block / 64) * 8 * (int)rr : 0;
    if (segs > 1) {
      P.ws_bytes = J * segs * (op == HF_REDUCER_ARGMAX ? 8 : 4);  // max/argmax: value and index
      P.fold_grid = J;  // one fold workgroup per row
    }
    P.macros = {{"HF_OP", op}, {"HF_BLOCK", block}, {"HF_V", V}, {"HF_ROWS", J},
                {"HF_KV", kv}, {"HF_TPR", tpr}, {"HF_RR_ROWS", rr}, {"HF_RR_PIPE", pipe},
                {"HF_RR_PIPE_K", std::max<long long>(1, pipe_k)}, {"HF_RSEG", segs}, {"HF_SEGKV", segkv}};
    P.info.vector_elems = V;
    P.info.rows = J;
    P.info.cols = K;
  } else {
    P.hero = HF_HERO_COLUMN_REDUCE;
    c = make_ctx(g, rin, order[0]);
    int V = c.general ? 1 : align_lanes(c, vec_width(it.dims[c.lane], std::max(1, 16 / stream_elem_bytes(g, c, 4))));
    c.V = V;
    long long Cc = J, Rr = K;
    // 32 column lanes: 128-bit lanes over 512-byte row segments, 8 row lanes
    // (measured 73% -> 76% of peak on f32[16384,4096] against 64 lanes)
    // (16 column lanes for 2048 columns or fewer: f32[16384,1024] took
    // 18.9 us with 32 lanes (128-row segments) and 13.7 with 16, and
    // f32[8192,2048] 14.1 against 13.7; 32 lanes stay for wider arrays.)
    int cl = (int)std::min<long long>(env_ll("HF_COL_CL", Cc <= 2048 ? 16 : 32), pow2_ceil(ceil_div(Cc, V)));
    int block = 256;
    int rl = block / cl;
    long long cb = (long long)cl * V;
    long long ncb = ceil_div(Cc, cb);
    // Segments of at least 128 rows (16 a row lane, two batches of loads):
    // with 4096 workgroups f32[4096,4096] got 32-row segments and took
    // 19.8 us, with 128-row ones (1024 workgroups) 13.8 us; at 2048 and
    // 8192 rows 128-row segments were also the fastest choice measured.
    long long target = env_ll("HF_COL_WGS", 4096);
    long long segs = std::max<long long>(1, std::min(target / ncb, ceil_div(Rr, std::getenv("HF_COL_WGS") ? rl : 128)));
    // At most 256 segments: the fold reads every segment of a column, and a
    // few narrow columns over many rows otherwise got thousands of them
    // (f32[1048576,16] 29.3 -> 14.0 us, f32[262144,64] 21.3 -> 13.8 us).
    if (!std::getenv("HF_COL_WGS")) segs = std::min<long long>(segs, 256);
    long long rs = Rr > 0 ? ceil_div(Rr, segs) : 0;
    segs = rs > 0 ? ceil_div(Rr, rs) : 1;
    P.grid = ncb * segs;
    P.block = block;
    P.lds_bytes = (int)(rl * cb * 4 + 4);
    if (segs > 1) {
      P.ws_bytes = segs * Cc * (op == HF_REDUCER_ARGMAX ? 8 : 4);  // max/argmax: value and index
      P.fold_grid = ceil_div(Cc, 64);
    }
    P.macros = {{"HF_OP", op}, {"HF_BLOCK", block}, {"HF_V", V}, {"HF_C", Cc}, {"HF_R", Rr},
                {"HF_CL", cl}, {"HF_RL", rl}, {"HF_CB", cb}, {"HF_NCB", ncb}, {"HF_S", segs},
                {"HF_RS", rs}, {"HF_CR_UNROLL", env_ll("HF_COL_UNROLL", 8)}};
    P.info.vector_elems = V;
    P.info.rows = Rr;
    P.info.cols = Cc;
    P.info.tile_rows = (int)rs;
    P.info.tile_cols = (int)cb;
  }
  P.ctx.push_back(c);
  // The epilogue: what follows the reduce, evaluated once per output element
  // with the reduced value as its leaf.
  if (g.reduce != g.root) P.ctx.push_back(make_ctx(g, g.root, -1, g.reduce));
  P.info.elements = it.numel();
  common_info(g, P);
  return P;
}

}  // namespace

bool is_streaming(const Graph &g, int p) {
  long long n = g.nodes[p].t.numel();
  long long out = g.nodes[g.root].t.numel();
  if (g.reduce >= 0) out = g.nodes[g.nodes[g.reduce].opd[0]].t.numel();
  return n >= 1024 && n * 4 >= out;
}

const char *hero_template_name(hf_hero h) {
  switch (h) {
    case HF_HERO_LOOP: return "loop";
    case HF_HERO_TRANSPOSE: return "transpose";
    case HF_HERO_ROW_REDUCE: return "reduce_row";
    case HF_HERO_COLUMN_REDUCE: return "reduce_col";
  }
  return "?";
}

// Hero selection (XLA:GPU Emitters, "Hero-based codegen"): a reduce root
// selects a reduction emitter, row or column by the physical layout of its
// input; a transpose whose reads are not coalesced in the output order
// selects the transpose emitter (shared memory fixes the read and write
// patterns); everything else is the loop emitter.
Plan make_plan(const Graph &g) {
  const Node &R = g.nodes[g.root];
  if (g.reduce >= 0) return plan_reduce(g);
  Ctx loop = make_ctx(g, g.root, phys_minor(R.t));
  if (!env_ll("HF_NO_TRANSPOSE_HERO", 0)) {
    Plan P;
    if (try_transpose(g, loop, &P)) return P;
  }
  return plan_loop(g, loop);
}

// ------------------------------------------------------------ constants
// Round-to-nearest-even of a double to a binary format with p significand
// bits and minimum normal exponent emin, working on the IEEE-754 binary64
// bit pattern; overflow goes to infinity.
static double round_bits(double x, int p, int emin, int emax) {
  if (std::isnan(x) || std::isinf(x) || x == 0.0) return x;
  uint64_t b;
  std::memcpy(&b, &x, 8);
  const uint64_t sign = b & (uint64_t(1) << 63);
  int e = (int)((b >> 52) & 0x7FF);
  uint64_t m = b & ((uint64_t(1) << 52) - 1);
  int ue;  // unbiased exponent of the leading bit
  if (e == 0) {  // double subnormal: normalise
    ue = -1022;
    while (!(m & (uint64_t(1) << 52))) {
      m <<= 1;
      --ue;
    }
  } else {
    m |= uint64_t(1) << 52;
    ue = e - 1023;
  }
  // keep p bits below and including the leading bit, fewer in the subnormal range
  int keep = p;
  if (ue < emin) keep = p - (emin - ue);
  if (keep <= 0) {
    // below half the smallest subnormal, or exactly half (ties to even -> 0)
    if (keep == 0 && m > (uint64_t(1) << 52)) {
      double r = std::ldexp(1.0, emin - (p - 1));
      return sign ? -r : r;
    }
    return sign ? -0.0 : 0.0;
  }
  int drop = 53 - keep;
  uint64_t q = m >> drop, rem = m & ((uint64_t(1) << drop) - 1), half = uint64_t(1) << (drop - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  double r = std::ldexp((double)q, ue - keep + 1);
  double maxf = std::ldexp(2.0 - std::ldexp(1.0, 1 - p), emax);
  if (r > maxf) r = INFINITY;
  return sign ? -r : r;
}

double reciprocal(float s) { return 1.0 / (double)s; }

double round_to_dtype(double x, hf_dtype dt) {
  switch (dt) {
    case HF_F32: return (double)(float)x;
    case HF_BF16: return round_bits(x, 8, -126, 127);
    case HF_F16: return round_bits(x, 11, -14, 15);
    default: return std::nearbyint(x);
  }
}

}  // namespace hf
