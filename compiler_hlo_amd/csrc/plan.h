// plan.h -- hero selection, partitioning, index maps and kernel geometry.
#pragma once

#include <map>
#include <set>
#include <string>
#include <vector>

#include "ir.h"

namespace hf {

// One component of an index vector, as a function of the variables of the
// space it is expressed in (i0, i1, ...): a variable, the constant 0 (a
// broadcast or size-1 dimension), or a general expression (after a reshape
// that is not a pure insertion/removal of size-1 dimensions).  A variable may
// carry an offset (a slice): `add` is known on the host, `dyn` names a
// wave-uniform value the kernel reads at launch (a dynamic_slice start).
struct Term {
  enum Kind { ZERO, VAR, EXPR } k = ZERO;
  int var = -1;
  std::string e;
  long long add = 0;
  std::string dyn;
};
using Index = std::vector<Term>;

std::string term_str(const Term &t);
// t + c + dyn (dyn: "" or the name of a run-time offset)
Term shifted(const Term &t, long long c, const std::string &dyn);
// Name of the kernel value holding the clamped start index of dim d of the
// dynamic_slice node n ("" when the start is known on the host).
std::string dyn_start_name(int n, int d);
std::string index_key(const Index &E);
Index identity_index(int rank);

// Output-to-input index map of operand `k` of node `n` read at E
// (XLA:GPU Emitters, "Indexing transforms").  Sets *general when the map
// changes how the lane variable `lane` moves through memory (a div/mod
// reshape; reverse, pad or concatenate of the lane's dim; lane < 0: of any
// dim): such a context runs one element per lane, or, as a loop (Ctx::gather),
// reads each lane's element on its own.
Index operand_index(const Graph &g, int n, int k, const Index &E, bool *general, int lane = -1);

// Physical stride (in elements) of every logical dim of t.
std::vector<long long> phys_strides(const Type &t);
// Most minor dim with extent > 1, or -1.
int phys_minor(const Type &t);

// One evaluation phase of a hero: `root` is evaluated at the identity index
// of its own space, lanes run along `lane`, `leaf` (if any) is read from LDS.
struct Ctx {
  int root = -1;
  int leaf = -1;
  int lane = -1;
  int V = 1;
  bool general = false;                       // an index map moves with the lane (or a div/mod reshape was met)
  bool gather = false;                        // general, yet V lanes: each lane's element read on its own
  std::vector<std::set<std::string>> maps;    // distinct index maps per node
  std::vector<char> in_ctx;
  std::vector<std::pair<int, Index>> param_reads;
  std::vector<int> part;                      // node -> partition
  std::vector<int> part_root;                 // partition -> root node
};

struct Plan {
  hf_hero hero = HF_HERO_LOOP;
  std::vector<Ctx> ctx;       // loop/reduce: 1; transpose: [0] load, [1] store
  int staged = -1;            // transpose: staged node
  int lane_in = -1, lane_out = -1;
  std::vector<int> u_dims;    // transpose: dims of the tile's U index, minor -> major (lane_out first)
  // reduce
  int rin = -1;               // reduce operand node
  std::vector<int> order;     // input dims with extent > 1, physical minor -> major
  // geometry
  std::vector<std::pair<std::string, long long>> macros;
  int block = 256;
  long long grid = 1;
  int lds_bytes = 0;
  long long ws_bytes = 0;     // workspace (column reduce)
  bool empty = false;         // nothing to launch (zero-size result)
  hf_plan_info info{};
  std::vector<int> quant_args;  // quant indices passed as per-axis arrays
  std::string kernel_name;      // set by generate_source
  std::string fold_name;        // column reduce with segments: the fold kernel
  long long fold_grid = 0;      // 0: no fold kernel
};

Plan make_plan(const Graph &g);
// A parameter the fusion streams (comparable in size to the result): read
// once, with the non-temporal hint.
bool is_streaming(const Graph &g, int param_node);
std::string generate_source(const Graph &g, Plan &P, const std::string &prelude,
                            const std::string &hero_text);
const char *hero_template_name(hf_hero h);

// Constants: round a double to an element type (RNE), the way a constant of
// that type holds it.
double round_to_dtype(double x, hf_dtype dt);
// 1/s rounded to the nearest double (IEEE double division).
double reciprocal(float s);

}  // namespace hf
