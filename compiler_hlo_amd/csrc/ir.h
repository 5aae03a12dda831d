// ir.h -- internal representation of one fusion, after intake.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "hlofusion.h"

namespace hf {

// Thrown by intake/planning; carries the status the C ABI returns.
struct Error {
  hf_status status;
  std::string msg;
};

[[noreturn]] void fail(hf_status st, const std::string &msg);

int dtype_bits(hf_dtype dt);
int dtype_bytes(hf_dtype dt);
int64_t storage_bytes(hf_dtype dt, int64_t n);
bool is_nibble(hf_dtype dt);
bool is_float(hf_dtype dt);
const char *dtype_name(hf_dtype dt);
const char *op_name(hf_op op);

// Quantization parameters of one quantized type, owned by the Graph.
struct Quant {
  int qdim = -1;                 // -1 per-tensor
  std::vector<float> scales;
  std::vector<int32_t> zero_points;
  int32_t smin = 0, smax = 0;
  hf_dtype storage = HF_S8;
};

struct Type {
  hf_dtype dt = HF_F32;
  int rank = 0;
  int64_t dims[HF_MAX_RANK] = {0};
  int m2m[HF_MAX_RANK] = {0};  // always filled (default layout when absent)
  int quant = -1;              // index into Graph::quants, -1 if not quantized

  int64_t numel() const {
    int64_t n = 1;
    for (int d = 0; d < rank; ++d) n *= dims[d];
    return n;
  }
  bool same_shape(const Type &o) const {
    if (rank != o.rank) return false;
    for (int d = 0; d < rank; ++d)
      if (dims[d] != o.dims[d]) return false;
    return true;
  }
};

struct Node {
  hf_op op = HF_PARAMETER;
  std::vector<int> opd;
  Type t;
  int param = -1;
  double cst = 0.0;
  std::vector<int64_t> attr;
  hf_reducer reducer = HF_REDUCER_ADD;
  double init = 0.0;
  std::vector<int> users;  // reachable users only
  bool live = false;       // reachable from the root
};

struct Graph {
  std::vector<Node> nodes;
  std::vector<Quant> quants;
  int root = -1;
  int reduce = -1;              // the reduce node (the hero), if any
  int n_params = 0;
  std::vector<int> param_node;  // parameter number -> node (-1 if unused)
};

// Intake: copy the C descriptor into a Graph and check every op's constraints.
Graph intake(const hf_fusion_desc *desc);

}  // namespace hf
