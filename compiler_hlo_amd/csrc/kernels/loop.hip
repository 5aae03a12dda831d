// loop.hip -- loop hero (XLA:GPU Emitters, "Loop emitter").
//
// The output is walked linearly in PHYSICAL order so that stores coalesce:
// the physical output is viewed as HF_ROWS rows of HF_COLS_V vectors of
// HF_V elements along the physically minor dimension (128-bit stores).
// Each thread keeps ONE column vector for its whole life and strides over
// rows, so every value that depends only on the column (per-axis scales,
// zero points, a bias broadcast along the rows) is loop-invariant and is
// loaded once per thread.  Per step a thread first issues the loads of
// HF_UNROLL rows (hf_loop_eval_fetch), then computes and stores them, so the
// loads of all those rows are in flight together.
//
// Provided by the generated code in front of this text:
//   HF_BLOCK, HF_V, HF_ROWS, HF_COLS_V, HF_TPR (threads per row segment),
//   HF_RPB (rows per block step), HF_NCH (column chunks), HF_UNROLL,
//   hf_val_t, hf_regs_t, hf_loop_eval_fetch(A, row, colv, R),
//   hf_loop_eval(A, row, colv, R, r), hf_loop_store(A, row, colv, r).
extern "C" __global__ __launch_bounds__(HF_BLOCK) void HF_KERNEL_NAME(HF_KERNEL_PARAMS) {
  const HfArgs A = HF_ARGS_INIT;
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x % HF_NCH;
  const int group = blockIdx.x / HF_NCH;
  const int ngroups = gridDim.x / HF_NCH;
  const int colv = chunk * HF_TPR + tid % HF_TPR;
  const int rsub = tid / HF_TPR;
  if (colv >= HF_COLS_V || rsub >= HF_RPB) return;
  const int rstep = ngroups * HF_RPB;
  int row = group * HF_RPB + rsub;
  for (; row + (HF_UNROLL - 1) * rstep < HF_ROWS; row += HF_UNROLL * rstep) {
    hf_regs_t R[HF_UNROLL];
#pragma unroll
    for (int u = 0; u < HF_UNROLL; ++u) hf_loop_eval_fetch(A, row + u * rstep, colv, R[u]);
    HF_LOADS_ISSUED();
#pragma unroll
    for (int u = 0; u < HF_UNROLL; ++u) {
      hf_val_t r[HF_V];
      hf_loop_eval(A, row + u * rstep, colv, R[u], r);
      hf_loop_store(A, row + u * rstep, colv, r);
    }
  }
  for (; row < HF_ROWS; row += rstep) {
    hf_regs_t R1;
    hf_loop_eval_fetch(A, row, colv, R1);
    hf_val_t r[HF_V];
    hf_loop_eval(A, row, colv, R1, r);
    hf_loop_store(A, row, colv, r);
  }
}
