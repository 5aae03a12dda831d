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
// With HF_PIPE > 0 (the planner's choice for 8-bit streams) the thread's
// HF_NR rows run as a software pipeline instead: the row-invariant loads first
// (hf_loop_inv), then the first HF_PIPE rows' loads; each row is computed and
// stored as soon as its own data is in, and the load of the row HF_PIPE
// further on is issued in its place.  The compute of a row then waits for
// that row only (vector-memory counters retire in issue order), while HBM
// keeps streaming the rows behind it.
//
// Provided by the generated code in front of this text:
//   HF_BLOCK, HF_V, HF_ROWS, HF_COLS_V, HF_TPR (threads per row segment),
//   HF_RPB (rows per block step), HF_NCH (column chunks), HF_UNROLL,
//   HF_PIPE, HF_RSTEP (rows between a thread's rows), HF_NR (rows a thread
//   takes, at most), hf_val_t, hf_regs_t, hf_loop_eval_fetch(A, row, colv, R),
//   hf_loop_eval(A, row, colv, R, r), hf_loop_store(A, row, colv, r); with
//   HF_PIPE also hf_inv_t, hf_loop_inv(A, row, colv, I), hf_loop_inv_pin(I)
//   and hf_loop_eval(A, row, colv, R, I, r).
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
#if HF_PIPE > 0
  // Rows row, row + HF_RSTEP, ...: HF_NR of them, or HF_NR - 1 when the
  // last one lies past HF_ROWS (only the last row is checked).
  constexpr int PD = HF_PIPE;
  hf_inv_t I;
  hf_loop_inv(A, row, colv, I);
  hf_regs_t R[PD];
#pragma unroll
  for (int p = 0; p < PD; ++p)
    if (p < HF_NR - 1 || row + p * HF_RSTEP < HF_ROWS) hf_loop_eval_fetch(A, row + p * HF_RSTEP, colv, R[p]);
  HF_LOADS_ISSUED();
#pragma unroll
  for (int i = 0; i < HF_NR; ++i) {
    const int r = row + i * HF_RSTEP;
    if (i < HF_NR - 1 || r < HF_ROWS) {
      hf_val_t v[HF_V];
      hf_loop_eval(A, r, colv, R[i % PD], I, v);
      if (i == 0) hf_loop_inv_pin(I);
      hf_loop_store(A, r, colv, v);
      if (i + PD < HF_NR - 1 || (i + PD < HF_NR && r + PD * HF_RSTEP < HF_ROWS))
        hf_loop_eval_fetch(A, r + PD * HF_RSTEP, colv, R[i % PD]);
      HF_LOADS_ISSUED();
    }
  }
  (void)rstep;
#else
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
#endif
}
