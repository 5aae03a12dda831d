// reduce_row.hip -- row reduction hero: the reduced dimensions are the
// physically minor ones, so each output element reduces one contiguous row
// (XLA:GPU Emitters, "Hero-based codegen": reductions use shuffles and shared
// memory).
//
// HF_TPR == HF_BLOCK: one workgroup per row (grid-strided over rows).  Each
// lane first issues the loads of all its chunks of the row (128-bit each),
// then accumulates them in registers; the wave reduces with DPP
// (hf_wave_reduce) and the waves combine through LDS.  Anything the prologue
// reads that depends only on the position in the row (a bias broadcast
// along the rows) is loop-invariant across rows.
// HF_TPR < 64: short rows; HF_BLOCK/HF_TPR rows per workgroup step, reduced
// within lane groups by cross-lane shuffles.
//
// Provided by the generated code: HF_OP, HF_BLOCK, HF_V, HF_ROWS, HF_KV
// (vectors per row), HF_TPR, hf_regs_t, hf_rr_eval_fetch(A, row, kv, R),
// hf_rr_eval(A, row, kv, R, x), hf_rr_store(A, row, acc).
extern "C" __global__ __launch_bounds__(HF_BLOCK) void HF_KERNEL_NAME(HF_KERNEL_PARAMS) {
  const HfArgs A = HF_ARGS_INIT;
#if HF_TPR == HF_BLOCK
  __shared__ float part[HF_BLOCK / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int ITERS = (HF_KV + HF_BLOCK - 1) / HF_BLOCK;
  for (int row = blockIdx.x; row < HF_ROWS; row += gridDim.x) {
    float acc[HF_V];
#pragma unroll
    for (int v = 0; v < HF_V; ++v) acc[v] = hf_red_identity<HF_OP>();
    if constexpr (HF_KV % HF_BLOCK == 0) {
      hf_regs_t R[ITERS];
#pragma unroll
      for (int it = 0; it < ITERS; ++it) hf_rr_eval_fetch(A, row, it * HF_BLOCK + (int)threadIdx.x, R[it]);
      HF_LOADS_ISSUED();
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        float x[HF_V];
        hf_rr_eval(A, row, it * HF_BLOCK + (int)threadIdx.x, R[it], x);
#pragma unroll
        for (int v = 0; v < HF_V; ++v) acc[v] = hf_red<HF_OP>(acc[v], x[v]);
      }
    } else {
      for (int kv = threadIdx.x; kv < HF_KV; kv += HF_BLOCK) {
        hf_regs_t R1;
        hf_rr_eval_fetch(A, row, kv, R1);
        float x[HF_V];
        hf_rr_eval(A, row, kv, R1, x);
#pragma unroll
        for (int v = 0; v < HF_V; ++v) acc[v] = hf_red<HF_OP>(acc[v], x[v]);
      }
    }
    float s = acc[0];
#pragma unroll
    for (int v = 1; v < HF_V; ++v) s = hf_red<HF_OP>(s, acc[v]);
    s = hf_wave_reduce<HF_OP>(s);
    if (lane == 0) part[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
      float t = part[0];
#pragma unroll
      for (int w = 1; w < HF_BLOCK / 64; ++w) t = hf_red<HF_OP>(t, part[w]);
      hf_rr_store(A, row, t);
    }
    __syncthreads();
  }
#else
  constexpr int RPB = HF_BLOCK / HF_TPR;
  const int sub = threadIdx.x % HF_TPR;
  const int rloc = threadIdx.x / HF_TPR;
  for (int row0 = blockIdx.x * RPB; row0 < HF_ROWS; row0 += gridDim.x * RPB) {
    const int row = row0 + rloc;
    float acc[HF_V];
#pragma unroll
    for (int v = 0; v < HF_V; ++v) acc[v] = hf_red_identity<HF_OP>();
    if (row < HF_ROWS) {
      for (int kv = sub; kv < HF_KV; kv += HF_TPR) {
        hf_regs_t R1;
        hf_rr_eval_fetch(A, row, kv, R1);
        float x[HF_V];
        hf_rr_eval(A, row, kv, R1, x);
#pragma unroll
        for (int v = 0; v < HF_V; ++v) acc[v] = hf_red<HF_OP>(acc[v], x[v]);
      }
    }
    float s = acc[0];
#pragma unroll
    for (int v = 1; v < HF_V; ++v) s = hf_red<HF_OP>(s, acc[v]);
    s = hf_group_reduce<HF_OP, HF_TPR>(s);
    if (sub == 0 && row < HF_ROWS) hf_rr_store(A, row, s);
  }
#endif
}
