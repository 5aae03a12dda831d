// reduce_col.hip -- column reduction hero: the kept dimensions are the
// physically minor ones, so each output element reduces a strided column.
//
// The reduced extent HF_R is split into HF_S segments of HF_RS rows.  A
// workgroup owns one segment and HF_CB consecutive columns; its HF_BLOCK
// threads form HF_RL row lanes x HF_CL column lanes, each column lane reading
// HF_V consecutive columns with one 128-bit load per row (coalesced along
// the row) and accumulating in registers.  The row lanes' partials are then
// written to LDS as an [HF_RL][HF_CB] tile and read back transposed, one
// column per thread, and reduced ("LDS transpose-then-reduce").  With more
// than one segment, each workgroup writes its column partials to the
// workspace; the last workgroup of a column block to finish (a device-scope
// atomic counter) folds the segments in segment order -- deterministic --
// writes the result and resets the counter for the next launch.
//
// Provided by the generated code: HF_OP, HF_BLOCK, HF_V, HF_C, HF_R, HF_CL,
// HF_RL, HF_CB, HF_NCB, HF_S, HF_RS, hf_cr_eval(A, r, c, x), hf_cr_store(A, c, acc).
extern "C" __global__ __launch_bounds__(HF_BLOCK) void hf_kernel(HF_KERNEL_PARAMS) {
  const HfArgs A = HF_ARGS_INIT;
  __shared__ float part[HF_RL * HF_CB];
  const int cb = blockIdx.x % HF_NCB, seg = blockIdx.x / HF_NCB;
  const int cl = threadIdx.x % HF_CL, rl = threadIdx.x / HF_CL;
  const int c = cb * HF_CB + cl * HF_V;
  float acc[HF_V];
#pragma unroll
  for (int v = 0; v < HF_V; ++v) acc[v] = hf_red_identity<HF_OP>();
  const int r_begin = seg * HF_RS;
  const int r_end = r_begin + HF_RS < HF_R ? r_begin + HF_RS : HF_R;
  if (c < HF_C) {
    int r = r_begin + rl;
    for (; r + 3 * HF_RL < r_end; r += 4 * HF_RL) {
      float x[4][HF_V];
#pragma unroll
      for (int u = 0; u < 4; ++u) hf_cr_eval(A, r + u * HF_RL, c, x[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < HF_V; ++v) acc[v] = hf_red<HF_OP>(acc[v], x[u][v]);
    }
    for (; r < r_end; r += HF_RL) {
      float x[HF_V];
      hf_cr_eval(A, r, c, x);
#pragma unroll
      for (int v = 0; v < HF_V; ++v) acc[v] = hf_red<HF_OP>(acc[v], x[v]);
    }
  }
#pragma unroll
  for (int v = 0; v < HF_V; ++v) part[rl * HF_CB + cl * HF_V + v] = acc[v];
  __syncthreads();
#if HF_S == 1
  for (int j = threadIdx.x; j < HF_CB; j += HF_BLOCK) {
    float s = part[j];
#pragma unroll
    for (int k = 1; k < HF_RL; ++k) s = hf_red<HF_OP>(s, part[k * HF_CB + j]);
    if (cb * HF_CB + j < HF_C) hf_cr_store(A, cb * HF_CB + j, s);
  }
#else
  float *ws = (float *)A.ws;
  unsigned int *counters = (unsigned int *)(ws + (long)HF_S * HF_C);
  for (int j = threadIdx.x; j < HF_CB; j += HF_BLOCK) {
    float s = part[j];
#pragma unroll
    for (int k = 1; k < HF_RL; ++k) s = hf_red<HF_OP>(s, part[k * HF_CB + j]);
    if (cb * HF_CB + j < HF_C) ws[(long)seg * HF_C + cb * HF_CB + j] = s;
  }
  __shared__ int is_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned int prev = __hip_atomic_fetch_add(&counters[cb], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    is_last = prev == HF_S - 1;
  }
  __syncthreads();
  if (is_last) {
    __threadfence();
    for (int j = threadIdx.x; j < HF_CB; j += HF_BLOCK) {
      const int col = cb * HF_CB + j;
      if (col < HF_C) {
        float s = hf_red_identity<HF_OP>();
        for (int k = 0; k < HF_S; ++k) s = hf_red<HF_OP>(s, ws[(long)k * HF_C + col]);
        hf_cr_store(A, col, s);
      }
    }
    if (threadIdx.x == 0) __hip_atomic_store(&counters[cb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#endif
}
