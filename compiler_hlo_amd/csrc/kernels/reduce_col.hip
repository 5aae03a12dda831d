// reduce_col.hip -- column reduction hero: the kept dimensions are the
// physically minor ones, so each output element reduces a strided column.
//
// Kernel 1 (HF_KERNEL_NAME): the reduced extent HF_R is split into HF_S
// segments of HF_RS rows.  A workgroup owns one segment and HF_CB
// consecutive columns; its HF_BLOCK threads form HF_RL row lanes x HF_CL
// column lanes, each column lane reading HF_V consecutive columns with one
// 128-bit load per row (coalesced along the row), HF_CR_UNROLL rows' loads
// in flight at a time, accumulating in registers.  The row lanes' partials are then
// written to LDS as an [HF_RL][HF_CB] tile and read back transposed, one
// column per thread, and reduced ("LDS transpose-then-reduce").  With one
// segment that is the result; otherwise the segment partial goes to the
// workspace and kernel 2 (HF_FOLD_NAME), launched right after on the same
// stream, folds the HF_S partials of each column in a fixed order --
// deterministic, and made visible by the kernel boundary rather than by
// device-wide cache write-backs inside kernel 1.
//
// Provided by the generated code: HF_OP, HF_BLOCK, HF_V, HF_C, HF_R, HF_CL,
// HF_RL, HF_CB, HF_NCB, HF_S, HF_RS, hf_regs_t, hf_cr_eval_fetch(A, r, c, R),
// hf_cr_eval(A, r, c, R, x), hf_cr_store(A, c, acc); for max/argmax (HF_OP 3)
// HF_ARG_V0 and hf_cr_store_arg(A, c, index) (which writes the index init
// where the index is still HF_ARG_NONE).
extern "C" __global__ __launch_bounds__(HF_BLOCK) void HF_KERNEL_NAME(HF_KERNEL_PARAMS) {
  const HfArgs A = HF_ARGS_INIT;
#if HF_OP == 3
  // max/argmax: the index of an element is its row r; each thread visits its
  // rows in increasing order.  The workspace holds the segments' maxima
  // ([HF_S][HF_C] floats) followed by their indices ([HF_S][HF_C] ints).
  __shared__ float pm[HF_RL * HF_CB];
  __shared__ int pk[HF_RL * HF_CB];
  {
    const int cb = blockIdx.x % HF_NCB, seg = blockIdx.x / HF_NCB;
    const int cl = threadIdx.x % HF_CL, rl = threadIdx.x / HF_CL;
    const int c = cb * HF_CB + cl * HF_V;
    float m[HF_V];
    int k[HF_V];
#pragma unroll
    for (int v = 0; v < HF_V; ++v) {
      m[v] = HF_ARG_V0;
      k[v] = HF_ARG_NONE;
    }
    const int r_begin = seg * HF_RS;
    const int r_end = r_begin + HF_RS < HF_R ? r_begin + HF_RS : HF_R;
    if (c < HF_C) {
      for (int r = r_begin + rl; r < r_end; r += HF_RL) {
        hf_regs_t R1;
        hf_cr_eval_fetch(A, r, c, R1);
        float x[HF_V];
        hf_cr_eval(A, r, c, R1, x);
#pragma unroll
        for (int v = 0; v < HF_V; ++v) hf_arg_step(m[v], k[v], x[v], r);
      }
    }
#pragma unroll
    for (int v = 0; v < HF_V; ++v) {
      pm[rl * HF_CB + cl * HF_V + v] = m[v];
      pk[rl * HF_CB + cl * HF_V + v] = k[v];
    }
    __syncthreads();
    for (int j = threadIdx.x; j < HF_CB; j += HF_BLOCK) {
      float mm = pm[j];
      int kk = pk[j];
      for (int q = 1; q < HF_RL; ++q) hf_arg_combine(mm, kk, pm[q * HF_CB + j], pk[q * HF_CB + j]);
      if (cb * HF_CB + j < HF_C) {
#if HF_S == 1
        hf_cr_store_arg(A, cb * HF_CB + j, kk);
#else
        ((float *)A.ws)[(long)seg * HF_C + cb * HF_CB + j] = mm;
        ((int *)A.ws)[(long)HF_S * HF_C + (long)seg * HF_C + cb * HF_CB + j] = kk;
#endif
      }
    }
  }
#else
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
    for (; r + (HF_CR_UNROLL - 1) * HF_RL < r_end; r += HF_CR_UNROLL * HF_RL) {
      hf_regs_t R[HF_CR_UNROLL];
#pragma unroll
      for (int u = 0; u < HF_CR_UNROLL; ++u) hf_cr_eval_fetch(A, r + u * HF_RL, c, R[u]);
      HF_LOADS_ISSUED();
#pragma unroll
      for (int u = 0; u < HF_CR_UNROLL; ++u) {
        float x[HF_V];
        hf_cr_eval(A, r + u * HF_RL, c, R[u], x);
#pragma unroll
        for (int v = 0; v < HF_V; ++v) acc[v] = hf_red<HF_OP>(acc[v], x[v]);
      }
    }
    for (; r < r_end; r += HF_RL) {
      hf_regs_t R1;
      hf_cr_eval_fetch(A, r, c, R1);
      float x[HF_V];
      hf_cr_eval(A, r, c, R1, x);
#pragma unroll
      for (int v = 0; v < HF_V; ++v) acc[v] = hf_red<HF_OP>(acc[v], x[v]);
    }
  }
#pragma unroll
  for (int v = 0; v < HF_V; ++v) part[rl * HF_CB + cl * HF_V + v] = acc[v];
  __syncthreads();
  for (int j = threadIdx.x; j < HF_CB; j += HF_BLOCK) {
    float s = part[j];
#pragma unroll
    for (int k = 1; k < HF_RL; ++k) s = hf_red<HF_OP>(s, part[k * HF_CB + j]);
    if (cb * HF_CB + j < HF_C) {
#if HF_S == 1
      hf_cr_store(A, cb * HF_CB + j, s);
#else
      ((float *)A.ws)[(long)seg * HF_C + cb * HF_CB + j] = s;
#endif
    }
  }
#endif  // HF_OP == 3
}

#if HF_S > 1
// Kernel 2: a workgroup folds the HF_S segment partials of 64 columns: its
// four waves take interleaved segments (coalesced 256-byte rows of the
// partial array, many loads in flight), then the four wave results are
// combined in wave order -- a fixed order, so the result is deterministic.
extern "C" __global__ __launch_bounds__(256) void HF_FOLD_NAME(HF_KERNEL_PARAMS) {
  const HfArgs A = HF_ARGS_INIT;
#if HF_OP == 3
  __shared__ float pm[4][64];
  __shared__ int pk[4][64];
  {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = blockIdx.x * 64 + lane;
    float m = HF_ARG_V0;
    int k = HF_ARG_NONE;
    if (col < HF_C)
      for (int q = wave; q < HF_S; q += 4)
        hf_arg_combine(m, k, ((const float *)A.ws)[(long)q * HF_C + col],
                       ((const int *)A.ws)[(long)HF_S * HF_C + (long)q * HF_C + col]);
    pm[wave][lane] = m;
    pk[wave][lane] = k;
    __syncthreads();
    if (wave == 0 && col < HF_C) {
      for (int w = 1; w < 4; ++w) hf_arg_combine(m, k, pm[w][lane], pk[w][lane]);
      hf_cr_store_arg(A, col, k);
    }
  }
#else
  __shared__ float part[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + lane;
  const float *ws = (const float *)A.ws;
  float s = hf_red_identity<HF_OP>();
  if (col < HF_C) {
    // the wave's segments k = wave, wave + 4, ...: up to 32 loads in flight,
    // then combined in segment order
    constexpr int NK = (HF_S + 3) / 4;
    constexpr int NB = NK < 32 ? NK : 32;
    for (int i0 = 0; i0 < NK; i0 += NB) {
      float t[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int k = wave + 4 * (i0 + i);
        t[i] = k < HF_S ? ws[(long)k * HF_C + col] : hf_red_identity<HF_OP>();
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) s = hf_red<HF_OP>(s, t[i]);
    }
  }
  part[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && col < HF_C)
    hf_cr_store(A, col, hf_red<HF_OP>(hf_red<HF_OP>(part[0][lane], part[1][lane]),
                                      hf_red<HF_OP>(part[2][lane], part[3][lane])));
#endif  // HF_OP == 3
}
#endif
