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
// HF_RSEG > 1: a few long rows; each row splits into HF_RSEG segments of
// HF_SEGKV vectors, one per workgroup step.  Each workgroup writes its
// segment's partial to the workspace ([HF_RSEG][HF_ROWS] values, then as
// many indices for max/argmax), and the fold kernel (HF_FOLD_NAME, launched
// next on the same stream) combines each row's partials in segment order.
//
// Provided by the generated code: HF_OP, HF_BLOCK, HF_V, HF_ROWS, HF_KV
// (vectors per row), HF_TPR, HF_RSEG, HF_SEGKV, hf_regs_t, hf_rr_eval_fetch(A, row, kv, R),
// hf_rr_eval(A, row, kv, R, x) (HF_V floats), hf_rr_store(A, row, acc); for max/argmax
// (HF_OP 3) HF_ARG_V0 and hf_rr_store_arg(A, row, index) (which writes the
// index init where the index is still HF_ARG_NONE).
extern "C" __global__ __launch_bounds__(HF_BLOCK) void HF_KERNEL_NAME(HF_KERNEL_PARAMS) {
  const HfArgs A = HF_ARGS_INIT;
#if HF_RSEG > 1
  {
    constexpr int NB = 8;  // loads in flight per thread
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#if HF_OP == 3
    __shared__ float sm[HF_BLOCK / 64];
    __shared__ int sk[HF_BLOCK / 64];
#else
    __shared__ float sp[HF_BLOCK / 64];
#endif
    for (int w = blockIdx.x; w < HF_ROWS * HF_RSEG; w += gridDim.x) {
      const int row = w / HF_RSEG, seg = w % HF_RSEG;
      const int kv0 = seg * HF_SEGKV;
      const int kv1 = kv0 + HF_SEGKV < HF_KV ? kv0 + HF_SEGKV : HF_KV;
#if HF_OP == 3
      float m = HF_ARG_V0;
      int k = HF_ARG_NONE;
#else
      float acc[HF_V];
#pragma unroll
      for (int v = 0; v < HF_V; ++v) acc[v] = hf_red_identity<HF_OP>();
#endif
      for (int base = kv0; base < kv1; base += NB * HF_BLOCK) {
        hf_regs_t R[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int kv = base + b * HF_BLOCK + (int)threadIdx.x;
          if (kv < kv1) hf_rr_eval_fetch(A, row, kv, R[b]);
        }
        HF_LOADS_ISSUED();
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int kv = base + b * HF_BLOCK + (int)threadIdx.x;
          if (kv < kv1) {
            float x[HF_V];
            hf_rr_eval(A, row, kv, R[b], x);
#pragma unroll
            for (int v = 0; v < HF_V; ++v) {
#if HF_OP == 3
              hf_arg_step(m, k, x[v], kv * HF_V + v);
#else
              acc[v] = hf_red<HF_OP>(acc[v], x[v]);
#endif
            }
          }
        }
      }
#if HF_OP == 3
      hf_arg_wave_reduce(m, k);
      if (lane == 0) {
        sm[wave] = m;
        sk[wave] = k;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        for (int q = 1; q < HF_BLOCK / 64; ++q) hf_arg_combine(m, k, sm[q], sk[q]);
        ((float *)A.ws)[(long)seg * HF_ROWS + row] = m;
        ((int *)A.ws)[(long)HF_RSEG * HF_ROWS + (long)seg * HF_ROWS + row] = k;
      }
#else
      float s = acc[0];
#pragma unroll
      for (int v = 1; v < HF_V; ++v) s = hf_red<HF_OP>(s, acc[v]);
      s = hf_wave_reduce<HF_OP>(s);
      if (lane == 0) sp[wave] = s;
      __syncthreads();
      if (threadIdx.x == 0) {
        float t = sp[0];
        for (int q = 1; q < HF_BLOCK / 64; ++q) t = hf_red<HF_OP>(t, sp[q]);
        ((float *)A.ws)[(long)seg * HF_ROWS + row] = t;
      }
#endif
      __syncthreads();  // the partials' LDS slots are reused next step
    }
  }
#elif HF_OP == 3
  // max/argmax: the index of element (row, kv, v) along the reduced dim is
  // kv * HF_V + v; each lane visits its elements in increasing index order.
  constexpr int RPB = HF_BLOCK / HF_TPR;
  constexpr int GW = HF_TPR < 64 ? HF_TPR : 64;  // lanes reduced by shuffles
  __shared__ float pm[HF_BLOCK / 64];
  __shared__ int pk[HF_BLOCK / 64];
  const int sub = threadIdx.x % HF_TPR, rloc = threadIdx.x / HF_TPR;
  for (int row0 = blockIdx.x * RPB; row0 < HF_ROWS; row0 += gridDim.x * RPB) {
    const int row = row0 + rloc;
    float m = HF_ARG_V0;
    int k = HF_ARG_NONE;
    if (row < HF_ROWS) {
      // the row's chunks in batches of up to 8 per thread, loads first
      constexpr int IT = (HF_KV + HF_TPR - 1) / HF_TPR;
      constexpr int NB = IT < 8 ? (IT > 0 ? IT : 1) : 8;
      for (int it0 = 0; it0 < IT; it0 += NB) {
        hf_regs_t R[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int kv = (it0 + b) * HF_TPR + sub;
          if (kv < HF_KV) hf_rr_eval_fetch(A, row, kv, R[b]);
        }
        HF_LOADS_ISSUED();
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int kv = (it0 + b) * HF_TPR + sub;
          if (kv < HF_KV) {
            float x[HF_V];
            hf_rr_eval(A, row, kv, R[b], x);
#pragma unroll
            for (int v = 0; v < HF_V; ++v) hf_arg_step(m, k, x[v], kv * HF_V + v);
          }
        }
      }
    }
    if constexpr (GW == 64) hf_arg_wave_reduce(m, k);
    else hf_arg_group_reduce<GW>(m, k);
    if (HF_TPR > 64) {  // one row per workgroup: combine the waves through LDS
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
      if (lane == 0) {
        pm[wave] = m;
        pk[wave] = k;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        for (int w = 1; w < HF_BLOCK / 64; ++w) hf_arg_combine(m, k, pm[w], pk[w]);
        hf_rr_store_arg(A, row, k);
      }
      __syncthreads();
    } else if (sub == 0 && row < HF_ROWS) {
      hf_rr_store_arg(A, row, k);
    }
  }
#else
#if HF_TPR == HF_BLOCK
  // Two result slots, alternating between a workgroup's consecutive steps, so
  // that one barrier per step is enough.
  constexpr int RR = HF_RR_ROWS;
  __shared__ float part[2][RR][HF_BLOCK / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int ITERS = (HF_KV + HF_BLOCK - 1) / HF_BLOCK;
  // acc[r] holds row row0 + r; rows past the end are neither read nor stored
  auto finish = [&](int row0, const float (&acc)[RR][HF_V], int slot) {
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      float s = acc[r][0];
#pragma unroll
      for (int v = 1; v < HF_V; ++v) s = hf_red<HF_OP>(s, acc[r][v]);
      s = hf_wave_reduce<HF_OP>(s);
      if (lane == 0) part[slot][r][wave] = s;
    }
    __syncthreads();
    if (threadIdx.x < RR && row0 + (int)threadIdx.x < HF_ROWS) {
      const int r = threadIdx.x;
      float t = part[slot][r][0];
#pragma unroll
      for (int w = 1; w < HF_BLOCK / 64; ++w) t = hf_red<HF_OP>(t, part[slot][r][w]);
      hf_rr_store(A, row0 + r, t);
    }
  };
#if HF_RR_PIPE
  {
    // Two rows in flight per workgroup: the loads of row + gridDim.x are
    // issued before row is accumulated.  Unrolled by two, so that the two
    // register sets swap roles without copies.  The loop holds no global
    // store (on this target stores and loads share one counter, and a
    // pending store would make every wait a full drain): the workgroup's
    // row results (at most HF_RR_PIPE_K) collect in LDS and are stored after
    // the last row.
    static_assert(RR == 1 && HF_KV % HF_BLOCK == 0 && ITERS <= 8, "pipelined rows take one batch each");
    __shared__ float res[HF_RR_PIPE_K];
    hf_regs_t R0[ITERS], R1[ITERS];
    auto fetch = [&](int row, hf_regs_t(&R)[ITERS]) {
#pragma unroll
      for (int b = 0; b < ITERS; ++b) hf_rr_eval_fetch(A, row, b * HF_BLOCK + (int)threadIdx.x, R[b]);
    };
    auto consume = [&](int row, int k, const hf_regs_t(&R)[ITERS], int slot) {
      float s = hf_red_identity<HF_OP>();
      {
        float x[HF_V];
        hf_rr_eval(A, row, (int)threadIdx.x, R[0], x);
        float acc[HF_V];
#pragma unroll
        for (int v = 0; v < HF_V; ++v) acc[v] = hf_red<HF_OP>(hf_red_identity<HF_OP>(), x[v]);
#pragma unroll
        for (int b = 1; b < ITERS; ++b) {
          hf_rr_eval(A, row, b * HF_BLOCK + (int)threadIdx.x, R[b], x);
#pragma unroll
          for (int v = 0; v < HF_V; ++v) acc[v] = hf_red<HF_OP>(acc[v], x[v]);
        }
        s = acc[0];
#pragma unroll
        for (int v = 1; v < HF_V; ++v) s = hf_red<HF_OP>(s, acc[v]);
      }
      s = hf_wave_reduce<HF_OP>(s);
      if (lane == 0) part[slot][0][wave] = s;
      __syncthreads();
      if (threadIdx.x == 0) {
        float t = part[slot][0][0];
#pragma unroll
        for (int w = 1; w < HF_BLOCK / 64; ++w) t = hf_red<HF_OP>(t, part[slot][0][w]);
        res[k] = t;
      }
    };
    // Every fetch inside the loop is unconditional (the next row is known to
    // exist), so that each wait counts only the other register set's loads;
    // the last row is accumulated on the way out.
    int row = blockIdx.x, k = 0;
    if (row < HF_ROWS) {
      fetch(row, R0);
      for (;;) {
        if (row + (int)gridDim.x >= HF_ROWS) {
          consume(row, k++, R0, 0);
          break;
        }
        fetch(row + gridDim.x, R1);
        HF_LOADS_ISSUED();
        consume(row, k++, R0, 0);
        row += gridDim.x;
        if (row + (int)gridDim.x >= HF_ROWS) {
          consume(row, k++, R1, 1);
          break;
        }
        fetch(row + gridDim.x, R0);
        HF_LOADS_ISSUED();
        consume(row, k++, R1, 1);
        row += gridDim.x;
      }
    }
    __syncthreads();
    for (int j = threadIdx.x; j < k; j += HF_BLOCK) hf_rr_store(A, blockIdx.x + j * gridDim.x, res[j]);
  }
#elif HF_KV % HF_BLOCK == 0
  {
    // RR rows per step; their chunks in batches of up to 8 loads per thread,
    // each batch's loads issued before its accumulation
    constexpr int NB0 = 8 / RR > 0 ? 8 / RR : 1;
    constexpr int NB = ITERS < NB0 ? ITERS : NB0;
    int slot = 0;
    for (int row0 = blockIdx.x * RR; row0 < HF_ROWS; row0 += gridDim.x * RR, slot ^= 1) {
      float acc[RR][HF_V];
#pragma unroll
      for (int r = 0; r < RR; ++r)
#pragma unroll
        for (int v = 0; v < HF_V; ++v) acc[r][v] = hf_red_identity<HF_OP>();
      for (int it0 = 0; it0 < ITERS; it0 += NB) {
        hf_regs_t R[RR][NB];
#pragma unroll
        for (int r = 0; r < RR; ++r)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            if ((RR == 1 || row0 + r < HF_ROWS) && (ITERS % NB == 0 || it0 + b < ITERS))
              hf_rr_eval_fetch(A, row0 + r, (it0 + b) * HF_BLOCK + (int)threadIdx.x, R[r][b]);
        HF_LOADS_ISSUED();
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
          for (int r = 0; r < RR; ++r) {
            if ((RR == 1 || row0 + r < HF_ROWS) && (ITERS % NB == 0 || it0 + b < ITERS)) {
              float x[HF_V];
              hf_rr_eval(A, row0 + r, (it0 + b) * HF_BLOCK + (int)threadIdx.x, R[r][b], x);
#pragma unroll
              for (int v = 0; v < HF_V; ++v) acc[r][v] = hf_red<HF_OP>(acc[r][v], x[v]);
            }
          }
        }
      }
      finish(row0, acc, slot);
    }
  }
#else
  {
    static_assert(RR == 1, "rows of unequal chunks take one row per step");
    int slot = 0;
    for (int row = blockIdx.x; row < HF_ROWS; row += gridDim.x, slot ^= 1) {
      float acc[1][HF_V];
#pragma unroll
      for (int v = 0; v < HF_V; ++v) acc[0][v] = hf_red_identity<HF_OP>();
      for (int kv = threadIdx.x; kv < HF_KV; kv += HF_BLOCK) {
        hf_regs_t R1;
        hf_rr_eval_fetch(A, row, kv, R1);
        float x[HF_V];
        hf_rr_eval(A, row, kv, R1, x);
#pragma unroll
        for (int v = 0; v < HF_V; ++v) acc[0][v] = hf_red<HF_OP>(acc[0][v], x[v]);
      }
      finish(row, acc, slot);
    }
  }
#endif
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
#endif  // HF_RSEG > 1, HF_OP == 3
}

#if HF_RSEG > 1
// The fold: one workgroup per row.  Thread t combines the row's partials of
// segments t, t + 256, ... in order; the waves reduce theirs with DPP and
// thread 0 combines the four waves in order, then applies the reduce's init
// and epilogue (hf_rr_store).  A fixed tree: the same result every launch.
extern "C" __global__ __launch_bounds__(256) void HF_FOLD_NAME(HF_KERNEL_PARAMS) {
  const HfArgs A = HF_ARGS_INIT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x;
#if HF_OP == 3
  __shared__ float pm[4];
  __shared__ int pk[4];
  float m = HF_ARG_V0;
  int k = HF_ARG_NONE;
  for (int q = threadIdx.x; q < HF_RSEG; q += 256)
    hf_arg_combine(m, k, ((const float *)A.ws)[(long)q * HF_ROWS + row],
                   ((const int *)A.ws)[(long)HF_RSEG * HF_ROWS + (long)q * HF_ROWS + row]);
  hf_arg_wave_reduce(m, k);
  if (lane == 0) {
    pm[wave] = m;
    pk[wave] = k;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) hf_arg_combine(m, k, pm[w], pk[w]);
    hf_rr_store_arg(A, row, k);
  }
#else
  __shared__ float part[4];
  float s = hf_red_identity<HF_OP>();
  for (int q = threadIdx.x; q < HF_RSEG; q += 256) s = hf_red<HF_OP>(s, ((const float *)A.ws)[(long)q * HF_ROWS + row]);
  s = hf_wave_reduce<HF_OP>(s);
  if (lane == 0) part[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0)
    hf_rr_store(A, row, hf_red<HF_OP>(hf_red<HF_OP>(part[0], part[1]), hf_red<HF_OP>(part[2], part[3])));
#endif
}
#endif
