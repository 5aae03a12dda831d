// transpose.hip -- transpose hero (XLA:GPU Emitters, "Transpose emitter").
//
// One workgroup per (batch, W-tile, U-tile).  U is the physically minor
// output dimension; W is the output dimension that the transposed operand
// stores contiguously.  Phase 1 reads the tile with 128-bit loads that are
// contiguous along W (coalesced in the INPUT), evaluates the staged node (the
// transpose and its prologue) and writes it to LDS in [w][u] order.  After a
// barrier, phase 2 reads the tile along U, evaluates the epilogue (everything
// between the staged node and the root) and writes 128-bit vectors that are
// contiguous along U (coalesced in the OUTPUT).  The LDS row pitch is the tile
// width plus one 4-byte word, so both the column writes of phase 1 and the
// row reads of phase 2 spread over all banks.  Full tiles (all but the ragged
// edge) take a path without bounds checks that issues every global load of
// the phase before the first use.
//
// Provided by the generated code: HF_BLOCK, HF_TU, HF_TW, HF_PITCH, HF_VIN,
// HF_VOUT, HF_DU, HF_DW, HF_NTU, HF_NTW, HF_ORDER (tile order), hf_tile_t,
// hf_val_t, hf_ldregs_t, hf_stregs_t, hf_tr_load_fetch / hf_tr_load (staged node at (b, w.., u)),
// hf_tr_eval_fetch / hf_tr_eval (root at (b, w, u..)), hf_tr_store.
extern "C" __global__ __launch_bounds__(HF_BLOCK) void HF_KERNEL_NAME(HF_KERNEL_PARAMS) {
  const HfArgs A = HF_ARGS_INIT;
  __shared__ hf_tile_t tile[HF_TW * HF_PITCH];
#if HF_ORDER == 3
  // XCD-contiguous: workgroup i runs on XCD i % 8, so XCD x takes the x-th
  // contiguous range of tiles in (batch, U-tile, W-tile) order, W fastest.
  // Tiles that share input lines (the W-neighbours of one U range, when the
  // input rows are not whole 128-byte lines) then read them through one L2.
  constexpr int NX = 8;
  const int n = (int)gridDim.x, x = (int)blockIdx.x % NX, q = n / NX, r = n % NX;
  const int bid = x * q + (x < r ? x : r) + (int)blockIdx.x / NX;
#else
  const int bid = blockIdx.x;
#endif
  const int b = bid / (HF_NTU * HF_NTW);
  const int t = bid % (HF_NTU * HF_NTW);
#if HF_ORDER == 0  // U-tiles fastest
  const int tu = t % HF_NTU, tw = t / HF_NTU;
#elif HF_ORDER == 1 || HF_ORDER == 3  // W-tiles fastest
  const int tw = t % HF_NTW, tu = t / HF_NTW;
#else  // diagonal: W-tiles fastest, U-tile shifted by the W-tile
  const int tw = t % HF_NTW, tu = (t / HF_NTW + tw) % HF_NTU;
#endif
  const int u0 = tu * HF_TU, w0 = tw * HF_TW;
  constexpr int WV = HF_TW / HF_VIN;          // load-phase vectors per tile row
  constexpr int UV = HF_TU / HF_VOUT;         // store-phase vectors per tile row
  constexpr int LIT = (HF_TU * WV + HF_BLOCK - 1) / HF_BLOCK;
  constexpr int SIT = (HF_TW * UV + HF_BLOCK - 1) / HF_BLOCK;
  const bool full = u0 + HF_TU <= HF_DU && w0 + HF_TW <= HF_DW;
  if (full && (HF_TU * WV) % HF_BLOCK == 0) {
    hf_ldregs_t R[LIT];
#pragma unroll
    for (int it = 0; it < LIT; ++it) {
      const int k = it * HF_BLOCK + (int)threadIdx.x;
      hf_tr_load_fetch(A, b, w0 + (k % WV) * HF_VIN, u0 + k / WV, R[it]);
    }
    HF_LOADS_ISSUED();
#pragma unroll
    for (int it = 0; it < LIT; ++it) {
      const int k = it * HF_BLOCK + (int)threadIdx.x;
      const int ul = k / WV, wl = (k % WV) * HF_VIN;
      hf_tile_t r[HF_VIN];
      hf_tr_load(A, b, w0 + wl, u0 + ul, R[it], r);
#pragma unroll
      for (int v = 0; v < HF_VIN; ++v) tile[(wl + v) * HF_PITCH + ul] = r[v];
    }
  } else {
    for (int k = threadIdx.x; k < HF_TU * WV; k += HF_BLOCK) {
      const int ul = k / WV, wl = (k % WV) * HF_VIN;
      if (u0 + ul < HF_DU && w0 + wl < HF_DW) {
        hf_ldregs_t R1;
        hf_tr_load_fetch(A, b, w0 + wl, u0 + ul, R1);
        hf_tile_t r[HF_VIN];
        hf_tr_load(A, b, w0 + wl, u0 + ul, R1, r);
#pragma unroll
        for (int v = 0; v < HF_VIN; ++v) tile[(wl + v) * HF_PITCH + ul] = r[v];
      }
    }
  }
  __syncthreads();
  if (full && (HF_TW * UV) % HF_BLOCK == 0) {
    hf_stregs_t R[SIT];
#pragma unroll
    for (int it = 0; it < SIT; ++it) {
      const int k = it * HF_BLOCK + (int)threadIdx.x;
      hf_tr_eval_fetch(A, b, w0 + k / UV, u0 + (k % UV) * HF_VOUT, R[it]);
    }
    HF_LOADS_ISSUED();
#pragma unroll
    for (int it = 0; it < SIT; ++it) {
      const int k = it * HF_BLOCK + (int)threadIdx.x;
      const int wl = k / UV, ul = (k % UV) * HF_VOUT;
      hf_val_t r[HF_VOUT];
      hf_tr_eval(A, tile, w0, u0, b, w0 + wl, u0 + ul, R[it], r);
      hf_tr_store(A, b, w0 + wl, u0 + ul, r);
    }
  } else {
    for (int k = threadIdx.x; k < HF_TW * UV; k += HF_BLOCK) {
      const int wl = k / UV, ul = (k % UV) * HF_VOUT;
      if (u0 + ul < HF_DU && w0 + wl < HF_DW) {
        hf_stregs_t R1;
        hf_tr_eval_fetch(A, b, w0 + wl, u0 + ul, R1);
        hf_val_t r[HF_VOUT];
        hf_tr_eval(A, tile, w0, u0, b, w0 + wl, u0 + ul, R1, r);
        hf_tr_store(A, b, w0 + wl, u0 + ul, r);
      }
    }
  }
}
