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
// row reads of phase 2 spread over all banks.
//
// Provided by the generated code: HF_BLOCK, HF_TU, HF_TW, HF_PITCH, HF_VIN,
// HF_VOUT, HF_DU, HF_DW, HF_NTU, HF_NTW, hf_tile_t, hf_val_t,
// hf_tr_load(A, b, w, u, r), hf_tr_eval(A, tile, w0, u0, b, w, u, r),
// hf_tr_store(A, b, w, u, r).
extern "C" __global__ __launch_bounds__(HF_BLOCK) void hf_kernel(HF_KERNEL_PARAMS) {
  const HfArgs A = HF_ARGS_INIT;
  __shared__ hf_tile_t tile[HF_TW * HF_PITCH];
  int bid = blockIdx.x;
  const int tu = bid % HF_NTU;
  bid /= HF_NTU;
  const int tw = bid % HF_NTW;
  const int b = bid / HF_NTW;
  const int u0 = tu * HF_TU, w0 = tw * HF_TW;
  constexpr int WV = HF_TW / HF_VIN;
#pragma unroll
  for (int k0 = 0; k0 < HF_TU * WV; k0 += HF_BLOCK) {
    const int k = k0 + (int)threadIdx.x;
    const int ul = k / WV, wl = (k % WV) * HF_VIN;
    if ((HF_TU * WV % HF_BLOCK == 0 || k < HF_TU * WV) && u0 + ul < HF_DU && w0 + wl < HF_DW) {
      hf_tile_t r[HF_VIN];
      hf_tr_load(A, b, w0 + wl, u0 + ul, r);
#pragma unroll
      for (int v = 0; v < HF_VIN; ++v) tile[(wl + v) * HF_PITCH + ul] = r[v];
    }
  }
  __syncthreads();
  constexpr int UV = HF_TU / HF_VOUT;
#pragma unroll
  for (int k0 = 0; k0 < HF_TW * UV; k0 += HF_BLOCK) {
    const int k = k0 + (int)threadIdx.x;
    const int wl = k / UV, ul = (k % UV) * HF_VOUT;
    if ((HF_TW * UV % HF_BLOCK == 0 || k < HF_TW * UV) && u0 + ul < HF_DU && w0 + wl < HF_DW) {
      hf_val_t r[HF_VOUT];
      hf_tr_eval(A, tile, w0, u0, b, w0 + wl, u0 + ul, r);
      hf_tr_store(A, b, w0 + wl, u0 + ul, r);
    }
  }
}
