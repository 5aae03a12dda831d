// common.hip -- device helpers shared by every generated fusion kernel.
//
// The library prepends this text to the generated code of each fusion and
// compiles the whole translation unit for gfx950 at hf_fusion_create time
// (-O3, -ffp-contract=off, no fast-math, packed-FP32 instructions disabled).
//
// Value convention inside a kernel: every floating-point element is carried
// in a 32-bit float that holds exactly a value of the node's declared element
// type (bf16 and f16 values are exact in f32); integer and quantized storage
// values are carried in int.  Each op rounds its result once to its declared
// type (StableHLO Specification, op semantics), so a bf16 op is an f32 op
// followed by a round-to-nearest-even to bf16.

typedef unsigned int hf_u32;
typedef unsigned short hf_u16;
typedef unsigned long long hf_u64;

// The generated code defines the kernel's parameter list (HF_KERNEL_PARAMS:
// one __restrict__ pointer per fusion parameter, the result, the per-axis
// quantization arrays and the workspace, so the compiler may assume they do
// not alias), the struct HfArgs that bundles them and HF_ARGS_INIT.

// ---------------------------------------------------------------- rounding
// bf16 RNE through the hardware pack-convert (v_cvt_pk_bf16_f32), back to f32.
__device__ __forceinline__ float hf_rnd_bf16(float x) {
  return __uint_as_float((hf_u32)__builtin_bit_cast(hf_u16, (__bf16)x) << 16);
}
__device__ __forceinline__ float hf_rnd_f16(float x) { return (float)(_Float16)x; }
__device__ __forceinline__ float hf_bf16_bits(hf_u32 bits16) { return __uint_as_float(bits16 << 16); }

// ------------------------------------------------------- IEEE max/min
// IEEE 754-2019 maximum/minimum (NaN-propagating, -0 < +0): v_maximum3_f32,
// v_minimum3_f32 on gfx950.
__device__ __forceinline__ float hf_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float hf_min(float a, float b) { return __builtin_elementwise_minimum(a, b); }

// ------------------------------------------------------- transcendentals
// exp whose result is rounded to bf16 afterwards: 2^(x*log2 e) on the
// hardware exp2 (v_exp_f32, about 1 ulp).  Relative error of the f32 value is
// below 2^-16 over the whole bf16 range, far under half a bf16 ulp (2^-9), so
// after rounding the bf16 result is within one bf16 ulp of the correctly
// rounded one.  Arguments below -126 are scaled so the hardware sees a normal
// result and the final multiply produces the subnormal.
__device__ __forceinline__ float hf_exp_for_bf16(float x) {
  float t = x * 1.44269504088896340736f;
  if (t < -126.0f) return __builtin_amdgcn_exp2f(t + 64.0f) * 5.42101086242752217e-20f;
  return __builtin_amdgcn_exp2f(t);
}

// ---------------------------------------------------------- reductions
// reducer codes: 0 add, 1 maximum, 2 minimum
template <int OP>
__device__ __forceinline__ float hf_red(float a, float b) {
  if constexpr (OP == 0) return a + b;
  else if constexpr (OP == 1) return hf_max(a, b);
  else return hf_min(a, b);
}
template <int OP>
__device__ __forceinline__ float hf_red_identity() {
  if constexpr (OP == 0) return -0.0f;  // -0 + x == x for every x, +0 and -0 included
  else if constexpr (OP == 1) return -__builtin_inff();
  else return __builtin_inff();
}

// Whole-wave (64 lanes) reduction: DPP within each row of 16 lanes
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror:4, row_ror:8 leave the
// row's result in every lane of the row), then the four row results are read
// with readlane and combined.  Every lane must be active.
#define HF_DPP(v, ctrl) \
  __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), (ctrl), 0xF, 0xF, false))
template <int OP>
__device__ __forceinline__ float hf_wave_reduce(float v) {
  v = hf_red<OP>(v, HF_DPP(v, 0xB1));   // quad_perm [1,0,3,2]
  v = hf_red<OP>(v, HF_DPP(v, 0x4E));   // quad_perm [2,3,0,1]
  v = hf_red<OP>(v, HF_DPP(v, 0x124));  // row_ror:4
  v = hf_red<OP>(v, HF_DPP(v, 0x128));  // row_ror:8
  float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return hf_red<OP>(hf_red<OP>(r0, r1), hf_red<OP>(r2, r3));
}

// Reduction over aligned groups of W lanes (W a power of two <= 64): the
// result ends up in every lane of the group.
template <int OP, int W>
__device__ __forceinline__ float hf_group_reduce(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = hf_red<OP>(v, __shfl_xor(v, o, W));
  return v;
}

// ------------------------------------------------------------ loads
// Vector loads of V consecutive elements starting at element offset `off`
// (off is a multiple of V, buffers are 16-byte aligned).
template <int V>
__device__ __forceinline__ void hf_ld_f32(const void *base, int off, float (&r)[V]) {
  const float *p = (const float *)base + off;
  if constexpr (V % 4 == 0) {
#pragma unroll
    for (int k = 0; k < V / 4; ++k) {
      float4 t = ((const float4 *)p)[k];
      r[4 * k] = t.x; r[4 * k + 1] = t.y; r[4 * k + 2] = t.z; r[4 * k + 3] = t.w;
    }
  } else if constexpr (V == 2) {
    float2 t = *(const float2 *)p;
    r[0] = t.x; r[1] = t.y;
  } else {
    r[0] = p[0];
  }
}
template <int V>
__device__ __forceinline__ void hf_ld_i32(const void *base, int off, int (&r)[V]) {
  const int *p = (const int *)base + off;
#pragma unroll
  for (int k = 0; k < V; ++k) r[k] = p[k];
}
// 16-bit floats: bf16 (F16=false) or f16 (F16=true)
template <int V, bool F16>
__device__ __forceinline__ void hf_ld_h(const void *base, int off, float (&r)[V]) {
  const hf_u16 *p = (const hf_u16 *)base + off;
  hf_u32 w[(V + 1) / 2];
  if constexpr (V % 8 == 0) {
#pragma unroll
    for (int k = 0; k < V / 8; ++k) {
      uint4 t = ((const uint4 *)p)[k];
      w[4 * k] = t.x; w[4 * k + 1] = t.y; w[4 * k + 2] = t.z; w[4 * k + 3] = t.w;
    }
  } else if constexpr (V == 4) {
    uint2 t = *(const uint2 *)p;
    w[0] = t.x; w[1] = t.y;
  } else if constexpr (V == 2) {
    w[0] = *(const hf_u32 *)p;
  } else {
    w[0] = p[0];
  }
#pragma unroll
  for (int k = 0; k < V; ++k) {
    hf_u32 h = (k & 1) ? (w[k / 2] >> 16) : (w[k / 2] & 0xFFFFu);
    if constexpr (F16) r[k] = (float)__builtin_bit_cast(_Float16, (hf_u16)h);
    else r[k] = __uint_as_float(h << 16);
  }
}
// 8-bit integers, sign- or zero-extended
template <int V, bool SIGNED>
__device__ __forceinline__ void hf_ld_b(const void *base, int off, int (&r)[V]) {
  const unsigned char *p = (const unsigned char *)base + off;
  hf_u32 w[(V + 3) / 4];
  if constexpr (V % 16 == 0) {
#pragma unroll
    for (int k = 0; k < V / 16; ++k) {
      uint4 t = ((const uint4 *)p)[k];
      w[4 * k] = t.x; w[4 * k + 1] = t.y; w[4 * k + 2] = t.z; w[4 * k + 3] = t.w;
    }
  } else if constexpr (V == 8) {
    uint2 t = *(const uint2 *)p;
    w[0] = t.x; w[1] = t.y;
  } else if constexpr (V == 4) {
    w[0] = *(const hf_u32 *)p;
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) w[0] = (k == 0 ? 0u : w[0]) | ((hf_u32)p[k] << (8 * k));
  }
#pragma unroll
  for (int k = 0; k < V; ++k) {
    hf_u32 b = (w[k / 4] >> (8 * (k & 3))) & 0xFFu;
    r[k] = SIGNED ? (int)(signed char)b : (int)b;
  }
}

// ------------------------------------------------------------ stores
template <int V>
__device__ __forceinline__ void hf_st_f32(void *base, int off, const float (&r)[V]) {
  float *p = (float *)base + off;
  if constexpr (V % 4 == 0) {
#pragma unroll
    for (int k = 0; k < V / 4; ++k)
      ((float4 *)p)[k] = make_float4(r[4 * k], r[4 * k + 1], r[4 * k + 2], r[4 * k + 3]);
  } else if constexpr (V == 2) {
    *(float2 *)p = make_float2(r[0], r[1]);
  } else {
    p[0] = r[0];
  }
}
// 16-bit floats: values are already exact in the target type.
template <bool F16>
__device__ __forceinline__ hf_u32 hf_h_bits(float x) {
  if constexpr (F16) return (hf_u32)__builtin_bit_cast(hf_u16, (_Float16)x);
  else return __float_as_uint(x) >> 16;
}
template <int V, bool F16>
__device__ __forceinline__ void hf_st_h(void *base, int off, const float (&r)[V]) {
  hf_u16 *p = (hf_u16 *)base + off;
  if constexpr (V >= 2) {
    hf_u32 w[V / 2];
#pragma unroll
    for (int k = 0; k < V / 2; ++k) {
      if constexpr (F16)
        w[k] = hf_h_bits<true>(r[2 * k]) | (hf_h_bits<true>(r[2 * k + 1]) << 16);
      else  // take the upper halves of both floats in one v_perm_b32
        w[k] = __builtin_amdgcn_perm(__float_as_uint(r[2 * k + 1]), __float_as_uint(r[2 * k]), 0x07060302u);
    }
    if constexpr (V % 8 == 0) {
#pragma unroll
      for (int k = 0; k < V / 8; ++k)
        ((uint4 *)p)[k] = make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
    } else if constexpr (V == 4) {
      *(uint2 *)p = make_uint2(w[0], w[1]);
    } else {
      *(hf_u32 *)p = w[0];
    }
  } else {
    p[0] = (hf_u16)hf_h_bits<F16>(r[0]);
  }
}
template <int V>
__device__ __forceinline__ void hf_st_b(void *base, int off, const int (&r)[V]) {
  unsigned char *p = (unsigned char *)base + off;
  if constexpr (V >= 4) {
    hf_u32 w[V / 4];
#pragma unroll
    for (int k = 0; k < V / 4; ++k)
      w[k] = ((hf_u32)r[4 * k] & 0xFFu) | (((hf_u32)r[4 * k + 1] & 0xFFu) << 8) |
             (((hf_u32)r[4 * k + 2] & 0xFFu) << 16) | ((hf_u32)r[4 * k + 3] << 24);
    if constexpr (V % 16 == 0) {
#pragma unroll
      for (int k = 0; k < V / 16; ++k)
        ((uint4 *)p)[k] = make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
    } else if constexpr (V == 8) {
      *(uint2 *)p = make_uint2(w[0], w[1]);
    } else {
      *(hf_u32 *)p = w[0];
    }
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) p[k] = (unsigned char)r[k];
  }
}
template <int V>
__device__ __forceinline__ void hf_st_i32(void *base, int off, const int (&r)[V]) {
  int *p = (int *)base + off;
#pragma unroll
  for (int k = 0; k < V; ++k) p[k] = r[k];
}

// -------------------------------------------------------- quantization
// uniform_quantize of one value: IEEE division by the scale, round half to
// even (v_rndne_f32), zero point added as an integer, clamp to the storage
// range.  The clamp is applied in float before the integer conversion, with
// the bounds shifted by the zero point (exact for these small integers).
__device__ __forceinline__ int hf_quantize(float y, float scale, int zp, int smin, int smax) {
  float t = y / scale;
  float r = __builtin_rintf(t);
  r = __builtin_fminf(__builtin_fmaxf(r, (float)(smin - zp)), (float)(smax - zp));
  return (int)r + zp;
}
