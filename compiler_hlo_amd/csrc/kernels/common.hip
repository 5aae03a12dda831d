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
typedef unsigned int hf_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int hf_u32x2 __attribute__((ext_vector_type(2)));

// The generated code defines the kernel's parameter list (HF_KERNEL_PARAMS:
// one __restrict__ pointer per fusion parameter, the result, the per-axis
// quantization arrays and the workspace, so the compiler may assume they do
// not alias), the struct HfArgs that bundles them and HF_ARGS_INIT.

// ---------------------------------------------------------------- rounding
// bf16 RNE in one instruction: v_cvt_pk_bf16_f32 of the pair (0, x) puts the
// rounded bf16 of x in the upper half and zero in the lower half, which is
// exactly the f32 bit pattern of the rounded value.
typedef __bf16 hf_bf16x2 __attribute__((ext_vector_type(2)));
typedef float hf_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float hf_rnd_bf16(float x) {
  const hf_f32x2 v = {0.0f, x};
  return __builtin_bit_cast(float, __builtin_convertvector(v, hf_bf16x2));
}
__device__ __forceinline__ float hf_rnd_f16(float x) { return (float)(_Float16)x; }
__device__ __forceinline__ float hf_bf16_bits(hf_u32 bits16) { return __uint_as_float(bits16 << 16); }

// ------------------------------------------------------- IEEE max/min
// IEEE 754-2019 maximum/minimum (NaN-propagating, -0 < +0): v_maximum3_f32,
// v_minimum3_f32 on gfx950.
__device__ __forceinline__ float hf_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float hf_min(float a, float b) { return __builtin_elementwise_minimum(a, b); }

// ------------------------------------------------------- transcendentals
// exp whose result is rounded to bf16 afterwards: (2^(x*log2(e)/2))^2 on the
// hardware exp2 (v_exp_f32, about 1 ulp).  The half-size argument keeps the
// exp2 result normal down to final results of 2^-252, and the IEEE square
// then produces subnormal results correctly -- no branch, no select.  The
// f32 value's relative error stays below 2^-16 over the whole bf16 range,
// far under half a bf16 ulp (2^-9), so after rounding the bf16 result is
// within one bf16 ulp of the correctly rounded one.
__device__ __forceinline__ float hf_exp_for_bf16(float x) {
  const float h = __builtin_amdgcn_exp2f(x * 0.72134752044448170368f);  // log2(e)/2
  return h * h;
}

// tanh of a bf16 value whose result is rounded to bf16.  Below 2^-4 in
// magnitude tanh(x) rounds to x itself (true for every bf16 input below
// 0.0903).  Otherwise (e - 1) / (e + 1) with e = e^(2|x|) from the hardware
// exp2 and reciprocal: there e - 1 >= 0.13, so the exp2 error stays near
// 2^-20 relative in the quotient, far under half a bf16 ulp (2^-9).  |x| is
// capped at 9, where the quotient already rounds to 1 and e stays finite; the
// cap is IEEE minimum, so a NaN stays NaN.  The sign is restored last
// (tanh(-0) = -0).  Exhaustive over the bf16 inputs the result rounds to the
// correctly rounded value.
__device__ __forceinline__ float hf_tanh_for_bf16(float x) {
  const float a = __builtin_elementwise_minimum(__builtin_fabsf(x), 9.0f);
  const float e = __builtin_amdgcn_exp2f(a * 2.8853900817779268f);  // 2 log2(e)
  const float t = (e - 1.0f) * __builtin_amdgcn_rcpf(e + 1.0f);
  return __builtin_copysignf(a < 0.0625f ? a : t, x);
}

__device__ __forceinline__ int hf_clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

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

// Max/argmax pairs (the variadic reduce of Operation semantics).  A thread
// folds its elements in increasing index order with the reducer body: the
// value replaces the running maximum when value >= max (so NaN never does,
// and later equal values win).  Partial results then combine by larger
// value, then larger index -- a commutative, associative choice that gives
// the sequential fold's answer.  Every partial starts from (value init,
// HF_ARG_NONE): HF_ARG_NONE means "no element has replaced the init yet" and
// loses every index tie, so the final pair holds the last index of the
// maximum whenever an element reached it.  The index init of the fold is
// written only where HF_ARG_NONE survives to the end (the store), which is
// exactly where the sequential fold never replaced its initial pair -- for
// any index init, also one inside the row.
#define HF_ARG_NONE (-2147483647 - 1)
__device__ __forceinline__ void hf_arg_step(float &m, int &k, float v, int j) {
  if (v >= m) {
    m = v;
    k = j;
  }
}
__device__ __forceinline__ void hf_arg_combine(float &m, int &k, float m2, int k2) {
  if (m2 > m || (m2 == m && k2 > k)) {
    m = m2;
    k = k2;
  }
}
// A whole wave's pairs by the DPP pattern of hf_wave_reduce; the result is
// returned in every lane.  Every lane must be active.
__device__ __forceinline__ void hf_arg_wave_reduce(float &m, int &k) {
#define HF_ARG_DPP(ctrl)                                                        \
  {                                                                            \
    const float m2 = HF_DPP(m, ctrl);                                          \
    const int k2 = __builtin_amdgcn_update_dpp(0, k, (ctrl), 0xF, 0xF, false); \
    hf_arg_combine(m, k, m2, k2);                                              \
  }
  HF_ARG_DPP(0xB1)   // quad_perm [1,0,3,2]
  HF_ARG_DPP(0x4E)   // quad_perm [2,3,0,1]
  HF_ARG_DPP(0x124)  // row_ror:4
  HF_ARG_DPP(0x128)  // row_ror:8
#undef HF_ARG_DPP
  float mr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0));
  int kr = __builtin_amdgcn_readlane(k, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16)
    hf_arg_combine(mr, kr, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), r)),
                   __builtin_amdgcn_readlane(k, r));
  m = mr;
  k = kr;
}
template <int W>  // across groups of W lanes (W a power of two <= 64)
__device__ __forceinline__ void hf_arg_group_reduce(float &m, int &k) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, W);
    const int k2 = __shfl_xor(k, o, W);
    hf_arg_combine(m, k, m2, k2);
  }
}

// ------------------------------------------------------------ loads
// Global loads are split from their use: a fetch function issues the raw
// loads of a whole hero step into registers (so every load of the step is in
// flight at once), the compute function unpacks them.  Raw vector loads move
// NB bytes (4..64) starting at a byte offset that is a multiple of NB.
// Streaming operands (each byte used once) are loaded and stored with the
// non-temporal hint: they stream through the caches instead of evicting
// what is reused (per-axis parameters, biases).  HF_NT_STORES = 0 turns the
// store hint off.
#ifndef HF_NT_STORES
#define HF_NT_STORES 1
#endif
template <int NB, bool NT = false>
__device__ __forceinline__ void hf_raw_ld(const void *base, long byte_off, hf_u32 (&w)[NB / 4]) {
  const char *p = (const char *)base + byte_off;
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int k = 0; k < NB / 16; ++k) {
      hf_u32x4 t;
      if constexpr (NT) t = __builtin_nontemporal_load((const hf_u32x4 *)p + k);
      else t = ((const hf_u32x4 *)p)[k];
      w[4 * k] = t.x; w[4 * k + 1] = t.y; w[4 * k + 2] = t.z; w[4 * k + 3] = t.w;
    }
  } else if constexpr (NB == 8) {
    hf_u32x2 t;
    if constexpr (NT) t = __builtin_nontemporal_load((const hf_u32x2 *)p);
    else t = *(const hf_u32x2 *)p;
    w[0] = t.x; w[1] = t.y;
  } else {
    static_assert(NB == 4, "raw loads move 4, 8 or a multiple of 16 bytes");
    if constexpr (NT) w[0] = __builtin_nontemporal_load((const hf_u32 *)p);
    else w[0] = *(const hf_u32 *)p;
  }
}
template <int V>
__device__ __forceinline__ void hf_unpack_f32(const hf_u32 (&w)[V], float (&r)[V]) {
#pragma unroll
  for (int k = 0; k < V; ++k) r[k] = __uint_as_float(w[k]);
}
template <int V>
__device__ __forceinline__ void hf_unpack_i32(const hf_u32 (&w)[V], int (&r)[V]) {
#pragma unroll
  for (int k = 0; k < V; ++k) r[k] = (int)w[k];
}
// 16-bit floats: bf16 (F16=false) or f16 (F16=true); V >= 2
template <int V, bool F16>
__device__ __forceinline__ void hf_unpack_h(const hf_u32 (&w)[V / 2], float (&r)[V]) {
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const hf_u32 x = w[k / 2];
    if constexpr (F16) r[k] = (float)__builtin_bit_cast(_Float16, (hf_u16)((k & 1) ? (x >> 16) : (x & 0xFFFFu)));
    else r[k] = __uint_as_float((k & 1) ? (x & 0xFFFF0000u) : (x << 16));
  }
}
// 8-bit integers, sign- or zero-extended; V >= 4
template <int V, bool SIGNED>
__device__ __forceinline__ void hf_unpack_b(const hf_u32 (&w)[V / 4], int (&r)[V]) {
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const hf_u32 b = (w[k / 4] >> (8 * (k & 3))) & 0xFFu;
    r[k] = SIGNED ? (int)(signed char)b : (int)b;
  }
}
// No v_dot2c_f32_bf16 here: on gfx950 an ordinary VALU instruction that
// reads its result within two instructions has been measured to get the
// register's old value, and the compiler inserts no wait for it.  A chain of
// v_dot2c accumulating into one register was unaffected.
// Keeps the machine scheduler from sinking the loads of a fetch phase below
// the compute that follows it (it otherwise trades memory-level parallelism
// for register pressure).
#define HF_LOADS_ISSUED() __builtin_amdgcn_sched_barrier(0)

__device__ __forceinline__ float hf_f16_bits(hf_u32 h) { return (float)__builtin_bit_cast(_Float16, (hf_u16)h); }

// ------------------------------------------------------------ stores
template <typename T>
__device__ __forceinline__ void hf_vst(T *p, T v) {
#if HF_NT_STORES
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}
template <int V>
__device__ __forceinline__ void hf_st_f32(void *base, int off, const float (&r)[V]) {
  float *p = (float *)base + off;
  if constexpr (V % 4 == 0) {
#pragma unroll
    for (int k = 0; k < V / 4; ++k)
      hf_vst((hf_u32x4 *)p + k, hf_u32x4{__float_as_uint(r[4 * k]), __float_as_uint(r[4 * k + 1]),
                                         __float_as_uint(r[4 * k + 2]), __float_as_uint(r[4 * k + 3])});
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
        hf_vst((hf_u32x4 *)p + k, hf_u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]});
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
    for (int k = 0; k < V / 4; ++k) {
      // low bytes of four values with three v_perm_b32: {r0, r1} and {r2, r3}
      // into the low halves, then both halves into one word
      const hf_u32 lo = __builtin_amdgcn_perm((hf_u32)r[4 * k + 1], (hf_u32)r[4 * k], 0x0C0C0400u);
      const hf_u32 hi = __builtin_amdgcn_perm((hf_u32)r[4 * k + 3], (hf_u32)r[4 * k + 2], 0x0C0C0400u);
      w[k] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
    if constexpr (V % 16 == 0) {
#pragma unroll
      for (int k = 0; k < V / 16; ++k)
        hf_vst((hf_u32x4 *)p + k, hf_u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]});
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
// 4-bit elements (si4/ui4), two per byte in linear order with the even index
// in the low half: element k of a run that starts at an even index sits at
// bits 4k of the run's little-endian words.
template <int V, bool SIGNED>
__device__ __forceinline__ void hf_unpack_n(const hf_u32 (&w)[(V + 7) / 8], int (&r)[V]) {
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const hf_u32 n = (w[k / 8] >> (4 * (k & 7))) & 0xFu;
    r[k] = SIGNED ? (int)(n ^ 8u) - 8 : (int)n;
  }
}
// One 4-bit element from its byte: the high half when its index is odd.
template <bool SIGNED>
__device__ __forceinline__ int hf_nibble(hf_u32 byte, int odd) {
  const hf_u32 n = (odd ? byte >> 4 : byte) & 0xFu;
  return SIGNED ? (int)(n ^ 8u) - 8 : (int)n;
}
// Store of V (even) 4-bit values at element offset off (even): whole bytes
// only, so lanes never share a byte.
template <int V>
__device__ __forceinline__ void hf_st_n(void *base, int off, const int (&r)[V]) {
  static_assert(V % 2 == 0, "4-bit stores move whole bytes");
  unsigned char *p = (unsigned char *)base + (off >> 1);
  if constexpr (V >= 8) {
    hf_u32 w[V / 8];
#pragma unroll
    for (int k = 0; k < V / 8; ++k) {
      hf_u32 x = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) x |= ((hf_u32)r[8 * k + j] & 0xFu) << (4 * j);
      w[k] = x;
    }
    if constexpr (V % 32 == 0) {
#pragma unroll
      for (int k = 0; k < V / 32; ++k)
        hf_vst((hf_u32x4 *)p + k, hf_u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]});
    } else if constexpr (V == 16) {
      *(uint2 *)p = make_uint2(w[0], w[1]);
    } else {
      *(hf_u32 *)p = w[0];
    }
  } else {
#pragma unroll
    for (int k = 0; k < V / 2; ++k)
      p[k] = (unsigned char)(((hf_u32)r[2 * k] & 0xFu) | (((hf_u32)r[2 * k + 1] & 0xFu) << 4));
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

// The same result for V values without a division: rcp is 1/scale rounded
// to the nearest double (computed on the host).  q = fl64(y * rcp) is within
// 2^-52 (relative) of y/scale, while y/scale -- a quotient of two f32 values
// -- is never closer than 2^-49 (relative) to the midpoint between two
// adjacent f32 values: its distance to a 25-bit midpoint m is
// |y - scale*m| / scale >= 2^(E-24)/2^24 for m in [2^E, 2^(E+1)).  So
// (float)q is exactly fl32(y/scale), the IEEE quotient, for all finite
// inputs, with no branch and four full-rate instructions.
//
// Rounding and conversion use one add: for |t| < 2^22, a = t + 1.5*2^23 lies
// in [2^23, 2^24) where floats are the integers, so the add rounds t to the
// nearest integer with ties to even (1.5*2^23 is even) and a is exactly
// 1.5*2^23 + rne(t); its low mantissa bits hold rne(t) in two's complement.
// The clamp is applied to a (bounds shifted by the same constant); |t| >=
// 2^22 lies far outside any storage range and clamps the same way.  A zero
// point is added after rounding, as an integer.  With LOW_BYTE, q keeps only
// a correct low byte (all an 8-bit store needs): for a zero point of 0 that
// is the low byte of a's bits, since 1.5*2^23's low byte is 0.
template <int V, bool LOW_BYTE = false>
__device__ __forceinline__ void hf_quantize_v(const float (&y)[V], const double (&rcp)[V], const int (&zp)[V],
                                              int smin, int smax, int (&q)[V]) {
  constexpr float M = 12582912.0f;  // 1.5 * 2^23
#pragma unroll
  for (int l = 0; l < V; ++l) {
    const float t = (float)((double)y[l] * rcp[l]);
    const float a = t + M;
    const float c = __builtin_fminf(__builtin_fmaxf(a, M + (float)(smin - zp[l])), M + (float)(smax - zp[l]));
    if constexpr (LOW_BYTE) q[l] = (int)__float_as_uint(c) + zp[l];
    else q[l] = (int)(__float_as_uint(c) - __float_as_uint(M)) + zp[l];
  }
}
