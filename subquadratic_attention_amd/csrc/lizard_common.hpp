// Device helpers shared by the Lizard attention kernels (gfx950 only).
//
// MFMA operand convention used everywhere in this library.  A 16x16 output
// tile C[m][n] = sum_k A[m][k] * B[n][k] is computed by one wavefront (64
// lanes).  Lane l works on row m = l % 16 of A and row n = l % 16 of B, and
// lane group g = l / 16 owns the contiguous quarter [g*K/4, (g+1)*K/4) of the
// contraction index k.  Because the contraction is a sum, any assignment of
// k to (lane group, step) works as long as A and B use the same one; this
// one keeps every lane's operand data contiguous (vector loads).  The output
// lands as C[4*g + r][l % 16] in accumulator register r (r = 0..3), which is
// the gfx950 layout of v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x4_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lizard {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// float -> bf16 conversion rounds to nearest even (gfx950 v_cvt_pk_bf16_f32).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// One token's log-gate in log2 units for the prefix sums.  Gates below
// 2^-100 are taken as 2^-100: any product through such a gate is below 1e-30
// and indistinguishable from a full reset, while the prefix stays small
// enough that differences of prefixes keep float precision.
constexpr float kMinLog2Gate = -100.0f;
__device__ __forceinline__ float log2_gate(float log_g) { return fmaxf(log_g * 1.4426950408889634f, kMinLog2Gate); }

// exp of a natural-log exponent via the hardware base-2 exponential.
__device__ __forceinline__ float exp_e(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float exp_2(float x) { return __builtin_amdgcn_exp2f(x); }

// The gate from its logit x (the gate projection's output): log sigmoid(x)
// = min(x, 0) - ln(1 + e^{-|x|}) in natural-log units, from the hardware
// base-2 exponential and logarithm (no overflow for either sign; +inf gives
// 0, a gate of one).  Its derivative is sigmoid(-x) = 1 / (1 + e^x).
__device__ __forceinline__ float log_sigmoid(float x) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
  return fminf(x, 0.f) - kLn2 * __builtin_amdgcn_logf(1.f + e);
}
__device__ __forceinline__ float sigmoid_neg(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * kLog2e));
}

// Per element type: elements per lane per MFMA step (KPL), the contraction
// length one MFMA covers (KSTEP = 4 * KPL), the fragment type and the op.
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 32;
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag load(const bf16* p) { return *reinterpret_cast<const frag*>(p); }
  static __device__ __forceinline__ frag zero() {
    frag z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = static_cast<bf16>(0.0f);
    return z;
  }
  // Build a fragment from 8 float values (one rounding each).
  static __device__ __forceinline__ frag pack(const float* x) {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = static_cast<bf16>(x[i]);
    return f;
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 4;
  typedef float frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ frag zero() { return 0.0f; }
  static __device__ __forceinline__ frag pack(const float* x) { return x[0]; }
};

// C += A * B^T over a contraction of length K, with A's row m and B's row n
// each given as a pointer to the start of that lane's k-quarter.
template <typename T, int K>
__device__ __forceinline__ f32x4 mma_rows(f32x4 c, const T* a_q, const T* b_q) {
  typedef Mfma<T> M;
  constexpr int STEPS = K / M::KSTEP;
#pragma unroll
  for (int e = 0; e < STEPS; ++e) c = M::mma(M::load(a_q + e * M::KPL), M::load(b_q + e * M::KPL), c);
  return c;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Max / sum across the 16 lanes of a lane group (lanes with equal l / 16).
__device__ __forceinline__ float group16_max(float x) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float group16_sum(float x) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// Reductions across the four 16-lane groups of a wavefront (lanes l, l^16,
// l^32, l^48).  (The gfx950 permlane16/32 swap builtins would do this on the
// VALU, but this compiler folds their two outputs into one, so the portable
// lane shuffle is used.)
__device__ __forceinline__ float xgroup_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float xgroup_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}

// Pack n float values (n = 4, 8, 16) into consecutive elements of type T and
// store them with 8/16-byte LDS or global writes.
template <typename T, int N> __device__ __forceinline__ void store_pack(T* dst, const float* v);
template <> __device__ __forceinline__ void store_pack<bf16, 4>(bf16* dst, const float* v) {
  bf16x4 p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = static_cast<bf16>(v[i]);
  *reinterpret_cast<bf16x4*>(dst) = p;
}
template <> __device__ __forceinline__ void store_pack<bf16, 8>(bf16* dst, const float* v) {
  bf16x8 p;
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = static_cast<bf16>(v[i]);
  *reinterpret_cast<bf16x8*>(dst) = p;
}
template <> __device__ __forceinline__ void store_pack<bf16, 16>(bf16* dst, const float* v) {
  store_pack<bf16, 8>(dst, v);
  store_pack<bf16, 8>(dst + 8, v + 8);
}
template <> __device__ __forceinline__ void store_pack<float, 4>(float* dst, const float* v) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
}
template <> __device__ __forceinline__ void store_pack<float, 8>(float* dst, const float* v) {
  store_pack<float, 4>(dst, v);
  store_pack<float, 4>(dst + 4, v + 4);
}
template <> __device__ __forceinline__ void store_pack<float, 16>(float* dst, const float* v) {
  store_pack<float, 8>(dst, v);
  store_pack<float, 8>(dst + 8, v + 8);
}

// Load n = 4 consecutive elements of type T as float (one 8/16-byte load).
template <typename T, int N> __device__ __forceinline__ void load_pack(const T* src, float* v);
template <> __device__ __forceinline__ void load_pack<bf16, 4>(const bf16* src, float* v) {
  const bf16x4 p = *reinterpret_cast<const bf16x4*>(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = static_cast<float>(p[i]);
}
template <> __device__ __forceinline__ void load_pack<float, 4>(const float* src, float* v) {
  const f32x4 p = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = p[i];
}

// The elements of a raw 16-byte vector of T, as float.
template <typename T> __device__ __forceinline__ void unpack16(uint4 raw, float* v);
template <> __device__ __forceinline__ void unpack16<bf16>(uint4 raw, float* v) {
  const bf16x8 p = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = static_cast<float>(p[i]);
}
template <> __device__ __forceinline__ void unpack16<float>(uint4 raw, float* v) {
  v[0] = __builtin_bit_cast(float, raw.x);
  v[1] = __builtin_bit_cast(float, raw.y);
  v[2] = __builtin_bit_cast(float, raw.z);
  v[3] = __builtin_bit_cast(float, raw.w);
}

// Order LDS traffic of one wavefront: writes before the fence are visible
// to reads after it from any lane of the same wavefront.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 16-byte global load / store of raw bits.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

}  // namespace lizard
