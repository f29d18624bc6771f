// Device-side building blocks for the gfx950 KDA kernels: element types,
// MFMA operand fragments, tile products and small reductions.
//
// Tile convention (wave64, 16x16 output tiles, fp32 accumulate):
//   * accumulator of a 16x16 tile: lane l holds rows 4*(l/16)+r (r = 0..3)
//     of column l%16  (f32x4).
//   * an operand "slab" covers 32 consecutive reduction indices.  Lane group
//     g = l/16 holds the 8 reduction indices
//         {4g, 4g+1, 4g+2, 4g+3, 16+4g, 16+4g+1, 16+4g+2, 16+4g+3}
//     of row l%16 (left operand) or column l%16 (right operand).  Both
//     operands use the same order, so the product is the plain sum over the
//     slab whatever order the hardware assigns inside one lane group.
//   * with this order two stacked accumulator tiles (rows 0..15 and 16..31)
//     are directly a right operand slab (or, read as a transpose, a left
//     operand slab): products chain without a trip through LDS.
//   * a "half slab" covers 16 reduction indices {4g..4g+3}.
//
// Element types: bf16 and fp16 slabs use v_mfma_f32_16x16x32_{bf16,f16},
// half slabs v_mfma_f32_16x16x16_{bf16,f16}; fp32 slabs use eight
// v_mfma_f32_16x16x4_f32.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---- scalar conversion -------------------------------------------------
template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return (T)x; }   // RNE

// ---- 4- and 8-element vectors of an element type -------------------------
template <typename T> struct Vec4;
template <> struct Vec4<float> { typedef f32x4 type; };
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<f16> { typedef f16x4 type; };
template <typename T> using V4 = typename Vec4<T>::type;

template <typename T> __device__ __forceinline__ V4<T> load4(const T* p) {
  return *reinterpret_cast<const V4<T>*>(p);
}
template <typename T> __device__ __forceinline__ void store4(T* p, V4<T> v) {
  *reinterpret_cast<V4<T>*>(p) = v;
}
template <typename V> __device__ __forceinline__ f32x4 widen4(V v) {
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <typename T> __device__ __forceinline__ V4<T> narrow4(f32x4 v) {
  return V4<T>{(T)v[0], (T)v[1], (T)v[2], (T)v[3]};
}

// ---- operand fragments ---------------------------------------------------
template <typename T> struct Slab;   // 8 reduction indices per lane
template <> struct Slab<bf16> { bf16x8 v; };
template <> struct Slab<f16> { f16x8 v; };
template <> struct Slab<float> { f32x4 lo, hi; };
template <typename T> struct Half { V4<T> v; };   // 4 reduction indices per lane

// Slab from two groups of 4 (indices 4g..4g+3 and 16+4g..16+4g+3).
template <typename T> __device__ __forceinline__ Slab<T> slab_of(V4<T> lo, V4<T> hi) {
  Slab<T> s;
  s.v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return s;
}
template <> __device__ __forceinline__ Slab<float> slab_of<float>(f32x4 lo, f32x4 hi) { return Slab<float>{lo, hi}; }
template <typename T> __device__ __forceinline__ Slab<T> make_slab(f32x4 lo, f32x4 hi) {
  return slab_of<T>(narrow4<T>(lo), narrow4<T>(hi));
}
// Split x = hi + lo with hi = round(x) and lo = round(x - hi) (both of type T).
template <typename T> __device__ __forceinline__ void make_slab_split(f32x4 lo4, f32x4 hi4, Slab<T>& h, Slab<T>& l) {
  const V4<T> a = narrow4<T>(lo4), b = narrow4<T>(hi4);
  h = slab_of<T>(a, b);
  l = make_slab<T>(lo4 - widen4(a), hi4 - widen4(b));
}

// Slab of a k-contiguous row: p points at element 0 of the 32-wide slab.
template <typename T> __device__ __forceinline__ Slab<T> load_slab(const T* p) {
  const int g = lane_id() >> 4;
  return slab_of<T>(load4(p + 4 * g), load4(p + 16 + 4 * g));
}
template <typename T> __device__ __forceinline__ Half<T> load_half(const T* p) {
  const int g = lane_id() >> 4;
  return Half<T>{load4(p + 4 * g)};
}

// acc += A(16 x 32 slab) * B(32 slab x 16)
__device__ __forceinline__ f32x4 mma(const Slab<bf16>& a, const Slab<bf16>& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Slab<f16>& a, const Slab<f16>& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Slab<float>& a, const Slab<float>& b, f32x4 acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[i], b.lo[i], acc, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[i], b.hi[i], acc, 0, 0, 0);
  return acc;
}
// acc += A(16 x 16 half) * B(16 half x 16)
__device__ __forceinline__ f32x4 mma(const Half<bf16>& a, const Half<bf16>& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a.v), __builtin_bit_cast(i16x4, b.v),
                                                  acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Half<f16>& a, const Half<f16>& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Half<float>& a, const Half<float>& b, f32x4 acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// exp(x) for x given in log2 units (x = ln-value * log2(e)); v_exp_f32.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ f32x4 exp2v(f32x4 x) {
  return f32x4{exp2_fast(x[0]), exp2_fast(x[1]), exp2_fast(x[2]), exp2_fast(x[3])};
}
constexpr float kLog2e = 1.4426950408889634f;
// Sigmoid(x) = 1 / (1 + e^{-x}) with v_exp_f32 and v_rcp_f32 (about 2 ulp;
// 0 and 1 at the far ends).
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + exp2_fast(-x * kLog2e));
}
// The layer's steps: lower bound of the decay gate g = gmin Sigmoid(exp(A) z)
// and the epsilon of the q/k row normalisation x / sqrt(sum x^2 + eps).
constexpr float kGateMin = -5.0f;
constexpr float kNormEps = 1e-6f;

__device__ __forceinline__ float absmax4(f32x4 v) {
  return fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
}
// max(m, |v[0]|, |v[1]|, |v[2]|, |v[3]|) for m >= 0, as two v_max3_f32 with
// abs modifiers on the new values.  For finite values the same as fmaxf over
// fabsf; it skips the canonicalising moves that fmaxf's NaN rules add to
// each operand (a NaN operand is dropped, as fmaxf drops it).
__device__ __forceinline__ float absmax_acc(float m, f32x4 v) {
  float r, s;
  asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(r) : "v"(v[0]), "v"(v[1]), "v"(m));
  asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(s) : "v"(v[2]), "v"(v[3]), "v"(r));
  return s;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// x from lane (l ^ ...) as selected by DPP control `ctrl` within the rows
// enabled by `row_mask`; lanes outside them (or with no source) keep x.
template <int ctrl, int row_mask = 0xf>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                                               ctrl, row_mask, 0xf, false));
}

// Maximum over the wave's 64 lanes with DPP moves (no LDS round trips),
// returned wave-uniform: pairs, quads, half rows and rows of 16 by lane
// permutations, then rows 0-1 and 2-3 by broadcasting lane 15 of a row into
// the next, then row 3 gets lane 31; lane 63 holds the result.
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));        // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));        // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));       // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));       // row_mirror
  x = fmaxf(x, dpp_f<0x142, 0xA>(x));  // row_bcast:15 into rows 1 and 3
  x = fmaxf(x, dpp_f<0x143, 0xC>(x));  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Power-of-two factor s with s * mx in [2^14, 2^15) (mx > 0 finite), so
// values scaled by s fit the fp16 range with their full precision; 1 for
// mx == 0 or non-finite mx.  Multiplying and dividing by s is exact.
__device__ __forceinline__ float fp16_range_scale(float mx) {
  const unsigned bits = __float_as_uint(mx);
  const int ex = (int)((bits >> 23) & 0xffu);
  if (mx <= 0.f || ex == 0xff) return 1.f;
  int k = 14 - (ex - 127);
  k = k < -100 ? -100 : (k > 100 ? 100 : k);
  return ldexpf(1.f, k);
}
// The same factor and its exact reciprocal.
__device__ __forceinline__ void fp16_range_scale2(float mx, float& s, float& inv) {
  const unsigned bits = __float_as_uint(mx);
  const int ex = (int)((bits >> 23) & 0xffu);
  int k = 14 - (ex - 127);
  k = k < -100 ? -100 : (k > 100 ? 100 : k);
  if (mx <= 0.f || ex == 0xff) k = 0;
  s = ldexpf(1.f, k);
  inv = ldexpf(1.f, -k);
}

}  // namespace kda
