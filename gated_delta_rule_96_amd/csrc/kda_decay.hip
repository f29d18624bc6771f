// Decay preparation: the lower-bounded gate and the chunk-local cumulative
// log-decay; and the opt-in range check of a given log-decay.
//
// Kimi K3 technical report summary, "Key claims" (section 2.1.1, Fig. 3) and
// "Method" (section 2.1): g = gmin * Sigmoid(exp(A) * z), gmin = -5, A a
// learnable scalar per head.  The chunkwise form rescales by exponentials of
// the running sum of g inside a chunk; this kernel produces that sum.  For
// the unbounded-decay comparison, the same page's predecessor gate (Kimi
// Linear's negative Softplus, no lower bound) as g = -Softplus(exp(A) * z).
//
// Layout [B, T, H, dk] with channels contiguous: one thread per
// (b, chunk, h, 8 consecutive channels) walks the chunk's rows in order,
// with one 16-byte load per row and sixteen rows in flight; a wave covers 512
// consecutive channels of a row (coalesced) and the scan needs no cross-lane
// traffic.  Memory-bound; all arithmetic fp32.
#include <stdlib.h>

#include <mutex>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kVE = 8;        // channels per thread
constexpr int kRowsU = 16;    // rows loaded together

// Eight consecutive elements of type T as fp32, and back (RNE).  Every
// element is read and written once: non-temporal accesses (streamed past
// the caches).
template <typename T> struct Eight;
template <> struct Eight<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float (&x)[kVE]) {
    const bf16x8 v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
#pragma unroll
    for (int i = 0; i < kVE; ++i) x[i] = (float)v[i];
  }
  static __device__ __forceinline__ void store(bf16* p, const float (&x)[kVE]) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < kVE; ++i) v[i] = (bf16)x[i];
    __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(p));
  }
};
template <> struct Eight<float> {
  static __device__ __forceinline__ void load(const float* p, float (&x)[kVE]) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float (&x)[kVE]) {
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4*>(p + 4));
  }
};

// kGate: 0 = g is an input, 1 = gmin * Sigmoid(exp(A) z), 2 = -Softplus(exp(A) z)
template <typename T, int kGate>
__global__ __launch_bounds__(256) void prepare_decay_kernel(const T* __restrict__ z, const float* __restrict__ A,
                                                            float gmin, T* __restrict__ g,
                                                            float* __restrict__ gcum, int T_len, int H, int dk,
                                                            int chunk, int nchunks, int blocks_per_bc) {
  const int bc = blockIdx.x / blocks_per_bc;
  const int hc = ((blockIdx.x % blocks_per_bc) * 256 + (int)threadIdx.x) * kVE;
  const int HD = H * dk;
  if (hc >= HD) return;
  const int b = bc / nchunks, ch = bc % nchunks;
  const int t0 = ch * chunk;
  const int t1 = min(t0 + chunk, T_len);
  const size_t base = (size_t)b * T_len * HD + hc;
  const float ea = kGate ? expf(A[hc / dk]) : 0.f;   // dk is a multiple of 8: one head per thread
  const float nea2 = -ea * 1.4426950408889634f;        // -exp(A) log2(e)
  float acc[kVE];
#pragma unroll
  for (int i = 0; i < kVE; ++i) acc[i] = 0.f;
  for (int t = t0; t < t1; t += kRowsU) {
    float x[kRowsU][kVE];
    // rows past the chunk's end re-read its last row (always in bounds)
    // and are not stored
#pragma unroll
    for (int u = 0; u < kRowsU; ++u) {
      const size_t idx = base + (size_t)min(t + u, t1 - 1) * HD;
      if (kGate) Eight<T>::load(z + idx, x[u]);
      else Eight<T>::load(g + idx, x[u]);
    }
#pragma unroll
    for (int u = 0; u < kRowsU; ++u) {
      const bool live = t + u < t1;
      const size_t idx = base + (size_t)(t + u) * HD;
      if (kGate) {
#pragma unroll
        for (int i = 0; i < kVE; ++i) {
          // bounded: gmin Sigmoid(a) = gmin / (1 + 2^{-a log2 e}) with v_exp_f32 and
          // v_rcp_f32 (a few ulp of fp32, far below the bf16 rounding of g);
          // Softplus(a) = max(a, 0) + log(1 + e^{-|a|}), no overflow for large |a|
          // (libm: near a = -inf it needs log1p's relative accuracy)
          float gf;
          if (kGate == 1) {
            gf = gmin * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(nea2 * x[u][i]));
          } else {
            const float a = ea * x[u][i];
            gf = -(fmaxf(a, 0.f) + log1pf(expf(-fabsf(a))));
          }
          x[u][i] = (float)from_f32<T>(gf);   // the rounded g is what the scan sums
        }
        if (g && live) Eight<T>::store(g + idx, x[u]);
      }
      if (gcum) {
#pragma unroll
        for (int i = 0; i < kVE; ++i) {
          acc[i] += x[u][i];
          x[u][i] = acc[i];
        }
        if (live) Eight<float>::store(gcum + idx, x[u]);
      }
    }
  }
}

template <typename T>
static hipError_t go_decay(const void* z, const float* A, float gmin, void* g, float* gcum, int B, int T_len,
                           int H, int dk, int chunk, int softplus, hipStream_t st) {
  const int nchunks = (T_len + chunk - 1) / chunk;
  const int bpb = (H * dk / kVE + 255) / 256;
  const size_t nblocks = (size_t)B * nchunks * bpb;
  if (nblocks > 0x7fffffffu || (H * dk) % kVE != 0) return hipErrorInvalidConfiguration;
  if (z && softplus)
    hipLaunchKernelGGL((prepare_decay_kernel<T, 2>), dim3((unsigned)nblocks), dim3(256), 0, st, (const T*)z,
                       A, gmin, (T*)g, gcum, T_len, H, dk, chunk, nchunks, bpb);
  else if (z)
    hipLaunchKernelGGL((prepare_decay_kernel<T, 1>), dim3((unsigned)nblocks), dim3(256), 0, st, (const T*)z,
                       A, gmin, (T*)g, gcum, T_len, H, dk, chunk, nchunks, bpb);
  else
    hipLaunchKernelGGL((prepare_decay_kernel<T, 0>), dim3((unsigned)nblocks), dim3(256), 0, st,
                       (const T*)nullptr, A, gmin, (T*)g, gcum, T_len, H, dk, chunk, nchunks, bpb);
  return hipGetLastError();
}

hipError_t launch_prepare_decay(int is_bf16, const void* z, const float* A, float gmin, void* g, float* gcum,
                                int B, int T_len, int H, int dk, int chunk, int softplus, hipStream_t st) {
  if (is_bf16) return go_decay<bf16>(z, A, gmin, g, gcum, B, T_len, H, dk, chunk, softplus, st);
  return go_decay<float>(z, A, gmin, g, gcum, B, T_len, H, dk, chunk, softplus, st);
}

// ---------------------------------------------------------------------------
// Range check of a log-decay input (the ABI's opt-in validation).
//   kBounded: every g in [gmin, 0] (the floor the bf16 rescaling relies on,
//             "Key claims" section 2.1.1); otherwise g <= 0 and finite.
//   gcum input (kCum): the per-row decay it encodes, the difference of
//             consecutive cumulative sums inside a chunk (the first row's
//             own value at a chunk start), in the same range up to the
//             rounding of the fp32 sums.
// A violation (NaN included) sets the flag word.
// ---------------------------------------------------------------------------
static __device__ unsigned int validate_flag;

template <typename T, bool kCum>
__global__ __launch_bounds__(256) void validate_decay_kernel(const T* __restrict__ g, const float* __restrict__ gcum,
                                                             int bounded, float gmin, int T_len, int HD,
                                                             int chunk, int nchunks, int blocks_per_bc,
                                                             unsigned int* __restrict__ flag) {
  const int bc = blockIdx.x / blocks_per_bc;
  const int hc = ((blockIdx.x % blocks_per_bc) * 256 + (int)threadIdx.x) * kVE;
  if (hc >= HD) return;
  const int b = bc / nchunks, ch = bc % nchunks;
  const int t0 = ch * chunk;
  const int t1 = min(t0 + chunk, T_len);
  const size_t base = (size_t)b * T_len * HD + hc;
  const float lo = bounded ? gmin : -INFINITY;
  bool bad = false;
  float prev[kVE];
#pragma unroll
  for (int i = 0; i < kVE; ++i) prev[i] = 0.f;
  for (int t = t0; t < t1; ++t) {
    float x[kVE];
    const size_t idx = base + (size_t)t * HD;
    if (kCum) Eight<float>::load(gcum + idx, x);
    else Eight<T>::load(g + idx, x);
#pragma unroll
    for (int i = 0; i < kVE; ++i) {
      float d = x[i], tol = 0.f;
      if (kCum) {
        d = x[i] - prev[i];
        tol = 1e-6f + (fabsf(x[i]) + fabsf(prev[i])) * 0x1p-20f;
        prev[i] = x[i];
      }
      // written so that a NaN fails
      bad = bad || !(d >= lo - tol && d <= tol && fabsf(x[i]) <= 3.0e38f);
    }
  }
  if (bad) atomicOr(flag, 1u);
}

__global__ void clear_flag_kernel(unsigned int* flag) { *flag = 0u; }

namespace {
void* g_flag_ptr[64];
std::mutex g_validate_mu;
}  // namespace

bool validate_requested() {
  const char* s = getenv("KDA_VALIDATE");
  return s && s[0] == '1' && s[1] == '\0';
}

template <typename T>
static hipError_t go_validate(const void* g, const float* gcum, int bounded, float gmin, int B, int T_len, int HD,
                              int chunk, hipStream_t st, unsigned int* flag) {
  const int nchunks = (T_len + chunk - 1) / chunk;
  const int bpb = (HD / kVE + 255) / 256;
  const size_t nblocks = (size_t)B * nchunks * bpb;
  if (nblocks > 0x7fffffffu || HD % kVE != 0) return hipErrorInvalidConfiguration;
  if (gcum)
    hipLaunchKernelGGL((validate_decay_kernel<T, true>), dim3((unsigned)nblocks), dim3(256), 0, st, (const T*)g,
                       gcum, bounded, gmin, T_len, HD, chunk, nchunks, bpb, flag);
  else
    hipLaunchKernelGGL((validate_decay_kernel<T, false>), dim3((unsigned)nblocks), dim3(256), 0, st, (const T*)g,
                       gcum, bounded, gmin, T_len, HD, chunk, nchunks, bpb, flag);
  return hipGetLastError();
}

hipError_t validate_decay(int is_bf16, const void* g, const float* gcum, int bounded, float gmin, int B, int T_len,
                          int HD, int chunk, hipStream_t st, int* in_range) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_validate_mu);
  if (!g_flag_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(validate_flag));
    if (e != hipSuccess) return e;
    g_flag_ptr[dev] = p;
  }
  unsigned int* flag = static_cast<unsigned int*>(g_flag_ptr[dev]);
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, st, flag);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = is_bf16 ? go_validate<bf16>(g, gcum, bounded, gmin, B, T_len, HD, chunk, st, flag)
              : go_validate<float>(g, gcum, bounded, gmin, B, T_len, HD, chunk, st, flag);
  if (e != hipSuccess) return e;
  unsigned int h = 0;
  e = hipMemcpyAsync(&h, flag, sizeof(h), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  *in_range = h == 0u;
  return hipSuccess;
}

}  // namespace kda
