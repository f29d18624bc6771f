// Decay preparation: the lower-bounded gate and the chunk-local cumulative
// log-decay.
//
// Kimi K3 technical report summary, "Key claims" (section 2.1.1, Fig. 3) and
// "Method" (section 2.1): g = gmin * Sigmoid(exp(A) * z), gmin = -5, A a
// learnable scalar per head.  The chunkwise form rescales by exponentials of
// the running sum of g inside a chunk; this kernel produces that sum.  For
// the unbounded-decay comparison, the same page's predecessor gate (Kimi
// Linear's negative Softplus, no lower bound) as g = -Softplus(exp(A) * z).
//
// Layout [B, T, H, dk] with channels contiguous: one thread per
// (b, chunk, h, channel) walks the chunk's rows in order, so every load and
// store instruction of a wave touches consecutive channels (coalesced) and
// the scan needs no cross-lane traffic.  Memory-bound; all arithmetic fp32.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// kGate: 0 = g is an input, 1 = gmin * Sigmoid(exp(A) z), 2 = -Softplus(exp(A) z)
template <typename T, int kGate>
__global__ __launch_bounds__(256) void prepare_decay_kernel(const T* __restrict__ z, const float* __restrict__ A,
                                                            float gmin, T* __restrict__ g,
                                                            float* __restrict__ gcum, int T_len, int H, int dk,
                                                            int chunk, int nchunks, int blocks_per_bc) {
  const int bc = blockIdx.x / blocks_per_bc;
  const int hc = (blockIdx.x % blocks_per_bc) * 256 + threadIdx.x;
  const int HD = H * dk;
  if (hc >= HD) return;
  const int b = bc / nchunks, ch = bc % nchunks;
  const int t0 = ch * chunk;
  const int t1 = min(t0 + chunk, T_len);
  size_t idx = ((size_t)b * T_len + t0) * (size_t)HD + hc;
  float ea = 0.f;
  if (kGate) ea = expf(A[hc / dk]);
  float acc = 0.f;
  for (int t = t0; t < t1; ++t, idx += HD) {
    float gv;
    if (kGate) {
      const float x = ea * to_f32(z[idx]);
      // Softplus(x) = max(x, 0) + log(1 + e^{-|x|}), no overflow for large |x|
      const float gf = kGate == 1 ? gmin / (1.0f + expf(-x)) : -(fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))));
      const T gt = from_f32<T>(gf);
      if (g) g[idx] = gt;
      gv = to_f32(gt);
    } else {
      gv = to_f32(g[idx]);
    }
    acc += gv;
    if (gcum) gcum[idx] = acc;
  }
}

template <typename T>
static hipError_t go_decay(const void* z, const float* A, float gmin, void* g, float* gcum, int B, int T_len,
                           int H, int dk, int chunk, int softplus, hipStream_t st) {
  const int nchunks = (T_len + chunk - 1) / chunk;
  const int bpb = (H * dk + 255) / 256;
  const size_t nblocks = (size_t)B * nchunks * bpb;
  if (nblocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
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

}  // namespace kda
