// Decode step: one new token per (batch, head) against the fp32 state.
//
// Recurrence (Kimi K3 technical report summary, "Key claims"/"Method",
// section 2.1; fixed-size state instead of a KV cache per "How a Frontier
// Model Gets Built...", "Technical Details"):
//     S' = Diag(exp(g)) S ;  u = beta (v - S'^T k) ;  S_new = S' + k u^T
//     o  = scale * S_new^T q = scale * (S'^T q + u (k . q))
// One pass over the state: every thread keeps its share of S' in
// registers, so the 4*dk*dv bytes of state are read once and written once.
//
// Work-group per (b, h), kDecThreads threads.  Thread t owns value columns
// 4*(t % (DV/4)) .. +3 and key rows  t/(DV/4) + RG*i, i = 0..DK/RG-1 with
// RG = kDecThreads/(DV/4) row groups: each wave reads whole 512-byte
// (DV = 128) state rows, so loads and stores are fully coalesced 16-byte
// accesses.  1024 threads keep 4 rows (16 values) of state per thread and
// two work-groups per CU resident, so the 8192 (b, h) of a B=256, H=32
// batch run in 16 full rounds (256 threads: 5 per CU, 6.4 rounds, and
// 3.6% slower).
//
// Layer variant (kLay): the layer's steps either side of the recurrence,
// selected per call, as in the prefill's layer variant:
//   - the decay input is z: g = gmin Sigmoid(exp(A[h]) z) in fp32;
//   - kDecNormQK: q and k divided by sqrt(sum of squares + 1e-6) in fp32
//     and rounded to the input type (the recurrence's input precision, as
//     in the prefill);
//   - og != nullptr: o <- Sigmoid(og) o, og [B,H,dv] of the input type.
// The norms are reduced by every wave from the staged rows (no extra
// barrier); all of it is a few hundred bytes per (b, h) against the 128 KiB
// of state, so the step stays bound by the state's HBM traffic.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kDecThreads = 1024;
constexpr int kDecNormQK = 2;   // the layer flag of the q/k row normalisation

// Round x to T's precision and back (identity for fp32).
template <typename T> __device__ __forceinline__ float round_to(float x) { return to_f32(from_f32<T>(x)); }

template <typename T, int DK, int DV, bool kLay>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          const T* __restrict__ v, const T* __restrict__ g,
                                                          const T* __restrict__ beta, float scale,
                                                          float* __restrict__ state, float* __restrict__ o,
                                                          const float* __restrict__ A, const T* __restrict__ og,
                                                          int flags, int H) {
  constexpr int CG = DV / 4;     // float4 column groups
  constexpr int RG = kDecThreads / CG;   // row groups
  constexpr int RPT = DK / RG;   // rows per thread
  static_assert(RPT >= 1 && DK % RG == 0, "shape");

  __shared__ float s_k[DK], s_q[DK], s_dec[DK], s_v[DV], s_u[DV];
  __shared__ f32x4 s_p[RG][CG], s_s[RG][CG];
  __shared__ float s_kq;

  const int tid = threadIdx.x;
  const size_t bh = blockIdx.x;
  float* S = state + bh * (size_t)(DK * DV);
  const int cg = tid % CG, rg = tid / CG;

  // Issue the state loads first; they are the bulk of the traffic.
  f32x4 x[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    x[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(rg + RG * i) * DV) + cg);

  const bool norm = kLay && (flags & kDecNormQK) != 0;   // uniform
  if (tid < DK) {
    s_k[tid] = to_f32(k[bh * DK + tid]);
    s_q[tid] = to_f32(q[bh * DK + tid]);
    float gv = to_f32(g[bh * DK + tid]);
    if (kLay) gv = kGateMin * sigmoid_fast(expf(A[bh % H]) * gv);   // g holds z
    s_dec[tid] = expf(gv);
  }
  if (tid < DV) s_v[tid] = to_f32(v[bh * DV + tid]);
  __syncthreads();

  // Row norms of q and k, reduced by every wave from the staged rows.
  float rk = 1.f, rq = 1.f;
  if (norm) {
    float sk = 0.f, sq = 0.f;
    for (int c = tid & 63; c < DK; c += 64) {
      sk = fmaf(s_k[c], s_k[c], sk);
      sq = fmaf(s_q[c], s_q[c], sq);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      sk += __shfl_xor(sk, off);
      sq += __shfl_xor(sq, off);
    }
    rk = 1.0f / sqrtf(sk + kNormEps);
    rq = 1.0f / sqrtf(sq + kNormEps);
  }
  // k and q as the recurrence uses them
  auto kn = [&](int c) { return norm ? round_to<T>(s_k[c] * rk) : s_k[c]; };
  auto qn = [&](int c) { return norm ? round_to<T>(s_q[c] * rq) : s_q[c]; };

  if (tid < 64) {  // k . q by wave 0
    float a = 0.f;
    for (int c = tid; c < DK; c += 64) a += kn(c) * qn(c);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a += __shfl_xor(a, off);
    if (tid == 0) s_kq = a;
  }

  f32x4 p = zero4(), s = zero4();
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg + RG * i;
    x[i] *= s_dec[c];
    p += kn(c) * x[i];
    s += qn(c) * x[i];
  }
  s_p[rg][cg] = p;
  s_s[rg][cg] = s;
  __syncthreads();

  if (tid < DV) {
    const int c4 = tid >> 2, e = tid & 3;
    float P = 0.f, Sq = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      P += s_p[r][c4][e];
      Sq += s_s[r][c4][e];
    }
    const float u = to_f32(beta[bh]) * (s_v[tid] - P);
    s_u[tid] = u;
    float ov = scale * (Sq + u * s_kq);
    if (kLay && og) ov *= sigmoid_fast(to_f32(og[bh * DV + tid]));
    o[bh * DV + tid] = ov;
  }
  __syncthreads();

  const f32x4 u4 = *reinterpret_cast<const f32x4*>(&s_u[4 * cg]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg + RG * i;
    f32x4 y = x[i] + kn(c) * u4;
    __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(S + (size_t)c * DV) + cg);
  }
}

template <typename T, int DK, int DV>
static hipError_t go_decode(const void* q, const void* k, const void* v, const void* g, const void* beta,
                            float scale, float* state, float* o, int B, int H, const DecodeLayer* lay,
                            hipStream_t st) {
  const unsigned nbh = (unsigned)B * (unsigned)H;
  if (lay)
    hipLaunchKernelGGL((decode_step_kernel<T, DK, DV, true>), dim3(nbh), dim3(kDecThreads), 0, st, (const T*)q,
                       (const T*)k, (const T*)v, (const T*)g, (const T*)beta, scale, state, o, lay->A,
                       (const T*)lay->og, lay->flags, H);
  else
    hipLaunchKernelGGL((decode_step_kernel<T, DK, DV, false>), dim3(nbh), dim3(kDecThreads), 0, st, (const T*)q,
                       (const T*)k, (const T*)v, (const T*)g, (const T*)beta, scale, state, o, nullptr, nullptr, 0,
                       H);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_decode(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                  float scale, float* state, float* o, int B, int H, int dk, int dv,
                                  const DecodeLayer* lay, hipStream_t st) {
  if (dk == 128 && dv == 128) return go_decode<T, 128, 128>(q, k, v, g, beta, scale, state, o, B, H, lay, st);
  if (dk == 128 && dv == 64) return go_decode<T, 128, 64>(q, k, v, g, beta, scale, state, o, B, H, lay, st);
  if (dk == 64 && dv == 128) return go_decode<T, 64, 128>(q, k, v, g, beta, scale, state, o, B, H, lay, st);
  return go_decode<T, 64, 64>(q, k, v, g, beta, scale, state, o, B, H, lay, st);
}

hipError_t launch_decode_step(int is_bf16, const void* q, const void* k, const void* v, const void* g,
                              const void* beta, float scale, float* state, float* o, int B, int H, int dk,
                              int dv, hipStream_t st, const DecodeLayer* lay) {
  static_assert(kDecNormQK == kDecodeLayerNormQK, "flag");
  if (is_bf16) return dispatch_decode<bf16>(q, k, v, g, beta, scale, state, o, B, H, dk, dv, lay, st);
  return dispatch_decode<float>(q, k, v, g, beta, scale, state, o, B, H, dk, dv, lay, st);
}

}  // namespace kda
