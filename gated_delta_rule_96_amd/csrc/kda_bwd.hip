// Backward of the chunked KDA prefill on gfx950 (fp32 arithmetic, fp32 MFMA).
//
// Kimi K3 technical report summary ("Method", section 2.1: the chunkwise
// form of the delta rule with channel-wise decay).  Per chunk with state S
// entering, N = dL/dS leaving and dO = dL/dO, and with L = I + Diag(beta) G,
// Kb = e^Gamma * K, Qb = e^Gamma * Q, Kh = e^(gamma - Gamma) * K (gamma the
// chunk's total decay), R = V - Kb S, U = L^-1 Diag(beta) R, the reverse-mode
// chain rule gives
//
//   dU  = scale M^T dO + Kh N,    Z = L^-T dU,    dV = beta * Z
//   dS  = e^gamma * N + scale Qb^T dO - W^T dU     (W = L^-1 Diag(beta) Kb)
//   dA  = -strict_lower(Z U^T),   dG = beta * dA,  dM = scale lower(dO U^T)
//   dQb = scale dO S^T,  dKb = -(beta * Z) S^T,  dKh = U N^T
//   dbeta = rowsum(Z * R) + rowsum(dA * G)
//
// and the gradients reach q, k and Gamma through the decay factors; dg is
// the reverse cumulative sum of dGamma over the chunk plus dgamma.
//
// Three kernels after a forward pass that keeps the state entering every
// chunk:
//   bwd_prep_kernel   per (chunk, head): G, M, L^-1, W, Kh, P = scale M^T dO,
//                     C = scale Qb^T dO and the chunk's decay references,
//                     to a per-chunk record.
//   bwd_state_kernel  per (head, 16 columns of dv): the sequential pass from
//                     the last chunk back, N <- e^gamma N + C - W^T (P + Kh N),
//                     writing N and dU = P + Kh N for every chunk.
//   bwd_grad_kernel   per (chunk, head): everything else.
//
// Pairwise decays e^(Gamma_r - Gamma_s) (s <= r) are split at the start of r's
// 16-row block a, ref_a = Gamma at row 16a - 1: e^(Gamma_r - ref_a) <= 1 and
// e^(ref_a - Gamma_s) <= 1 for s before the block, <= e^80 inside it (the
// bounded gate keeps a 16-row block's decay above -80), so every factor is a
// finite fp32.  Gamma is accumulated in fp64; the record keeps the block
// references and gamma in fp64 and Gamma as fp32 offsets from its block's
// reference (|.| <= 80), so each exponent is rounded to fp32 once.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kCh = 64;        // chunk rows
constexpr int kP64 = kCh + 4;  // row stride of 64-wide LDS matrices

__device__ __forceinline__ f32x4 mfma4(f32x4 a, f32x4 b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
  return c;
}

// 16x16 tile products, k in [k0, k1) (multiples of 16).  Lane group g = l/16
// supplies reduction indices 16j + 4g + {0..3} of row (A) / column (B) l%16.
//   mm_nt: A(row, k) = A[row * as + k],  B(k, col) = Bt[col * bs + k]
//   mm_nn: A(row, k) = A[row * as + k],  B(k, col) = Bn[k * bs + col]
//   mm_tt: A(row, k) = At[k * as + row], B(k, col) = Bt[col * bs + k]
__device__ __forceinline__ f32x4 mm_nt(f32x4 acc, const float* A, int as, const float* Bt, int bs, int k0, int k1) {
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const float* a = A + r * as + 4 * g;
  const float* b = Bt + r * bs + 4 * g;

  for (int k = k0; k < k1; k += 16) acc = mfma4(*(const f32x4*)(a + k), *(const f32x4*)(b + k), acc);
  return acc;
}
__device__ __forceinline__ f32x4 mm_nn(f32x4 acc, const float* A, int as, const float* Bn, int bs, int k0, int k1) {
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const float* a = A + r * as + 4 * g;
  const float* b = Bn + (4 * g) * bs + r;

  for (int k = k0; k < k1; k += 16) {
    const float* bk = b + k * bs;
    acc = mfma4(*(const f32x4*)(a + k), f32x4{bk[0], bk[bs], bk[2 * bs], bk[3 * bs]}, acc);
  }
  return acc;
}
__device__ __forceinline__ f32x4 mm_tt(f32x4 acc, const float* At, int as, const float* Bt, int bs, int k0, int k1) {
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const float* a = At + (4 * g) * as + r;
  const float* b = Bt + r * bs + 4 * g;

  for (int k = k0; k < k1; k += 16) {
    const float* ak = a + k * as;
    acc = mfma4(f32x4{ak[0], ak[as], ak[2 * as], ak[3 * as]}, *(const f32x4*)(b + k), acc);
  }
  return acc;
}

// Accumulator tile -> matrix: row-major D[row * ds + col], transposed Dt[col * ds + row].
__device__ __forceinline__ void st_rm(float* D, int ds, f32x4 v) {
  const int l = lane_id(), c = l & 15, r0 = 4 * (l >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) D[(r0 + i) * ds + c] = v[i];
}
__device__ __forceinline__ void st_tr(float* Dt, int ds, f32x4 v) {
  const int l = lane_id();
  *(f32x4*)(Dt + (l & 15) * ds + 4 * (l >> 4)) = v;
}

// e^x with the rounding of x * log2(e) compensated (first order): without it
// |x| ~ 80 loses ~5e-6 of relative precision.
__device__ __forceinline__ float ex(float x) {
  constexpr float kL2eLo = 1.925963e-08f;   // log2(e) - fp32(log2(e))
  constexpr float kLn2 = 0.6931472f;
  const float t = x * kLog2e;
  const float e = fmaf(x, kLog2e, -t) + x * kL2eLo;
  return exp2_fast(t) * fmaf(e, kLn2, 1.f);
}

// Record of one (chunk, head), fp32 words.
template <int DK, int DV>
struct Rec {
  static constexpr size_t G = 0;                        // [64][64] raw Gram, strictly lower
  static constexpr size_t LINV = G + kCh * kCh;         // [64][64] (I + Diag(beta) G)^-1
  static constexpr size_t GLOC = LINV + kCh * kCh;      // [64][DK] Gamma - ref_(block)
  static constexpr size_t REF = GLOC + kCh * DK;        // [4][DK] fp64 ref_a (ref_0 = 0)
  static constexpr size_t GAM = REF + 8 * DK;           // [DK] fp64 gamma
  static constexpr size_t KH = GAM + 2 * DK;            // [64][DK] e^(gamma - Gamma) k
  static constexpr size_t WT = KH + kCh * DK;           // [DK][64] W transposed
  static constexpr size_t P = WT + DK * kCh;            // [64][DV] scale M^T dO
  static constexpr size_t C = P + kCh * DV;             // [DK][DV] scale Qb^T dO
  static constexpr size_t WORDS = C + DK * DV;
};

template <typename T>
__device__ __forceinline__ float ldf(const T* p, size_t i) { return to_f32(p[i]); }

// 8 (4) consecutive elements as fp32, one or two 16-byte loads (8-byte for 4 bf16)
__device__ __forceinline__ void ld8(const float* p, float* o) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[i] = a[i];
    o[4 + i] = b[i];
  }
}
__device__ __forceinline__ void ld8(const bf16* p, float* o) {
  const bf16x8 v = *(const bf16x8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
}
__device__ __forceinline__ f32x4 ld4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 ld4(const bf16* p) { return widen4(*(const bf16x4*)p); }
__device__ __forceinline__ void st8(float* p, const float* v) {
  *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
  *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
// Loads of rows that may lie past the end of the sequence: the caller
// points p at row 0 instead of such a row (always a valid address) and
// passes ok = false, and the values become zero.  The load itself is not
// inside a branch, so a run of them is issued together; behind a branch
// every load was followed by its own wait for memory.
template <typename T>
__device__ __forceinline__ void ld8z(const T* p, bool ok, float* o) {
  ld8(p, o);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = ok ? o[i] : 0.f;
}
template <typename T>
__device__ __forceinline__ f32x4 ld4z(const T* p, bool ok) {
  const f32x4 x = ld4(p);
  return f32x4{ok ? x[0] : 0.f, ok ? x[1] : 0.f, ok ? x[2] : 0.f, ok ? x[3] : 0.f};
}
template <typename T>
__device__ __forceinline__ float ldfz(const T* p, size_t i, bool ok) {
  const float x = ldf(p, i);
  return ok ? x : 0.f;
}

// ---------------------------------------------------------------------------
// Per-chunk preparation.
template <typename TIn, int DK, int DV>
struct PrepLds {
  static constexpr int PK = DK + 4, PV = DV + 4;
  static constexpr int M0 = 64 * PK > DK * kP64 ? 64 * PK : DK * kP64;
  static constexpr int M1 = M0 > DV * kP64 ? M0 : DV * kP64;
  static constexpr int RS = M1 > 2 * kCh * kP64 ? M1 : 2 * kCh * kP64;   // also holds two [64][68]
  static constexpr int R0 = 0, R1 = RS, R2 = 2 * RS, R3 = 3 * RS, RL = 4 * RS;
  static constexpr int REF = RL + kCh * kP64;   // [4][DK] fp64
  static constexpr int GAM = REF + 8 * DK;      // [DK] fp64
  static constexpr int BETA = GAM + 2 * DK;     // [64]
  static constexpr int WORDS = BETA + kCh;
};

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                       const TIn* __restrict__ g, const TIn* __restrict__ beta,
                                                       const float* __restrict__ dO, float scale, int T, int H,
                                                       int nch, float* __restrict__ rec) {
  using LD = PrepLds<TIn, DK, DV>;
  using RC = Rec<DK, DV>;
  constexpr int PK = LD::PK;
  constexpr int NT = DK / 16;   // column tiles of a [64][DK] matrix
  constexpr int NV = DV / 16;
  __shared__ __align__(16) float sm[LD::WORDS];
  const int tid = threadIdx.x, w = tid >> 6;
  const int n = blockIdx.x, bh = n / nch, c = n % nch;
  const int b = bh / H, h = bh % H;
  const int t0 = c * kCh, L = min(kCh, T - t0);
  float* out = rec + (size_t)n * RC::WORDS;
  auto row = [&](int r) { return ((size_t)b * T + t0 + r) * H + h; };   // token-major row index
  auto rowc = [&](int r) { return row(r < L ? r : 0); };   // row 0 stands in past the end

  float* sGl = sm + LD::R0;   // Gamma - ref [64][PK]
  double* sRef = reinterpret_cast<double*>(sm + LD::REF);
  double* sGam = reinterpret_cast<double*>(sm + LD::GAM);
  float* sBeta = sm + LD::BETA;
  // exponents from the fp64 references, rounded once
  auto dref = [&](int a, int bs, int cc) { return (float)(sRef[a * DK + cc] - sRef[bs * DK + cc]); };
  auto gam_minus = [&](int a, int cc) { return (float)(sGam[cc] - sRef[a * DK + cc]); };
  auto ref_plus = [&](int a, int cc, float gl) { return (float)(sRef[a * DK + cc] + (double)gl); };

  constexpr int V8 = DK / 8;
  // stage g, k and q with 16-byte loads (rows past the end are zero)
  float* sKe = sm + LD::R1;
  float* sQe = sm + LD::R2;
  float* sKF = sm + LD::R3;
#pragma unroll
  for (int e = tid; e < kCh * V8; e += 256) {
    const int r = e / V8, c0 = (e % V8) * 8;
    float x[8], kk[8], qq[8];
    ld8z(g + rowc(r) * DK + c0, r < L, x);
    ld8z(k + rowc(r) * DK + c0, r < L, kk);
    ld8z(q + rowc(r) * DK + c0, r < L, qq);
    st8(sGl + r * PK + c0, x);
    st8(sKe + r * PK + c0, kk);
    st8(sQe + r * PK + c0, qq);
  }
  if (tid < kCh) sBeta[tid] = ldfz(beta, rowc(tid), tid < L);
  __syncthreads();
  // decay scan (fp64) per channel, in place: Gamma - ref of the row's block
  if (tid < DK) {
    double acc = 0.0, ref[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll   // (static block index of ref, no select chains)
    for (int r = 0; r < kCh; ++r) {
      acc += (double)sGl[r * PK + tid];
      sGl[r * PK + tid] = (float)(acc - ref[r >> 4]);
      if ((r & 15) == 15 && r < kCh - 1) ref[(r + 1) >> 4] = acc;
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) sRef[a * DK + tid] = ref[a];
    sGam[tid] = acc;
  }
  __syncthreads();
  // Ke = k e^(Gamma - ref), Qe = q e^(Gamma - ref), in place
  for (int e = tid; e < kCh * V8; e += 256) {
    const int r = e / V8, c0 = (e % V8) * 8;
    float gl[8], kk[8], qq[8];
    ld8(sGl + r * PK + c0, gl);
    ld8(sKe + r * PK + c0, kk);
    ld8(sQe + r * PK + c0, qq);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float f = ex(gl[i]);
      kk[i] *= f;
      qq[i] *= f;
    }
    st8(sKe + r * PK + c0, kk);
    st8(sQe + r * PK + c0, qq);
  }

  // Gram tiles: G(a, bb) = sum_c Ke[r][c] KF_a[s][c] (bb <= a), same for M with Qe;
  // KF_a[s][c] = k[s][c] e^(ref_a - Gamma_s) for s < 16(a+1).
  f32x4 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    __syncthreads();
    {   // rows s < 16 (a + 1): every k load is issued before the first use
      constexpr int NPC = kCh * V8 / 256;
      float kk[NPC][8];
#pragma unroll
      for (int j = 0; j < NPC; ++j) {
        const int e = tid + 256 * j, s = e / V8, c0 = (e % V8) * 8;
        if (e < 16 * (a + 1) * V8) ld8z(k + rowc(s) * DK + c0, s < L, kk[j]);
      }
#pragma unroll
      for (int j = 0; j < NPC; ++j) {
        const int e = tid + 256 * j, s = e / V8, c0 = (e % V8) * 8, bs = s >> 4;
        if (e < 16 * (a + 1) * V8) {
          float gl[8];
          ld8(sGl + s * PK + c0, gl);
#pragma unroll
          for (int i = 0; i < 8; ++i) kk[j][i] *= ex((a == bs ? 0.f : dref(a, bs, c0 + i)) - gl[i]);
          st8(sKF + s * PK + c0, kk[j]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = w + 4 * j;
      acc[a][j] = zero4();
      if (t < 2 * (a + 1)) {
        const bool isG = t <= a;
        const int bb = isG ? t : t - a - 1;
        acc[a][j] = mm_nt(zero4(), (isG ? sKe : sQe) + 16 * a * PK, PK, sKF + 16 * bb * PK, PK, 0, DK);
      }
    }
  }
  __syncthreads();
  // G and M^T to LDS (R1: G [64][68] then MT [64][68]), G and M to nothing else
  float* sG = sm + LD::R1;
  float* sMT = sm + LD::R1 + kCh * kP64;
  for (int e = tid; e < 2 * kCh * kP64; e += 256) sm[LD::R1 + e] = 0.f;
  __syncthreads();
  {
    const int l = lane_id(), cl = l & 15, r0 = 4 * (l >> 4);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = w + 4 * j;
        if (t < 2 * (a + 1)) {
          const bool isG = t <= a;
          const int bb = isG ? t : t - a - 1;
          f32x4 v = acc[a][j];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool keep = bb < a || (isG ? (r0 + i > cl) : (r0 + i >= cl));
            v[i] = keep ? v[i] : 0.f;
          }
          if (isG) st_rm(sG + 16 * a * kP64 + 16 * bb, kP64, v);
          else st_tr(sMT + 16 * bb * kP64 + 16 * a, kP64, v);
        }
      }
    }
  }
  __syncthreads();
  // G to the record
  for (int e = tid; e < kCh * kCh; e += 256) out[RC::G + e] = sG[(e / kCh) * kP64 + (e % kCh)];

  // (I + Diag(beta) G)^-1: diagonal 16x16 blocks by forward substitution
  // (wave 0, lane = (block, column)), then off-diagonal blocks by levels.
  float* sLi = sm + LD::RL;
  float* sKbT = sm + LD::R2;   // [DK][68] beta e^Gamma k, transposed
  for (int e = tid; e < kCh * kP64; e += 256) sLi[e] = 0.f;
  __syncthreads();
  if (w == 0) {
    const int l = lane_id(), a = l >> 4, j = l & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int ri = 16 * a + i;
      float s = (i == j) ? 1.f : 0.f;
      float t = 0.f;
#pragma unroll
      for (int p = 0; p < i; ++p) t += sG[ri * kP64 + 16 * a + p] * x[p];
      x[i] = s - sBeta[ri] * t;
      sLi[ri * kP64 + 16 * a + j] = x[i];
    }
  } else {
    constexpr int NP = (kCh * V8 + 191) / 192;   // pieces per thread of waves 1-3
    float kk[NP][8];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int e = tid - 64 + 192 * j, s = e < kCh * V8 ? e / V8 : 0, c0 = (e % V8) * 8;
      ld8z(k + rowc(s) * DK + c0, e < kCh * V8 && s < L, kk[j]);
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int e = tid - 64 + 192 * j, s = e / V8, c0 = (e % V8) * 8;
      if (e < kCh * V8) {
        float gl[8];
        ld8(sGl + s * PK + c0, gl);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          sKbT[(c0 + i) * kP64 + s] = sBeta[s] * kk[j][i] * ex(ref_plus(s >> 4, c0 + i, gl[i]));
      }
    }
  }
  __syncthreads();
  float* sTmp = sm + LD::R3;   // per-wave 16x16 scratch (row-major, stride 16)
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    const int bb = w, a = w + d;
    const bool act = a < 4;
    if (act) {
      f32x4 t = zero4();
      for (int cc = bb; cc < a; ++cc)
        t = mm_nn(t, sG + 16 * a * kP64 + 16 * cc, kP64, sLi + 16 * cc * kP64 + 16 * bb, kP64, 0, 16);
      const int l = lane_id(), r0 = 4 * (l >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] *= sBeta[16 * a + r0 + i];
      st_rm(sTmp + w * 256, 16, t);
    }
    __syncthreads();
    if (act) {
      f32x4 x = mm_nn(zero4(), sLi + 16 * a * kP64 + 16 * a, kP64, sTmp + w * 256, 16, 0, 16);
      st_rm(sLi + 16 * a * kP64 + 16 * bb, kP64, -x);
    }
    __syncthreads();
  }
  for (int e = tid; e < kCh * kCh; e += 256) out[RC::LINV + e] = sLi[(e / kCh) * kP64 + (e % kCh)];

  // W = Linv (beta Kb): wave w owns rows 16w..16w+15
  f32x4 wt[NT];
#pragma unroll
  for (int T_ = 0; T_ < NT; ++T_)
    wt[T_] = mm_nt(zero4(), sLi + 16 * w * kP64, kP64, sKbT + 16 * T_ * kP64, kP64, 0, 16 * (w + 1));
  // dO^T scaled (R3; the inverse's scratch is no longer read)
  float* sdOT = sm + LD::R3;
  {
    constexpr int NDO = kCh * DV / 8 / 256;
    static_assert(NDO * 2048 == kCh * DV, "pieces per thread");
    float x[NDO][8];
#pragma unroll
    for (int j = 0; j < NDO; ++j) {
      const int e = tid + 256 * j, r = e / (DV / 8), j0 = (e % (DV / 8)) * 8;
      ld8z(dO + rowc(r) * DV + j0, r < L, x[j]);
    }
#pragma unroll
    for (int j = 0; j < NDO; ++j) {
      const int e = tid + 256 * j, r = e / (DV / 8), j0 = (e % (DV / 8)) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) sdOT[(j0 + i) * kP64 + r] = scale * x[j][i];
    }
  }
  __syncthreads();
  float* sWT = sm + LD::R2;
  {
    const int l = lane_id();
#pragma unroll
    for (int T_ = 0; T_ < NT; ++T_) {
      st_tr(sWT + 16 * T_ * kP64 + 16 * w, kP64, wt[T_]);
      *(f32x4*)(out + RC::WT + (size_t)(16 * T_ + (l & 15)) * kCh + 16 * w + 4 * (l >> 4)) = wt[T_];
    }
  }
  // P = scale M^T dO: rows s of block w, r >= 16w
  f32x4 pt[NV];
#pragma unroll
  for (int J = 0; J < NV; ++J) pt[J] = mm_nt(zero4(), sMT + 16 * w * kP64, kP64, sdOT + 16 * J * kP64, kP64, 16 * w, kCh);
  // Kh to the record; gather Gamma offsets for Qb (R0 is rewritten next)
  {
    constexpr int NPC = kCh * V8 / 256;
    float kk[NPC][8];
#pragma unroll
    for (int j = 0; j < NPC; ++j) {
      const int e = tid + 256 * j, r = e / V8, c0 = (e % V8) * 8;
      ld8z(k + rowc(r) * DK + c0, r < L, kk[j]);
    }
#pragma unroll
    for (int j = 0; j < NPC; ++j) {
      const int e = tid + 256 * j, r = e / V8, c0 = (e % V8) * 8;
      float gl[8];
      ld8(sGl + r * PK + c0, gl);
      st8(out + RC::GLOC + r * DK + c0, gl);
#pragma unroll
      for (int i = 0; i < 8; ++i) kk[j][i] *= ex(gam_minus(r >> 4, c0 + i) - gl[i]);
      st8(out + RC::KH + r * DK + c0, kk[j]);
    }
  }
  for (int e = tid; e < 10 * DK; e += 256) out[RC::REF + e] = sm[LD::REF + e];   // fp64 refs and gamma
  constexpr int PER = kCh * V8 / 256;   // groups of 8 per thread
  float qb[PER][8];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = tid + 256 * j, r = e / V8, c0 = (e % V8) * 8;
    float gl[8];
    ld8z(q + rowc(r) * DK + c0, r < L, qb[j]);
    ld8(sGl + r * PK + c0, gl);
#pragma unroll
    for (int i = 0; i < 8; ++i) qb[j][i] *= ex(ref_plus(r >> 4, c0 + i, gl[i]));
  }
  __syncthreads();
  float* sQbT = sm + LD::R0;
  {
    const int l = lane_id();
#pragma unroll
    for (int J = 0; J < NV; ++J) {
      const int r0 = 16 * w + 4 * (l >> 4), cl = 16 * J + (l & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) out[RC::P + (size_t)(r0 + i) * DV + cl] = pt[J][i];
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = tid + 256 * j, r = e / V8, c0 = (e % V8) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) sQbT[(c0 + i) * kP64 + r] = qb[j][i];
  }
  __syncthreads();
  // C = scale Qb^T dO   [DK][DV] (dO^T carries the scale); wave w owns tiles w, w+4, ...
  {
    const int l = lane_id(), r0 = 4 * (l >> 4), cl = l & 15;
    for (int t = w; t < NT * NV; t += 4) {
      const int Tr = t / NV, J = t % NV;
      const f32x4 v = mm_nt(zero4(), sQbT + 16 * Tr * kP64, kP64, sdOT + 16 * J * kP64, kP64, 0, kCh);
#pragma unroll
      for (int i = 0; i < 4; ++i) out[RC::C + (size_t)(16 * Tr + r0 + i) * DV + 16 * J + cl] = v[i];
    }
  }
}

// ---------------------------------------------------------------------------
// Reverse pass of the state gradient: one work-group per (head, 16 columns).
template <int DK, int DV>
struct StateLds {
  static constexpr int PK = DK + 4;
  static constexpr int KH = 0;                       // [64][PK]
  static constexpr int WT = KH + kCh * PK;           // [DK][68]
  static constexpr int NT_ = WT + DK * kP64;         // N^T slice [16][PK]
  static constexpr int XT = NT_ + 16 * PK;           // dU^T slice [16][68]
  static constexpr int WORDS = XT + 16 * kP64;
};

template <int DK, int DV>
__global__ __launch_bounds__(256) void bwd_state_kernel(const float* __restrict__ rec, const float* __restrict__ dht,
                                                        float* __restrict__ dN, float* __restrict__ dU,
                                                        float* __restrict__ dh0, int nch, int nbh) {
  using LD = StateLds<DK, DV>;
  using RC = Rec<DK, DV>;
  constexpr int PK = LD::PK;
  constexpr int NS = DV / 16;
  __shared__ __align__(16) float sm[LD::WORDS];
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id();
  // The NS work-groups of a head run on one XCD (work-group i runs on XCD
  // i % 8): each reads the head's whole Kh and W^T every chunk, which then
  // come from that XCD's L2 after one read from memory.  (With the groups
  // of a head on consecutive work-groups, i.e. on all eight XCDs, every
  // XCD fetched every head's records: about 17 GB per call at B1 H32 T64K.)
  const int xg = blockIdx.x & 7, rest = blockIdx.x >> 3;
  const int js = rest % NS, bh = xg + 8 * (rest / NS), j0 = 16 * js;
  if (bh >= nbh) return;   // (the grid rounds the heads up to a multiple of 8)
  float* sKh = sm + LD::KH;
  float* sWT = sm + LD::WT;
  float* sNT = sm + LD::NT_;
  float* sXT = sm + LD::XT;
  const int cl = l & 15, r0 = 4 * (l >> 4);

  for (int e = tid; e < 16 * DK; e += 256) {
    const int cc = e / 16, j = e % 16;
    sNT[j * PK + cc] = dht ? dht[((size_t)bh * DK + cc) * DV + j0 + j] : 0.f;
  }
  // Chunk c - 1's record slices are loaded into registers while chunk c is
  // computed, so the step does not wait for a memory round trip: Kh and W^T
  // (16-byte pieces of the whole matrices), this lane's P and C values and
  // the fp64 gamma of its key rows.
  constexpr int NKW = kCh * DK / 4 / 256;   // 16-byte pieces per thread
  constexpr int NM = DK / 64;               // key-row tiles per wave
  static_assert(NKW * 256 * 4 == kCh * DK && NM * 64 == DK, "record slices split evenly over the threads");
  f32x4 pkh[NKW], pwt[NKW];
  float pp[4], pcv[NM][4];
  double pg[NM][4];
  auto load_rec = [&](int c) {
    const float* rc = rec + ((size_t)bh * nch + c) * RC::WORDS;
#pragma unroll
    for (int i = 0; i < NKW; ++i) {
      const int e = tid + 256 * i;
      pkh[i] = *(const f32x4*)(rc + RC::KH + 4 * e);
      pwt[i] = *(const f32x4*)(rc + RC::WT + 4 * e);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) pp[i] = rc[RC::P + (size_t)(16 * w + r0 + i) * DV + j0 + cl];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cc = 16 * (w + 4 * m) + r0 + i;
        pcv[m][i] = rc[RC::C + (size_t)cc * DV + j0 + cl];
        pg[m][i] = reinterpret_cast<const double*>(rc + RC::GAM)[cc];
      }
  };
  load_rec(nch - 1);
  for (int c = nch - 1; c >= 0; --c) {
    const size_t n = (size_t)bh * nch + c;
    // the previous step's readers of Kh and W^T passed its last barrier
#pragma unroll
    for (int i = 0; i < NKW; ++i) {
      const int e = tid + 256 * i;
      const int r = (4 * e) / DK, cc = (4 * e) % DK;
      *(f32x4*)(sKh + r * PK + cc) = pkh[i];
      const int cw = (4 * e) / kCh, rw = (4 * e) % kCh;
      *(f32x4*)(sWT + cw * kP64 + rw) = pwt[i];
    }
    f32x4 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = pp[i];
    f32x4 base[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) base[m][i] = pcv[m][i];
    float eg[NM][4];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) eg[m][i] = ex((float)pg[m][i]);
    if (c > 0) load_rec(c - 1);
    __syncthreads();   // also orders the previous iteration's N^T writes
    // the gradient leaving chunk c
    for (int e = tid; e < 16 * DK; e += 256) {
      const int cc = e / 16, j = e % 16;
      dN[(n * DK + cc) * DV + j0 + j] = sNT[j * PK + cc];
    }
    // dU rows of block w: P + Kh N
    x = mm_nt(x, sKh + 16 * w * PK, PK, sNT, PK, 0, DK);
    st_tr(sXT + 16 * w, kP64, x);
#pragma unroll
    for (int i = 0; i < 4; ++i) dU[(n * kCh + 16 * w + r0 + i) * DV + j0 + cl] = x[i];
    __syncthreads();
    // N <- e^gamma N + C - W^T dU, rows of tiles w, w+4
    f32x4 nn[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int Tc = w + 4 * m;
      const f32x4 old = *(const f32x4*)(sNT + cl * PK + 16 * Tc + r0);
#pragma unroll
      for (int i = 0; i < 4; ++i) base[m][i] += eg[m][i] * old[i];
      nn[m] = base[m] - mm_nt(zero4(), sWT + 16 * Tc * kP64, kP64, sXT, kP64, 0, kCh);
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NM; ++m) st_tr(sNT + 16 * (w + 4 * m), PK, nn[m]);
  }
  __syncthreads();
  if (dh0)
    for (int e = tid; e < 16 * DK; e += 256) {
      const int cc = e / 16, j = e % 16;
      dh0[((size_t)bh * DK + cc) * DV + j0 + j] = sNT[j * PK + cc];
    }
}

// ---------------------------------------------------------------------------
// Per-chunk gradients.
template <int DK, int DV>
struct GradLds {
  static constexpr int PK = DK + 4, PV = DV + 4;
  static constexpr int RS0 = (64 * PK > DK * kP64 ? 64 * PK : DK * kP64);
  static constexpr int RS1 = (64 * PV > DV * kP64 ? 64 * PV : DV * kP64);
  static constexpr int RS2 = RS0 > RS1 ? RS0 : RS1;
  static constexpr int RS = RS2 > 2 * kCh * kP64 ? RS2 : 2 * kCh * kP64;   // also holds two [64][68]
  static constexpr int R0 = 0, R1 = RS, R2 = 2 * RS, R3 = 3 * RS, RL = 4 * RS;
  static constexpr int REF = RL + kCh * kP64;   // [4][DK] fp64
  static constexpr int GAM = REF + 8 * DK;      // [DK] fp64
  static constexpr int BETA = GAM + 2 * DK;     // [64]
  static constexpr int DB = BETA + kCh;         // [64] dbeta
  static constexpr int DGS = DB + kCh;          // [DK] e^gamma sum_j N S
  static constexpr int WORDS = DGS + DK;
};

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(256) void bwd_grad_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v, const TIn* __restrict__ beta,
    const float* __restrict__ dO, const float* __restrict__ h0, const float* __restrict__ snap,
    const float* __restrict__ rec, const float* __restrict__ dNb, const float* __restrict__ dUb, float scale, int T,
    int H, int nch, float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dg,
    float* __restrict__ dbeta) {
  using LD = GradLds<DK, DV>;
  using RC = Rec<DK, DV>;
  constexpr int PK = LD::PK, PV = LD::PV;
  constexpr int NT = DK / 16, NV = DV / 16;
  __shared__ __align__(16) float sm[LD::WORDS];
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id();
  const int cl = l & 15, g4 = l >> 4, r0 = 4 * g4;
  const int n = blockIdx.x, bh = n / nch, c = n % nch;
  const int b = bh / H, h = bh % H;
  const int t0 = c * kCh, L = min(kCh, T - t0);
  const int nbh = (int)(gridDim.x / nch);
  const float* rc = rec + (size_t)n * RC::WORDS;
  auto row = [&](int r) { return ((size_t)b * T + t0 + r) * H + h; };
  auto rowc = [&](int r) { return row(r < L ? r : 0); };   // row 0 stands in past the end
  const float* S = c == 0 ? (h0 ? h0 + (size_t)bh * DK * DV : nullptr) : snap + ((size_t)(c - 1) * nbh + bh) * DK * DV;
  const float* Nn = dNb + (size_t)n * DK * DV;

  double* sRef = reinterpret_cast<double*>(sm + LD::REF);
  double* sGam = reinterpret_cast<double*>(sm + LD::GAM);
  auto dref = [&](int a, int bs, int cc) { return (float)(sRef[a * DK + cc] - sRef[bs * DK + cc]); };
  auto gam_minus = [&](int a, int cc) { return (float)(sGam[cc] - sRef[a * DK + cc]); };
  auto ref_plus = [&](int a, int cc, float gl) { return (float)(sRef[a * DK + cc] + (double)gl); };
  float* sBeta = sm + LD::BETA;
  float* sDb = sm + LD::DB;
  float* sDgs = sm + LD::DGS;
  float* sS = sm + LD::R0;     // [DK][PV] over R0..R1
  float* sLi = sm + LD::RL;    // [64][68]
  // The chunk's state S, L^-1 and dU^T go to LDS; every load is issued
  // before the first LDS write, so the work-group waits for one round trip
  // (its 4 waves cannot hide a chain of them).
  constexpr int NSS = DK * DV / 4 / 256, NLI = kCh * kCh / 4 / 256, NDU = kCh * DV / 8 / 256;
  static_assert(NSS * 1024 == DK * DV && NLI * 1024 == kCh * kCh && NDU * 2048 == kCh * DV, "pieces per thread");
  float* sdUT = sm + LD::R3;   // dU^T
  constexpr int NREF = (10 * DK + 255) / 256;   // fp64 block references and gamma, as words
  {
    f32x4 sv[NSS], li[NLI];
    float du[NDU][8], refv[NREF];
#pragma unroll
    for (int i = 0; i < NREF; ++i) refv[i] = rc[RC::REF + min(tid + 256 * i, 10 * DK - 1)];
#pragma unroll
    for (int i = 0; i < NSS; ++i) sv[i] = S ? *(const f32x4*)(S + 4 * (tid + 256 * i)) : zero4();
#pragma unroll
    for (int i = 0; i < NLI; ++i) li[i] = *(const f32x4*)(rc + RC::LINV + 4 * (tid + 256 * i));
#pragma unroll
    for (int i = 0; i < NDU; ++i) {
      const int e = tid + 256 * i, r = e / (DV / 8), j0 = (e % (DV / 8)) * 8;
      ld8(dUb + ((size_t)n * kCh + r) * DV + j0, du[i]);
    }
#pragma unroll
    for (int i = 0; i < NREF; ++i)
      if (tid + 256 * i < 10 * DK) sm[LD::REF + tid + 256 * i] = refv[i];
    if (tid < kCh) {
      sBeta[tid] = ldfz(beta, rowc(tid), tid < L);
      sDb[tid] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < NSS; ++i) {
      const int e = tid + 256 * i, cc = (4 * e) / DV, j = (4 * e) % DV;
      *(f32x4*)(sS + cc * PV + j) = sv[i];
    }
#pragma unroll
    for (int i = 0; i < NLI; ++i) {
      const int e = tid + 256 * i, r = (4 * e) / kCh, s = (4 * e) % kCh;
      *(f32x4*)(sLi + r * kP64 + s) = li[i];
    }
#pragma unroll
    for (int i = 0; i < NDU; ++i) {
      const int e = tid + 256 * i, r = e / (DV / 8), j0 = (e % (DV / 8)) * 8;
#pragma unroll
      for (int x = 0; x < 8; ++x) sdUT[(j0 + x) * kP64 + r] = du[i][x];
    }
  }
  // this wave's rows of Kb and scale * dO as left operands (Kb takes the
  // block references, which are in LDS only after the barrier)
  const int ra = 16 * w + cl;   // operand row of this lane
  f32x4 kba[NT], doa[NV], gla[NT];
#pragma unroll
  for (int J = 0; J < NT; ++J) {
    const int c0 = 16 * J + 4 * g4;
    kba[J] = ld4z(k + rowc(ra) * DK + c0, ra < L);
    gla[J] = ld4(rc + RC::GLOC + ra * DK + c0);
  }
#pragma unroll
  for (int J = 0; J < NV; ++J) doa[J] = scale * ld4z(dO + rowc(ra) * DV + 16 * J + 4 * g4, ra < L);
  __syncthreads();
#pragma unroll
  for (int J = 0; J < NT; ++J)
#pragma unroll
    for (int i = 0; i < 4; ++i) kba[J][i] *= ex(ref_plus(w, 16 * J + 4 * g4 + i, gla[J][i]));

  // e^gamma sum_j N S per key row (threads: row = tid / 2, half of the columns)
  {
    const int cc = tid >> 1, half = tid & 1;
    float s = 0.f;
    if (cc < DK) {
      const float* np = Nn + (size_t)cc * DV + half * (DV / 2);
      f32x4 nv[DV / 8];
#pragma unroll
      for (int i = 0; i < DV / 8; ++i) nv[i] = *(const f32x4*)(np + 4 * i);
#pragma unroll
      for (int i = 0; i < DV / 8; ++i) {
        const f32x4 sv = *(const f32x4*)(sS + cc * PV + half * (DV / 2) + 4 * i);
#pragma unroll
        for (int x = 0; x < 4; ++x) s += nv[i][x] * sv[x];
      }
    }
    s += __shfl_xor(s, 1);
    if (cc < DK && half == 0) sDgs[cc] = ex((float)sGam[cc]) * s;
  }
  // R = V - Kb S, dQb = scale dO S^T (rows of block w)
  f32x4 R[NV], dQb[NT];
#pragma unroll
  for (int J = 0; J < NV; ++J)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + r0 + i;
      R[J][i] = ldfz(v, rowc(r) * DV + 16 * J + cl, r < L);
    }
#pragma unroll
  for (int J = 0; J < NV; ++J) {
    f32x4 acc = zero4();
    const float* b0 = sS + (4 * g4) * PV + 16 * J + cl;
#pragma unroll
    for (int K = 0; K < NT; ++K) {
      const float* bk = b0 + 16 * K * PV;
      acc = mfma4(kba[K], f32x4{bk[0], bk[PV], bk[2 * PV], bk[3 * PV]}, acc);
    }
    R[J] -= acc;
  }
#pragma unroll
  for (int K = 0; K < NT; ++K) {
    f32x4 acc = zero4();
    const float* bt = sS + (16 * K + cl) * PV + 4 * g4;
#pragma unroll
    for (int J = 0; J < NV; ++J) acc = mfma4(doa[J], *(const f32x4*)(bt + 16 * J), acc);
    dQb[K] = acc;
  }
  // (beta R)^T -> R2, then U = Linv (beta R)
  float* sRT = sm + LD::R2;
#pragma unroll
  for (int J = 0; J < NV; ++J) {
    f32x4 br;
#pragma unroll
    for (int i = 0; i < 4; ++i) br[i] = sBeta[16 * w + r0 + i] * R[J][i];
    st_tr(sRT + 16 * J * kP64 + 16 * w, kP64, br);
  }
  __syncthreads();
  f32x4 U[NV], Z[NV];
#pragma unroll
  for (int J = 0; J < NV; ++J) U[J] = mm_nt(zero4(), sLi + 16 * w * kP64, kP64, sRT + 16 * J * kP64, kP64, 0, 16 * (w + 1));
  // Z = Linv^T dU (rows of block w: s >= 16w)
#pragma unroll
  for (int J = 0; J < NV; ++J) Z[J] = mm_tt(zero4(), sLi + 16 * w, kP64, sdUT + 16 * J * kP64, kP64, 16 * w, kCh);
  // dv = beta Z; dbeta part sum_j Z R
  {
    float db[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J < NV; ++J) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + r0 + i;
        db[i] += Z[J][i] * R[J][i];
        if (r < L) dv[row(r) * DV + 16 * J + cl] = sBeta[r] * Z[J][i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = db[i];
      x += __shfl_xor(x, 1);
      x += __shfl_xor(x, 2);
      x += __shfl_xor(x, 4);
      x += __shfl_xor(x, 8);
      if (cl == 0) sDb[16 * w + r0 + i] += x;   // one lane per row
    }
  }
  __syncthreads();
  // Z row-major -> R2; dKb' = Z S^T
  float* sZ = sm + LD::R2;
#pragma unroll
  for (int J = 0; J < NV; ++J) st_rm(sZ + 16 * w * PV + 16 * J, PV, Z[J]);
  __syncthreads();
  f32x4 dKb[NT];
#pragma unroll
  for (int K = 0; K < NT; ++K) dKb[K] = mm_nt(zero4(), sZ + 16 * w * PV, PV, sS + 16 * K * PV, PV, 0, DV);
  __syncthreads();
  // N row-major over R0..R1; U row-major -> R3
  float* sN = sm + LD::R0;
  float* sU = sm + LD::R3;
  for (int e = tid; e < DK * DV / 4; e += 256) {
    const int cc = (4 * e) / DV, j = (4 * e) % DV;
    *(f32x4*)(sN + cc * PV + j) = *(const f32x4*)(Nn + 4 * e);
  }
#pragma unroll
  for (int J = 0; J < NV; ++J) st_rm(sU + 16 * w * PV + 16 * J, PV, U[J]);
  __syncthreads();
  // dKh = U N^T
  f32x4 dKh[NT];
#pragma unroll
  for (int K = 0; K < NT; ++K) dKh[K] = mm_nt(zero4(), sU + 16 * w * PV, PV, sN + 16 * K * PV, PV, 0, DV);
  // dA' = Z U^T, dM' = scale dO U^T on tiles (w, bb <= w)
  f32x4 dA[4], dM[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    dA[bb] = zero4();
    dM[bb] = zero4();
    if (bb <= w) {
      dA[bb] = mm_nt(zero4(), sZ + 16 * w * PV, PV, sU + 16 * bb * PV, PV, 0, DV);
      const float* bt = sU + (16 * bb + cl) * PV + 4 * g4;
      f32x4 acc = zero4();
#pragma unroll
      for (int J = 0; J < NV; ++J) acc = mfma4(doa[J], *(const f32x4*)(bt + 16 * J), acc);
      dM[bb] = acc;
    }
  }
  // masks; dG = beta dA with dA = -Z U^T strictly lower; dbeta += sum_s dA G
  {
    float db[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + r0 + i, s = 16 * bb + cl;
        const bool strict = bb < w || (bb == w && r0 + i > cl);
        const bool low = bb < w || (bb == w && r0 + i >= cl);
        const float a_ = strict ? -dA[bb][i] : 0.f;
        db[i] += a_ * (strict ? rc[RC::G + r * kCh + s] : 0.f);
        dA[bb][i] = sBeta[r] * a_;
        dM[bb][i] = low ? dM[bb][i] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = db[i];
      x += __shfl_xor(x, 1);
      x += __shfl_xor(x, 2);
      x += __shfl_xor(x, 4);
      x += __shfl_xor(x, 8);
      if (cl == 0) sDb[16 * w + r0 + i] += x;
    }
  }
  __syncthreads();   // Z, U, N no longer read
  // dG, dM row-major -> R2; transposed -> R3 (upper parts zero)
  float* sdG = sm + LD::R2;
  float* sdM = sm + LD::R2 + kCh * kP64;
  float* sdGT = sm + LD::R3;
  float* sdMT = sm + LD::R3 + kCh * kP64;
  for (int e = tid; e < 2 * kCh * kP64; e += 256) {
    sm[LD::R2 + e] = 0.f;
    sm[LD::R3 + e] = 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    if (bb <= w) {
      st_rm(sdG + 16 * w * kP64 + 16 * bb, kP64, dA[bb]);
      st_rm(sdM + 16 * w * kP64 + 16 * bb, kP64, dM[bb]);
      st_tr(sdGT + 16 * bb * kP64 + 16 * w, kP64, dA[bb]);
      st_tr(sdMT + 16 * bb * kP64 + 16 * w, kP64, dM[bb]);
    }
  }
  // own-position decay offsets
  f32x4 gl[NT];
#pragma unroll
  for (int K = 0; K < NT; ++K) {
#pragma unroll
    for (int i = 0; i < 4; ++i) gl[K][i] = rc[RC::GLOC + (size_t)(16 * w + r0 + i) * DK + 16 * K + cl];
  }
  // decayed products, one row block a at a time
  // Row side of row block a: every wave takes NT / 4 channel tiles of every
  // block (rx1, rx2), handed to the block's owner wave through LDS after the
  // loop; the column side stays with the owner of the column rows.
  constexpr int NTW = NT / 4;
  static_assert(NTW * 4 == NT, "dk must be a multiple of 64");
  f32x4 dkcol[NT], rx1[4][NTW], rx2[4][NTW];
#pragma unroll
  for (int K = 0; K < NT; ++K) dkcol[K] = zero4();
  float* sKFT = sm + LD::R0;                // [DK][68]: k_s e^(ref_a - Gamma_s), s < 16(a+1)
  float* sKeT = sm + LD::R1;                // [DK][20]: k_r e^(Gamma_r - ref_a), r in block a
  float* sQeT = sm + LD::R1 + DK * 20;      // [DK][20]: q_r e^(Gamma_r - ref_a)
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    __syncthreads();
    // Pieces e = tid + 256 j (row s = e / (DK / 8), 8 channels from c0) with
    // s < 16 (a + 1): k and the decay offsets, plus q for the rows of block
    // a (piece jq); all loads are issued before the LDS writes.
    {
      constexpr int NPC = kCh * (DK / 8) / 256;
      static_assert(NPC * 256 == kCh * (DK / 8), "pieces per thread");
      const int lo = 16 * a * (DK / 8), hi = lo + 16 * (DK / 8), jq = lo / 256;
      float kk[NPC][8], gv[NPC][8], qq[8];
#pragma unroll
      for (int j = 0; j < NPC; ++j) {
        const int e = tid + 256 * j, s = e / (DK / 8), c0 = (e % (DK / 8)) * 8;
        if (e < hi) {
          ld8z(k + rowc(s) * DK + c0, s < L, kk[j]);
          ld8(rc + RC::GLOC + (size_t)s * DK + c0, gv[j]);
          if (j == jq && e >= lo) {
            ld8z(q + rowc(s) * DK + c0, s < L, qq);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NPC; ++j) {
        const int e = tid + 256 * j, s = e / (DK / 8), c0 = (e % (DK / 8)) * 8, bs = s >> 4;
        if (e < hi) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            sKFT[(c0 + i) * kP64 + s] = kk[j][i] * ex((a == bs ? 0.f : dref(a, bs, c0 + i)) - gv[j][i]);
          if (j == jq && e >= lo) {   // k_r e^(Gamma_r - ref_a), q_r e^(Gamma_r - ref_a), r in block a
            const int rl = s - 16 * a;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float f = ex(gv[j][i]);
              sKeT[(c0 + i) * 20 + rl] = kk[j][i] * f;
              sQeT[(c0 + i) * 20 + rl] = qq[i] * f;
            }
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < NTW; ++kk) {   // row side: rows of block a, this wave's channel tiles
      const int K = w * NTW + kk;
      rx1[a][kk] = mm_nt(zero4(), sdG + 16 * a * kP64, kP64, sKFT + 16 * K * kP64, kP64, 0, 16 * (a + 1));
      rx2[a][kk] = mm_nt(zero4(), sdM + 16 * a * kP64, kP64, sKFT + 16 * K * kP64, kP64, 0, 16 * (a + 1));
    }
    if (w <= a) {   // column side: rows s of block w against rows r of block a
#pragma unroll
      for (int K = 0; K < NT; ++K) {
        const f32x4 x1 = mm_nt(zero4(), sdGT + 16 * w * kP64 + 16 * a, kP64, sKeT + 16 * K * 20, 20, 0, 16);
        const f32x4 x2 = mm_nt(zero4(), sdMT + 16 * w * kP64 + 16 * a, kP64, sQeT + 16 * K * 20, 20, 0, 16);
        f32x4 fa;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int cc = 16 * K + cl;
          const float d = (a == w) ? 0.f : dref(a, w, cc);
          fa[i] = ex(d - gl[K][i]);
        }
        dkcol[K] += fa * (x1 + x2);
      }
    }
  }
  __syncthreads();
  // q and k rows of the chunk as fp32 (zero past the end) into R2 / R3, free
  // after the decayed products, for the own-row terms below
  float* sQr = sm + LD::R2;
  float* sKr = sm + LD::R3;
  {
    constexpr int NPC = kCh * (DK / 8) / 256;
    float qv[NPC][8], kv[NPC][8];
#pragma unroll
    for (int j = 0; j < NPC; ++j) {
      const int e = tid + 256 * j, s = e / (DK / 8), c0 = (e % (DK / 8)) * 8;
      ld8z(q + rowc(s) * DK + c0, s < L, qv[j]);
      ld8z(k + rowc(s) * DK + c0, s < L, kv[j]);
    }
#pragma unroll
    for (int j = 0; j < NPC; ++j) {
      const int e = tid + 256 * j, s = e / (DK / 8), c0 = (e % (DK / 8)) * 8;
      st8(sQr + s * PK + c0, qv[j]);
      st8(sKr + s * PK + c0, kv[j]);
    }
  }
  // row-side products to R0 / R1 ([64][PK], free after the loop), then each
  // wave takes its own rows and applies their decay factors
  float* sX1 = sm + LD::R0;
  float* sX2 = sm + LD::R1;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int kk = 0; kk < NTW; ++kk) {
      st_rm(sX1 + 16 * a * PK + 16 * (w * NTW + kk), PK, rx1[a][kk]);
      st_rm(sX2 + 16 * a * PK + 16 * (w * NTW + kk), PK, rx2[a][kk]);
    }
  __syncthreads();
  f32x4 dqm[NT], dkrow[NT];
#pragma unroll
  for (int K = 0; K < NT; ++K) {
    const f32x4 e4 = f32x4{ex(gl[K][0]), ex(gl[K][1]), ex(gl[K][2]), ex(gl[K][3])};
    const float* x1 = sX1 + (16 * w + r0) * PK + 16 * K + cl;
    const float* x2 = sX2 + (16 * w + r0) * PK + 16 * K + cl;
    dkrow[K] = e4 * f32x4{x1[0], x1[PK], x1[2 * PK], x1[3 * PK]};
    dqm[K] = e4 * f32x4{x2[0], x2[PK], x2[2 * PK], x2[3 * PK]};
  }
  __syncthreads();   // R0 and R1 are rewritten below
  // combine.  dg_r = sum_{r' >= r} (q dq + k dk_plus - k dk_col)_{r'}
  //              + sum_{r' < r} k e^(gamma - Gamma) dKh_{r'} + e^gamma sum_j N S:
  // the Kh term, which enters both dGamma (-) and dgamma (+), is summed over
  // the rows before r instead, so the two large sums never cancel.
  // Pairwise terms cancel between the row and column sides; both use the same
  // rounded factors.
  float* sdGam = sm + LD::R0;   // [64][PK] reverse-summed part
  float* sHk = sm + LD::R1;     // [64][PK] forward-summed part
#pragma unroll
  for (int K = 0; K < NT; ++K) {
    const int cc = 16 * K + cl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + r0 + i;
      const float E = ex(ref_plus(w, cc, gl[K][i]));
      const float Eh = ex(gam_minus(w, cc) - gl[K][i]);
      const float qv = sQr[r * PK + cc];
      const float kv = sKr[r * PK + cc];
      const float dqv = E * dQb[K][i] + dqm[K][i];
      const float dkp = -sBeta[r] * E * dKb[K][i] + dkrow[K][i];
      const float hk = Eh * dKh[K][i];
      const float dkm = dkcol[K][i] + hk;
      if (r < L) {
        dq[row(r) * DK + cc] = dqv;
        dk[row(r) * DK + cc] = dkp + dkm;
      }
      sdGam[r * PK + cc] = qv * dqv + kv * (dkp - dkcol[K][i]);
      sHk[r * PK + cc] = kv * hk;
    }
  }
  __syncthreads();
  if (tid < DK) {   // row sums in fp64, one rounding per output (dg spans orders of magnitude)
    double rev = 0.0;
    for (int r = 0; r < kCh; ++r) rev += (double)sdGam[r * PK + tid];
    double fw = (double)sDgs[tid];
    for (int r = 0; r < L; ++r) {
      dg[row(r) * DK + tid] = (float)(rev + fw);
      rev -= (double)sdGam[r * PK + tid];
      fw += (double)sHk[r * PK + tid];
    }
  }
  if (tid < L) dbeta[row(tid)] = sDb[tid];
}

template <typename TIn, int DK, int DV>
hipError_t bwd_t(const void* q, const void* k, const void* v, const void* g, const void* beta, const float* dO,
                 float scale, const float* h0, const float* dht, const float* snap, float* rec, float* dNb,
                 float* dUb, int B, int T, int H, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                 float* dh0, hipStream_t st) {
  const int nch = (T + kCh - 1) / kCh;
  const int nbh = B * H;
  const unsigned nrec = (unsigned)(nch * nbh);
  const TIn* qq = (const TIn*)q;
  const TIn* kk = (const TIn*)k;
  hipLaunchKernelGGL((bwd_prep_kernel<TIn, DK, DV>), dim3(nrec), dim3(256), 0, st, qq, kk, (const TIn*)g,
                     (const TIn*)beta, dO, scale, T, H, nch, rec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_state_kernel<DK, DV>), dim3((nbh + 7) / 8 * 8 * (DV / 16)), dim3(256), 0, st,
                     (const float*)rec, dht, dNb, dUb, dh0, nch, nbh);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_grad_kernel<TIn, DK, DV>), dim3(nrec), dim3(256), 0, st, qq, kk, (const TIn*)v,
                     (const TIn*)beta, dO, h0, snap, (const float*)rec, (const float*)dNb, (const float*)dUb, scale, T,
                     H, nch, dq, dk, dv, dg, dbeta);
  return hipGetLastError();
}

template <typename TIn>
hipError_t bwd_d(int dk_, int dv_, const void* q, const void* k, const void* v, const void* g, const void* beta,
                 const float* dO, float scale, const float* h0, const float* dht, const float* snap, float* rec,
                 float* dNb, float* dUb, int B, int T, int H, float* dq, float* dk, float* dv, float* dg,
                 float* dbeta, float* dh0, hipStream_t st) {
#define KDA_BWD_CASE(A, Bv)                                                                                    \
  if (dk_ == A && dv_ == Bv)                                                                                   \
    return bwd_t<TIn, A, Bv>(q, k, v, g, beta, dO, scale, h0, dht, snap, rec, dNb, dUb, B, T, H, dq, dk, dv, dg, \
                             dbeta, dh0, st);
  KDA_BWD_CASE(128, 128)
  KDA_BWD_CASE(128, 64)
  KDA_BWD_CASE(64, 128)
  KDA_BWD_CASE(64, 64)
#undef KDA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace

size_t bwd_record_words(int dk, int dv) {
  return (size_t)2 * kCh * kCh + (size_t)kCh * dk + 10 * (size_t)dk + (size_t)kCh * dk + (size_t)dk * kCh +
         (size_t)kCh * dv + (size_t)dk * dv;
}

hipError_t launch_bwd_chunks(int is_bf16, const void* q, const void* k, const void* v, const void* g,
                             const void* beta, const float* dO, float scale, const float* h0, const float* dht,
                             const float* snap, float* rec, float* dN, float* dU, int B, int T, int H, int dk,
                             int dv, float* dq, float* dk_, float* dv_, float* dg, float* dbeta, float* dh0,
                             hipStream_t st) {
  if (is_bf16)
    return bwd_d<bf16>(dk, dv, q, k, v, g, beta, dO, scale, h0, dht, snap, rec, dN, dU, B, T, H, dq, dk_, dv_, dg,
                       dbeta, dh0, st);
  return bwd_d<float>(dk, dv, q, k, v, g, beta, dO, scale, h0, dht, snap, rec, dN, dU, B, T, H, dq, dk_, dv_, dg,
                      dbeta, dh0, st);
}

}  // namespace kda
