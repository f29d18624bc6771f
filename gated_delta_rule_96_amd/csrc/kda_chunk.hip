// Chunked KDA prefill on gfx950: an intra-chunk kernel (parallel over every
// chunk of every head) followed by a state pass (sequential over chunks,
// parallel over heads), or both fused into one persistent kernel.
//
// Method (Kimi K3 technical report summary, page "Kimi K3 Technical Report -
// Open Frontier Intelligence"): "Key claims" section 2.1 (delta-rule state
// with channel-wise decay), section 2.1.1 / Fig. 3 (log-decay floored at
// gmin = -5 so that the reciprocal rescaling factors stay inside the bf16
// range and every causal tile, diagonal ones included, is a dense matrix
// product), "Method" section 2.1 (chunkwise-parallel form).
//
// Per (b, h) and chunk of C = 64 rows, Gamma = inclusive cumsum of g inside
// the chunk, S the state entering the chunk:
//   A[r,s]  = beta_r sum_c k_rc k_sc e^{Gamma_rc - Gamma_sc}      s <  r
//   M[r,s]  =        sum_c q_rc k_sc e^{Gamma_rc - Gamma_sc}      s <= r
//   Tm      = (I + A)^-1 Diag(beta)
//   W       = Tm (e^Gamma * K)          Ut = Tm V
//   U       = Ut - W S
//   O       = scale (e^Gamma * Q) S + scale M U
//   S      <- e^{Gamma_C} * S + (e^{Gamma_C - Gamma} * K)^T U
// Everything that does not depend on S (A, M, Tm, W, Ut) is built by the
// intra-chunk kernel; the state pass does the four S-dependent products.
//
// Rescaling (the point of the bounded decay): a tile of A or M whose rows
// lie in 16-row sub-chunk a is a plain product of
//   row operand  k_r (or q_r) * e^{Gamma_r - Gamma_p}   in [e^-80, 1]
//   col operand  k_s         * e^{Gamma_p - Gamma_s}
// with p = 16a - 1 (the row just before the sub-chunk).  For s in an
// earlier sub-chunk the column factor is <= 1; in the same sub-chunk it is
// <= e^80, inside the bf16 range (max e^88.7), so these operands are bf16.
// Entries above the diagonal of the diagonal tiles are finite and are
// discarded with a select.
//
// Precision policy with bf16 inputs (fp32 state, fp32 output):
//   * A: bf16 operands.  M: bf16 operands off the block diagonal; on the
//     diagonal tiles each operand is split into bf16 hi + lo and three
//     products are summed (the diagonal term q_r.k_r dominates the output).
//   * every other product uses fp16 operands (11-bit significand) with
//     fp32 accumulation.  Quantities whose range is not bounded by the
//     normalised inputs (V, Ut, S, U) are first scaled by a power of two
//     chosen from their current maximum (exact), so fp16 never overflows.
// With fp32 inputs every operand is fp32 (v_mfma_f32_16x16x4_f32).
//
// Workspace record per (b, h, chunk), every matrix stored as 16x16 tiles in
// MFMA lane order (tile = 64 lanes x 4 consecutive values; the two tiles of
// an operand slab interleaved lane by lane, tile_elem), so the state pass
// reads each operand slab with one contiguous 16-byte load per lane:
//   W  : tile (ct, rt) lane l = -W[16rt + l%16][16ct + 4(l/16) + i]      (Op)
//   Q  : tile (ct, rt) lane l = Qbar[16rt + l%16][16ct + 4(l/16) + i]    (Op)
//        with Qbar = scale e^Gamma * Q
//   K  : tile (st, ct) lane l = Khat[16st + 4(l/16) + i][16ct + l%16]    (Op)
//   M  : tile (kt, rt) lane l = scale M[16rt + l%16][16kt + 4(l/16) + i] (Op)
//        (tiles above the diagonal are zero)
//   (tile order: tile_cr / tile_k below, the two tiles of one operand slab
//   next to each other)
//   dec: fp32 [dk] = e^{Gamma_C};  uinv: fp32, 1 / (scale factor of U)
//   U  : tile (st, jt) lane l = Ut[16st + 4(l/16) + i][16jt + l%16] * su (Op),
//        tiles column-block major (index 4 jt + st)
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kC = 64;   // chunk rows
constexpr int kNW = 8;                // waves per work-group (every kernel here)
constexpr int kThreads = 64 * kNW;

// Cycle stamps, compiled in only with KDA_CYCLE_STAMPS (a profiling build of
// the library; the product build has empty marks and identical code).  Each
// wave of the fused kernel adds up the shader-clock cycles (s_memtime)
// between consecutive marks into the slot named by the later mark and, when
// it leaves, lane 0 writes its sums to g_stamps[(block * kNW + wave) * 32 +
// slot].  Slot kStampRole says which loop the wave ran (1 producer, 2 state
// pass owner, 3 state pass staging), slot kStampCount how many items or
// chunks it handled.  Reading the clock waits for the wave's outstanding
// LDS and scalar accesses, so stamped runs are a few percent slower.
constexpr int kStampSlots = 32, kStampRole = 29, kStampCount = 30;
constexpr int kStampMaxWgs = 256;   // the fused grid (one work-group per CU)
#ifdef KDA_CYCLE_STAMPS
__device__ unsigned long long g_stamps[kStampMaxWgs * kNW * kStampSlots];
struct Stamps {
  unsigned long long acc[kStampSlots];
  unsigned long long last;
  __device__ Stamps() : last(__builtin_amdgcn_s_memtime()) {
#pragma unroll
    for (int i = 0; i < kStampSlots; ++i) acc[i] = 0;
  }
  template <int i> __device__ __forceinline__ void mark() {
    const unsigned long long now = __builtin_amdgcn_s_memtime();
    acc[i] += now - last;
    last = now;
  }
  template <int i> __device__ __forceinline__ void add(unsigned long long n) { acc[i] += n; }
  __device__ __forceinline__ void flush() {
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0 && blockIdx.x < kStampMaxWgs) {
#pragma unroll
      for (int i = 0; i < kStampSlots; ++i) g_stamps[((size_t)blockIdx.x * kNW + w) * kStampSlots + i] = acc[i];
    }
  }
};
#else
struct Stamps {
  template <int i> __device__ __forceinline__ void mark() {}
  template <int i> __device__ __forceinline__ void add(unsigned long long) {}
  __device__ __forceinline__ void flush() {}
};
#endif

template <typename TIn> struct Policy;
template <> struct Policy<float> {
  using Op = float;
  using Gram = float;
  static constexpr bool kMixed = false;
};
template <> struct Policy<bf16> {
  using Op = f16;
  using Gram = bf16;
  static constexpr bool kMixed = true;
};

template <typename TIn, int DK, int DV>
struct Rec {
  using Op = typename Policy<TIn>::Op;
  static constexpr size_t W = 0;                               // Op elements
  static constexpr size_t Q = (size_t)DK * kC;
  static constexpr size_t K = 2 * (size_t)DK * kC;
  static constexpr size_t M = 3 * (size_t)DK * kC;
  static constexpr size_t DEC_OFF_BYTES = (M + (size_t)kC * kC) * sizeof(Op);   // fp32 [DK]
  static constexpr size_t UINV_OFF_BYTES = DEC_OFF_BYTES + 4 * (size_t)DK;      // fp32, 16 bytes
  static constexpr size_t U_OFF_BYTES = UINV_OFF_BYTES + 16;                    // Op [C*DV]
  static constexpr size_t BYTES = (U_OFF_BYTES + (size_t)kC * DV * sizeof(Op) + 255) / 256 * 256;
  static_assert(U_OFF_BYTES % 16 == 0, "record alignment");
};

// Record tile order.  The state pass reads operand slabs made of two tiles
// that are consecutive along the reduction index (reduction tiles 2s and
// 2s + 1); those two tiles get consecutive indices (2j, 2j + 1), whose
// values tile_elem interleaves per lane.
//   W, Q, M tile (ct, rt), reduction tile ct, 4 row tiles rt
__host__ __device__ constexpr int tile_cr(int ct, int rt) { return (ct >> 1) * 8 + rt * 2 + (ct & 1); }
//   K tile (st, ct), reduction tile st, NCT column tiles ct
template <int NCT> __host__ __device__ constexpr int tile_k(int st, int ct) {
  return (st >> 1) * (2 * NCT) + ct * 2 + (st & 1);
}

// Element offset of lane `lane`'s 4 values of record tile t (tiles of 256
// elements, 64 lanes x 4 consecutive values).  The two tiles of an operand
// slab, 2j and 2j + 1, are interleaved lane by lane: a lane's 8 values of
// slab j are contiguous (16 bytes in fp16), so the state pass reads a slab
// with one 16-byte load.
__host__ __device__ constexpr int tile_elem(int t, int lane) { return (t >> 1) * 512 + lane * 8 + (t & 1) * 4; }

// A lane's values of record tiles 2j (lo) and 2j + 1 (hi) at p = the even
// tile's tile_elem: one 16-byte store for 2-byte elements (half-filled
// 8-byte stores cost the record writes twice the requests), two for fp32.
template <typename T> __device__ __forceinline__ void store_pair(T* p, f32x4 lo, f32x4 hi) {
  if constexpr (sizeof(T) == 2) {
    const V4<T> a = narrow4<T>(lo), b = narrow4<T>(hi);
    typedef T T8 __attribute__((ext_vector_type(8)));
    *reinterpret_cast<T8*>(p) = T8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  } else {
    store4<T>(p, narrow4<T>(lo));
    store4<T>(p + 4, narrow4<T>(hi));
  }
}

typedef float raw16 __attribute__((ext_vector_type(4)));   // 16 raw bytes

// Element x of 16 raw bytes holding values of type T, as fp32.
template <typename T> __device__ __forceinline__ float raw_elem(raw16 v, int x);
template <> __device__ __forceinline__ float raw_elem<float>(raw16 v, int x) { return v[x]; }
template <> __device__ __forceinline__ float raw_elem<bf16>(raw16 v, int x) {
  return (float)__builtin_bit_cast(bf16x8, v)[x];
}

// acc = sum over the first 16*n16 reduction indices of pa-row . pb-row
// (both rows k-contiguous): the lower-triangular ranges of the chunk.
// The odd 16 of the range goes through a half-width MFMA into an
// accumulator of its own, added with a VALU op: the result of one MFMA shape
// is never fed to an MFMA of another shape as its accumulator (with such a
// hand-off, rows of the result came out wrong, differently from run to run).
template <typename T>
__device__ __forceinline__ f32x4 tri_mma(const T* pa, const T* pb, int n16) {
  f32x4 acc = zero4();
  int k = 0;
  for (; k + 2 <= n16; k += 2) acc = mma(load_slab(pa + 16 * k), load_slab(pb + 16 * k), acc);
  if (k < n16) acc = acc + mma(load_half(pa + 16 * k), load_half(pb + 16 * k), zero4());
  return acc;
}

// Right operand half slab read down a column of a row-major fp32 matrix:
// lane (g, j) gets p[(4g + i) * ld + j], i = 0..3.
__device__ __forceinline__ Half<float> load_half_col(const float* p, int ld) {
  const int l = lane_id(), j = l & 15, g4 = 4 * (l >> 4);
  return Half<float>{f32x4{p[(g4 + 0) * ld + j], p[(g4 + 1) * ld + j], p[(g4 + 2) * ld + j], p[(g4 + 3) * ld + j]}};
}

__device__ __forceinline__ float block_max(float x, float* sred) {
  x = wave_max_dpp(x);
  if ((threadIdx.x & 63) == 0) sred[threadIdx.x >> 6] = x;
  __syncthreads();
  float m = sred[0];
#pragma unroll
  for (int i = 1; i < kNW; ++i) m = fmaxf(m, sred[i]);
  __syncthreads();
  return m;
}

// Tiles (x, r) of a 64-row x (16 * nx) output split over the 8 waves, j-th
// tile of wave w: with 4 tiles per wave, wave w takes column-tile x = w and
// every row block r; with 2, the pairs of row blocks {0,3} and {1,2}.  The
// lower-triangular products cost r + 1 units, so every wave gets the same.
__device__ __forceinline__ void wave_tile(int w, int j, int per_wave, int& x, int& r) {
  if (per_wave == 4) {
    x = w;
    r = j;
  } else {
    x = w >> 1;
    r = (w & 1) ? 1 + j : (j ? 3 : 0);
  }
}

// The layer's steps either side of the path, fused into the kernel (all
// optional, selected per call; every test on them is wave-uniform):
//   kLayerGateZ   the decay input is z: g = gmin Sigmoid(exp(A[h]) z), fp32,
//                 in the staging of the scan (no separate decay pass)
//   kLayerNormQK  q and k rows divided by sqrt(sum of squares + 1e-6) before
//                 use, in fp32, then rounded to the input type
//   og != nullptr output gate: o <- Sigmoid(og) * o, og [B,T,H,dv] of the
//                 input type
constexpr int kLayerGateZ = 1, kLayerNormQK = 2;
struct Layer {
  const float* A;
  const void* og;
  int flags;
};

// Row-wise L2 normalisation of 16 raw bytes of a row that is spread over G
// consecutive lanes (G a power of two dividing 64): every lane of the
// group returns its elements divided by the row's norm.
template <typename TIn, int G>
__device__ __forceinline__ raw16 l2norm_part(raw16 v) {
  constexpr int VE = 16 / sizeof(TIn);
  float ss = 0.f;
#pragma unroll
  for (int x = 0; x < VE; ++x) ss = fmaf(raw_elem<TIn>(v, x), raw_elem<TIn>(v, x), ss);
  if constexpr (G <= 16) {
    // within a row of 16 lanes by DPP moves (pairs, quads, half rows, rows:
    // the same sums in the same order as an xor butterfly, without the LDS
    // round trip of a lane shuffle)
    if (G >= 2) ss += dpp_f<0xB1>(ss);    // quad_perm [1,0,3,2]
    if (G >= 4) ss += dpp_f<0x4E>(ss);    // quad_perm [2,3,0,1]
    if (G >= 8) ss += dpp_f<0x141>(ss);   // row_half_mirror
    if (G >= 16) ss += dpp_f<0x140>(ss);  // row_mirror
  } else {
#pragma unroll
    for (int off = 1; off < G; off <<= 1) ss += __shfl_xor(ss, off);
  }
  const float inv = 1.0f / sqrtf(ss + kNormEps);
  raw16 out;
  if constexpr (sizeof(TIn) == 4) {
#pragma unroll
    for (int x = 0; x < 4; ++x) out[x] = v[x] * inv;
  } else {
    bf16x8 o8;
#pragma unroll
    for (int x = 0; x < 8; ++x) o8[x] = from_f32<bf16>(raw_elem<TIn>(v, x) * inv);
    out = __builtin_bit_cast(raw16, o8);
  }
  return out;
}

// One chunk's raw inputs in registers (rows past the end of the sequence
// are zero): 16-byte vectors of k, q, g and v rows (k, q, g row-major over
// the threads, v column-block-major), and beta.  Inputs are read once, so
// their loads are non-temporal: they do not displace the chunk records that
// producers and consumers exchange through the L2.
template <typename TIn, int DK, int DV>
struct InRegs {
  static constexpr int VE = 16 / sizeof(TIn);
  static constexpr int NK = kC * DK / VE / kThreads;
  static constexpr int NV = kC * DV / VE / kThreads;
  static_assert(NK * kThreads * VE == kC * DK && NV * kThreads * VE == kC * DV, "shape");
  raw16 k[NK], q[NK], g[NK], v[NV];
  TIn beta;   // raw: converted when staged, so that no wait follows its load
};

// Parts of the inputs (bit mask of load_inputs): the next chunk's loads
// can be issued in portions spread over the current chunk's phases.
constexpr int kLoadK = 1, kLoadQ = 2, kLoadG = 4, kLoadV = 8, kLoadBeta = 16, kLoadAll = 31;

template <typename TIn, int DK, int DV, int kParts = kLoadAll>
__device__ __forceinline__ void load_inputs(InRegs<TIn, DK, DV>& in, const TIn* __restrict__ q,
                                            const TIn* __restrict__ k, const TIn* __restrict__ v,
                                            const TIn* __restrict__ g, const TIn* __restrict__ beta, int b, int h,
                                            int T_len, int H, int t0, int Lrows) {
  using IR = InRegs<TIn, DK, DV>;
  constexpr int VE = IR::VE;
  const int tid = threadIdx.x;
  const size_t tokk = (size_t)H * DK, tokv = (size_t)H * DV;
  const size_t base_k = ((size_t)b * T_len + t0) * tokk + (size_t)h * DK;
  const size_t base_v = ((size_t)b * T_len + t0) * tokv + (size_t)h * DV;
  const raw16 zero16 = raw16{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < IR::NK; ++i) {
    const int n = tid + kThreads * i;
    const int r = n / (DK / VE), c = (n % (DK / VE)) * VE;
    const bool ok = r < Lrows;
    const size_t off = base_k + r * tokk + c;
    if (kParts & kLoadK) in.k[i] = ok ? __builtin_nontemporal_load(reinterpret_cast<const raw16*>(k + off)) : zero16;
    if (kParts & kLoadQ) in.q[i] = ok ? __builtin_nontemporal_load(reinterpret_cast<const raw16*>(q + off)) : zero16;
    if (kParts & kLoadG)
      in.g[i] = (ok && g) ? __builtin_nontemporal_load(reinterpret_cast<const raw16*>(g + off)) : zero16;
  }
  // v: consecutive lanes take consecutive rows of one column block, so that
  // the transposed LDS staging of V is free of bank conflicts
#pragma unroll
  for (int i = 0; i < IR::NV; ++i) {
    const int n = tid + kThreads * i;
    const int r = n % kC, c = (n / kC) * VE;
    if (kParts & kLoadV)
      in.v[i] = r < Lrows ? __builtin_nontemporal_load(reinterpret_cast<const raw16*>(v + base_v + r * tokv + c)) : zero16;
  }
  if (kParts & kLoadBeta)
    in.beta = (tid < kC && tid < Lrows) ? beta[((size_t)b * T_len + t0 + tid) * H + h] : (TIn)0.f;
}

// 2^x for x given in fp64, rounded to fp32 with about one ulp of error
// whatever the size of x: x = n + f with n = floor(x) exact, 2^f by
// v_exp_f32 on f in [0, 1), then an exact scaling by 2^n (results below
// the fp32 range flush towards zero).
__device__ __forceinline__ float exp2_split(double x) {
  const double n = floor(x);
  const int ni = n < -400.0 ? -400 : (n > 400.0 ? 400 : (int)n);
  return ldexpf(exp2_fast((float)(x - n)), ni);
}

// Per-channel factors built from the chunk's block starts, fp32 rows of
// [kNBlk][DK]; Gamma_p(a) = Gamma at row 16a - 1 (0 for a = 0; Gamma_p(4) =
// Gamma_C at the chunk's last row), T_a = Gamma_p(a+1) - Gamma_p(a):
constexpr int kBlkF = 0;     // rows 0-3   e^{Gamma_p(a)}
constexpr int kBlkE = 4;     // rows 4-7   (unused: Khat is formed from the scan registers)
constexpr int kBlkD = 8;     // rows 8-13  e^{Gamma_p(a) - Gamma_p(b+1)}, off-diagonal
                             //            tiles (a, b) in kTileA/kTileB order 4..9
constexpr int kBlkDec = 14;  // row 14     e^{Gamma_C}
constexpr int kBlkM = 15;    // rows 15-18 e^{-T_a} (bounded decay only: <= e^80)
constexpr int kNBlk = 19;

// ---------------------------------------------------------------------------
// Intra-chunk work: one work-group (8 waves) per (b*h, chunk).
// G = Gamma - Gamma_p(a) for a row in 16-row block a (a sum of at most 16
// decays, kept in fp32; G <= 0 and G decreases along the block); everything
// else is a product of
//   KP = k e^{G},  QP = q e^{G},  KE = k e^{T_a - G}      (fp32, all three
// bounded by |k| or |q|: two exponentials per element) and per-channel
// factors of the block starts (BLK):
//   A, M tile (a, b), b < a: row operand KP or QP (block a), column operand
//                            KE * e^{Gamma_p(a) - Gamma_p(b+1)} (block b)
//   diagonal tile (a, a):    bounded decay (g >= -5): column operand
//                            KE * e^{-T_a} <= e^80 |k|, inside the bf16 range;
//                            unbounded decay (kUnb): position-pair sums
//                            sum_c k_rc k_sc e^{G_rc - G_sc} in fp32
//   Qbar = scale e^{Gamma_p(a)} QP,  Kbar = e^{Gamma_p(a)} KP,
//   Khat = e^{Gamma_C - Gamma_p(a+1)} KE
// LDS regions, reused across phases (lifetimes in brackets):
//   P0 : g, then G (fp32 [C][LG])                        [phase 0]
//        -> KP (fp32 [C][LG])                              [0 - 2b]
//   P1 : k, q (input type, [C][LK] each)                   [phase 0]
//        -> QP at 0, KE at PB (fp32 [C][LG] each)          [0 - 1]
//        -> Kbar^T (Op [DK][LB]) at 0, V^T (Op [DV][LB]) at KT   [2b - 3]
//   X  : (phase 0: diagonal A tiles where A goes; the block totals where X
//        goes), then A and X fp32 [C][LA]                  [1 - 2b]
//        -> Tm (Op [C][LB]) where A was                     [2b - 3]
//   BLK: fp32 [kNBlk][DK] per-channel factors                [0 - 2b]
//   MD : (kUnb) M's diagonal tiles by position pairs       [0 - 1]
// Phases: 0 stage inputs, block scans, exponentials, factors (kUnb: and the
// diagonal tiles by position pairs); Khat goes to the record straight from
// the scan registers (a thread holds 16 rows of one channel, four rows per
// record lane); 1 Gram tiles (A -> LDS, scale M -> record), then each wave
// that held a diagonal tile inverts that block of I + A while the others
// write Qbar and e^{Gamma_C} to the record; 2b Kbar^T and V^T staged,
// off-diagonal blocks of the inverse, Tm; 3 W = Tm Kbar, Ut = Tm V to the
// record.
// ---------------------------------------------------------------------------
template <typename TIn, int DK, int DV>
struct IntraLds {
  using Op = typename Policy<TIn>::Op;
  static constexpr int PI = 16 / sizeof(TIn), PO = 16 / sizeof(Op);
  static constexpr int LG = DK + 4;     // fp32 rows (G, KP, QP, KE)
  static constexpr int LK = DK + PI;    // k / q rows (input type)
  static constexpr int LB = kC + PO;    // channel-major Op rows (Kbar^T, V^T) and Tm rows
  static constexpr int LA = kC + 4;     // A / X rows (fp32)
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t r16(size_t a) { return (a + 15) / 16 * 16; }
  static constexpr size_t PB = (size_t)kC * LG * 4;                       // one fp32 [C][LG] array
  static constexpr size_t KIN = r16((size_t)kC * LK * sizeof(TIn));       // one staged input array
  static constexpr size_t KT = r16((size_t)DK * LB * sizeof(Op));         // Kbar^T
  static constexpr size_t P0 = 0;
  static constexpr size_t P1 = P0 + PB;
  static constexpr size_t P1_SIZE = mx(mx(2 * KIN, 2 * PB), KT + (size_t)DV * LB * sizeof(Op));
  static constexpr size_t X = P1 + P1_SIZE;
  static constexpr size_t X_SIZE = 2 * (size_t)kC * LA * 4;
  static constexpr size_t BLK = X + X_SIZE;
  static constexpr size_t BETA = BLK + (size_t)kNBlk * DK * 4;
  static constexpr size_t RED = BETA + kC * 4;
  static constexpr size_t MD = RED + 16 * 4;
  static constexpr size_t BYTES = MD + 4 * 256 * 4;
  static_assert((size_t)kC * LB * sizeof(Op) <= (size_t)kC * LA * 4, "Tm fits where A was");
  static_assert(4 * (size_t)DK * 4 <= (size_t)kC * LA * 4, "block totals fit in X");
};

// Small per-wave tables are packed into 64-bit immediates, 4 bits per
// entry, so a lookup with a wave-uniform index is scalar shifts.  (As
// __constant__ arrays, each lookup was a vector load followed by a wait for
// every outstanding vector access, the next chunk's input loads included.)
__device__ __forceinline__ int nib(unsigned long long tab, int i) { return (int)((tab >> (4 * i)) & 0xfu); }
// The 10 tiles (a, b) of the lower 4x4 block triangle: diagonal first.
//   a: 0 1 2 3 1 2 3 2 3 3     b: 0 1 2 3 0 0 0 1 1 2
constexpr unsigned long long kTileA = 0x3323213210ull;
constexpr unsigned long long kTileB = 0x2110003210ull;
// Gram tiles of wave w (-1: none): a diagonal tile (the costlier kind, with
// split operands) for waves 0-3; two off-diagonal tiles of one row block for
// waves 4 and 5 (they share the row operand); one for waves 6 and 7.
//   first tile: 0 1 2 3 5 6 4 9     second tile (15: none): - - - - 7 8 - -
constexpr unsigned long long kWaveTile0 = 0x94653210ull;
constexpr unsigned long long kWaveTile1 = 0xff87ffffull;

// Builds the record of the chunk of head (b, h) that starts at token t0 and
// has Lrows rows (1 .. 64; the rest of the 64-row tile is zero) at `rec`.  Called by a
// whole work-group of kThreads threads; `smem` holds IntraLds::BYTES.
// `in` holds the chunk's inputs (load_inputs).  `slot(step)` (step an
// std::integral_constant) is called by every thread: kSlotPeek once the
// inputs are staged, kSlotCheck before the barrier that ends phase 0 and
// kSlotOk after it; if that returns false nothing is written.  From then on `in` is free (v is read from it once
// more, before the last call): `prefetch(parts)` is called by every thread
// at four points of the later phases, with kLoadK | kLoadBeta, kLoadQ,
// kLoadG, kLoadV in turn (as std::integral_constant), e.g. to load the next
// chunk's inputs into `in` in portions while this one is computed.
// kLay: the layer steps (Layer) may be requested; without it their code is
// compiled out of the other kernels.
constexpr int kSlotPeek = 0, kSlotCheck = 1, kSlotOk = 2;

template <typename TIn, int DK, int DV, bool kUnb, bool kLay, typename Slot, typename Prefetch>
__device__ __forceinline__ bool produce_chunk(char* smem, InRegs<TIn, DK, DV>& in, const float* __restrict__ gcum,
                                              float scale, int b, int h, int T_len, int H, int t0, int Lrows,
                                              char* __restrict__ rec, Slot slot, Prefetch prefetch, Stamps& stp,
                                              Layer lay = Layer{nullptr, nullptr, 0}) {
  using P = Policy<TIn>;
  using Op = typename P::Op;
  using Gm = typename P::Gram;
  using L = IntraLds<TIn, DK, DV>;
  using R = Rec<TIn, DK, DV>;
  using IR = InRegs<TIn, DK, DV>;
  constexpr int VE = 16 / sizeof(TIn);   // input elements per 16-byte vector
  constexpr int NQT = (DK / 16) * 4;     // 16x16 tiles of a [C][DK] matrix
  constexpr int NQW = NQT / kNW;         // ... per wave
  float* sG = reinterpret_cast<float*>(smem + L::P0);     // g, G (phase 0)
  float* sKP = reinterpret_cast<float*>(smem + L::P0);
  TIn* sK = reinterpret_cast<TIn*>(smem + L::P1);         // phase 0
  TIn* sQ = reinterpret_cast<TIn*>(smem + L::P1 + L::KIN);
  float* sQP = reinterpret_cast<float*>(smem + L::P1);
  float* sKE = reinterpret_cast<float*>(smem + L::P1 + L::PB);
  Op* sKbt = reinterpret_cast<Op*>(smem + L::P1);          // phases 2b-3
  Op* sVt = reinterpret_cast<Op*>(smem + L::P1 + L::KT);
  float* sA = reinterpret_cast<float*>(smem + L::X);
  float* sX = sA + kC * L::LA;
  float* sMd = reinterpret_cast<float*>(smem + L::MD);    // [4][16][16], phase 0-1 (kUnb)
  float* sTot = sX;                                       // [4][DK], phase 0
  Op* sTm = reinterpret_cast<Op*>(smem + L::X);           // phases 2b-3
  float* sBeta = reinterpret_cast<float*>(smem + L::BETA);
  float* sBlk = reinterpret_cast<float*>(smem + L::BLK);
  float* sRed = reinterpret_cast<float*>(smem + L::RED);

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = 4 * (lane >> 4);
  const size_t tokk = (size_t)H * DK;
  const size_t base_k = ((size_t)b * T_len + t0) * tokk + (size_t)h * DK;
  // (no barrier here: a caller running several chunks in one work-group
  // passes a barrier between them, after the previous chunk's last LDS
  // access; the fused loop's hand-off has one)
  stp.mark<0>();   // producer slots: 0 entry, 1-8 phase work, 17-24 their barriers, 9 phase 3, 10 publish
  Op* rW = reinterpret_cast<Op*>(rec) + R::W;
  Op* rQ = reinterpret_cast<Op*>(rec) + R::Q;
  Op* rK = reinterpret_cast<Op*>(rec) + R::K;
  float* rDec = reinterpret_cast<float*>(rec + R::DEC_OFF_BYTES);
  Op* rM = reinterpret_cast<Op*>(rec) + R::M;
  Op* rU = reinterpret_cast<Op*>(rec + R::U_OFF_BYTES);
  float* rUinv = reinterpret_cast<float*>(rec + R::UINV_OFF_BYTES);

  // ---- phase 0: stage k, q, beta (and g) from the input registers
  const bool normqk = kLay && (lay.flags & kLayerNormQK) != 0;   // uniform
  const bool gatez = kLay && (lay.flags & kLayerGateZ) != 0;
  const float ea = gatez ? expf(lay.A[h]) : 0.f;   // exp(A), once per chunk
#pragma unroll
  for (int i = 0; i < IR::NK; ++i) {
    const int n = tid + kThreads * i;
    const int r = n / (DK / VE), c = (n % (DK / VE)) * VE;
    *reinterpret_cast<raw16*>(sK + r * L::LK + c) = normqk ? l2norm_part<TIn, DK / VE>(in.k[i]) : in.k[i];
    *reinterpret_cast<raw16*>(sQ + r * L::LK + c) = normqk ? l2norm_part<TIn, DK / VE>(in.q[i]) : in.q[i];
    if (!gcum) {
      float gv[VE];
#pragma unroll
      for (int x = 0; x < VE; ++x) {
        gv[x] = raw_elem<TIn>(in.g[i], x);
        // (rows past the end of the sequence keep g = 0: no decay there)
        if (gatez) gv[x] = r < Lrows ? kGateMin * sigmoid_fast(ea * gv[x]) : 0.f;
      }
#pragma unroll
      for (int x = 0; x < VE; x += 4)
        *reinterpret_cast<f32x4*>(sG + r * L::LG + c + x) = f32x4{gv[x], gv[x + 1], gv[x + 2], gv[x + 3]};
    }
  }
  if (tid < kC) sBeta[tid] = to_f32(in.beta);
  stp.mark<1>();
  __syncthreads();
  stp.mark<17>();
  slot(std::integral_constant<int, kSlotPeek>{});

  // Block scans: thread (block a, channel c) forms G for its 16 rows (local
  // sums in row order, or differences of the given cumulative sums), the two
  // exponentials and the products with its k and q.
  const bool scan = tid < 4 * DK;   // wave-uniform (4 DK is a multiple of 64)
  float kp[16], qp[16], ke[16];
  if (scan) {
    const int c = tid % DK, a = tid / DK;
    float x[16];
    if (gcum) {
      const int pr = min(16 * a - 1, Lrows - 1);
      const float g0 = pr >= 0 ? gcum[base_k + (size_t)pr * tokk + c] : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = gcum[base_k + (size_t)min(16 * a + i, Lrows - 1) * tokk + c] - g0;
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = sG[(16 * a + i) * L::LG + c];
#pragma unroll
      for (int i = 1; i < 16; ++i) x[i] += x[i - 1];
    }
    sTot[a * DK + c] = x[15];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (kUnb) sG[(16 * a + i) * L::LG + c] = x[i] * kLog2e;   // for the position pairs
      const float kv = to_f32(sK[(16 * a + i) * L::LK + c]), qv = to_f32(sQ[(16 * a + i) * L::LK + c]);
      const float ep = exp2_fast(x[i] * kLog2e), ee = exp2_fast((x[15] - x[i]) * kLog2e);
      kp[i] = kv * ep;
      qp[i] = qv * ep;
      ke[i] = kv * ee;
    }
  }
  slot(std::integral_constant<int, kSlotCheck>{});
  stp.mark<2>();
  __syncthreads();   // staged g read (kUnb: G written); block totals written
  stp.mark<18>();
  if (!slot(std::integral_constant<int, kSlotOk>{})) return false;
  if (kUnb) {
    // Diagonal tiles by position pairs, fp32: entry (i, j), j <= i, of tile
    // a is sum_c y_rc k_sc e^{G_rc - G_sc} (r = 16a + i, s = 16a + j, y = k
    // for A, q for M; the factor is <= 1 since G decreases along a block).
    // Wave w takes tile w / 2 and 8 of its rows, paired (i, 15 - i) so that
    // both waves of a tile have the same number of entries.  A goes where
    // A will be, scale M to the diagonal-tile area in X.
    const int a = w >> 1;
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const int e = lane + 64 * e2, slot = e >> 4, j = e & 15;
      const int pr = (w & 1) * 4 + (slot >> 1);
      const int i = (slot & 1) ? 15 - pr : pr;
      const int r = 16 * a + i, sc = 16 * a + j;
      float accA = 0.f, accM = 0.f;
      if (j <= i) {
        for (int c = 0; c < DK; c += 4) {
          const f32x4 ex = exp2v(*reinterpret_cast<const f32x4*>(sG + r * L::LG + c) -
                                 *reinterpret_cast<const f32x4*>(sG + sc * L::LG + c));
          const f32x4 ks = widen4(load4(sK + sc * L::LK + c)) * ex;
          const f32x4 kr = widen4(load4(sK + r * L::LK + c)), qr = widen4(load4(sQ + r * L::LK + c));
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            accA = fmaf(kr[u], ks[u], accA);
            accM = fmaf(qr[u], ks[u], accM);
          }
        }
      }
      sA[r * L::LA + sc] = j < i ? sBeta[r] * accA : 0.f;
      sMd[a * 256 + i * 16 + j] = j <= i ? accM * scale : 0.f;
    }
    __syncthreads();   // G, staged k and q read
  }
  if (scan) {
    const int c = tid % DK, a = tid / DK;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sKP[(16 * a + i) * L::LG + c] = kp[i];
      sQP[(16 * a + i) * L::LG + c] = qp[i];
      sKE[(16 * a + i) * L::LG + c] = ke[i];
    }
    // factors from the block starts, summed in fp64 (natural log units):
    // thread group a builds one kind of row
    double bs[5];
    if (gcum) {
#pragma unroll
      for (int j = 0; j < 5; ++j) {
        const int pr = min(j < 4 ? 16 * j - 1 : kC - 1, Lrows - 1);
        bs[j] = pr >= 0 ? (double)gcum[base_k + (size_t)pr * tokk + c] : 0.0;
      }
    } else {
      bs[0] = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) bs[j + 1] = bs[j] + (double)sTot[j * DK + c];
    }
    constexpr double l2e = 1.4426950408889634;
    {   // Khat rows of this thread's block and channel, straight to the record:
        // lane group g of tile (a, c / 16) holds rows 16a + 4g .. + 3
      const double bn = a == 0 ? bs[1] : (a == 1 ? bs[2] : (a == 2 ? bs[3] : bs[4]));   // Gamma_p(a + 1)
      const float e = exp2_split((bs[4] - bn) * l2e);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4<Op>(rK + tile_elem(tile_k<DK / 16>(a, c / 16), (c % 16) + 16 * g),
                   narrow4<Op>(f32x4{ke[4 * g] * e, ke[4 * g + 1] * e, ke[4 * g + 2] * e, ke[4 * g + 3] * e}));
    }
    if (a == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sBlk[(kBlkF + j) * DK + c] = exp2_split(bs[j] * l2e);
    } else if (a == 2) {
      const int ta[6] = {1, 2, 3, 2, 3, 3}, tb[6] = {0, 0, 0, 1, 1, 2};
#pragma unroll
      for (int j = 0; j < 6; ++j) sBlk[(kBlkD + j) * DK + c] = exp2_split((bs[ta[j]] - bs[tb[j] + 1]) * l2e);
    } else {
      sBlk[kBlkDec * DK + c] = exp2_split(bs[4] * l2e);
      // e^{-T_a} from the same fp32 totals as KE's exponents
#pragma unroll
      for (int j = 0; j < 4; ++j) sBlk[(kBlkM + j) * DK + c] = exp2_split(-(double)sTot[j * DK + c] * l2e);
    }
  }
  stp.mark<3>();
  __syncthreads();
  stp.mark<19>();
  prefetch(std::integral_constant<int, kLoadK | kLoadBeta>{});

  // ---- phase 1: Gram tiles (A -> LDS, scale M -> record)
  {
    const int t0i = nib(kWaveTile0, w), t1i1 = nib(kWaveTile1, w), t1i = t1i1 == 15 ? -1 : t1i1;
    const int ntile = t0i < 0 ? 0 : (t1i < 0 ? 1 : 2);   // wave-uniform
    if (kUnb && t0i >= 0 && t0i < 4) {
      // diagonal tile from the position pairs of phase 0: scale M to the record
      // (lane holds M[16a + l16][16a + g4 + i]); A is already in place
      const float* md = sMd + t0i * 256 + l16 * 16 + g4;
      store4<Op>(rM + tile_elem(tile_cr(t0i, t0i), lane), narrow4<Op>(f32x4{md[0], md[1], md[2], md[3]}));
    } else if (ntile > 0) {
      // both tiles of a wave share the row block a, hence the row operand
      const int a = nib(kTileA, t0i);
      const int bb0 = nib(kTileB, t0i), bb1 = ntile > 1 ? nib(kTileB, t1i) : bb0;
      const bool diag = a == bb0;   // only single-tile waves hold a diagonal tile
      const int r = 16 * a + l16, s0 = 16 * bb0 + l16, s1 = 16 * bb1 + l16;
      const float* d0p = sBlk + (diag ? kBlkM + a : kBlkD + t0i - 4) * DK;
      const float* d1p = sBlk + (kBlkD + (ntile > 1 ? t1i - 4 : 0)) * DK;
      f32x4 accA0 = zero4(), accM0 = zero4(), accA1 = zero4(), accM1 = zero4();
      // One straight-line slab loop per kind of wave (kind 0: the diagonal
      // tile with split operands for M, 1: one tile, 2: two tiles of the
      // same row block), chosen once, with the next slab's operands read
      // from LDS while the current slab's are converted and multiplied
      // (with the kind tested inside the loop every slab's reads waited for
      // the previous slab's products).
      auto tiles = [&](auto kind) {
        // the products KE x factor are rounded before they are split (no
        // contraction into the split's subtraction), the same arithmetic in
        // every instantiation
#pragma clang fp contract(off)
        constexpr int K = decltype(kind)::value, NR = K == 2 ? 12 : 8, NSL = DK / 32;
        auto ld = [&](const float* p) { return *reinterpret_cast<const f32x4*>(p); };
        // a slab's operands: KP and QP of row r, KE of rows s0 (and s1) with
        // their per-channel factors, each as the halves c0 and c1 = c0 + 16
        auto load = [&](int sl, f32x4 (&x)[NR]) {
          const int c0 = 32 * sl + g4, c1 = c0 + 16;
          x[0] = ld(sKP + r * L::LG + c0);
          x[1] = ld(sKP + r * L::LG + c1);
          x[2] = ld(sQP + r * L::LG + c0);
          x[3] = ld(sQP + r * L::LG + c1);
          x[4] = ld(sKE + s0 * L::LG + c0);
          x[5] = ld(sKE + s0 * L::LG + c1);
          x[6] = ld(d0p + c0);
          x[7] = ld(d0p + c1);
          if constexpr (K == 2) {
            x[8] = ld(sKE + s1 * L::LG + c0);
            x[9] = ld(sKE + s1 * L::LG + c1);
            x[10] = ld(d1p + c0);
            x[11] = ld(d1p + c1);
          }
        };
        f32x4 xb[2][NR];
        load(0, xb[0]);
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
          if (sl + 1 < NSL) load(sl + 1, xb[(sl + 1) & 1]);
          const f32x4(&x)[NR] = xb[sl & 1];
          const Slab<Gm> RK = make_slab<Gm>(x[0], x[1]);
          // column operand: KE times e^{-T_a} (diagonal) or e^{Gamma_p(a) - Gamma_p(b+1)}
          const f32x4 ck0 = x[4] * x[6], ck1 = x[5] * x[7];
          if constexpr (K == 0) {
            Slab<Gm> CKh, CKl, RQh, RQl;
            make_slab_split<Gm>(ck0, ck1, CKh, CKl);
            make_slab_split<Gm>(x[2], x[3], RQh, RQl);
            accA0 = mma(CKh, RK, accA0);
            accM0 = mma(CKh, RQh, accM0);
            accM0 = mma(CKl, RQh, accM0);
            accM0 = mma(CKh, RQl, accM0);
          } else {
            const Slab<Gm> RQ = make_slab<Gm>(x[2], x[3]);
            const Slab<Gm> CK = make_slab<Gm>(ck0, ck1);
            accA0 = mma(CK, RK, accA0);   // A^T tile: lane holds A[r][16bb + g4 + i]
            accM0 = mma(CK, RQ, accM0);   // M^T tile: lane holds M[r][16bb + g4 + i]
            if constexpr (K == 2) {
              const Slab<Gm> CK1 = make_slab<Gm>(x[8] * x[10], x[9] * x[11]);
              accA1 = mma(CK1, RK, accA1);
              accM1 = mma(CK1, RQ, accM1);
            }
          }
        }
      };
      if (P::kMixed && diag) tiles(std::integral_constant<int, 0>{});
      else if (ntile > 1) tiles(std::integral_constant<int, 2>{});
      else tiles(std::integral_constant<int, 1>{});
      const float br = sBeta[r];
      for (int ti = 0; ti < ntile; ++ti) {
        const int bb = ti ? bb1 : bb0;
        const f32x4 accA = ti ? accA1 : accA0, accM = ti ? accM1 : accM0;
        f32x4 arow, mrow;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int sc = 16 * bb + g4 + i;
          arow[i] = sc < r ? br * accA[i] : 0.f;
          mrow[i] = sc <= r ? accM[i] : 0.f;
        }
        *reinterpret_cast<f32x4*>(sA + r * L::LA + 16 * bb + g4) = arow;
        store4<Op>(rM + tile_elem(tile_cr(bb, a), lane), narrow4<Op>(mrow * scale));
      }
    }
  }
  if (w >= 2) {   // the six tiles above the diagonal of the record's M are zero
    // (the mirror of lower tile (a, b): row block b, column block a)
    const int zt = w - 2, kt = nib(kTileA, 4 + zt), rt = nib(kTileB, 4 + zt);
    store4<Op>(rM + tile_elem(tile_cr(kt, rt), lane), narrow4<Op>(zero4()));
  }
  if (w < 4) {
    // The wave that held diagonal tile (a, a) (or, kUnb, any wave a < 4:
    // the tiles were written in phase 0) inverts that block: X_aa =
    // (I + A_aa)^-1 by forward substitution, lane j % 16 = column j (lanes
    // of the same column compute the same values; those of lanes 0-15 are
    // stored).  Row by row: x_i = -sum_{m<i} A_im x_m for i != j (x_m = 0
    // for m < j), a 16-byte read of row i per four terms.  This wave wrote
    // the block (or it was complete at the last barrier): LDS accesses of
    // one wave are performed in order.
    const int a = w;
    const float* Ab = sA + 16 * a * L::LA + 16 * a;
    const int j = lane & 15;
    float x[16];
    x[0] = j == 0 ? 1.f : 0.f;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      float s = 0.f;
#pragma unroll
      for (int q4 = 0; 4 * q4 < i; ++q4) {
        const f32x4 ar = *reinterpret_cast<const f32x4*>(Ab + i * L::LA + 4 * q4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * q4 + e < i) s = fmaf(ar[e], x[4 * q4 + e], s);
      }
      x[i] = i == j ? 1.f : 0.f - s;
    }
    if (lane < 16) {
      float* Xb = sX + 16 * a * L::LA + 16 * a;
#pragma unroll
      for (int i = 0; i < 16; ++i) Xb[i * L::LA + j] = x[i];
    }
  } else {
    // Qbar tiles and e^{Gamma_C} to the record, by tile pairs (ct = 2c2,
    // 2c2 + 1; rt) that one 16-byte store per lane writes: waves 4 and 5
    // (two Gram tiles each) take NQT / 16 pairs, waves 6 and 7 (one)
    // 3 NQT / 16, in groups of up to two pairs whose operands are read
    // before their stores.
    auto qbar = [&](auto cnt, int m0) {
      constexpr int N = decltype(cnt)::value, NG = N % 2 == 0 ? 2 : N;
      static_assert(N % NG == 0, "groups");
#pragma unroll
      for (int g0 = 0; g0 < N; g0 += NG) {
        f32x4 qv[NG][2], fv[NG][2];
#pragma unroll
        for (int n = 0; n < NG; ++n) {
          const int m = m0 + g0 + n, c2 = m >> 2, rt = m & 3;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int ct = 2 * c2 + e;
            fv[n][e] = *reinterpret_cast<const f32x4*>(sBlk + (kBlkF + rt) * DK + 16 * ct + g4);
            qv[n][e] = *reinterpret_cast<const f32x4*>(sQP + (16 * rt + l16) * L::LG + 16 * ct + g4);
          }
        }
#pragma unroll
        for (int n = 0; n < NG; ++n) {
          const int m = m0 + g0 + n, c2 = m >> 2, rt = m & 3;
          store_pair<Op>(rQ + tile_elem(tile_cr(2 * c2, rt), lane), qv[n][0] * (fv[n][0] * scale),
                         qv[n][1] * (fv[n][1] * scale));
        }
      }
    };
    if (w < 6) qbar(std::integral_constant<int, NQT / 16>{}, (w - 4) * (NQT / 16));
    else qbar(std::integral_constant<int, 3 * NQT / 16>{}, NQT / 8 + (w - 6) * (3 * NQT / 16));
    if (tid >= 6 * 64 && tid < 6 * 64 + DK) rDec[tid - 6 * 64] = sBlk[kBlkDec * DK + tid - 6 * 64];
  }
  // V's range (for its fp16 staging): wave maxima of the chunk's v, combined
  // after the barrier
  float vmax = 0.f;
#pragma unroll
  for (int i = 0; i < IR::NV; ++i)
#pragma unroll
    for (int x = 0; x < VE; ++x) vmax = fmaxf(vmax, fabsf(raw_elem<TIn>(in.v[i], x)));
  vmax = wave_max_dpp(vmax);
  if (lane == 0) sRed[w] = vmax;
  prefetch(std::integral_constant<int, kLoadQ>{});
  stp.mark<4>();
  __syncthreads();   // A and the diagonal blocks of X complete; QP, KE dead
  stp.mark<20>();
  prefetch(std::integral_constant<int, kLoadG>{});

  // ---- phase 2b: Kbar^T and V^T (range-scaled) into P1, then the
  // off-diagonal blocks of X, then Tm = X Diag(beta) where A was
  float sv = 1.f;
  if (P::kMixed) {
    float m = sRed[0];
#pragma unroll
    for (int i = 1; i < kNW; ++i) m = fmaxf(m, sRed[i]);
    sv = fp16_range_scale(m);
  }
#pragma unroll
  for (int j = 0; j < NQW; ++j) {   // Kbar tile (ct, rt) staged transposed
    int ct, rt;
    wave_tile(w, j, NQW, ct, rt);
    const int row = 16 * rt + l16, col = 16 * ct + g4;
    const f32x4 f = *reinterpret_cast<const f32x4*>(sBlk + (kBlkF + rt) * DK + col);
    const V4<Op> kb = narrow4<Op>(*reinterpret_cast<const f32x4*>(sKP + row * L::LG + col) * f);
#pragma unroll
    for (int i = 0; i < 4; ++i) sKbt[(col + i) * L::LB + row] = kb[i];
  }
  constexpr int NVV = kC * DV / VE;
  {
    raw16 vreg[IR::NV];
#pragma unroll
    for (int i = 0; i < IR::NV; ++i) vreg[i] = in.v[i];
    prefetch(std::integral_constant<int, kLoadV>{});
#pragma unroll
    for (int i = 0; i < IR::NV; ++i) {   // consecutive lanes hold consecutive rows (see load_inputs)
      const int n = tid + kThreads * i;
      if (n < NVV) {
        const int r = n % kC, c = (n / kC) * VE;
#pragma unroll
        for (int x = 0; x < VE; ++x) sVt[(c + x) * L::LB + r] = from_f32<Op>(raw_elem<TIn>(vreg[i], x) * sv);
      }
    }
  }
  // off-diagonal blocks by distance d = a - b: X_ab = -X_aa sum_{c=b}^{a-1} A_ac X_cb
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int bb = w, a = w + d;
      f32x4 y = zero4();
      for (int c = bb; c < a; ++c)
        y = mma(load_half(sA + (16 * a + l16) * L::LA + 16 * c), load_half_col(sX + 16 * c * L::LA + 16 * bb, L::LA), y);
      const f32x4 xr = mma(load_half(sX + (16 * a + l16) * L::LA + 16 * a), Half<float>{y}, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) sX[(16 * a + g4 + i) * L::LA + 16 * bb + l16] = -xr[i];
    }
    if (d == 1) stp.mark<5>();
    else if (d == 2) stp.mark<6>();
    else stp.mark<7>();
    __syncthreads();
    if (d == 1) stp.mark<21>();
    else if (d == 2) stp.mark<22>();
    else stp.mark<23>();
  }
  static_assert(kC * kC == 8 * kThreads, "Tm: 8 entries per thread");
  {   // A is dead: Tm takes its place (8 consecutive entries of a row per thread)
    const int r = tid >> 3, s0 = (tid & 7) * 8;
    f32x4 x[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const f32x4 xv = *reinterpret_cast<const f32x4*>(sX + r * L::LA + s0 + 4 * h2);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(sBeta + s0 + 4 * h2);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[h2][i] = s0 + 4 * h2 + i <= r ? xv[i] * bv[i] : 0.f;
    }
    store4<Op>(sTm + r * L::LB + s0, narrow4<Op>(x[0]));
    store4<Op>(sTm + r * L::LB + s0 + 4, narrow4<Op>(x[1]));
  }
  stp.mark<8>();
  __syncthreads();   // Tm, Kbar^T, V^T complete
  stp.mark<24>();

  // ---- phase 3: W = Tm Kbar (as W^T tiles) and Ut = Tm V into the record
  // (the record holds -W)
  if constexpr (NQW == 4) {
    // tile pairs (ct = 2cp, 2cp + 1; rt), one 16-byte store per lane each:
    // wave w takes column pair w / 2 and row tiles {0, 3} (even w) or
    // {1, 2} (odd w), five 16-wide steps per column either way
    const int cp = w >> 1;
    auto wpair = [&](auto rtc) {
      constexpr int rt = decltype(rtc)::value;
      const f32x4 a0 = tri_mma(sKbt + (32 * cp + l16) * L::LB, sTm + (16 * rt + l16) * L::LB, rt + 1);
      const f32x4 a1 = tri_mma(sKbt + (32 * cp + 16 + l16) * L::LB, sTm + (16 * rt + l16) * L::LB, rt + 1);
      store_pair<Op>(rW + tile_elem(tile_cr(2 * cp, rt), lane), -a0, -a1);
    };
    if (w & 1) {
      wpair(std::integral_constant<int, 1>{});
      wpair(std::integral_constant<int, 2>{});
    } else {
      wpair(std::integral_constant<int, 0>{});
      wpair(std::integral_constant<int, 3>{});
    }
  } else {
#pragma unroll
    for (int j = 0; j < NQW; ++j) {   // W^T tile (ct, rt)
      int ct, rt;
      wave_tile(w, j, NQW, ct, rt);
      const f32x4 acc = tri_mma(sKbt + (16 * ct + l16) * L::LB, sTm + (16 * rt + l16) * L::LB, rt + 1);
      store4<Op>(rW + tile_elem(tile_cr(ct, rt), lane), narrow4<Op>(-acc));
    }
  }
  constexpr int NUT = (DV / 16) * 4;
  constexpr int NUW = NUT / kNW;
  f32x4 ut[NUW];
  float umax = 0.f;
#pragma unroll
  for (int j = 0; j < NUW; ++j) {   // Ut tile (st, jt)
    int jt, st;
    wave_tile(w, j, NUW, jt, st);
    ut[j] = tri_mma(sTm + (16 * st + l16) * L::LB, sVt + (16 * jt + l16) * L::LB, st + 1) * (1.f / sv);
    umax = fmaxf(umax, absmax4(ut[j]));
  }
  // Ut into the record as Op, range-scaled by su (exact power of two)
  float su = 1.f, suinv = 1.f;
  if (P::kMixed) fp16_range_scale2(block_max(umax, sRed + 8), su, suinv);
  if constexpr (NUW == 4) {   // wave w holds tiles 4w .. 4w + 3: two pairs
#pragma unroll
    for (int j = 0; j < 4; j += 2) store_pair<Op>(rU + tile_elem(4 * w + j, lane), ut[j] * su, ut[j + 1] * su);
  } else {
#pragma unroll
    for (int j = 0; j < NUW; ++j) {
      int jt, st;
      wave_tile(w, j, NUW, jt, st);
      store4<Op>(rU + tile_elem(jt * 4 + st, lane), narrow4<Op>(ut[j] * su));
    }
  }
  if (tid == 0) *rUinv = suinv;
  stp.mark<9>();
  return true;
}

// Two-stage schedule, stage 1: one work-group per (b*h, chunk), records for
// every chunk of every head in the workspace.  kUnb: decay not bounded below
// (diagonal tiles by position pairs).
template <typename TIn, int DK, int DV, bool kUnb>
__global__ __launch_bounds__(kThreads) void intra_chunk_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                               const TIn* __restrict__ v, const TIn* __restrict__ g,
                                                               const float* __restrict__ gcum,
                                                               const TIn* __restrict__ beta, float scale,
                                                               char* __restrict__ ws, int T_len, int H, int nchunks) {
  __shared__ __align__(16) char smem[IntraLds<TIn, DK, DV>::BYTES];
  const int ch = blockIdx.x % nchunks, bh = blockIdx.x / nchunks;
  InRegs<TIn, DK, DV> in;
  const int t0 = ch * kC, rows = min(kC, T_len - t0);
  load_inputs<TIn, DK, DV>(in, q, k, v, g, beta, bh / H, bh % H, T_len, H, t0, rows);
  Stamps stp;
  produce_chunk<TIn, DK, DV, kUnb, false>(smem, in, gcum, scale, bh / H, bh % H, T_len, H, t0, rows,
                                   ws + ((size_t)bh * nchunks + ch) * Rec<TIn, DK, DV>::BYTES, [](auto) { return true; },
                                   [](auto) {}, stp);
}

// ---------------------------------------------------------------------------
// State pass over one head's chunks.  Waves 0..3 (one per SIMD) own the
// value columns: wave w keeps the dk x 16 slice of S it owns in fp32
// accumulators for the whole sequence; waves 4..7 stage the records: each
// chunk's record is copied into LDS once, and the next chunk's copy is
// prefetched into their registers while the owners compute the current one.
// Operand slabs are lane-interleaved in the record (tile_elem), so every
// slab is one 16-byte LDS read.  When two records do not fit in LDS (fp32
// inputs), one buffer is staged between two barriers.
//
// kRing = false: records of every chunk are stored one after another at
//   recbase (two-stage schedule).
// kRing = true : chunk c is in slot c % R of a ring at recbase, published by a
//   producer work-group through ready[c % R] = ((c + 1) << 4) | (producer's
//   XCD); after the chunk has been read, done[0] = c + 1 hands the slot back.
// ---------------------------------------------------------------------------
struct Ring {
  int* ready;   // this head's R slot flags
  int* done;    // this consumer's progress counter
  int* err;     // set on a wait that exceeded its bound
  int* cxcc;    // this consumer's XCD + 1, published at its start
  int R;
};

constexpr int kSpinLimit = 1 << 20;   // about a second of polling before giving up

// Position of stream chunk c of a head: first token, rows, sequence and the
// chunk's index within it.  Without packed sequences (var->n == 0) chunk c
// is tokens 64c .. of the one sequence; with them, sequence i owns stream
// chunks cc[i] .. cc[i+1]-1.  Callers visit chunks in increasing order and
// keep `seq` between calls (start at 0): it only moves forward, past the
// sequences that end at or before c (empty ones included), so a sequence
// change costs a few scalar loads and the usual call none beyond one.
struct ChunkPos {
  int t0, rows, seq, j;
};
__device__ __forceinline__ ChunkPos chunk_pos(const VarSeg* var, int c, int T_len, int& seq) {
  if (var == nullptr || var->n == 0) return ChunkPos{c * kC, min(kC, T_len - c * kC), 0, c};
  while (seq + 1 < var->n && var->cc[seq + 1] <= c) ++seq;
  const int j = c - var->cc[seq], t0 = var->cu[seq] + j * kC;
  return ChunkPos{t0, min(kC, var->cu[seq + 1] - t0), seq, j};
}
constexpr int kFlagBase = 32;         // first flag word of the fused schedule's control block
constexpr int kFlagLine = 32;         // ints per 128-byte cache line

// The XCD (accelerator complex die, each with its own L2) this wave runs on.
__device__ __forceinline__ int xcc_id() { return __builtin_amdgcn_s_getreg((15 << 11) | 20) & 0xf; }

// A flag word read from this XCD's L2 (the load misses the CU's L1: sc0).
// Sees every store that has reached this L2, i.e. stores made by work-groups
// on the same XCD; a device-scope load (sc1) may go out to memory instead,
// which costs a fabric round trip.
__device__ __forceinline__ int load_flag_l2(const int* p) {
  int v;
  asm volatile("global_load_dword %0, %1, off sc0\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}

// Polls *p until it is >= target and returns the value seen.  Executed by
// every lane of one whole wave: all lanes load the same word and the loop
// condition goes through readfirstlane, so the loop is wave-uniform (no
// lane-divergent loop inside code that also holds barriers).  Polls read
// this XCD's L2; every 4th poll is a device-scope load (the writer may run
// on another XCD), and every 64th checks the error word.  kSleep: pause between polls
// (units of 64 cycles).  Returns -1 after kSpinLimit polls, or as soon as
// another work-group reported an error; sets *err on a timeout.
template <int kSleep = 2>
__device__ __forceinline__ int spin_until_geq(const int* p, int target, int* err) {
  for (int it = 0; it < kSpinLimit; ++it) {
    const bool dev = (it & 3) == 3;
    const int v = __builtin_amdgcn_readfirstlane(dev ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                                     : load_flag_l2(p));
    if (v >= target) return v;
    if ((it & 63) == 63) {
      const int e = __builtin_amdgcn_readfirstlane(__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (e != 0) return -1;
    }
    __builtin_amdgcn_s_sleep(kSleep);
  }
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return -1;
}

// Waits until every vector memory access this wave issued has completed
// (stores acknowledged by the L2, loads returned); also a compiler barrier.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Buffer resource word 3 for raw dword access on gfx950, and the cache
// policy bit sc0 of a buffer load (served by this XCD's L2, not the CU's L1).
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kCachePolicySc0 = 1;

constexpr size_t kLdsMax = 160 * 1024;
constexpr int kOwners = 4;   // waves that own value columns, 16 each

// The state pass of one head runs on NS work-groups (value-column blocks
// of dv / NS = 64 columns), each staging the record's shared part (W, Qbar,
// Khat, M, dec, uinv), its own Ut columns and (output gate) the chunk's og
// rows of its columns.  LDS: NBUF such buffers (two when they fit, so that
// the next chunk is staged while the current one is computed) + abort word.
template <typename TIn, int DK, int DV>
struct ConsumerLds {
  using R = Rec<TIn, DK, DV>;
  using Op = typename Policy<TIn>::Op;
  static constexpr int NS = DV / (16 * kOwners);
  static constexpr size_t SH = R::U_OFF_BYTES;
  static constexpr size_t UPART = (size_t)kC * (DV / NS) * sizeof(Op);
  static constexpr size_t USED = SH + UPART;
  static constexpr size_t OG_OFF = USED;                              // og [kC][DV / NS] of TIn
  static constexpr size_t OGB = (size_t)kC * (DV / NS) * sizeof(TIn);
  static constexpr size_t BUF = (USED + OGB + 255) / 256 * 256;
  static constexpr int NBUF = 2 * BUF + 16 <= kLdsMax ? 2 : 1;
  static constexpr size_t BYTES = NBUF * BUF + 16;
  static_assert(NS * 16 * kOwners == DV, "dv must be 64 or 128");
  static_assert(BUF + 16 <= kLdsMax, "record does not fit in LDS");
  static_assert(SH % 16 == 0 && UPART % 16 == 0 && OGB % 16 == 0, "16-byte staging");
};

// The state pass's fp16 domain: Sh = sigma S and Uh = sigma U with sigma a
// power of two.  kFp16Safe bounds what converts to fp16 without overflow.
constexpr float kFp16Safe = 65000.f;
// Exponent k with m * 2^k in [2^12, 2^13) for finite m > 0; 0 otherwise.
__device__ __forceinline__ int fp16_domain_exp(float m) {
  const int ex = (int)((__float_as_uint(m) >> 23) & 0xffu);
  if (!(m > 0.f) || ex == 0xff) return 0;
  const int k = 12 - (ex - 127);
  return k < -100 ? -100 : (k > 100 ? 100 : k);
}
// Exponent step moving a domain maximum m into [2^12, 2^13), limited so that
// sigma = 2^se stays within 2^-120 .. 2^120 (a state that has decayed to
// nothing keeps its last sigma).
__device__ __forceinline__ int domain_rescale_exp(float m, int se) {
  const int k = fp16_domain_exp(m);
  return (se + k > 120 || se + k < -120) ? 0 : k;
}

// One lane's slab of 8 reduction indices, stored contiguously (tile_elem).
template <typename T> __device__ __forceinline__ Slab<T> load_slab8(const T* p);
template <> __device__ __forceinline__ Slab<f16> load_slab8<f16>(const f16* p) {
  return Slab<f16>{*reinterpret_cast<const f16x8*>(p)};
}
template <> __device__ __forceinline__ Slab<float> load_slab8<float>(const float* p) {
  return Slab<float>{load4(p), load4(p + 4)};
}

// Prefix-state snapshots: with p != nullptr and every > 0, the state after
// chunk c (c + 1 a multiple of `every`, and not the sequence's end, which
// is ht) is written to p + ((c + 1) / every - 1) * nbh * dk * dv + bh * dk * dv
// ([snapshot][b * H + h][dk][dv], fp32).
struct Snap {
  float* p;
  int every;
  int nbh;
};

// kLay: the output gate may be requested; kSeg: snapshots and packed
// sequences may be requested (each compiled out otherwise).  cbase: the
// ring's chunk count before this head (a ring serves the heads of several
// rounds in turn; its flags and progress count on across them).  Returns
// false if the chain stopped early (a hand-off wait gave up).
template <typename TIn, int DK, int DV, bool kRing, bool kLay, bool kSeg>
__device__ __forceinline__ bool consume_chain(char* smem, const char* __restrict__ recbase, Ring ring, int vb,
                                              const float* __restrict__ h0, float* __restrict__ ht,
                                              float* __restrict__ o, int b, int h, int T_len, int H,
                                              int nchunks, int cbase, Snap snap, Stamps& stp,
                                              Layer lay = Layer{nullptr, nullptr, 0}, const VarSeg* var = nullptr) {
  using P = Policy<TIn>;
  using Op = typename P::Op;
  using R = Rec<TIn, DK, DV>;
  using CL = ConsumerLds<TIn, DK, DV>;
  constexpr int NBUF = CL::NBUF;
  constexpr int NCT = DK / 16;
  constexpr int NV16 = CL::USED / 16;
  constexpr int NSH16 = CL::SH / 16;
  constexpr int kHelpers = kThreads - 64 * kOwners;   // threads of the staging waves
  constexpr int PPT = (NV16 + kHelpers - 1) / kHelpers;
  int* sAbort = reinterpret_cast<int*>(smem + NBUF * CL::BUF);

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = 4 * (lane >> 4);
  const bool owner = w < kOwners;   // wave-uniform
  const int jl0 = owner ? w : 0;                   // local column tile
  const int jt0 = vb * kOwners + jl0;              // column tile of the head
  const size_t bh = (size_t)b * H + h;
  auto rec_of = [&](int c) { return recbase + (size_t)(kRing ? (cbase + c) % ring.R : c) * R::BYTES; };
  auto buf_of = [&](int c) { return smem + (size_t)(NBUF == 2 ? (c & 1) : 0) * CL::BUF; };

  // A producer on this XCD wrote the chunk into the L2 this work-group
  // reads through, so only the CU's L1 may hold stale lines of the slot: an
  // L1 invalidate suffices.  Otherwise an agent-scope acquire.
  const int my_xcc = xcc_id();
  if (kRing && tid == 0) __hip_atomic_store(ring.cxcc, my_xcc + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) *sAbort = 0;
  __syncthreads();   // B0

  // Owners and staging waves run separate loops (so that their registers
  // are allocated separately) with the same barriers per chunk c:
  //   X_c  chunk c is staged in its buffer; every wave then reads the abort
  //        word and leaves if it is set
  //   Y_c  (one buffer only) the owners are done with chunk c
  // With two buffers, chunk c + 1 is staged into the other buffer while the
  // owners compute chunk c: the owners passed X_c only after finishing chunk
  // c - 1, the buffer's previous content.  Each staging wave polls the ring
  // by itself (a wave-uniform bounded spin) and sets the abort word before
  // the next X if the wait failed; the word is only ever set, so every wave
  // sees the same verdict after X.
  if (!owner) {
    const int htid = tid - 64 * kOwners;
    raw16 pre[PPT];
    // output gate rows of the chunk (kLay with og): [kC][DV / NS] of TIn,
    // OPT 16-byte pieces per thread, read once (non-temporal)
    constexpr int ROWP = (DV / CL::NS) * (int)sizeof(TIn) / 16, OPT = (int)(CL::OGB / 16) / kHelpers;
    static_assert(OPT * kHelpers * 16 == (int)CL::OGB, "og staging");
    raw16 ogp[OPT];
    const bool gate = kLay && lay.og != nullptr;   // uniform
    bool ok = true;
    // true once chunk c is published and may be read.  `seen` is chunk c's
    // ready word as read one chunk earlier (device scope: an L2 copy of the
    // word can lag behind the producer's agent-scope store); if it already
    // shows the chunk, there is no polling at all.
    auto ready_wait = [&](int c, int seen) -> bool {
      if (!kRing) return true;
      const int cg = cbase + c;
      const int v = seen >= ((cg + 1) << 4) ? seen : spin_until_geq(ring.ready + cg % ring.R, (cg + 1) << 4, ring.err);
      if (v < 0) return false;
      if ((v & 15) == my_xcc) asm volatile("buffer_inv sc0" ::: "memory");
      else __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return true;
    };
    auto peek = [&](int c) -> int {   // chunk c's ready word, read now, used a chunk later
      return (kRing && c < nchunks)
                 ? __hip_atomic_load(ring.ready + (cbase + c) % ring.R, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                 : 0;
    };
    // staged vector n: the shared part, then this work-group's Ut columns
    const int uoff16 = (int)((R::U_OFF_BYTES + (size_t)vb * CL::UPART) / 16) - NSH16;
    // With two buffers the record goes straight from memory into chunk c's
    // LDS buffer (16-byte direct-to-LDS loads: lane l of a wave's load
    // writes 16 bytes at the wave's base + 16 l; lanes that are switched off
    // write nothing), so the staging waves hold no record in registers and
    // issue no LDS writes for it; with one buffer it waits in registers for
    // the owners to finish the chunk before.
    auto load = [&](int c) {
      const raw16* rec = reinterpret_cast<const raw16*>(rec_of(c));
      if constexpr (NBUF == 2) {
        raw16* buf = reinterpret_cast<raw16*>(buf_of(c)) + (htid & ~63);
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
          const int n = htid + kHelpers * i;
          if (n < NV16) __builtin_amdgcn_global_load_lds(rec + (n < NSH16 ? n : n + uoff16), buf + kHelpers * i, 16, 0, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
          const int n = htid + kHelpers * i;
          if (n < NV16) pre[i] = rec[n < NSH16 ? n : n + uoff16];
        }
      }
      if (gate) {   // chunk c starts at token 64 c (the layer variant takes no packed sequences)
        const TIn* og = reinterpret_cast<const TIn*>(lay.og);
#pragma unroll
        for (int i = 0; i < OPT; ++i) {
          const int pc = htid + kHelpers * i, row = pc / ROWP, col = (pc % ROWP) * (16 / (int)sizeof(TIn));
          const int tr = c * kC + row;
          ogp[i] = tr < T_len ? __builtin_nontemporal_load(reinterpret_cast<const raw16*>(
                                    og + (((size_t)b * T_len + tr) * H + h) * DV + vb * (DV / CL::NS) + col))
                              : raw16{0.f, 0.f, 0.f, 0.f};
        }
      }
    };
    auto stage = [&](int c) {
      char* buf = buf_of(c);
      if constexpr (NBUF != 2) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
          const int n = htid + kHelpers * i;
          if (n < NV16) reinterpret_cast<raw16*>(buf)[n] = pre[i];
        }
      }
      if (gate) {
#pragma unroll
        for (int i = 0; i < OPT; ++i) reinterpret_cast<raw16*>(buf + CL::OG_OFF)[htid + kHelpers * i] = ogp[i];
      }
      // every load of chunk c has returned its data (and the direct-to-LDS
      // loads have written it) before the next X, where the owners start
      // reading it and its slot is handed back
      wait_vmem();
    };
    ok = ready_wait(0, 0);
    int seen_next = peek(1);
    if (ok) {
      load(0);
      stage(0);
    } else if (lane == 0) {
      *sAbort = 1;
    }
    // staging slots: 0 loop top, 1 barrier X, 2 abort word, progress
    // store and peek, 3 ready wait, 4 load issue, 5 stage (loads' wait, LDS writes)
    stp.add<kStampRole>(3);
    for (int c = 0; c < nchunks; ++c) {
      stp.mark<0>();
      __syncthreads();   // X_c
      stp.mark<1>();
      if (__builtin_amdgcn_readfirstlane(*sAbort)) return false;
      // chunk c has been read completely: hand its slot back
      if (kRing && htid == 0)
        __hip_atomic_store(ring.done, cbase + c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int seen = __builtin_amdgcn_readfirstlane(seen_next);
      seen_next = peek(c + 2);
      stp.mark<2>();
      if (c + 1 < nchunks) {
        ok = ready_wait(c + 1, seen);
        stp.mark<3>();
        if (ok) load(c + 1);
        else if (lane == 0) *sAbort = 1;
        stp.mark<4>();
        if (NBUF == 1) __syncthreads();   // Y_c
        if (ok) stage(c + 1);
        stp.mark<5>();
      } else if (NBUF == 1) {
        __syncthreads();   // Y_c
      }
      stp.add<kStampCount>(1);
    }
    return true;
  }

  // Packed sequences (extended variant): the state restarts at every
  // sequence's first chunk from its own h0 and is written to its own ht
  // after its last.
  const bool packed = kSeg && var != nullptr && var->n > 0;   // uniform
  // S from h0 (one wave-uniform branch around unconditional loads), used
  // before the loop, so that no wait inside the loop is tied to its loads
  f32x4 S[NCT];
  const size_t sbase = bh * DK * DV;
  auto load_state = [&](const float* src) {   // src: this (b, h)'s dk x dv state, or null
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) S[ct] = zero4();
    if (src) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[ct][i] = src[(size_t)(16 * ct + g4 + i) * DV + 16 * jt0 + l16];
    }
  };
  float m0 = 0.f;
  if (!packed) {
    load_state(h0 ? h0 + sbase : nullptr);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) m0 = absmax_acc(m0, S[ct]);
    m0 = wave_max_dpp(m0);
  }

  // O of the chunk at tokens t0 .. t0 + rows - 1, as 16-byte non-temporal
  // vectors (written once, not re-read)
  auto store_out = [&](int t0, int rows, const f32x4 (&Ov)[4]) {
    float* orow = o + (((size_t)b * T_len + t0 + l16) * H + h) * DV + 16 * jt0 + g4;
    const size_t ors = (size_t)16 * H * DV;   // 16 rows
    const bool full = rows == kC;             // uniform; only a sequence's last chunk is partial
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
      if (full || 16 * rt + l16 < rows) __builtin_nontemporal_store(Ov[rt], reinterpret_cast<f32x4*>(orow + rt * ors));
  };

  const bool mixed = P::kMixed;
  // sigma = 2^sig_e: the owner holds Sh = sigma S.  Sigma is chosen at every
  // chunk from the state alone (its maximum moved into [2^12, 2^13)), so a
  // run split into several calls at chunk boundaries does the same
  // arithmetic as one call.
  int sig_e = 0;
  // Packed sequences: the current sequence's stream chunks [c_beg, c_end)
  // and tokens [t_beg, t_end) stay in registers; the sequence table is read
  // when a sequence starts.  snap_left: chunks to the sequence's next
  // snapshot.  (Reading the table, and dividing for the snapshot test, at
  // every chunk cost the state pass 10%.)
  int seq = -1, c_beg = 0, c_end = 0, t_beg = 0, t_end = 0;
  int snap_left = snap.every;
  // The products run in the sigma domain (bf16 mode): Sh = sigma S and
  // Uh = sigma U are fp16 operands as they are (fp16 has the same relative
  // precision at every normal magnitude; sigma keeps the largest values in
  // range), and the record holds -W, so the MFMAs accumulating onto sigma
  // Ut give Uh directly.  A chunk's sigma and fp16 Sh depend on the state
  // alone, so they are formed at the end of the chunk before (ahead of the
  // barrier the owners then wait at), and here for the first chunk.
  float sig = 1.f, isig = 1.f;
  V4<Op> Sb[NCT];
  auto prepare_state = [&]() {
    if (mixed) {
      const int k = domain_rescale_exp(m0, sig_e);
      if (k != 0) {
        const float f = ldexpf(1.f, k);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) S[ct] = S[ct] * f;
        sig_e += k;
      }
    }
    sig = ldexpf(1.f, sig_e);
    isig = ldexpf(1.f, -sig_e);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) Sb[ct] = narrow4<Op>(S[ct]);
  };
  if (!packed) prepare_state();
  // owner slots: 0 loop top, 1 barrier X, 2 abort word, 3 the U
  // accumulators, 4 U and Qbar products issued, 5 Khat/M/decay reads and the
  // U range, 6 state update, output and stores, 7 snapshots and the next
  // chunk's sigma and Sh
  stp.add<kStampRole>(2);
  for (int c = 0; c < nchunks; ++c) {
    stp.mark<0>();
    __syncthreads();   // X_c
    stp.mark<1>();
    if (__builtin_amdgcn_readfirstlane(*sAbort)) return false;
    stp.mark<2>();
    const char* buf = buf_of(c);
    const Op* sW = reinterpret_cast<const Op*>(buf) + R::W;
    const Op* sQ = reinterpret_cast<const Op*>(buf) + R::Q;
    const Op* sK = reinterpret_cast<const Op*>(buf) + R::K;
    const Op* sM = reinterpret_cast<const Op*>(buf) + R::M;
    const float* sDec = reinterpret_cast<const float*>(buf + R::DEC_OFF_BYTES);
    const float uinv = *reinterpret_cast<const float*>(buf + R::UINV_OFF_BYTES);
    const Op* sU = reinterpret_cast<const Op*>(buf + CL::SH);   // local column tiles, 4 jl + st
    if (packed && c >= c_end) {   // a sequence starts: its range, its own initial state, sigma from it
      do {
        ++seq;
        c_beg = var->cc[seq];
        c_end = var->cc[seq + 1];
      } while (c >= c_end);   // (past empty sequences)
      t_beg = var->cu[seq];
      t_end = var->cu[seq + 1];
      snap_left = snap.every;
      load_state(h0 ? h0 + ((size_t)seq * H + h) * DK * DV : nullptr);
      m0 = 0.f;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) m0 = absmax_acc(m0, S[ct]);
      m0 = wave_max_dpp(m0);
      sig_e = 0;
      prepare_state();
    }
    const int j = packed ? c - c_beg : c;                        // chunk of the sequence
    const int t0 = packed ? t_beg + j * kC : c * kC;
    const int rows = min(kC, (packed ? t_end : T_len) - t0);
    const bool seq_last = packed ? c + 1 == c_end : (c + 1) * kC >= T_len;   // uniform

    // Uh = sigma Ut - W Sh and the Qbar Sh part of O, row block by row
    // block (both need only Sh); O^T = Sh^T Qbar^T + Uh^T (scale M)^T:
    // lane l holds row 16rt + l%16, columns 16jt + 4(l/16) .. +3.
    const float cu = sig * uinv;
    f32x4 Uh[4], accO[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      Uh[st] = widen4(load4(sU + tile_elem(jl0 * 4 + st, lane))) * cu;
      accO[st] = zero4();
    }
    stp.mark<3>();
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      Slab<Op> Wa[DK / 32], Qa[DK / 32];
#pragma unroll
      for (int sl = 0; sl < DK / 32; ++sl) {
        Wa[sl] = load_slab8<Op>(sW + tile_elem(tile_cr(2 * sl, st), lane));
        Qa[sl] = load_slab8<Op>(sQ + tile_elem(tile_cr(2 * sl, st), lane));
      }
#pragma unroll
      for (int sl = 0; sl < DK / 32; ++sl) {
        const Slab<Op> sb = slab_of<Op>(Sb[2 * sl], Sb[2 * sl + 1]);
        Uh[st] = mma(Wa[sl], sb, Uh[st]);
        accO[st] = mma(sb, Qa[sl], accO[st]);
      }
    }
    stp.mark<4>();
    // Khat, M and e^{Gamma_C} for the rest of the chunk, read while the
    // products above run (the owner has the registers to spare)
    Slab<Op> Ka[NCT][2], Ma[6];
    f32x4 dv[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) Ka[ct][sl] = load_slab8<Op>(sK + tile_elem(tile_k<NCT>(2 * sl, ct), lane));
      dv[ct] = *reinterpret_cast<const f32x4*>(sDec + 16 * ct + g4);
    }
#pragma unroll
    for (int rt = 0, m = 0; rt < 4; ++rt)
#pragma unroll
      for (int sl = 0; sl < (rt < 2 ? 1 : 2); ++sl, ++m) Ma[m] = load_slab8<Op>(sM + tile_elem(tile_cr(2 * sl, rt), lane));
    // Uh must fit fp16.  It does unless U is more than 8x larger than S
    // (or the input holds inf/NaN): then Uh is scaled into range by a power
    // of two r (wave-uniform branch).
    float umax = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st) umax = absmax_acc(umax, Uh[st]);
    int re = 0;
    if (mixed) {
      umax = wave_max_dpp(umax);
      if (!(umax <= kFp16Safe)) re = fp16_domain_exp(umax);
    }
    const float r = ldexpf(1.f, re), ir = ldexpf(1.f, -re);
    stp.mark<5>();
    // The rest of the chunk, one straight-line block per case (so that the
    // output work and stores can be scheduled into the gaps of the state
    // update's products).  Sh <- e^{Gamma_C} Sh + Khat^T Uh: MFMAs
    // accumulating onto the decayed state; the (scale M) Uh part of O onto
    // the Qbar Sh part.  With Uh scaled by r, both are unscaled in fp32.
    auto tail = [&](auto kScaled) {
      constexpr bool scl = decltype(kScaled)::value;
      V4<Op> Ub[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) Ub[st] = narrow4<Op>(scl ? Uh[st] * r : Uh[st]);
      f32x4 accS[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) accS[ct] = scl ? S[ct] * dv[ct] * r : S[ct] * dv[ct];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) accS[ct] = mma(Ka[ct][sl], slab_of<Op>(Ub[2 * sl], Ub[2 * sl + 1]), accS[ct]);
      f32x4 Ov[4];
#pragma unroll
      for (int rt = 0, m = 0; rt < 4; ++rt) {
        const int nms = rt < 2 ? 1 : 2;   // slabs of M's row block rt that are not all zero
        f32x4 am = scl ? zero4() : accO[rt];
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
          if (sl < nms) am = mma(slab_of<Op>(Ub[2 * sl], Ub[2 * sl + 1]), Ma[m + sl], am);
        m += nms;
        Ov[rt] = (scl ? accO[rt] + am * ir : am) * isig;
      }
      if (kLay && lay.og) {   // output gate: o <- Sigmoid(og) o, og rows staged with the record
        const TIn* sOg = reinterpret_cast<const TIn*>(buf + CL::OG_OFF);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const f32x4 gz = widen4(load4(sOg + (16 * rt + l16) * (DV / CL::NS) + 16 * jl0 + g4));
#pragma unroll
          for (int i = 0; i < 4; ++i) Ov[rt][i] *= sigmoid_fast(gz[i]);
        }
      }
      store_out(t0, rows, Ov);
      float smax = 0.f;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        S[ct] = scl ? accS[ct] * ir : accS[ct];
        smax = absmax_acc(smax, S[ct]);
      }
      m0 = mixed ? wave_max_dpp(smax) : 0.f;   // the next chunk's sigma comes from it
    };
    if (__builtin_amdgcn_readfirstlane(re)) tail(std::true_type{});
    else tail(std::false_type{});
    stp.mark<6>();
    if (kSeg && snap.p && snap.every > 0 && --snap_left == 0) {
      snap_left = snap.every;
      if (!seq_last) {   // the state after chunk j of the sequence, (j + 1) a multiple of every
        const int si = (packed ? var->sb[seq] : 0) + (j + 1) / snap.every - 1;
        float* sp = snap.p + ((size_t)si * snap.nbh + bh) * DK * DV;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) sp[(size_t)(16 * ct + g4 + i) * DV + 16 * jt0 + l16] = S[ct][i] * isig;
      }
    }
    if (packed && seq_last && ht) {   // the sequence's final state
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ht[((size_t)seq * H + h) * DK * DV + (size_t)(16 * ct + g4 + i) * DV + 16 * jt0 + l16] = S[ct][i] * isig;
    }
    // the next chunk's sigma and Sh (a sequence's first chunk forms its own;
    // none after the last chunk, whose state goes out as it is)
    if (c + 1 < nchunks && !(packed && seq_last)) prepare_state();
    stp.mark<7>();
    stp.add<kStampCount>(1);
    if (NBUF == 1) __syncthreads();   // Y_c
  }

  if (ht && !packed) {
    const float isig = ldexpf(1.f, -sig_e);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) ht[sbase + (size_t)(16 * ct + g4 + i) * DV + 16 * jt0 + l16] = S[ct][i] * isig;
  }
  return true;
}

// Two-stage schedule, stage 2: NS work-groups per head.
template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(kThreads) void state_pass_kernel(const char* __restrict__ ws,
                                                              const float* __restrict__ h0, float* __restrict__ ht,
                                                              float* __restrict__ o, int T_len, int H, int nchunks,
                                                              Snap snap) {
  using CL = ConsumerLds<TIn, DK, DV>;
  __shared__ __align__(16) char smem[CL::BYTES];
  const int bh = blockIdx.x / CL::NS, vb = blockIdx.x % CL::NS;
  Stamps stp;
  consume_chain<TIn, DK, DV, false, false, false>(smem, ws + (size_t)bh * nchunks * Rec<TIn, DK, DV>::BYTES,
                                           Ring{nullptr, nullptr, nullptr, nullptr, 1}, vb, h0, ht, o, bh / H,
                                           bh % H, T_len, H, nchunks, 0, snap, stp);
}

// ---------------------------------------------------------------------------
// Fused single-pass schedule: one persistent work-group per CU.  Heads are
// dealt to the 8 XCDs (work-group i runs on XCD i % 8); on each XCD the
// first work-groups are state-pass consumers (NS per head, resident for
// the whole call) and the rest are producers that share the (chunk, head)
// items of that XCD's heads, in chunk-major order, round robin, and write
// each chunk's record into the head's ring of R slots.  Records
// therefore live only in L2 / Infinity Cache between producer and consumer.
// A producer loads its next item's inputs in four portions issued during
// the current item's phases, so that the loads overlap the compute and no
// phase waits for one large burst of requests to be accepted.
// Ordering: producer stores, then a release in every wave, then
// ready[slot] = (c + 1) << 4 | XCD; the consumer polls ready, then an
// acquire, then reads.  Work-group i is dispatched to XCD i % 8, so a head's
// producers and its consumer normally share one L2: then the release is a
// wait for the stores to reach the L2 and the acquire an L1 invalidate.
// Both sides check where they actually run (the XCC_ID hardware register;
// the consumer publishes its XCD, the producer tags the flag with its own)
// and use agent-scope fences whenever the two differ.  A slot is reused only after every
// consumer of the head stored done >= c + 1 for the chunk that held it.
// Every wait is bounded (kSpinLimit); on a timeout the work-group sets the
// error word and leaves, so the grid always drains.
//
// ctrl layout (ints):
//   [0..7]   unused                     [8] error word (status of the call)
//   [32 ..)  ready[nheads][kFlagLine] (a head's R <= kFlagLine slot words),
//            then done[nheads * NS][kFlagLine] (one word used), then
//            cxcc[nheads][NS]
// Every head's ready words and every consumer's progress word have a cache
// line of their own: waves that poll different words (and the error word)
// then never queue behind each other on one line.
// [32 ..) is zeroed before every launch; [0..16) once per API call
// (launch_clear_status), so an error word set by any launch of a call stays
// set until the caller reads it, and every later launch of the call gives
// up at its first wait.  A launch runs its heads in rounds of nheads head
// slots; a slot's ready and progress words count its ring's chunks across
// the rounds.
// ---------------------------------------------------------------------------
template <typename TIn, int DK, int DV>
struct FusedLds {
  static constexpr size_t A = IntraLds<TIn, DK, DV>::BYTES, B = ConsumerLds<TIn, DK, DV>::BYTES;
  static constexpr size_t BYTES = (A > B ? A : B) + 16;
};

// kRounds: the launch may hold more heads than one round (otherwise
// nbh_run == nheads, and the round arithmetic is compiled out).
template <typename TIn, int DK, int DV, bool kUnb, bool kLay, bool kSeg, bool kRounds>
__global__ __launch_bounds__(kThreads) void fused_fwd_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                             const TIn* __restrict__ v, const TIn* __restrict__ g,
                                                             const float* __restrict__ gcum,
                                                             const TIn* __restrict__ beta, float scale,
                                                             const float* __restrict__ h0, float* __restrict__ ht,
                                                             float* __restrict__ o, int T_len, int H, int nchunks,
                                                             int head0, int nheads, int nbh_run,
                                                             char* __restrict__ ring, int* __restrict__ ctrl, int R,
                                                             Snap snap, Layer lay, VarSeg var) {
  using Rc = Rec<TIn, DK, DV>;
  __shared__ __align__(16) char smem[FusedLds<TIn, DK, DV>::BYTES];
  const VarSeg* vp = kSeg ? &var : nullptr;   // packed sequences (snapshot variant only)
  int* sWord = reinterpret_cast<int*>(smem + FusedLds<TIn, DK, DV>::BYTES - 16);
  const int xcd = blockIdx.x & 7, li = blockIdx.x >> 3;
  // The launch's nbh_run heads (from head0) go in rounds of nheads: head
  // slot j (0 <= j < nheads) of round r is head head0 + r nheads + j; slot j
  // keeps its ring, flags and state-pass work-groups for every round.
  const int rounds = kRounds ? (nbh_run + nheads - 1) / nheads : 1;
  const int last_n = kRounds ? nbh_run - (rounds - 1) * nheads : nheads;   // heads of the last round
  const int nloc = nheads > xcd ? (nheads - xcd + 7) / 8 : 0;              // slots j = xcd + 8m of this XCD
  const int nloc_last = kRounds ? (last_n > xcd ? (last_n - xcd + 7) / 8 : 0) : nloc;   // ... in the last round
  constexpr int NS = ConsumerLds<TIn, DK, DV>::NS;
  int* err = ctrl + 8;
  int* ready = ctrl + kFlagBase;
  int* done = ready + nheads * kFlagLine;
  int* cxcc = done + nheads * NS * kFlagLine;
  Stamps stp;

  if (li < nloc * NS) {   // state pass vb of head slot jh, one head per round
    const int jh = xcd + 8 * (li / NS), vb = li % NS;
    const Ring rg{ready + jh * kFlagLine, done + (jh * NS + vb) * kFlagLine, err, cxcc + jh * NS + vb, R};
    for (int r = 0; r < rounds && (r + 1 < rounds || jh < last_n); ++r) {
      const int bh = head0 + r * nheads + jh;
      if (!consume_chain<TIn, DK, DV, true, kLay, kSeg>(smem, ring + (size_t)jh * R * Rc::BYTES, rg, vb, h0, ht, o,
                                                        bh / H, bh % H, T_len, H, nchunks, r * nchunks, snap, stp,
                                                        lay, vp))
        break;
    }
    stp.flush();
    return;
  }

  // producer p of this XCD's P producers: items p, p + P, p + 2P, ... of
  // this XCD's head slots, round by round and chunk-major within a round
  // (item = (r nchunks + chunk) nloc + local slot in the full rounds).  A
  // slot's ring counts its chunks across rounds: ring chunk cg = r nchunks
  // + chunk.  No deadlock: the smallest item any producer waits on only
  // needs chunks of smaller items, and every smaller item is finished
  // because each producer handles its items in increasing order.
  const int per_round = nloc * nchunks;
  const int total = (rounds - 1) * per_round + nloc_last * nchunks;
  const int P = (int)(gridDim.x >> 3) - nloc * NS;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int my_xcc = xcc_id();
  struct Item {
    int r, c, pl;   // round, chunk of the head, local head slot
  };
  auto item_of = [&](int i) -> Item {
    if (!kRounds) return Item{0, i / nloc, i % nloc};
    const int r = min(i / per_round, rounds - 1), rem = i - r * per_round;
    if (r + 1 < rounds) return Item{r, rem / nloc, rem % nloc};
    return Item{r, rem / nloc_last, rem % nloc_last};
  };
  InRegs<TIn, DK, DV> in;
  int it = li - nloc * NS;
  stp.add<kStampRole>(1);
  if (it >= total) {
    stp.flush();
    return;
  }
  // sequence cursors of this item and of the next one (reset when the
  // round changes: chunk indices start again from 0)
  int seq_cur = 0, seq_next = 0, r_cur = 0, r_next = 0;
  Item xc = item_of(it);   // this item (the next one is carried over)
  {
    const int bh = head0 + xc.r * nheads + xcd + 8 * xc.pl;
    r_next = xc.r;
    const ChunkPos ps = chunk_pos(vp, xc.c, T_len, seq_next);
    load_inputs<TIn, DK, DV>(in, q, k, v, g, beta, bh / H, bh % H, T_len, H, ps.t0, ps.rows);
  }
  // Publishes ring chunk cg of slot pl (its record stores were issued by
  // every wave).  Release: if the slot's consumers run on this XCD they read
  // through the same L2, so it is enough that every wave's record stores
  // have reached the L2; otherwise an agent-scope release (L2 write-back).
  // A consumer's XCD word is written at its start, so a slot whose
  // consumers were seen on this XCD is remembered (bit of same_mask).
  // Its barrier also separates the item's last LDS accesses from the next
  // item's first (produce_chunk has no barrier of its own at entry).
  unsigned same_mask = 0;
  auto publish = [&](int cg, int pl) {
    const int pj = xcd + 8 * pl;
    bool same = pl < 32 && ((same_mask >> pl) & 1u);
    if (!same) {
      same = true;
      for (int vb = 0; vb < NS; ++vb)
        same = same && __builtin_amdgcn_readfirstlane(__hip_atomic_load(cxcc + pj * NS + vb, __ATOMIC_RELAXED,
                                                                        __HIP_MEMORY_SCOPE_AGENT)) == my_xcc + 1;
      if (same && pl < 32) same_mask |= 1u << pl;
    }
    if (same) wait_vmem();
    else __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (w == 0 && lane == 0)
      __hip_atomic_store(ready + pj * kFlagLine + cg % R, ((cg + 1) << 4) | my_xcc, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  };
  for (;;) {
    const Item x = xc;
    const int c = x.c, cg = x.r * nchunks + c, jh = xcd + 8 * x.pl, bh = head0 + x.r * nheads + jh;
    const int nxt = it + P;
    if (x.r != r_cur) {
      r_cur = x.r;
      seq_cur = 0;
    }
    const ChunkPos pc = chunk_pos(vp, c, T_len, seq_cur);
    // the next item and its position, once per item (its table reads wait
    // for the LDS accesses in flight, so not inside the phases)
    Item xn = x;
    ChunkPos pn = pc;
    if (nxt < total) {
      xn = item_of(nxt);
      if (xn.r != r_next) {
        r_next = xn.r;
        seq_next = 0;
      }
      pn = chunk_pos(vp, xn.c, T_len, seq_next);
    }
    // The ring slot of ring chunk cg is free once the slot's consumers have
    // read ring chunk cg - R.  Wave 0 reads their progress words from this
    // XCD's L2 once the inputs are staged (after the input registers are
    // consumed: vector loads complete in order), checks them at the end of
    // the block scans, polling only if the slot is still taken, and leaves
    // its verdict in LDS for the other waves to read after the next barrier.
    int seen[NS] = {};
    auto slot = [&](auto step) -> bool {
      constexpr int s = decltype(step)::value;
      if (cg < R) return true;
      if (s == kSlotPeek && w == 0) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(done + jh * NS * kFlagLine, (short)0, NS * kFlagLine * 4, kBufferRsrcWord3);
#pragma unroll
        for (int vb = 0; vb < NS; ++vb)
          seen[vb] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * vb * kFlagLine, 0, kCachePolicySc0);
      } else if (s == kSlotCheck && w == 0) {
        bool ok = true;
#pragma unroll
        for (int vb = 0; vb < NS; ++vb)
          if (ok && __builtin_amdgcn_readfirstlane(seen[vb]) < cg - R + 1)
            ok = spin_until_geq(done + (jh * NS + vb) * kFlagLine, cg - R + 1, err) >= 0;
        if (lane == 0) *sWord = ok ? 1 : 0;
      } else if (s == kSlotOk) {
        return __builtin_amdgcn_readfirstlane(*sWord) != 0;
      }
      return true;
    };
    // the next item's inputs, loaded in portions during this item's phases
    auto prefetch = [&](auto parts) {
      if (nxt < total) {
        const int bn = head0 + xn.r * nheads + xcd + 8 * xn.pl;
        load_inputs<TIn, DK, DV, decltype(parts)::value>(in, q, k, v, g, beta, bn / H, bn % H, T_len, H, pn.t0,
                                                         pn.rows);
      }
    };
    if (!produce_chunk<TIn, DK, DV, kUnb, kLay>(smem, in, gcum, scale, bh / H, bh % H, T_len, H, pc.t0, pc.rows,
                                    ring + ((size_t)jh * R + cg % R) * Rc::BYTES, slot, prefetch, stp, lay)) {
      stp.flush();
      return;
    }
    // Published as soon as its stores are in the L2.  (Deferring this until
    // the next item's inputs were staged let the stores drain in the
    // background but made every record visible some 4-5k cycles later; the
    // consumers then waited for records and the producers for ring slots.)
    publish(cg, x.pl);
    stp.mark<10>();
    stp.add<kStampCount>(1);
    if (nxt >= total) {
      stp.flush();
      return;
    }
    it = nxt;
    xc = xn;
  }
}

__global__ void clear_ints_kernel(int* p, int n) {   // also zero-fills fp32 buffers
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
constexpr int kRingSlots = 9;         // ring slots per head (fused schedule)
static_assert(kRingSlots <= kFlagLine, "a head's ready words share one line");
constexpr int kMaxWgPerXcd = 32;      // MI355X: 256 CUs in 8 XCDs

// Heads one fused launch can serve with `per_xcd` work-groups per XCD:
// keep at least a quarter of each XCD (and >= 2 work-groups) as producers.
static int fused_heads_per_launch(int per_xcd, int ns) {
  const int prod = per_xcd / 4 > 2 ? per_xcd / 4 : 2;
  const int hx = (per_xcd - prod) / ns;
  return hx > 0 ? 8 * hx : 0;
}

// Heads per round for nbh heads (at most cap per round, wgs work-groups,
// ns state-pass work-groups per head).  A round of nh heads takes, per
// chunk of its heads, about max(t_chain, nh t_item / (wgs - ns nh)): one
// chunk of a head's state pass, or the producers' share of the records
// (t_item: one record on one producer work-group).  The number of rounds L
// minimising L times that maximum gives the batch; measured t_item / t_chain
// is about 5.7 (d_k = d_v = 128), so a round of about 32 heads keeps both
// sides busy, and 64 heads run as two rounds of 32 rather than one with
// half the work-groups holding state passes.  The rounds share one launch:
// the producers go on to the next round's records while the last chunks of
// the round before are still in the state passes.
static int fused_launch_batch(int nbh, int cap, int wgs, int ns) {
  constexpr double kItemOverChain = 5.7;
  int best = nbh < cap ? nbh : cap;
  double best_cost = 1e300;
  for (int L = (nbh + cap - 1) / cap; L <= nbh; ++L) {
    int nh = (nbh + L - 1) / L;
    if (nh > 8) nh = (nh + 7) / 8 * 8;   // whole rounds over the 8 XCDs
    if (nh > cap) nh = cap;
    const int launches = (nbh + nh - 1) / nh, prod = wgs - ns * nh;
    if (prod > 0) {
      const double per = nh * kItemOverChain / prod;
      const double cost = launches * (per > 1.0 ? per : 1.0);
      if (cost < best_cost * (1.0 - 1e-9)) {
        best_cost = cost;
        best = nh;
      }
    }
    if (nh <= 8) break;
  }
  return best;
}

template <typename TIn, int DK, int DV>
static size_t fused_ctrl_bytes(int nheads) {
  constexpr int NS = ConsumerLds<TIn, DK, DV>::NS;
  return ((size_t)(kFlagBase + nheads * kFlagLine + NS * nheads * kFlagLine + NS * nheads) * 4 + 255) / 256 * 256;
}

template <typename TIn, int DK, int DV>
static size_t fused_ws_bytes(int nbh) {
  const int cap = fused_heads_per_launch(kMaxWgPerXcd, ConsumerLds<TIn, DK, DV>::NS);
  const int nh = nbh < cap ? nbh : cap;
  return fused_ctrl_bytes<TIn, DK, DV>(nh) + (size_t)nh * kRingSlots * Rec<TIn, DK, DV>::BYTES;
}

template <typename TIn, int DK, int DV>
static hipError_t go_fused(const void* q, const void* k, const void* v, const void* g, const float* gcum,
                           const void* beta, float scale, const float* h0, float* ht, float* o, int B, int T_len,
                           int H, void* ws, size_t ws_bytes, bool unb, float* snap, int snap_every, Layer lay,
                           hipStream_t st, const VarSeg* var) {
  // packed sequences: every head's stream is the sequences' chunks in order
  const bool packed = var != nullptr && var->n > 0;
  const int nchunks = packed ? var->cc[var->n] : (T_len + kC - 1) / kC;
  if (packed && (B != 1 || unb || gcum)) return hipErrorInvalidValue;
  if (nchunks <= 0) return hipSuccess;
  static const VarSeg kNoVar{};
  const int nbh = B * H;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  int per_xcd = cus / 8;
  if (per_xcd > kMaxWgPerXcd) per_xcd = kMaxWgPerXcd;
  constexpr int NS = ConsumerLds<TIn, DK, DV>::NS;
  const int cap = fused_heads_per_launch(per_xcd, NS);
  if (cap <= 0) return hipErrorInvalidConfiguration;
  int batch = fused_launch_batch(nbh, cap, 8 * per_xcd, NS);
  // what the workspace can hold
  while (batch > 0 && fused_ctrl_bytes<TIn, DK, DV>(batch) + (size_t)batch * kRingSlots * Rec<TIn, DK, DV>::BYTES > ws_bytes)
    --batch;
  if (batch <= 0) return hipErrorInvalidValue;
  int* ctrl = reinterpret_cast<int*>(ws);
  char* ring = reinterpret_cast<char*>(ws) + fused_ctrl_bytes<TIn, DK, DV>(batch);
  // one launch: rounds of `batch` heads (slot j of every round shares ring j)
  const int nh = nbh < batch ? nbh : batch;
  const int nflags = nh * kFlagLine + NS * nh * kFlagLine + NS * nh;   // ctrl[kFlagBase ..)
  hipLaunchKernelGGL(clear_ints_kernel, dim3((nflags + 255) / 256), dim3(256), 0, st, ctrl + kFlagBase, nflags);
  // four variants: plain, unbounded decay, layer steps, snapshots / packed sequences
  const bool with_lay = lay.flags != 0 || lay.og != nullptr;
  const bool with_seg = (snap != nullptr && snap_every > 0) || packed;
  if ((unb && (with_lay || with_seg)) || (with_lay && with_seg)) return hipErrorInvalidValue;
  // (the plain, layer and packed-sequence variants also come as one-round
  // kernels, used when the heads fit one round: the round arithmetic cost
  // the plain one 1% at 32 heads, and spilled in the others' chunk loops)
  const bool multi = nbh > nh;
  auto kern = unb ? fused_fwd_kernel<TIn, DK, DV, true, false, false, true>
              : with_lay ? (multi ? fused_fwd_kernel<TIn, DK, DV, false, true, false, true>
                                  : fused_fwd_kernel<TIn, DK, DV, false, true, false, false>)
              : with_seg ? (multi ? fused_fwd_kernel<TIn, DK, DV, false, false, true, true>
                                  : fused_fwd_kernel<TIn, DK, DV, false, false, true, false>)
                         : (multi ? fused_fwd_kernel<TIn, DK, DV, false, false, false, true>
                                  : fused_fwd_kernel<TIn, DK, DV, false, false, false, false>);
  hipLaunchKernelGGL(kern, dim3(8 * per_xcd), dim3(kThreads), 0, st, (const TIn*)q, (const TIn*)k, (const TIn*)v,
                     (const TIn*)g, gcum, (const TIn*)beta, scale, h0, ht, o, T_len, H, nchunks, 0, nh, nbh, ring,
                     ctrl, kRingSlots, Snap{snap, snap_every, nbh}, lay, packed ? *var : kNoVar);
  return hipGetLastError();
}

template <typename TIn, int DK, int DV>
static hipError_t go_stages(const void* q, const void* k, const void* v, const void* g, const float* gcum,
                            const void* beta, float scale, const float* h0, float* ht, float* o, int B, int T_len,
                            int H, void* ws, int stages, bool unb, float* snap, int snap_every, hipStream_t st) {
  const int nchunks = (T_len + kC - 1) / kC;
  const unsigned nbh = (unsigned)B * (unsigned)H;
  if (stages & 1) {
    auto kern = unb ? intra_chunk_kernel<TIn, DK, DV, true> : intra_chunk_kernel<TIn, DK, DV, false>;
    hipLaunchKernelGGL(kern, dim3(nchunks * nbh), dim3(kThreads), 0, st, (const TIn*)q, (const TIn*)k,
                       (const TIn*)v, (const TIn*)g, gcum, (const TIn*)beta, scale, (char*)ws, T_len, H, nchunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & 2) {
    hipLaunchKernelGGL((state_pass_kernel<TIn, DK, DV>), dim3(ConsumerLds<TIn, DK, DV>::NS * nbh), dim3(kThreads), 0, st,
                       (const char*)ws, h0, ht, o, T_len, H, nchunks, Snap{snap, snap_every, (int)nbh});
    return hipGetLastError();
  }
  return hipSuccess;
}

#define KDA_DISPATCH_D(FN, ...)                                   \
  do {                                                            \
    if (dk == 128 && dv == 128) return FN<TIn, 128, 128>(__VA_ARGS__); \
    if (dk == 128 && dv == 64) return FN<TIn, 128, 64>(__VA_ARGS__);   \
    if (dk == 64 && dv == 128) return FN<TIn, 64, 128>(__VA_ARGS__);   \
    return FN<TIn, 64, 64>(__VA_ARGS__);                          \
  } while (0)

template <typename TIn>
static size_t ws_fused_t(int nbh, int dk, int dv) { KDA_DISPATCH_D(fused_ws_bytes, nbh); }
template <typename TIn>
static size_t rec_bytes_t(int dk, int dv) {
  if (dk == 128 && dv == 128) return Rec<TIn, 128, 128>::BYTES;
  if (dk == 128 && dv == 64) return Rec<TIn, 128, 64>::BYTES;
  if (dk == 64 && dv == 128) return Rec<TIn, 64, 128>::BYTES;
  return Rec<TIn, 64, 64>::BYTES;
}

size_t fwd_record_bytes(int is_bf16, int dk, int dv) {
  return is_bf16 ? rec_bytes_t<bf16>(dk, dv) : rec_bytes_t<float>(dk, dv);
}
size_t fwd_fused_workspace_bytes(int is_bf16, int nbh, int dk, int dv) {
  return is_bf16 ? ws_fused_t<bf16>(nbh, dk, dv) : ws_fused_t<float>(nbh, dk, dv);
}

template <typename TIn>
static hipError_t fused_t(const void* q, const void* k, const void* v, const void* g, const float* gcum,
                          const void* beta, float scale, const float* h0, float* ht, float* o, int B, int T_len,
                          int H, int dk, int dv, void* ws, size_t wsb, bool unb, float* snap, int snap_every,
                          Layer lay, hipStream_t st, const VarSeg* var) {
  KDA_DISPATCH_D(go_fused, q, k, v, g, gcum, beta, scale, h0, ht, o, B, T_len, H, ws, wsb, unb, snap, snap_every,
                 lay, st, var);
}
template <typename TIn>
static hipError_t stages_t(const void* q, const void* k, const void* v, const void* g, const float* gcum,
                           const void* beta, float scale, const float* h0, float* ht, float* o, int B, int T_len,
                           int H, int dk, int dv, void* ws, int stages, bool unb, float* snap, int snap_every,
                           hipStream_t st) {
  KDA_DISPATCH_D(go_stages, q, k, v, g, gcum, beta, scale, h0, ht, o, B, T_len, H, ws, stages, unb, snap, snap_every,
                 st);
}

hipError_t launch_fwd_fused(int is_bf16, const void* q, const void* k, const void* v, const void* g,
                            const float* gcum, const void* beta, float scale, const float* h0, float* ht, float* o,
                            int B, int T_len, int H, int dk, int dv, void* ws, size_t ws_bytes, int unbounded,
                            float* snap, int snap_every, const float* A, const void* og, int layer_flags,
                            hipStream_t st, const VarSeg* var) {
  const bool u = unbounded != 0;
  const Layer lay{A, og, layer_flags};
  if (is_bf16)
    return fused_t<bf16>(q, k, v, g, gcum, beta, scale, h0, ht, o, B, T_len, H, dk, dv, ws, ws_bytes, u, snap,
                         snap_every, lay, st, var);
  return fused_t<float>(q, k, v, g, gcum, beta, scale, h0, ht, o, B, T_len, H, dk, dv, ws, ws_bytes, u, snap,
                        snap_every, lay, st, var);
}

hipError_t launch_fwd_stages(int is_bf16, const void* q, const void* k, const void* v, const void* g,
                             const float* gcum, const void* beta, float scale, const float* h0, float* ht, float* o,
                             int B, int T_len, int H, int dk, int dv, void* ws, int stages, int unbounded,
                             float* snap, int snap_every, hipStream_t st) {
  const bool u = unbounded != 0;
  if (is_bf16)
    return stages_t<bf16>(q, k, v, g, gcum, beta, scale, h0, ht, o, B, T_len, H, dk, dv, ws, stages, u, snap,
                          snap_every, st);
  return stages_t<float>(q, k, v, g, gcum, beta, scale, h0, ht, o, B, T_len, H, dk, dv, ws, stages, u, snap,
                         snap_every, st);
}

}  // namespace kda

namespace kda {
hipError_t launch_zero_words(void* p, size_t nwords, hipStream_t st) {
  if (nwords == 0) return hipSuccess;
  if (nwords > 0x7fffffffu) return hipErrorInvalidValue;
  const int n = (int)nwords;
  hipLaunchKernelGGL(clear_ints_kernel, dim3((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096), dim3(256), 0, st,
                     reinterpret_cast<int*>(p), n);
  return hipGetLastError();
}
}  // namespace kda

namespace kda {

// Status words of a prefill workspace (ints [0..16): the error word and
// spare words) cleared once at the start of an API call.
hipError_t launch_clear_status(void* ws, hipStream_t st) {
  hipLaunchKernelGGL(clear_ints_kernel, dim3(1), dim3(64), 0, st, reinterpret_cast<int*>(ws), 16);
  return hipGetLastError();
}

}  // namespace kda

#ifdef KDA_CYCLE_STAMPS
#include "kda_stamps.h"
extern "C" int kda_stamps_read(unsigned long long* host, size_t count) {
  static_assert(KDA_STAMP_WGS == kda::kStampMaxWgs && KDA_STAMP_SLOTS == kda::kStampSlots &&
                    KDA_STAMP_ROLE == kda::kStampRole && KDA_STAMP_COUNT == kda::kStampCount,
                "stamp layout");
  constexpr size_t kTotal = (size_t)kda::kStampMaxWgs * kda::kNW * kda::kStampSlots;
  if (host == nullptr) return KDA_ERR_NULL;
  if (count != kTotal) return KDA_ERR_SHAPE;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(kda::g_stamps), kTotal * sizeof(unsigned long long)) == hipSuccess
             ? KDA_OK
             : KDA_ERR_HIP;
}
#endif
