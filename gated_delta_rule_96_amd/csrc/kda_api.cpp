// C ABI of libkda.so (declared in include/kda.h): synchronous argument
// validation, then dispatch to the gfx950 kernels on the caller's stream.
// Nothing here allocates device memory or keeps mutable global state.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_launch.h"

namespace {

constexpr int kChunk = 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool supported_d(int d) { return d == 64 || d == 128; }
bool valid_dtype(int dt) { return dt == KDA_F32 || dt == KDA_BF16; }

// Largest element count of any [B, T, H, d] tensor accepted (64-bit offsets
// are used throughout; this only rejects sizes whose byte count overflows).
bool size_ok(long long a, long long b, long long c, long long d) {
  const long long lim = (1LL << 62);
  long long x = a;
  for (long long y : {b, c, d}) {
    if (y <= 0 || x > lim / y) return false;
    x *= y;
  }
  return true;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_str(int s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "a size is non-positive or too large";
    case KDA_ERR_DTYPE: return "dtype is not KDA_F32 or KDA_BF16";
    case KDA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case KDA_ERR_UNSUPPORTED: return "unsupported dk/dv/chunk (dk, dv in {64,128}; chunk 64)";
    case KDA_ERR_WORKSPACE: return "workspace missing or smaller than kda_fwd_workspace_bytes";
    case KDA_ERR_RANGE: return "input value out of range (log-decay outside [gmin, 0], or gmin outside [-5, 0))";
    case KDA_ERR_HIP: return "HIP launch failed";
    case KDA_ERR_INCOMPLETE:
      return "the fused prefill gave up on a hand-off wait (GPU shared with other work?): outputs incomplete";
    default: return "unknown status";
  }
}

namespace {

constexpr float kGmin = -5.0f;   // the gate's floor ("Key claims", section 2.1.1)

// Opt-in range check (KDA_VALIDATE=1): the log-decay input of a bounded
// call in [-5, 0] (bounded != 0), or <= 0 (unbounded call); finite.
int check_range(int dtype, const void* g, const float* gcum, int bounded, int B, int T, int H, int dk,
                void* stream) {
  if (!kda::validate_requested()) return KDA_OK;
  int ok = 0;
  const hipError_t e = kda::validate_decay(dtype == KDA_BF16, g, gcum, bounded, kGmin, B, T, H * dk, kChunk,
                                           static_cast<hipStream_t>(stream), &ok);
  if (e != hipSuccess) return KDA_ERR_HIP;
  return ok ? KDA_OK : KDA_ERR_RANGE;
}

int prepare_decay_impl(const void* z, const float* A, float gmin, void* g, float* gcum, int dtype, int B, int T,
                       int H, int dk, int chunk, int softplus, void* stream) {
  if (!valid_dtype(dtype)) return KDA_ERR_DTYPE;
  if (B <= 0 || T <= 0 || H <= 0 || dk <= 0 || chunk <= 0 || !size_ok(B, T, H, dk)) return KDA_ERR_SHAPE;
  if (!supported_d(dk) || chunk != kChunk) return KDA_ERR_UNSUPPORTED;
  // the bounded gate's floor must keep 16 rows of decay inside the bf16
  // range the prefill's rescaled tiles rely on (16 * 5 = 80 < 88.7)
  if (z && !softplus && !(gmin >= kGmin && gmin < 0.f)) return KDA_ERR_RANGE;
  if (z) {
    if (!A || (!g && !gcum)) return KDA_ERR_NULL;
  } else {
    if (!g || !gcum) return KDA_ERR_NULL;
  }
  if ((z && !aligned16(z)) || (g && !aligned16(g)) || (gcum && !aligned16(gcum)) || (A && !aligned16(A)))
    return KDA_ERR_ALIGN;
  hipError_t e = kda::launch_prepare_decay(dtype == KDA_BF16, z, A, gmin, g, gcum, B, T, H, dk, chunk, softplus,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}
}  // namespace

int kda_prepare_decay(const void* z, const float* A, float gmin, void* g, float* gcum, int dtype, int B, int T,
                      int H, int dk, int chunk, void* stream) {
  return prepare_decay_impl(z, A, gmin, g, gcum, dtype, B, T, H, dk, chunk, 0, stream);
}

int kda_prepare_decay_softplus(const void* z, const float* A, void* g, float* gcum, int dtype, int B, int T, int H,
                               int dk, int chunk, void* stream) {
  if (!z) return KDA_ERR_NULL;
  return prepare_decay_impl(z, A, 0.f, g, gcum, dtype, B, T, H, dk, chunk, 1, stream);
}

size_t kda_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype) {
  if (!valid_dtype(dtype) || B <= 0 || T <= 0 || H <= 0 || !supported_d(dk) || !supported_d(dv) ||
      chunk != kChunk || !size_ok(B, T, H, dk))
    return 0;
  return kda::fwd_fused_workspace_bytes(dtype == KDA_BF16, B * H, dk, dv);
}

size_t kda_fwd_stages_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype) {
  if (!valid_dtype(dtype) || B <= 0 || T <= 0 || H <= 0 || !supported_d(dk) || !supported_d(dv) ||
      chunk != kChunk || !size_ok(B, T, H, dk))
    return 0;
  const size_t nchunks = ((size_t)T + kChunk - 1) / kChunk;
  return (size_t)B * (size_t)H * nchunks * kda::fwd_record_bytes(dtype == KDA_BF16, dk, dv);
}

namespace {

// Shared validation of the prefill calls; `stages` is 3 for kda_fwd_chunked
// (the stage mask, without the unbounded-decay bit).
int check_fwd(const void* q, const void* k, const void* v, const void* g, const float* gcum, const void* beta,
              const float* h0, const float* ht, const float* o, int dtype, int B, int T, int H, int dk, int dv,
              int chunk, const void* workspace, int stages) {
  if (!valid_dtype(dtype)) return KDA_ERR_DTYPE;
  if (B <= 0 || T <= 0 || H <= 0 || dk <= 0 || dv <= 0 || chunk <= 0 || !size_ok(B, T, H, dk) ||
      !size_ok(B, T, H, dv) || (long long)B * H * ((T + kChunk - 1) / kChunk) > 2147483647LL || stages < 1 ||
      stages > 3)
    return KDA_ERR_SHAPE;
  if (!supported_d(dk) || !supported_d(dv) || chunk != kChunk) return KDA_ERR_UNSUPPORTED;
  if ((stages & 1) && (!q || !k || !v || !beta || (!g && !gcum))) return KDA_ERR_NULL;
  if ((stages & 2) && !o) return KDA_ERR_NULL;
  if (!workspace) return KDA_ERR_WORKSPACE;
  for (const void* p : {(const void*)q, k, v, beta, g, (const void*)gcum, (const void*)h0, (const void*)ht,
                        (const void*)o})
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERR_ALIGN;
  return KDA_OK;
}

// The scratch of the allocation-free prefill stands in for the workspace
// in the shared checks (never dereferenced on the host).
const void* const kNoAllocWs = reinterpret_cast<const void*>(static_cast<uintptr_t>(256));

}  // namespace

namespace {
int fwd_fused_impl(const void* q, const void* k, const void* v, const void* g, const float* gcum, const void* beta,
                   float scale, const float* h0, float* ht, float* o, int dtype, int B, int T, int H, int dk, int dv,
                   int chunk, void* workspace, size_t workspace_bytes, int unbounded, void* stream) {
  const int st = check_fwd(q, k, v, g, gcum, beta, h0, ht, o, dtype, B, T, H, dk, dv, chunk, workspace, 3);
  if (st != KDA_OK) return st;
  if (workspace_bytes < kda_fwd_workspace_bytes(B, T, H, dk, dv, chunk, dtype)) return KDA_ERR_WORKSPACE;
  const int rs = check_range(dtype, g, gcum, !unbounded, B, T, H, dk, stream);
  if (rs != KDA_OK) return rs;
  hipError_t e = kda::launch_clear_status(workspace, static_cast<hipStream_t>(stream));
  if (e == hipSuccess)
    e = kda::launch_fwd_fused(dtype == KDA_BF16, q, k, v, g, gcum, beta, scale, h0, ht, o, B, T, H, dk, dv,
                              workspace, workspace_bytes, unbounded, nullptr, 0, nullptr, nullptr, 0,
                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}
}  // namespace

int kda_fwd_chunked(const void* q, const void* k, const void* v, const void* g, const float* gcum,
                    const void* beta, float scale, const float* h0, float* ht, float* o, int dtype, int B, int T,
                    int H, int dk, int dv, int chunk, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_fused_impl(q, k, v, g, gcum, beta, scale, h0, ht, o, dtype, B, T, H, dk, dv, chunk, workspace,
                        workspace_bytes, 0, stream);
}

int kda_fwd_chunked_noalloc(const void* q, const void* k, const void* v, const void* g, const float* gcum,
                            const void* beta, float scale, const float* h0, float* ht, float* o, int dtype, int B,
                            int T, int H, int dk, int dv, int chunk, void* stream) {
  const int st = check_fwd(q, k, v, g, gcum, beta, h0, ht, o, dtype, B, T, H, dk, dv, chunk, kNoAllocWs, 3);
  if (st != KDA_OK) return st;
  // the scratch holds at least one head's ring for every supported size
  // (more heads run as further rounds of the launch); checked for completeness
  if (kda_fwd_workspace_bytes(1, 1, 1, dk, dv, chunk, dtype) > kda::kNoAllocScratchBytes) return KDA_ERR_WORKSPACE;
  const int rs = check_range(dtype, g, gcum, 1, B, T, H, dk, stream);
  if (rs != KDA_OK) return rs;
  void* scr = nullptr;
  hipError_t e = kda::noalloc_scratch(&scr);
  if (e == hipSuccess) e = kda::launch_clear_status(scr, static_cast<hipStream_t>(stream));
  if (e == hipSuccess)
    e = kda::launch_fwd_fused(dtype == KDA_BF16, q, k, v, g, gcum, beta, scale, h0, ht, o, B, T, H, dk, dv, scr,
                              kda::kNoAllocScratchBytes, 0, nullptr, 0, nullptr, nullptr, 0,
                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_fwd_chunked_unbounded(const void* q, const void* k, const void* v, const void* g, const float* gcum,
                              const void* beta, float scale, const float* h0, float* ht, float* o, int dtype, int B,
                              int T, int H, int dk, int dv, int chunk, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return fwd_fused_impl(q, k, v, g, gcum, beta, scale, h0, ht, o, dtype, B, T, H, dk, dv, chunk, workspace,
                        workspace_bytes, 1, stream);
}

int kda_fwd_chunked_stages(const void* q, const void* k, const void* v, const void* g, const float* gcum,
                           const void* beta, float scale, const float* h0, float* ht, float* o, int dtype, int B,
                           int T, int H, int dk, int dv, int chunk, void* workspace, size_t workspace_bytes,
                           int stages, void* stream) {
  const int mask = stages & ~KDA_STAGES_UNBOUNDED;
  if ((stages & KDA_STAGES_UNBOUNDED) && mask < 1) return KDA_ERR_SHAPE;
  const int st = check_fwd(q, k, v, g, gcum, beta, h0, ht, o, dtype, B, T, H, dk, dv, chunk, workspace, mask);
  if (st != KDA_OK) return st;
  if (workspace_bytes < kda_fwd_stages_workspace_bytes(B, T, H, dk, dv, chunk, dtype)) return KDA_ERR_WORKSPACE;
  if (mask & 1) {
    const int rs = check_range(dtype, g, gcum, !(stages & KDA_STAGES_UNBOUNDED), B, T, H, dk, stream);
    if (rs != KDA_OK) return rs;
  }
  hipError_t e = kda::launch_fwd_stages(dtype == KDA_BF16, q, k, v, g, gcum, beta, scale, h0, ht, o, B, T, H, dk, dv,
                                        workspace, mask, (stages & KDA_STAGES_UNBOUNDED) ? 1 : 0, nullptr, 0,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_fwd_chunked_layer(const void* q, const void* k, const void* v, const void* z, const float* A,
                          const void* beta, const void* og, float scale, const float* h0, float* ht, float* o,
                          int flags, int dtype, int B, int T, int H, int dk, int dv, int chunk, void* workspace,
                          size_t workspace_bytes, void* stream) {
  const int st = check_fwd(q, k, v, z, nullptr, beta, h0, ht, o, dtype, B, T, H, dk, dv, chunk, workspace, 3);
  if (st != KDA_OK) return st;
  if (!z || !A) return KDA_ERR_NULL;
  if (flags & ~KDA_LAYER_QK_L2NORM) return KDA_ERR_SHAPE;
  if ((og && !aligned16(og)) || !aligned16(A)) return KDA_ERR_ALIGN;
  if (workspace_bytes < kda_fwd_workspace_bytes(B, T, H, dk, dv, chunk, dtype)) return KDA_ERR_WORKSPACE;
  const int lf = 1 /* g is z */ | ((flags & KDA_LAYER_QK_L2NORM) ? 2 : 0);
  hipError_t e = kda::launch_clear_status(workspace, static_cast<hipStream_t>(stream));
  if (e == hipSuccess)
    e = kda::launch_fwd_fused(dtype == KDA_BF16, q, k, v, z, nullptr, beta, scale, h0, ht, o, B, T, H, dk, dv,
                              workspace, workspace_bytes, 0, nullptr, 0, A, og, lf, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

const int* kda_fwd_status_word(const void* workspace) {
  return workspace ? static_cast<const int*>(workspace) + 8 : nullptr;
}

int kda_fwd_status(const void* workspace, void* stream) {
  if (!workspace) {   // the allocation-free prefill's scratch on the current device
    void* scr = nullptr;
    if (kda::noalloc_scratch(&scr) != hipSuccess) return KDA_ERR_HIP;
    workspace = scr;
  }
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERR_ALIGN;
  int word = 0;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&word, kda_fwd_status_word(workspace), sizeof(int), hipMemcpyDeviceToHost, hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return KDA_ERR_HIP;
  return word != 0 ? KDA_ERR_INCOMPLETE : KDA_OK;
}

long long kda_fwd_varlen_snapshots(const int* cu_seqlens, int N, int snap_every, int chunk) {
  if (!cu_seqlens || N <= 0 || snap_every <= 0 || chunk != kChunk) return -1;
  long long n = 0;
  for (int i = 0; i < N; ++i) {
    const long long len = (long long)cu_seqlens[i + 1] - cu_seqlens[i];
    if (len < 0) return -1;
    const long long nch = (len + kChunk - 1) / kChunk;   // snapshots at chunk ends before the last
    n += nch > 0 ? (nch - 1) / snap_every : 0;
  }
  return n;
}

int kda_fwd_chunked_varlen(const void* q, const void* k, const void* v, const void* g, const float* gcum,
                           const void* beta, float scale, const int* cu_seqlens, int N, const float* h0, float* ht,
                           float* o, float* snap, int snap_every, int dtype, int T, int H, int dk, int dv, int chunk,
                           void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_fwd(q, k, v, g, gcum, beta, h0, ht, o, dtype, 1, T, H, dk, dv, chunk, workspace, 3);
  if (st != KDA_OK) return st;
  if (!cu_seqlens) return KDA_ERR_NULL;
  // a packed gcum restarts at multiples of 64 of the packed axis, not at
  // each sequence's own chunks: only g is accepted here
  if (gcum) return KDA_ERR_UNSUPPORTED;
  if (N <= 0 || cu_seqlens[0] != 0 || cu_seqlens[N] != T || snap_every < 0) return KDA_ERR_SHAPE;
  for (int i = 0; i < N; ++i)
    if (cu_seqlens[i + 1] < cu_seqlens[i]) return KDA_ERR_SHAPE;
  if ((long long)N * H > 2147483647LL / ((long long)dk * dv)) return KDA_ERR_SHAPE;
  if (snap && snap_every > 0 && !aligned16(snap)) return KDA_ERR_ALIGN;
  // the workspace sized for one sequence of T tokens serves every call below
  if (workspace_bytes < kda_fwd_workspace_bytes(1, T, H, dk, dv, chunk, dtype)) return KDA_ERR_WORKSPACE;
  const int rs = check_range(dtype, g, nullptr, 1, 1, T, H, dk, stream);
  if (rs != KDA_OK) return rs;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (kda::launch_clear_status(workspace, hs) != hipSuccess) return KDA_ERR_HIP;
  const size_t esz = dtype == KDA_BF16 ? 2 : 4;
  const size_t hk = (size_t)H * dk, hv = (size_t)H * dv, sd = (size_t)H * dk * dv;
  const bool snaps = snap && snap_every > 0;
  if (N <= kda::kMaxVarSeq) {
    // one fused launch for all sequences: their chunks, in order, are every
    // head's stream (the launch carries the sequence table)
    kda::VarSeg vs{};
    vs.n = N;
    long long nch_total = 0, nsnap = 0;
    for (int i = 0; i <= N; ++i) {
      vs.cu[i] = cu_seqlens[i];
      vs.cc[i] = (int)nch_total;
      vs.sb[i] = (int)nsnap;
      if (i == N) break;
      const long long len = cu_seqlens[i + 1] - cu_seqlens[i];
      const long long nch = (len + kChunk - 1) / kChunk;
      nch_total += nch;
      if (snaps && nch > 0) nsnap += (nch - 1) / snap_every;
    }
    for (int i = 0; i < N; ++i) {   // sequences without tokens: ht = h0 (or zero)
      if (cu_seqlens[i + 1] != cu_seqlens[i]) continue;
      const float* h0_i = h0 ? h0 + i * sd : nullptr;
      float* ht_i = ht ? ht + i * sd : nullptr;
      hipError_t e = hipSuccess;
      if (ht_i && h0_i && ht_i != h0_i)
        e = hipMemcpyAsync(ht_i, h0_i, sd * sizeof(float), hipMemcpyDeviceToDevice, hs);
      else if (ht_i && !h0_i)
        e = kda::launch_zero_words(ht_i, sd, hs);
      if (e != hipSuccess) return KDA_ERR_HIP;
    }
    if (nch_total == 0) return KDA_OK;
    const hipError_t e = kda::launch_fwd_fused(dtype == KDA_BF16, q, k, v, g, nullptr, beta, scale, h0, ht, o, 1, T, H,
                                               dk, dv, workspace, workspace_bytes, 0, snaps ? snap : nullptr,
                                               snaps ? snap_every : 0, nullptr, nullptr, 0, hs, &vs);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }
  // more sequences than one launch carries: one fused launch per sequence
  long long snap_off = 0;
  for (int i = 0; i < N; ++i) {
    const size_t t0 = (size_t)cu_seqlens[i];
    const int len = cu_seqlens[i + 1] - cu_seqlens[i];
    const float* h0_i = h0 ? h0 + i * sd : nullptr;
    float* ht_i = ht ? ht + i * sd : nullptr;
    hipError_t e = hipSuccess;
    if (len == 0) {   // empty sequence: the final state is the initial one
      if (ht_i && h0_i && ht_i != h0_i)
        e = hipMemcpyAsync(ht_i, h0_i, sd * sizeof(float), hipMemcpyDeviceToDevice, hs);
      else if (ht_i && !h0_i)
        e = kda::launch_zero_words(ht_i, sd, hs);
    } else {
      auto at = [&](const void* p, size_t per_token) {
        return p ? static_cast<const void*>(static_cast<const char*>(p) + t0 * per_token * esz) : nullptr;
      };
      e = kda::launch_fwd_fused(dtype == KDA_BF16, at(q, hk), at(k, hk), at(v, hv), at(g, hk),
                                nullptr, at(beta, (size_t)H), scale, h0_i, ht_i,
                                o + t0 * hv, 1, len, H, dk, dv, workspace, workspace_bytes, 0,
                                snaps ? snap + (size_t)snap_off * sd : nullptr, snaps ? snap_every : 0, nullptr,
                                nullptr, 0, hs);
      if (snaps) {
        const long long nch = ((long long)len + kChunk - 1) / kChunk;
        snap_off += (nch - 1) / snap_every;
      }
    }
    if (e != hipSuccess) return KDA_ERR_HIP;
  }
  return KDA_OK;
}

int kda_decode_step(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                    float* state, float* o, int dtype, int B, int H, int dk, int dv, void* stream) {
  if (!valid_dtype(dtype)) return KDA_ERR_DTYPE;
  if (B <= 0 || H <= 0 || dk <= 0 || dv <= 0 || !size_ok(B, H, dk, dv)) return KDA_ERR_SHAPE;
  if (!supported_d(dk) || !supported_d(dv)) return KDA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_NULL;
  for (const void* p : {q, k, v, g, beta, (const void*)state, (const void*)o})
    if (!aligned16(p)) return KDA_ERR_ALIGN;
  if ((long long)B * H > 2147483647LL) return KDA_ERR_SHAPE;
  const int rs = check_range(dtype, g, nullptr, 1, B, 1, H, dk, stream);
  if (rs != KDA_OK) return rs;
  hipError_t e = kda::launch_decode_step(dtype == KDA_BF16, q, k, v, g, beta, scale, state, o, B, H, dk, dv,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_decode_step_layer(const void* q, const void* k, const void* v, const void* z, const float* A,
                          const void* beta, const void* og, float scale, float* state, float* o, int flags,
                          int dtype, int B, int H, int dk, int dv, void* stream) {
  if (!valid_dtype(dtype)) return KDA_ERR_DTYPE;
  if (B <= 0 || H <= 0 || dk <= 0 || dv <= 0 || !size_ok(B, H, dk, dv)) return KDA_ERR_SHAPE;
  if (!supported_d(dk) || !supported_d(dv)) return KDA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !z || !A || !beta || !state || !o) return KDA_ERR_NULL;
  if (flags & ~KDA_LAYER_QK_L2NORM) return KDA_ERR_SHAPE;
  for (const void* p : {q, k, v, z, beta, (const void*)A, (const void*)state, (const void*)o})
    if (!aligned16(p)) return KDA_ERR_ALIGN;
  if (og && !aligned16(og)) return KDA_ERR_ALIGN;
  if ((long long)B * H > 2147483647LL) return KDA_ERR_SHAPE;
  const kda::DecodeLayer lay{A, og, (flags & KDA_LAYER_QK_L2NORM) ? kda::kDecodeLayerNormQK : 0};
  hipError_t e = kda::launch_decode_step(dtype == KDA_BF16, q, k, v, z, beta, scale, state, o, B, H, dk, dv,
                                         static_cast<hipStream_t>(stream), &lay);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"

namespace {

// Backward workspace, in order: the forward's own workspace, its output and
// final state (scratch), the states entering chunks 1.., per-chunk records,
// the state gradient leaving every chunk and dU of every chunk.  Each part
// starts on a 256-byte boundary.
struct BwdLayout {
  size_t fwd, o, ht, snap, rec, dn, du, total;
};
size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
BwdLayout bwd_layout(int B, int T, int H, int dk, int dv, int dtype) {
  const size_t nbh = (size_t)B * H, nch = ((size_t)T + kChunk - 1) / kChunk;
  BwdLayout L{};
  size_t off = 0;
  auto put = [&](size_t bytes) {
    const size_t at = off;
    off += up256(bytes);
    return at;
  };
  L.fwd = put(kda_fwd_workspace_bytes(B, T, H, dk, dv, kChunk, dtype));
  L.o = put((size_t)B * T * H * dv * 4);
  L.ht = put(nbh * dk * dv * 4);
  L.snap = put((nch - 1) * nbh * dk * dv * 4);
  L.rec = put(nch * nbh * kda::bwd_record_words(dk, dv) * 4);
  L.dn = put(nch * nbh * dk * dv * 4);
  L.du = put(nch * nbh * kChunk * dv * 4);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

size_t kda_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype) {
  if (B <= 0 || T <= 0 || H <= 0 || !supported_d(dk) || !supported_d(dv) || chunk != kChunk || !valid_dtype(dtype))
    return 0;
  return bwd_layout(B, T, H, dk, dv, dtype).total;
}

int kda_bwd_chunked(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                    const float* h0, const float* dout, const float* dht, float* dq, float* dk_, float* dv_,
                    float* dg, float* dbeta, float* dh0, int dtype, int B, int T, int H, int dk, int dv, int chunk,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_fwd(q, k, v, g, nullptr, beta, h0, nullptr, dout, dtype, B, T, H, dk, dv, chunk, workspace, 3);
  if (st != KDA_OK) return st;
  if (!g || !dout || !dq || !dk_ || !dv_ || !dg || !dbeta) return KDA_ERR_NULL;
  for (const void* p : {(const void*)dht, (const void*)dq, (const void*)dk_, (const void*)dv_, (const void*)dg,
                        (const void*)dbeta, (const void*)dh0})
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  const BwdLayout lay = bwd_layout(B, T, H, dk, dv, dtype);
  if (workspace_bytes < lay.total) return KDA_ERR_WORKSPACE;
  st = check_range(dtype, g, nullptr, 1, B, T, H, dk, stream);
  if (st != KDA_OK) return st;
  char* ws = static_cast<char*>(workspace);
  const int nch = (T + kChunk - 1) / kChunk;
  float* snap = nch > 1 ? reinterpret_cast<float*>(ws + lay.snap) : nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the forward recompute's status word is the workspace's (its forward
  // part comes first): kda_fwd_status reads it
  if (kda::launch_clear_status(ws + lay.fwd, s) != hipSuccess) return KDA_ERR_HIP;
  hipError_t e = kda::launch_fwd_fused(dtype == KDA_BF16, q, k, v, g, nullptr, beta, scale, h0,
                                       reinterpret_cast<float*>(ws + lay.ht), reinterpret_cast<float*>(ws + lay.o), B,
                                       T, H, dk, dv, ws + lay.fwd, lay.o - lay.fwd, 0, snap, snap ? 1 : 0, nullptr,
                                       nullptr, 0, s);
  if (e != hipSuccess) return KDA_ERR_HIP;
  e = kda::launch_bwd_chunks(dtype == KDA_BF16, q, k, v, g, beta, dout, scale, h0, dht, snap,
                             reinterpret_cast<float*>(ws + lay.rec), reinterpret_cast<float*>(ws + lay.dn),
                             reinterpret_cast<float*>(ws + lay.du), B, T, H, dk, dv, dq, dk_, dv_, dg, dbeta, dh0, s);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
