/*
 * kda.h -- C ABI of libkda.so, the MI355X (gfx950) Kimi Delta Attention
 * (KDA) forward library.
 *
 * The method (Kimi K3 technical report summary, page "Kimi K3 Technical
 * Report - Open Frontier Intelligence"):
 *   - "Key claims", section 2.1: KDA is the sequence mixer of a 3:1
 *     KDA : Gated-MLA hybrid; it is a delta-rule attention with a fixed-size
 *     per-head recurrent state and channel-wise decay.  Per head and token t,
 *     with S in R^{dk x dv} (key channels as rows):
 *         S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *         o_t = scale * S_t^T q_t              (scale is 1/sqrt(dk) in the model)
 *   - "Key claims", section 2.1.1 and Fig. 3; "Method", section 2.1: the
 *     log-decay is g = gmin * Sigmoid(exp(A) * z) with gmin = -5 and a
 *     learnable per-head A.  The floor keeps the reciprocal rescaling
 *     factors of the chunkwise form inside the bf16 range, so every causal
 *     tile is a dense matrix product.
 *   - "Method", section 2.1: the chunkwise-parallel form (prefill);
 *     page "How a Frontier Model Gets Built, Read from the Kimi K3 Report",
 *     "Technical Details": the fixed-size running state replaces the KV
 *     cache (decode step, state carry between calls).
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller,
 *     contiguous row-major, 16-byte aligned.  Nothing is retained after the
 *     call returns.  The library never allocates device memory; its only
 *     device state is in its code object (one copy per GPU): a word used by
 *     the opt-in range check and the scratch of kda_fwd_chunked_noalloc.
 *     Calls are re-entrant.
 *   - Layouts: q, k, g, z : [B, T, H, dk];  v, o : [B, T, H, dv];
 *     beta : [B, T, H];  A : [H] (fp32);  states h0 / ht / state :
 *     [B, H, dk, dv] fp32 (key channel = row, value channel = column).
 *     Decode inputs drop the T axis: q, k, g : [B, H, dk]; v, o : [B, H, dv];
 *     beta : [B, H].
 *   - `dtype` (kda_dtype) is the element type of q, k, v, g, z and beta.
 *     The output o, the states and gcum are always fp32 (the outputs of the
 *     method have a heavy tail, max|o| of 10-20 times rms(o) on long
 *     sequences, so a bf16 output alone would carry errors of several
 *     percent of rms(o)).  Supported: dk, dv in {64, 128}; chunk == 64.
 *     Any T >= 1 is accepted.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call
 *     validates its arguments synchronously on the host; on any error
 *     nothing is enqueued and no output is touched.  On success the work is
 *     enqueued on `stream` and the call returns without synchronising.
 *     Device faults surface at the caller's next synchronisation.
 *   - Return value: a kda_status code (0 = KDA_OK).
 *   - Opt-in range check: with KDA_VALIDATE=1 in the environment, every call
 *     that takes a log-decay g (or gcum) first checks it on the device and
 *     returns KDA_ERR_RANGE without enqueuing anything if a value is outside
 *     [gmin, 0] with gmin = -5 (the floor that keeps 16 rows of decay inside
 *     the bf16 range, "Key claims" section 2.1.1), or is not finite; the
 *     unbounded-decay calls accept any finite g <= 0.  For gcum the per-row
 *     decays it encodes (differences of consecutive sums inside a chunk)
 *     are checked, up to the rounding of the fp32 sums.  The check
 *     synchronises `stream` and uses one library-owned device word per GPU
 *     (checks running at once on one GPU are serialised).  Without it the
 *     range is a precondition: a g below -5.5 overflows the rescaled bf16
 *     tiles (inf/NaN outputs).
 *   - Status of the fused prefill: its kernels hand work between
 *     work-groups with bounded waits (about a second).  If one expires (the
 *     GPU shared with other work that holds CUs), the call stops early and
 *     sets the status word of its workspace; the outputs are then
 *     incomplete.  The word is cleared at the start of every call and stays
 *     set for the rest of it; read it with kda_fwd_status (synchronous) or
 *     kda_fwd_status_word (its device address, for an asynchronous copy).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  KDA_ERR_SHAPE = 2,       /* a size is non-positive or too large                 */
  KDA_ERR_DTYPE = 3,       /* dtype is not a kda_dtype value                      */
  KDA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                    */
  KDA_ERR_UNSUPPORTED = 5, /* dk / dv / chunk outside the supported set           */
  KDA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than kda_fwd_workspace_bytes */
  KDA_ERR_RANGE = 7,       /* a value outside its documented range (KDA_VALIDATE=1 */
                           /* checks, and gmin of kda_prepare_decay)              */
  KDA_ERR_HIP = 8,         /* a HIP launch failed (hipGetLastError)               */
  KDA_ERR_INCOMPLETE = 9   /* kda_fwd_status: a hand-off wait of the fused        */
                           /* prefill expired; the call's outputs are incomplete  */
} kda_status;

typedef enum kda_dtype { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Returns KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* kda_status_str(int status);

/*
 * Decay preparation ("Key claims", section 2.1.1; "Method", section 2.1).
 *   z != NULL : gate mode.  g[b,t,h,c] = gmin * Sigmoid(exp(A[h]) * z[b,t,h,c])
 *               computed in fp32 and rounded (RNE) to `dtype`; written to g
 *               when g != NULL.  A must be non-NULL.
 *   z == NULL : g is an input (A is ignored).
 *   gcum != NULL : gcum[b,t,h,c] = inclusive sum of g over the rows of t's
 *               chunk of `chunk` tokens up to t (the rounded g in gate mode),
 *               accumulated in fp32.
 * At least one output (g in gate mode, or gcum) must be requested.
 * gmin must lie in [-5, 0) (a lower floor would take 16 rows of decay out
 * of the bf16 range the prefill's rescaled tiles rely on; the unbounded
 * comparison has its own gate below).
 * Errors: KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_DTYPE, KDA_ERR_ALIGN,
 *         KDA_ERR_UNSUPPORTED (dk, chunk), KDA_ERR_RANGE (gmin), KDA_ERR_HIP.
 */
int kda_prepare_decay(const void* z, const float* A, float gmin, void* g, float* gcum,
                      int dtype, int B, int T, int H, int dk, int chunk, void* stream);

/*
 * Decay preparation with the predecessor's unbounded gate ("Key claims",
 * section 2.1.1: Kimi Linear's negative Softplus log-decay, which K3
 * replaces with the bounded one): g[b,t,h,c] = -Softplus(exp(A[h]) *
 * z[b,t,h,c]), Softplus(x) = log(1 + e^x), in fp32, rounded (RNE) to dtype;
 * g has no lower bound.  Outputs, layout and errors as kda_prepare_decay in
 * gate mode (z and A required).  For kda_fwd_chunked_unbounded.
 */
int kda_prepare_decay_softplus(const void* z, const float* A, void* g, float* gcum, int dtype,
                               int B, int T, int H, int dk, int chunk, void* stream);

/* Bytes of device workspace kda_fwd_chunked needs for these sizes (0 if
 * the sizes are invalid or unsupported): ring buffers of a few chunk
 * records per head for at most one round of heads (the fused kernel runs
 * more heads as further rounds of the same launch, reusing the rings) plus
 * control words, independent of T (about 45 MiB at B*H >= 84, dk = dv =
 * 128, bf16). */
size_t kda_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype);

/* Bytes of device workspace kda_fwd_chunked_stages needs: one record per
 * (b, h, chunk), i.e. proportional to B*H*T (0 if invalid). */
size_t kda_fwd_stages_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype);

/*
 * Chunked prefill ("Method", section 2.1): o[b,t,h,:] = scale * S_t^T q_t
 * for every token, with S_0 = h0[b,h] (zero state if h0 == NULL) and the
 * recurrence above.  The final state S_T is written to ht when ht != NULL;
 * ht may alias h0 (in-place carry from one segment of a sequence to the
 * next).  g is the log-decay input; if gcum != NULL (fp32, from
 * kda_prepare_decay with the same chunk) it is used instead and g may be
 * NULL.  workspace (device, >= kda_fwd_workspace_bytes, 256-byte aligned)
 * holds per-chunk intermediates in flight; its contents on entry are
 * ignored.  Calls that share one workspace must not overlap on the device
 * (one stream, or synchronised streams).  Schedule: one persistent kernel
 * per batch of heads, whose work-groups hand chunk records from producers
 * to the state pass through the workspace; the kernel needs every one of
 * its work-groups resident at once (one per CU), so it must not share the
 * GPU with other work that holds CUs for long; if a hand-off wait exceeds
 * its bound (about a second) the kernel stops early and sets the status
 * word of the workspace, leaving the outputs incomplete (kda_fwd_status).
 * Precondition: g in [gmin, 0] with gmin = -5 (checked under KDA_VALIDATE=1).
 * Errors: KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_DTYPE, KDA_ERR_ALIGN,
 *         KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_RANGE, KDA_ERR_HIP.
 */
int kda_fwd_chunked(const void* q, const void* k, const void* v, const void* g,
                    const float* gcum, const void* beta, float scale, const float* h0,
                    float* ht, float* o, int dtype, int B, int T, int H, int dk, int dv,
                    int chunk, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_fwd_chunked without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same computation, kernels and results
 * as kda_fwd_chunked (bit for bit); the ring buffers and control words live
 * in a library-owned device array of 40 MiB per GPU (a file-scope array in
 * the code object, held until the process ends; no allocation by this call
 * or by the library).  The array holds the rings of 34 heads (fp32 inputs,
 * dk = dv = 128) to 70 heads (bf16 inputs): more heads run as further
 * rounds of the one launch, so no supported size is refused for lack of
 * scratch.
 * Every call on one GPU uses that GPU's array: calls that overlap on one
 * GPU (unordered streams) race and must not be issued.  Status:
 * kda_fwd_status(NULL, stream) reads this array's status word (current
 * device).
 * Errors: as kda_fwd_chunked without KDA_ERR_WORKSPACE for a missing
 * workspace.
 */
int kda_fwd_chunked_noalloc(const void* q, const void* k, const void* v, const void* g,
                            const float* gcum, const void* beta, float scale, const float* h0,
                            float* ht, float* o, int dtype, int B, int T, int H, int dk, int dv,
                            int chunk, void* stream);

/*
 * kda_fwd_chunked for a log-decay with no lower bound (g <= 0, e.g. from
 * kda_prepare_decay_softplus): the comparison point of "Key claims",
 * section 2.1.1 / Fig. 3, where an unbounded decay rules out the rescaled
 * dense diagonal tiles.  The diagonal 16x16 tiles of the two intra-chunk
 * Gram matrices are then sums over position pairs in fp32 (each pair's
 * decay factor formed directly, never above 1); everything else is
 * unchanged.  Arguments, layouts, workspace, errors as kda_fwd_chunked;
 * precondition: g <= 0 and finite (checked under KDA_VALIDATE=1).
 */
int kda_fwd_chunked_unbounded(const void* q, const void* k, const void* v, const void* g,
                              const float* gcum, const void* beta, float scale, const float* h0,
                              float* ht, float* o, int dtype, int B, int T, int H, int dk,
                              int dv, int chunk, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * The same computation as kda_fwd_chunked on a two-kernel schedule with
 * every chunk record stored in the workspace (>= kda_fwd_stages_workspace_bytes):
 * bit 0 of `stages` = the intra-chunk kernel (reads q, k, v, g/gcum, beta;
 * writes the workspace), bit 1 = the state pass (reads the workspace and h0;
 * writes o and ht).  Running stage 2 alone requires a workspace filled by
 * stage 1 with the same sizes, inputs and scale.  No inter-work-group
 * waits; for profiling each stage and for callers that schedule the stages
 * themselves.  Same results as kda_fwd_chunked up to nothing: both
 * schedules run the same per-chunk arithmetic.
 * Adding KDA_STAGES_UNBOUNDED to `stages` runs the unbounded-decay
 * intra-chunk kernel of kda_fwd_chunked_unbounded.
 * Errors: as kda_fwd_chunked, plus KDA_ERR_SHAPE for stages outside 1..3
 * (with or without KDA_STAGES_UNBOUNDED).
 */
#define KDA_STAGES_UNBOUNDED 4
int kda_fwd_chunked_stages(const void* q, const void* k, const void* v, const void* g,
                           const float* gcum, const void* beta, float scale, const float* h0,
                           float* ht, float* o, int dtype, int B, int T, int H, int dk, int dv,
                           int chunk, void* workspace, size_t workspace_bytes, int stages,
                           void* stream);

/*
 * Chunked prefill with the layer's steps on either side fused in (the
 * prologue and epilogue of the path):
 *   - the decay gate: z (instead of g, same layout) and A [H] fp32 are
 *     given; g = -5 Sigmoid(exp(A[h]) z) is formed in fp32 inside the
 *     kernel's scan ("Key claims", section 2.1.1; "Method", section 2.1);
 *   - flags & KDA_LAYER_QK_L2NORM: q and k rows are divided by
 *     sqrt(sum of squares + 1e-6) in the kernel, in fp32, then rounded to
 *     dtype (keys of the delta rule are unit vectors);
 *   - og != NULL ([B,T,H,dv] of dtype): output gate, o = Sigmoid(og) * o
 *     (the pages mention KDA's output gating without defining it; this is
 *     the elementwise sigmoid gate they name for MLA, section 2.1.2).
 * Other arguments, layouts, workspace and errors as kda_fwd_chunked (g and
 * gcum are replaced by z and A); KDA_ERR_NULL for z or A NULL,
 * KDA_ERR_SHAPE for unknown flag bits.
 */
#define KDA_LAYER_QK_L2NORM 1
int kda_fwd_chunked_layer(const void* q, const void* k, const void* v, const void* z,
                          const float* A, const void* beta, const void* og, float scale,
                          const float* h0, float* ht, float* o, int flags, int dtype, int B, int T,
                          int H, int dk, int dv, int chunk, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Variable-length packed prefill with prefix-state snapshots ("Key claims",
 * Infrastructure: states kept at prefix boundaries for reuse; "Method",
 * section 2.1).  N sequences are packed along the token axis: q, k, g
 * [1,T,H,dk], v [1,T,H,dv], beta [1,T,H], o [1,T,H,dv] fp32, gcum (if used)
 * [1,T,H,dk]; sequence i is tokens cu_seqlens[i] .. cu_seqlens[i+1]-1 of
 * them, with its own chunks (every chunk starts at the sequence start), its
 * own initial state h0[i] and final state ht[i] ([N,H,dk,dv] fp32; NULL h0:
 * zero states; ht may alias h0).  cu_seqlens is a HOST array of N+1 ints
 * with cu_seqlens[0] = 0, non-decreasing, cu_seqlens[N] = T; empty
 * sequences are allowed (ht[i] = h0[i]).
 * Snapshots: when snap != NULL and snap_every > 0, the state after every
 * snap_every chunks of a sequence (after tokens 64 j snap_every, j = 1, 2,
 * ..., strictly before the sequence's end) is written to snap
 * [S,H,dk,dv] fp32, sequences in order, snapshots in order within one;
 * S = kda_fwd_varlen_snapshots(cu_seqlens, N, snap_every, chunk).
 * workspace: kda_fwd_workspace_bytes(1, T, H, dk, dv, chunk, dtype) bytes.
 * Up to 128 sequences: one fused launch for all of them (each head's chunks
 * of every sequence, in order, with the state restarted at each sequence's
 * first chunk); more sequences: one fused launch per non-empty sequence, in
 * order on `stream`.  The status word (kda_fwd_status) covers the call.  gcum must be NULL (a
 * gcum of the packed axis restarts at multiples of 64 tokens, not at each
 * sequence's own chunks): KDA_ERR_UNSUPPORTED otherwise.
 * Errors: as kda_fwd_chunked; KDA_ERR_NULL for cu_seqlens == NULL,
 * KDA_ERR_SHAPE for inconsistent cu_seqlens or snap_every < 0,
 * KDA_ERR_ALIGN for an unaligned snap, KDA_ERR_UNSUPPORTED for gcum.
 */
int kda_fwd_chunked_varlen(const void* q, const void* k, const void* v, const void* g,
                           const float* gcum, const void* beta, float scale,
                           const int* cu_seqlens, int N, const float* h0, float* ht, float* o,
                           float* snap, int snap_every, int dtype, int T, int H, int dk, int dv,
                           int chunk, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Status of the last call that used `workspace` (a workspace of the fused
 * prefill calls: kda_fwd_chunked, _unbounded, _layer, _varlen, or of
 * kda_bwd_chunked, whose forward recompute it covers): synchronises
 * `stream`, then returns KDA_OK, or KDA_ERR_INCOMPLETE if a hand-off wait
 * of that call expired (its outputs are incomplete).  workspace NULL: the
 * scratch of kda_fwd_chunked_noalloc on the current device.  Errors:
 * KDA_ERR_ALIGN (workspace not 256-byte aligned), KDA_ERR_HIP.
 */
int kda_fwd_status(const void* workspace, void* stream);

/* Device address of the status word of `workspace` (one int; non-zero =
 * KDA_ERR_INCOMPLETE as above), for an asynchronous read ordered after the
 * call on its stream.  NULL for a NULL workspace. */
const int* kda_fwd_status_word(const void* workspace);

/* Number of snapshots kda_fwd_chunked_varlen writes for these sequences
 * (host computation; -1 for invalid arguments, including snap_every <= 0). */
long long kda_fwd_varlen_snapshots(const int* cu_seqlens, int N, int snap_every, int chunk);

/*
 * Decode step (page "How a Frontier Model Gets Built...", "Technical
 * Details": fixed-size running state instead of a KV cache): one new token
 * per (b, h).  state [B,H,dk,dv] fp32 is read and overwritten in place with
 * S_t; o[b,h,:] = scale * S_t^T q.
 * Precondition: g in [gmin, 0] with gmin = -5 (checked under KDA_VALIDATE=1).
 * Errors: KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_DTYPE, KDA_ERR_ALIGN,
 *         KDA_ERR_UNSUPPORTED, KDA_ERR_RANGE, KDA_ERR_HIP.
 */
int kda_decode_step(const void* q, const void* k, const void* v, const void* g,
                    const void* beta, float scale, float* state, float* o, int dtype,
                    int B, int H, int dk, int dv, void* stream);

/*
 * Decode step with the layer's steps on either side fused in, as
 * kda_fwd_chunked_layer does for the prefill (so that a sequence prefilled
 * with the layer call continues with the same arithmetic):
 *   - z [B,H,dk] of dtype instead of g, A [H] fp32: g = -5 Sigmoid(exp(A[h]) z)
 *     in fp32 ("Key claims", section 2.1.1; "Method", section 2.1);
 *   - flags & KDA_LAYER_QK_L2NORM: q and k rows divided by
 *     sqrt(sum of squares + 1e-6) in fp32, then rounded to dtype;
 *   - og != NULL ([B,H,dv] of dtype): o = Sigmoid(og) * o.
 * Other arguments, layouts and errors as kda_decode_step; z is not range
 * checked (the gate maps every finite z into [-5, 0]); KDA_ERR_NULL for z
 * or A NULL, KDA_ERR_SHAPE for unknown flag bits, KDA_ERR_ALIGN for A or og
 * not 16-byte aligned.
 */
int kda_decode_step_layer(const void* q, const void* k, const void* v, const void* z,
                          const float* A, const void* beta, const void* og, float scale,
                          float* state, float* o, int flags, int dtype, int B, int H, int dk,
                          int dv, void* stream);

/*
 * Backward of the chunked prefill: gradients of a loss L with respect to the
 * inputs of kda_fwd_chunked, given dout = dL/do and dht = dL/dht (Kimi K3
 * technical report summary, "Method", section 2.1: the chunkwise form; its
 * gradient by the reverse-mode chain rule, chunk by chunk from the last).
 *
 * Inputs as kda_fwd_chunked (q, k, g [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H];
 * dtype KDA_F32 or KDA_BF16; g in [-5, 0), the bounded gate) plus dout
 * [B,T,H,dv] fp32 and dht [B,H,dk,dv] fp32 (NULL = no gradient reaches the
 * final state); h0 NULL = zero initial state.
 * Outputs, all fp32, overwritten: dq, dk, dg [B,T,H,dk]; dv [B,T,H,dv];
 * dbeta [B,T,H]; dh0 [B,H,dk,dv] (NULL = not written).  dg is the gradient
 * with respect to the per-token decay g (apply the gate's own derivative
 * for z and A).
 * The call recomputes the forward pass (keeping the state entering every
 * chunk) inside `workspace` of at least kda_bwd_workspace_bytes bytes
 * (256-byte aligned, owned by the caller, contents undefined afterwards);
 * it allocates nothing and returns without synchronising.  The recompute
 * is the fused prefill: kda_fwd_status(workspace) reports whether it
 * completed (gradients are meaningless otherwise).
 * Errors: as kda_fwd_chunked, KDA_ERR_NULL also for a NULL dout or output.
 */
size_t kda_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype);
int kda_bwd_chunked(const void* q, const void* k, const void* v, const void* g, const void* beta,
                    float scale, const float* h0, const float* dout, const float* dht, float* dq,
                    float* dk_, float* dv_, float* dg, float* dbeta, float* dh0, int dtype, int B,
                    int T, int H, int dk, int dv, int chunk, void* workspace,
                    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
