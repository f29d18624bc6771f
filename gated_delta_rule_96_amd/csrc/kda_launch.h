// Internal host-side launch interface between the C ABI (kda_api.cpp) and
// the kernel translation units.  Arguments are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Decay preparation: gate (z != nullptr; softplus != 0 selects the unbounded
// -Softplus gate instead of gmin * Sigmoid) and/or chunk-local cumsum.
hipError_t launch_prepare_decay(int is_bf16, const void* z, const float* A, float gmin, void* g,
                                float* gcum, int B, int T, int H, int dk, int chunk, int softplus,
                                hipStream_t stream);

// Opt-in range check of a log-decay input (KDA_VALIDATE=1 in the
// environment: validate_requested()).  bounded != 0: every g in [gmin, 0];
// otherwise g <= 0; finite in both cases.  With gcum != nullptr the per-row
// decays it encodes are checked instead of g.  g / gcum are [B, T, HD]
// (HD = H * dk).  Synchronises `stream`; *in_range = 1 if every value passes.
bool validate_requested();
hipError_t validate_decay(int is_bf16, const void* g, const float* gcum, int bounded, float gmin, int B, int T,
                          int HD, int chunk, hipStream_t stream, int* in_range);

// Bytes of one per-chunk record of the prefill workspace.
size_t fwd_record_bytes(int is_bf16, int dk, int dv);
// Workspace of the fused single-pass schedule (ring buffers + control words).
size_t fwd_fused_workspace_bytes(int is_bf16, int nbh, int dk, int dv);

// Up to kMaxVarSeq packed sequences of one variable-length prefill, carried
// in the fused kernel's launch arguments: sequence i is tokens cu[i] ..
// cu[i+1]-1 of the packed axis, its chunks (every chunk starts at the
// sequence start) are stream chunks cc[i] .. cc[i+1]-1 of every head, and its
// first snapshot is snapshot sb[i].  n = 0: one plain sequence per (b, h).
constexpr int kMaxVarSeq = 128;
struct VarSeg {
  int n;
  int cu[kMaxVarSeq + 1];
  int cc[kMaxVarSeq + 1];
  int sb[kMaxVarSeq + 1];
};

// Chunked prefill, fused schedule (one persistent kernel per batch of heads).
// unbounded != 0: the decay may go below -5 (diagonal tiles by position pairs).
// snap != nullptr, snap_every > 0: states after every snap_every chunks
// (excluding the end) to snap[j][b * H + h][dk][dv].
// var != nullptr (B = 1): the packed sequences above, h0 / ht [n][H][dk][dv]
// (h0 nullable), snapshots numbered per sequence from sb[i]; sequences
// without tokens are not touched.
// layer_flags (1: g is z, gate with A fused into the scan; 2: q/k rows L2
// normalised in-kernel) and og (output gate pre-activation, nullable).
hipError_t launch_fwd_fused(int is_bf16, const void* q, const void* k, const void* v, const void* g,
                            const float* gcum, const void* beta, float scale, const float* h0, float* ht, float* o,
                            int B, int T, int H, int dk, int dv, void* workspace, size_t workspace_bytes,
                            int unbounded, float* snap, int snap_every, const float* A, const void* og,
                            int layer_flags, hipStream_t stream, const VarSeg* var = nullptr);

// Chunked prefill, two-stage schedule: bit 0 intra-chunk kernel, bit 1 state pass.
hipError_t launch_fwd_stages(int is_bf16, const void* q, const void* k, const void* v, const void* g,
                             const float* gcum, const void* beta, float scale, const float* h0, float* ht, float* o,
                             int B, int T, int H, int dk, int dv, void* workspace, int stages, int unbounded,
                             float* snap, int snap_every, hipStream_t stream);

// Zero-fills nwords 4-byte words on the stream (a kernel, not a memset node).
hipError_t launch_zero_words(void* p, size_t nwords, hipStream_t stream);

// Zeroes the status words (the first 16 ints, error word at [8]) of a
// prefill workspace; called once per API call, before its launches.
hipError_t launch_clear_status(void* ws, hipStream_t stream);

// Library-owned scratch of the allocation-free prefill (a file-scope device
// array, one per GPU): its device address on the current device, fetched
// with hipGetSymbolAddress on the first call there.  40 MiB hold the ring of
// 34 heads with fp32 inputs at dk = dv = 128 (the largest record, 1.16 MB per
// head) and 70 heads with bf16 inputs; larger batches of heads run as
// further launches of the same kernel.
constexpr size_t kNoAllocScratchBytes = (size_t)40 << 20;
hipError_t noalloc_scratch(void** ptr);


// The decode step's layer steps: g holds z and the gate is formed from
// A [H] fp32; flags & kDecodeLayerNormQK normalises the q and k rows; og
// [B,H,dv] of the input type (or null) gates the output.
constexpr int kDecodeLayerNormQK = 2;
struct DecodeLayer {
  const float* A;
  const void* og;
  int flags;
};

// One decode token per (b, h), state updated in place (lay: the layer
// variant, or null for the plain step).
hipError_t launch_decode_step(int is_bf16, const void* q, const void* k, const void* v,
                              const void* g, const void* beta, float scale, float* state, float* o,
                              int B, int H, int dk, int dv, hipStream_t stream,
                              const DecodeLayer* lay = nullptr);

// Backward: fp32 words of one per-chunk record, and the three kernels after
// a forward pass that kept the state entering every chunk in snap
// ([chunk - 1][b * H + h][dk][dv]).  rec, dN ([chunk][dk][dv] per head) and
// dU ([chunk][64][dv] per head) are workspace.
size_t bwd_record_words(int dk, int dv);
hipError_t launch_bwd_chunks(int is_bf16, const void* q, const void* k, const void* v, const void* g,
                             const void* beta, const float* dO, float scale, const float* h0, const float* dht,
                             const float* snap, float* rec, float* dN, float* dU, int B, int T, int H, int dk,
                             int dv, float* dq, float* dk_, float* dv_, float* dg, float* dbeta, float* dh0,
                             hipStream_t st);

}  // namespace kda
