// Internal host-side interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// Validated problem, in host-friendly form.
struct Problem {
  int B, T, H, dk, dv, chunk;
  int nseq;                   // number of independent sequences (B or varlen)
  bool varlen;
  const int32_t* cu_seqlens;  // device
  int seg_req;                // gdn_problem::seg_chunks (0 automatic,
                              // > 0 chunks per segment, < 0 never split)
  int io;                     // gdn_dtype
  int gdt;                    // gdn_dtype of beta / log_alpha
  int gate;                   // gdn_gate
  int lnh;                    // log2 of the delta steps per token (Householder
                              // products); T counts steps, q / o / log alpha
                              // / cu_seqlens count tokens.  0 otherwise.
  bool qknorm;                // forward only: q and k rows L2-normalised
  const int32_t* parent;      // forward only: draft trees, one per chunk
                              // (device, node parents inside each tree)
  const void* beta_w;         // forward and decode: write strength of the
                              // decoupled erase/write rule (gate_dtype, like
                              // beta, which is then the erase strength);
                              // nullptr: beta does both
  int conv_w;                 // forward, per-token gates: > 0 fuses the short
                              // causal convolution of k and v (width conv_w,
                              // fp32 taps [H, d, conv_w]) and SiLU into the
                              // prep's staging, k rows then L2-normalised;
                              // q arrives processed.  0 otherwise.
  const float* conv_tk;       // device taps of k and v
  const float* conv_tv;
  // derived
  int64_t nchunks;            // chunk slots per head (upper bound in varlen)
  int seg;                    // chunks per segment of the forward state pass
                              // (0: one segment per sequence)
  int64_t nsegs;              // segment slots (upper bound in varlen)
};

// Segment length the forward state pass uses for this problem (0 = whole
// sequences), from the sizes and the requested seg_req (gdn_api.hip).
int plan_segments(const Problem& p);
// Segment slots for p.seg (upper bound in varlen).
int64_t seg_slots_host(const Problem& p);

// Stage timing (gdn_api.hip): no-ops unless gdn_profile_enable(1).
void prof_begin(int stage, hipStream_t s);
void prof_end(int stage, hipStream_t s);

// Brackets one kernel launch with prof_begin / prof_end.
struct StageScope {
  int stage;
  hipStream_t stream;
  StageScope(int st, hipStream_t s) : stage(st), stream(s) { prof_begin(st, s); }
  ~StageScope() { prof_end(stage, stream); }
};

// Decode launcher (gdn_decode.hip).
hipError_t launch_decode(const Problem& p, const void* q, const void* k,
                         const void* v, const void* beta, const void* la,
                         float* state, void* o, hipStream_t s);

// Decode with Householder-product transitions (gdn_decode.hip).
hipError_t launch_decode_product(const Problem& p, int nh, const void* q, const void* k,
                                 const void* v, const void* beta, const void* la,
                                 float* state, void* o, hipStream_t s);

// Draft-tree commit (gdn_tree.hip).
hipError_t launch_tree_commit(const Problem& p, const int32_t* parent,
                              const int32_t* accepted, const void* k, const void* v,
                              const void* beta, const void* la, float* state,
                              hipStream_t s);

// q, k, v prologue (gdn_prologue.hip): y = silu(conv(x)) with taps [H, D, W]
// (taps == nullptr: y = x), rows L2-normalised when `normalize`; x, y
// [B * T, H, D] in p.io.
hipError_t launch_prologue(const Problem& p, int D, int W, const void* x, const float* taps,
                           bool normalize, void* y, hipStream_t s);
// Adjoint of the prologue path (dz, then dx with per-block tap partials,
// then the partials summed in block order); workspace: dz in fp32 and the
// partials.
size_t prologue_bwd_workspace_bytes(const Problem& p, int D, int W);
hipError_t launch_prologue_bwd(const Problem& p, int D, int W, const void* x, const float* taps,
                               bool normalize, const void* dy, void* dx, float* dtaps, void* ws,
                               hipStream_t s);

// Forward (gdn_fwd.hip).
size_t fwd_workspace_bytes(const Problem& p);
hipError_t launch_fwd(const Problem& p, const void* q, const void* k,
                      const void* v, const void* beta, const void* la,
                      const float* s0, void* o, float* s_final, void* ws,
                      hipStream_t s);

// Backward (gdn_bwd.hip).  bwd_supported: whether the per-chunk gradient
// kernel's LDS plan fits for these sizes (fp32 inputs with the per-channel
// gate at dk = 128 need chunk <= 32).
bool bwd_supported(const Problem& p);
size_t bwd_workspace_bytes(const Problem& p);
hipError_t launch_bwd(const Problem& p, const void* q, const void* k,
                      const void* v, const void* beta, const void* la,
                      const float* s0, const void* d_o, const float* ds_final,
                      void* dq, void* dk, void* dv, float* dbeta, float* dla,
                      float* ds0, void* ws, hipStream_t s);

}  // namespace gdn
