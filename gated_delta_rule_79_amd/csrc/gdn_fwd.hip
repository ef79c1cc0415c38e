// Chunkwise-parallel forward of the gated delta rule.
//
// "Gated Delta Networks: Improving Mamba2 with Delta Rule" (paper review),
// "Method" and "Goal": the gate is folded into DeltaNet's chunkwise algorithm
// (WY representation + UT transform) so that the recurrence stays a sequence
// of matrix products.  Unrolling S_t = S_{t-1} a_t (I - b_t k_t k_t^T)
// + b_t v_t k_t^T over one chunk of c tokens, with the stored state M = S^T,
// the chunk-local inclusive cumulative log-gate g and gamma = exp(g):
//
//   A_ri = b_r exp(g_r - g_i) k_r.k_i  (i < r),    T = (I + A)^-1
//   W = T diag(b gamma) K,   U = T diag(b) V,      E = U - W M0
//   O = diag(gamma) Q M0 + P E,  P_ri = exp(g_r - g_i) q_r.k_i  (i <= r)
//   M_c = gamma_c M0 + (K (.) exp(g_c - g))^T E
//
// (the per-channel gate moves every exp(g_r - g_i) inside the k-sums).
//
// Kernels, in launch order:
//   prep (one workgroup per chunk and head, all in parallel): cumulative gate,
//     K K^T and Q K^T on the matrix cores, the unit lower-triangular inverse T
//     (16x16 diagonal blocks by column substitution, off-diagonal blocks by
//     block rows on fp32 MFMA), W and U products; writes every operand the
//     state pass needs already in MFMA fragment order.
//   The state pass carries M across the chunks of each sequence.  Over one
//   chunk M -> (gamma_c I - K~^T W) M + K~^T U is affine in M, so so is the
//   map over a run of chunks (a segment): M_end = Phi M_start + M0.  When the
//   (sequence, head) chains alone cannot fill the GPU, the chains are cut
//   into segments and the pass runs in three launches:
//   trans   (per segment, head and group of 16-column tiles): M0 from a zero
//           state with U, and Phi by running the identity's columns through
//           the same chain without U.
//   combine (per sequence, head and dv tile): M_{j+1} = Phi_j M_j + M0_j
//           over the segments, the entering state of each segment.
//   scan    (per segment, head and group of eight 16-column dv tiles, one
//           wave per tile): E = U - W M, O = Q~ M + P E, M <- gamma_c M
//           + K~^T E from the segment's entering state; writes O and the
//           final state.  Unsplit chains run the scan alone from S0.
//   The state tile and E accumulators are fed straight back as MFMA operands
//   in a permuted K order (see perm_k), so the sequential chain never goes
//   through LDS; the per-chunk operands are staged into LDS by direct
//   global-to-LDS loads, double-buffered one chunk ahead.  dv columns are
//   independent, so tiles need no communication.

#include "gdn_fwd_kernels.hpp"

namespace gdn {

// ------------------------------------------------------------ chunk map ---

namespace {

// Exclusive prefix sum over one 256-wide block; returns the thread's offset
// and adds the block total to *carry (all threads see the same value).
__device__ int block_excl_scan(int x, int* s_scan, int* carry) {
  const int tid = threadIdx.x;
  s_scan[tid] = x;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int y = tid >= d ? s_scan[tid - d] : 0;
    __syncthreads();
    s_scan[tid] += y;
    __syncthreads();
  }
  const int excl = *carry + s_scan[tid] - x;
  const int total = s_scan[255];
  __syncthreads();
  if (tid == 0) *carry += total;
  __syncthreads();
  return excl;
}

// Varlen chunk map and, for L > 0, the segment table: sequence n owns chunk
// slots [first[n], first[n+1]) and segment slots [sfirst[n], sfirst[n+1]),
// at least one segment even when it has no chunk.
// cu counts tokens; with 2^lnh delta steps per token the table counts steps.
__global__ __launch_bounds__(256) void chunk_map_kernel(
    const int32_t* __restrict__ cu, int nseq, int T, int C, int64_t nslots,
    int4* __restrict__ tab, int32_t* __restrict__ first, int L, int64_t nsegs,
    int4* __restrict__ stab, int32_t* __restrict__ sfirst, int lnh) {
  const int tid = threadIdx.x;
  for (int64_t i = tid; i < nslots; i += 256) tab[i] = make_int4(-1, 0, 0, 0);
  if (L > 0)
    for (int64_t i = tid; i < nsegs; i += 256) stab[i] = make_int4(-1, 0, 0, 0);
  __shared__ int s_scan[256];
  __shared__ int s_carry[2];
  if (tid < 2) s_carry[tid] = 0;
  __syncthreads();
  for (int base = 0; base < nseq; base += 256) {
    const int n = base + tid;
    int cnt = 0, st = 0, en = 0;
    if (n < nseq) {
      const int tt = T >> lnh;  // tokens
      st = min(max(cu[n], 0), tt);
      en = min(max(cu[n + 1], st), tt);
      st <<= lnh;
      en <<= lnh;
      cnt = (en - st + C - 1) / C;
    }
    const int excl = block_excl_scan(cnt, s_scan, &s_carry[0]);
    const int c0 = static_cast<int>(min<int64_t>(excl, nslots));
    const int c1 = static_cast<int>(min<int64_t>(static_cast<int64_t>(excl) + cnt, nslots));
    if (n < nseq) {
      first[n] = c0;
      for (int j = 0; j < c1 - c0; ++j)
        tab[c0 + j] = make_int4(n, st + j * C, min(C, en - st - j * C), 0);
    }
    if (L > 0) {
      const int ns = n < nseq ? max(1, (c1 - c0 + L - 1) / L) : 0;
      const int sx = block_excl_scan(ns, s_scan, &s_carry[1]);
      if (n < nseq) {
        sfirst[n] = static_cast<int>(min<int64_t>(sx, nsegs));
        for (int j = 0; j < ns; ++j) {
          const int64_t slot = static_cast<int64_t>(sx) + j;
          if (slot < nsegs)
            stab[slot] = make_int4(n, c0 + j * L, min(c0 + (j + 1) * L, c1), j);
        }
      }
    }
  }
  if (tid == 0) {
    first[nseq] = static_cast<int>(min<int64_t>(s_carry[0], nslots));
    if (L > 0) sfirst[nseq] = static_cast<int>(min<int64_t>(s_carry[1], nsegs));
  }
}

}  // namespace

hipError_t launch_chunk_map(const Problem& p, char* map_base, hipStream_t s) {
  const ChunkMap m = make_chunk_map(p, map_base);
  const SegMap sm = make_seg_map(p, map_base, p.seg);
  StageScope scope(GDN_STAGE_CHUNK_MAP, s);
  hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(256), 0, s, p.cu_seqlens,
                     p.nseq, p.T, p.chunk, p.nchunks,
                     const_cast<int4*>(m.tab), const_cast<int32_t*>(m.first),
                     p.seg, p.nsegs, const_cast<int4*>(sm.tab),
                     const_cast<int32_t*>(sm.first), p.lnh);
  return hipGetLastError();
}


// ------------------------------------------------------------ dispatch ---

namespace {

template <int C, int DK, typename IO, int GATE>
hipError_t run_fwd(const Problem& p, const void* q, const void* k,
                   const void* v, const void* beta, const void* la,
                   const float* s0, void* o, float* s_final, char* ws,
                   hipStream_t s) {
  constexpr int ob = opstore<IO>::bytes;
  const FwdLayout L(C, DK, p.dv, ob, GATE == GDN_GATE_CHANNEL);
  char* map_base = ws;
  char* ops = ws + chunk_map_bytes(p);
  const FwdBuffers buf = make_buffers(ops, L);
  const SegBuffers sb = make_seg_buffers(p, ops + size_t(p.nchunks) * p.H * L.per_ch, ob);
  const ChunkMap map = make_chunk_map(p, map_base);
  const SegMap sm = make_seg_map(p, map_base, p.seg);
  const int ndvt = p.dv / 16;
  hipError_t e;
  if (p.varlen) {
    e = launch_chunk_map(p, map_base, s);
    if (e != hipSuccess) return e;
  }
  if (p.nchunks > 0) {
    StageScope scope(GDN_STAGE_FWD_PREP, s);
    if constexpr (GATE == GDN_GATE_CHANNEL)
      hipLaunchKernelGGL((fwd_prep_kernel<C, DK, IO, GATE, false, kPrepChWaves>),
                         dim3(static_cast<unsigned>(p.nchunks * p.H)), dim3(64 * kPrepChWaves),
                         0, s, map, p.H, p.dv, p.nchunks, q, k, v, beta, la,
                         p.gdt == GDN_BF16, buf, p.beta_w);
    else
      if (p.conv_w > 0)
        hipLaunchKernelGGL((fwd_prep_sg_kernel<C, DK, IO, GATE, false, true>),
                           dim3(static_cast<unsigned>(p.nchunks * p.H)),
                           dim3(64 * prep_waves(C)), 0, s, map, p.H, p.dv, p.nchunks, q, k, v,
                           beta, la, p.gdt == GDN_BF16, buf, p.lnh, p.qknorm, p.parent,
                           p.beta_w, p.conv_w, p.conv_tk, p.conv_tv);
      else
        hipLaunchKernelGGL((fwd_prep_sg_kernel<C, DK, IO, GATE>),
                           dim3(static_cast<unsigned>(p.nchunks * p.H)),
                           dim3(64 * prep_waves(C)), 0, s, map, p.H, p.dv, p.nchunks, q, k, v,
                           beta, la, p.gdt == GDN_BF16, buf, p.lnh, p.qknorm, p.parent,
                           p.beta_w);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.seg > 0 && p.nchunks > 0) {
    {
      StageScope scope(GDN_STAGE_FWD_TRANS, s);
      const int64_t ngrp = (ndvt + DK / 16 + kTransGroup - 1) / kTransGroup;
      hipLaunchKernelGGL((fwd_trans_kernel<C, DK, IO, GATE>),
                         dim3(static_cast<unsigned>(p.nsegs * p.H * ngrp)),
                         dim3(64 * kTransWaves), 0, s, map, sm, p.H, p.dv, p.nchunks,
                         buf, sb, false);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    {
      StageScope scope(GDN_STAGE_FWD_COMBINE, s);
      hipLaunchKernelGGL((fwd_combine_kernel<DK, IO>),
                         dim3(static_cast<unsigned>(p.nseq * p.H * ndvt)),
                         dim3(64 * ((DK + 31) / 32)), 0, s, map, sm, p.H, p.dv,
                         s0, sb);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const int64_t nwork = p.nsegs * p.H * ((ndvt + kScanGroup - 1) / kScanGroup);
  StageScope scope(GDN_STAGE_FWD_SCAN, s);
  hipLaunchKernelGGL((fwd_scan_kernel<C, DK, IO, GATE>),
                     dim3(static_cast<unsigned>(nwork)), dim3(64 * kScanWaves), 0, s,
                     map, sm, p.H, p.dv, p.nchunks, q, s0, o, s_final, buf, sb,
                     static_cast<float*>(nullptr), p.lnh);
  return hipGetLastError();
}

template <int C, int DK, typename IO>
hipError_t fwd_gate(const Problem& p, const void* q, const void* k,
                    const void* v, const void* beta, const void* la,
                    const float* s0, void* o, float* sf, char* ws,
                    hipStream_t s) {
  switch (p.gate) {
    case GDN_GATE_NONE:
      return run_fwd<C, DK, IO, GDN_GATE_NONE>(p, q, k, v, beta, la, s0, o, sf, ws, s);
    case GDN_GATE_SCALAR:
      return run_fwd<C, DK, IO, GDN_GATE_SCALAR>(p, q, k, v, beta, la, s0, o, sf, ws, s);
    default:
      return run_fwd<C, DK, IO, GDN_GATE_CHANNEL>(p, q, k, v, beta, la, s0, o, sf, ws, s);
  }
}

template <int C, int DK>
hipError_t fwd_types(const Problem& p, const void* q, const void* k,
                     const void* v, const void* beta, const void* la,
                     const float* s0, void* o, float* sf, char* ws,
                     hipStream_t s) {
  if (p.io == GDN_BF16)
    return fwd_gate<C, DK, bf16_t>(p, q, k, v, beta, la, s0, o, sf, ws, s);
  return fwd_gate<C, DK, f32_t>(p, q, k, v, beta, la, s0, o, sf, ws, s);
}

template <int C>
hipError_t fwd_dk(const Problem& p, const void* q, const void* k,
                  const void* v, const void* beta, const void* la,
                  const float* s0, void* o, float* sf, char* ws,
                  hipStream_t s) {
  switch (p.dk) {
    case 16: return fwd_types<C, 16>(p, q, k, v, beta, la, s0, o, sf, ws, s);
    case 32: return fwd_types<C, 32>(p, q, k, v, beta, la, s0, o, sf, ws, s);
    case 64: return fwd_types<C, 64>(p, q, k, v, beta, la, s0, o, sf, ws, s);
    default: return fwd_types<C, 128>(p, q, k, v, beta, la, s0, o, sf, ws, s);
  }
}

}  // namespace

size_t fwd_workspace_bytes(const Problem& p) {
  const FwdLayout L(p.chunk, p.dk, p.dv, p.io == GDN_BF16 ? 2 : 4,
                    p.gate == GDN_GATE_CHANNEL);
  return chunk_map_bytes(p) + size_t(p.nchunks) * p.H * L.per_ch +
         seg_buffer_bytes(p, p.io == GDN_BF16 ? 2 : 4);
}

hipError_t launch_fwd(const Problem& p, const void* q, const void* k,
                      const void* v, const void* beta, const void* la,
                      const float* s0, void* o, float* s_final, void* ws,
                      hipStream_t s) {
  char* w = static_cast<char*>(ws);
  switch (p.chunk) {
    case 16: return fwd_dk<16>(p, q, k, v, beta, la, s0, o, s_final, w, s);
    case 32: return fwd_dk<32>(p, q, k, v, beta, la, s0, o, s_final, w, s);
    default: return fwd_dk<64>(p, q, k, v, beta, la, s0, o, s_final, w, s);
  }
}

}  // namespace gdn
