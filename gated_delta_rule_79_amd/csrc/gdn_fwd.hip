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
// Two kernels:
//   prep (one workgroup per chunk and head, all in parallel): cumulative gate,
//     K K^T and Q K^T on the matrix cores, the unit lower-triangular inverse T
//     in LDS (16x16 diagonal blocks by column substitution, then block rows),
//     W and U products; writes every operand the state pass needs already in
//     MFMA fragment order.
//   scan (one wave per sequence, head and 16-column slab of dv): carries the
//     fp32 state slab in registers across the chunks of the sequence.  Each
//     chunk is E = U - W M, O = Q~ M + P E, M <- gamma_c M + K~^T E.  The
//     state and E accumulators are fed straight back as MFMA operands in a
//     permuted K order (see perm_k), so the sequential chain never goes
//     through LDS.  dv columns are independent, so slabs need no
//     communication.

#include "gdn_fwd_kernels.hpp"

namespace gdn {

// ------------------------------------------------------------ chunk map ---

namespace {

__global__ __launch_bounds__(256) void chunk_map_kernel(
    const int32_t* __restrict__ cu, int nseq, int T, int C, int64_t nslots,
    int4* __restrict__ tab, int32_t* __restrict__ first) {
  const int tid = threadIdx.x;
  for (int64_t i = tid; i < nslots; i += 256) tab[i] = make_int4(-1, 0, 0, 0);
  __shared__ int s_scan[256];
  __shared__ int s_carry;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < nseq; base += 256) {
    const int n = base + tid;
    int cnt = 0, st = 0, en = 0;
    if (n < nseq) {
      st = min(max(cu[n], 0), T);
      en = min(max(cu[n + 1], st), T);
      cnt = (en - st + C - 1) / C;
    }
    s_scan[tid] = cnt;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int y = tid >= d ? s_scan[tid - d] : 0;
      __syncthreads();
      s_scan[tid] += y;
      __syncthreads();
    }
    const int excl = s_carry + s_scan[tid] - cnt;
    if (n < nseq) {
      first[n] = static_cast<int>(min<int64_t>(excl, nslots));
      for (int j = 0; j < cnt; ++j) {
        const int64_t slot = static_cast<int64_t>(excl) + j;
        if (slot < nslots)
          tab[slot] = make_int4(n, st + j * C, min(C, en - st - j * C), 0);
      }
    }
    __syncthreads();
    if (tid == 0) s_carry += s_scan[255];
    __syncthreads();
  }
  if (tid == 0) first[nseq] = static_cast<int>(min<int64_t>(s_carry, nslots));
}

}  // namespace

hipError_t launch_chunk_map(const Problem& p, char* map_base, hipStream_t s) {
  ChunkMap m = make_chunk_map(p, map_base);
  StageScope scope(GDN_STAGE_CHUNK_MAP, s);
  hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(256), 0, s, p.cu_seqlens,
                     p.nseq, p.T, p.chunk, p.nchunks,
                     const_cast<int4*>(m.tab), const_cast<int32_t*>(m.first));
  return hipGetLastError();
}


// ------------------------------------------------------------ dispatch ---

namespace {

template <int C, int DK, typename IO, int GATE>
hipError_t run_fwd(const Problem& p, const void* q, const void* k,
                   const void* v, const void* beta, const void* la,
                   const float* s0, void* o, float* s_final, char* ws,
                   hipStream_t s) {
  const FwdLayout L(C, DK, p.dv, opstore<IO>::bytes, GATE == GDN_GATE_CHANNEL);
  char* map_base = ws;
  char* ops = ws + chunk_map_bytes(p);
  const FwdBuffers buf = make_buffers(ops, L);
  const ChunkMap map = make_chunk_map(p, map_base);
  if (p.varlen) {
    hipError_t e = launch_chunk_map(p, map_base, s);
    if (e != hipSuccess) return e;
  }
  if (p.nchunks > 0) {
    StageScope scope(GDN_STAGE_FWD_PREP, s);
    hipLaunchKernelGGL((fwd_prep_kernel<C, DK, IO, GATE>),
                       dim3(static_cast<unsigned>(p.nchunks * p.H)), dim3(256),
                       0, s, map, p.H, p.dv, p.nchunks, q, k, v, beta, la,
                       p.gdt == GDN_BF16, buf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nwork = static_cast<int64_t>(p.nseq) * p.H * (p.dv / 16);
  // q through a buffer resource when its byte size fits the 32-bit range
  const int64_t qb = static_cast<int64_t>(p.B) * p.T * p.H * DK * io<IO>::bytes;
  const uint32_t q_bytes = qb < (int64_t(1) << 31) ? static_cast<uint32_t>(qb) : 0u;
  StageScope scope(GDN_STAGE_FWD_SCAN, s);
  hipLaunchKernelGGL((fwd_scan_kernel<C, DK, IO, GATE>),
                     dim3(static_cast<unsigned>(nwork)), dim3(128), 0, s, map,
                     p.H, p.dv, p.nchunks, q, q_bytes, s0, o, s_final, buf,
                     static_cast<float*>(nullptr));
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
  return chunk_map_bytes(p) + size_t(p.nchunks) * p.H * L.per_ch;
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
