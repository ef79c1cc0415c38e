// Shared pieces of the chunkwise forward and backward kernels: chunk
// bookkeeping, the varlen chunk map, workspace layout and fragment helpers.
#pragma once

#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

// ------------------------------------------------------------ chunk map ---
// A chunk slot c (per head) covers tokens [tok0, tok0 + len) of one sequence.
// Dense batches compute it; varlen batches read a table that
// build_chunk_map fills on the device from cu_seqlens.

struct ChunkMap {
  int varlen;
  int T, C, nt;                 // dense: tokens per sequence, chunk, chunks/seq
  const int4* tab;              // varlen: [nchunks] (seq, tok0, len, -); seq < 0 unused
  const int32_t* first;         // varlen: [nseq + 1] first chunk slot of each seq
};

struct ChunkInfo {
  int seq;       // sequence index (dense: batch index); < 0 = unused slot
  int64_t tok0;  // global token index of the chunk's first token
  int len;       // tokens in the chunk, 1..C
};

__device__ inline ChunkInfo chunk_info(const ChunkMap& m, int c) {
  ChunkInfo r;
  if (!m.varlen) {
    const int b = c / m.nt, j = c % m.nt;
    r.seq = b;
    r.tok0 = static_cast<int64_t>(b) * m.T + static_cast<int64_t>(j) * m.C;
    r.len = min(m.C, m.T - j * m.C);
  } else {
    const int4 e = m.tab[c];
    r.seq = e.x;
    r.tok0 = e.y;
    r.len = e.z;
  }
  return r;
}

// Chunks of one sequence: slots [c_begin, c_end).
__device__ inline void seq_chunks(const ChunkMap& m, int seq, int* c_begin,
                                  int* c_end) {
  if (!m.varlen) {
    *c_begin = seq * m.nt;
    *c_end = (seq + 1) * m.nt;
  } else {
    *c_begin = m.first[seq];
    *c_end = m.first[seq + 1];
  }
}

// --------------------------------------------------------- XCD mapping ---
// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2.  Map the linear workgroup id so that consecutive work items land on the
// same XCD (they read the same per-chunk operands).
__device__ inline int xcd_swizzle(int L, int N) {
  if ((N & 7) != 0) return L;
  return (L & 7) * (N >> 3) + (L >> 3);
}

// ------------------------------------------------------- fragment maps ---
// An MFMA operand fragment covers 16 rows and a 32-wide K block; lane l holds
// row l%16 and K-slots 8*(l/16) .. +7.  The fragments written for the state
// recurrence use a permuted K order: slot s of lane group g stands for
//   k = 4g + s        (s < 4)
//   k = 16 + 4g + s-4 (s >= 4)
// within the block, which is exactly the set of rows that lane holds in the
// accumulators of two stacked 16x16 output tiles.  The accumulators can
// therefore be fed back as the other operand without any data movement.
__device__ __host__ inline int perm_k(int g, int s) {
  return s < 4 ? 4 * g + s : 16 + 4 * g + (s - 4);
}

template <typename OP> struct opstore;
template <> struct opstore<bf16_t> {
  using vec = bf16x8;
  static constexpr int bytes = 2;
};
template <> struct opstore<f32_t> {
  using vec = floatx8;
  static constexpr int bytes = 4;
};

// -------------------------------------------------------- workspace ---
// Per chunk-head (slot c of head h, index ch = h * nchunks + c) the forward
// keeps, in the operand type OP (bf16 or fp32):
//   Wn  : -W fragments      [NB][NKD][64 lanes][8]   (W = T diag(b g) K)
//   Qg  : Q~ fragments      [NB][NKD][64][8]         (Q~ = gamma (.) Q)
//   Kg  : K~^T fragments    [DK/16][NKC][64][8]      (K~ = K (.) e^{g_C - g})
//   P   : P fragments       [NB][NKC][64][8]         (masked decayed Q K^T)
// and in fp32:
//   U   : U accumulators    [NB][dv/16][64][4]       (U = T diag(b) V)
//   gam : per-row decay of the state over the chunk, [DK]
struct FwdLayout {
  int C, DK, dv, ob;           // chunk, key dim, value dim, operand bytes
  int NB, NKD, NKC;            // C/16, ceil(DK/32), ceil(C/32)
  size_t w, q, k, p, u, g;     // bytes per chunk-head of each buffer
  size_t per_ch;               // sum, 256-aligned pieces
  __host__ __device__ FwdLayout(int C_, int DK_, int dv_, int ob_)
      : C(C_), DK(DK_), dv(dv_), ob(ob_) {
    NB = C / 16;
    NKD = (DK + 31) / 32;
    NKC = (C + 31) / 32;
    w = al(size_t(NB) * NKD * 512 * ob);
    q = w;
    k = al(size_t(DK / 16) * NKC * 512 * ob);
    p = al(size_t(NB) * NKC * 512 * ob);
    u = al(size_t(C) * dv * 4);
    g = al(size_t(DK) * 4);
    per_ch = w + q + k + p + u + g;
  }
  __host__ __device__ static size_t al(size_t x) { return (x + 255) & ~size_t(255); }
};

struct FwdBuffers {
  char* base;     // per-chunk operand area
  size_t per_ch;
  size_t off_w, off_q, off_k, off_p, off_u, off_g;
  __device__ char* at(int64_t ch, size_t off) const {
    return base + static_cast<size_t>(ch) * per_ch + off;
  }
};

inline FwdBuffers make_buffers(char* base, const FwdLayout& L) {
  FwdBuffers b;
  b.base = base;
  b.per_ch = L.per_ch;
  b.off_w = 0;
  b.off_q = b.off_w + L.w;
  b.off_k = b.off_q + L.q;
  b.off_p = b.off_k + L.k;
  b.off_u = b.off_p + L.p;
  b.off_g = b.off_u + L.u;
  return b;
}

// Host: bytes of the varlen chunk map (table + first-chunk index).
inline size_t chunk_map_bytes(const Problem& p) {
  if (!p.varlen) return 0;
  return FwdLayout::al(size_t(p.nchunks) * 16) + FwdLayout::al(size_t(p.nseq + 1) * 4);
}

// Host: fill a ChunkMap pointing into workspace `map_base`.
inline ChunkMap make_chunk_map(const Problem& p, char* map_base) {
  ChunkMap m{};
  m.varlen = p.varlen ? 1 : 0;
  m.T = p.T;
  m.C = p.chunk;
  m.nt = (p.T + p.chunk - 1) / p.chunk;
  if (p.varlen) {
    m.tab = reinterpret_cast<const int4*>(map_base);
    m.first = reinterpret_cast<const int32_t*>(
        map_base + FwdLayout::al(size_t(p.nchunks) * 16));
  }
  return m;
}

// Device: build the varlen chunk map (one workgroup).  Lengths are clamped
// into [0, T] so malformed cu_seqlens cannot send later kernels out of
// bounds; chunks beyond the slot budget are dropped.
hipError_t launch_chunk_map(const Problem& p, char* map_base, hipStream_t s);

}  // namespace gdn
