// Shared pieces of the chunkwise forward and backward kernels: chunk
// bookkeeping, the varlen chunk map, workspace layout and fragment helpers.
#pragma once

#include <algorithm>

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

// Read-only table entry through the constant address space: with a uniform
// index this is a scalar load, which leaves the vector memory counter (and
// so the waits on in-flight copies) alone.
__device__ inline int ld_table(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)(p))[i];
}
__device__ inline int4 ld_table(const int4* p, int64_t i) {
  const int32_t* q = reinterpret_cast<const int32_t*>(p) + 4 * i;
  return make_int4(ld_table(q, 0), ld_table(q, 1), ld_table(q, 2), ld_table(q, 3));
}

__device__ inline ChunkInfo chunk_info(const ChunkMap& m, int c) {
  ChunkInfo r;
  if (!m.varlen) {
    const int b = c / m.nt, j = c % m.nt;
    r.seq = b;
    r.tok0 = static_cast<int64_t>(b) * m.T + static_cast<int64_t>(j) * m.C;
    r.len = min(m.C, m.T - j * m.C);
  } else {
    const int4 e = ld_table(m.tab, c);
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
    *c_begin = ld_table(m.first, seq);
    *c_end = ld_table(m.first, seq + 1);
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

// ------------------------------------------------- operand load/store ---

template <typename OP> using opvec = typename opstore<OP>::vec;

// Accumulator tile stored in the operand type (4 values per lane).
template <typename OP> struct acc4;
template <> struct acc4<bf16_t> { using type = bf16x4; };
template <> struct acc4<f32_t> { using type = floatx4; };

__device__ inline floatx4 to_f4(const bf16x4& x) {
  return floatx4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
__device__ inline floatx4 to_f4(const floatx4& x) { return x; }
template <typename OP> __device__ inline typename acc4<OP>::type from_f4(const floatx4& x);
template <> __device__ inline bf16x4 from_f4<bf16_t>(const floatx4& x) {
  return bf16x4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
}
template <> __device__ inline floatx4 from_f4<f32_t>(const floatx4& x) { return x; }

template <typename OP>
__device__ inline opvec<OP> zero_vec() { return frag<OP>::zero(); }

// 8 consecutive elements at element offset `off` of a global array in the
// operand type (16-byte aligned for bf16, 32-byte for fp32).
template <typename OP>
__device__ inline opvec<OP> gload8(const void* base, int64_t off) {
  return *reinterpret_cast<const opvec<OP>*>(
      static_cast<const char*>(base) + off * opstore<OP>::bytes);
}

// Two runs of 4 elements (offsets a and b) joined into one operand vector.
__device__ inline bf16x8 join44(const uint2& a, const uint2& b) {
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}
template <typename OP>
__device__ inline opvec<OP> gload4x2(const void* base, int64_t a, int64_t b) {
  const char* p = static_cast<const char*>(base);
  if constexpr (opstore<OP>::bytes == 2) {
    return join44(*reinterpret_cast<const uint2*>(p + a * 2),
                  *reinterpret_cast<const uint2*>(p + b * 2));
  } else {
    const floatx4 x = *reinterpret_cast<const floatx4*>(p + a * 4);
    const floatx4 y = *reinterpret_cast<const floatx4*>(p + b * 4);
    return floatx8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  }
}

template <typename OP>
__device__ inline void to_floats(const opvec<OP>& v, float* out) {
#pragma unroll
  for (int s = 0; s < 8; ++s) out[s] = (float)v[s];
}

// Pack two stacked accumulator tiles into one operand fragment (permuted K).
template <typename OP>
__device__ inline opvec<OP> pack2(const floatx4& lo, const floatx4& hi) {
  float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return frag<OP>::from_floats(v);
}

// ------------------------------------------------------ buffer access ---
// Raw buffer resources (base, byte size): loads past the end return zero and
// offsets are 32-bit, so address arithmetic stays in one VGPR.
constexpr int kBufFlags = 0x00020000;  // dword 3 of a raw gfx9 descriptor

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0,
                                           static_cast<int>(bytes), kBufFlags);
}

// An offset past every range set up here: such a load reads zero and
// touches no memory.
constexpr uint32_t kOob = 0x80000000u;

// 16 bytes at byte offset `off` of a buffer (zero when out of range).
__device__ inline uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// 8 consecutive operand elements at byte offset `off` of a buffer.
template <typename OP>
__device__ inline opvec<OP> bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (opstore<OP>::bytes == 2) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  } else {
    const floatx4 x = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    const floatx4 y =
        __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
    return floatx8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  }
}

// A gate value (bf16 or fp32 by a run-time flag) requested without a branch:
// both widths are loaded, the other one from an empty range, so no wait for
// the data is placed before gate_value() uses it.  Element `i` of the `n`
// elements at p; i >= n reads zero.
struct RawGate {
  uint16_t h16;
  uint32_t f32;
};
__device__ inline RawGate gate_issue(const void* p, uint32_t n, uint32_t i, bool bf16) {
  const uint32_t j = i < n ? i : kOob / 4;
  return {__builtin_amdgcn_raw_buffer_load_b16(make_rsrc(p, bf16 ? 2 * n : 0), 2 * j, 0, 0),
          __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p, bf16 ? 0 : 4 * n), 4 * j, 0, 0)};
}
__device__ inline float gate_value(const RawGate& g, bool bf16) {
  return bf16 ? bf16_bits_to_float(g.h16) : __uint_as_float(g.f32);
}

// Two runs of 4 operand elements at byte offsets a and b of a buffer.
template <typename OP>
__device__ inline opvec<OP> bload4x2(__amdgpu_buffer_rsrc_t r, uint32_t a, uint32_t b) {
  if constexpr (opstore<OP>::bytes == 2) {
    const uint2 x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, a, 0, 0));
    const uint2 y = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, b, 0, 0));
    return join44(x, y);
  } else {
    const floatx4 x = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, a, 0, 0));
    const floatx4 y = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, b, 0, 0));
    return floatx8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  }
}

// -------------------------------------------------------- workspace ---
// Per chunk-head (slot c of head h, index ch = h * nchunks + c) the forward
// keeps, in the operand type OP (bf16 for bf16 inputs, fp32 for fp32):
//   Wn  : -W fragments      [NB][NKD][64 lanes][8]   (W = T diag(b g) K)
//   Kg  : K~^T fragments    [DK/16][NKC][64][8]      (K~ = K (.) e^{g_C - g})
//   P   : P fragments       [NB][NKC][64][8]         (masked decayed Q K^T)
//   U   : U accumulators    [NB][dv/16][64][4]       (U = T diag(b) V)
//   Qg  : Q~ fragments      [NB][NKD][64][8]         (per-channel gate only:
//                                                     Q~ = Q (.) e^{g})
// and in fp32 the decays  [C] gamma_r = e^{g_r}, then [DK] the per-row decay
// of the state over the whole chunk.
struct FwdLayout {
  int C, DK, dv, ob;           // chunk, key dim, value dim, operand bytes
  int NB, NKD, NKC, NDT;       // C/16, ceil(DK/32), ceil(C/32), DK/16
  size_t w, k, p, u, q, g;     // bytes per chunk-head of each buffer
  // backward only: the reverse recurrence's operands (see gdn_bwd.hip)
  size_t kf, wt, pt, qt;
  size_t per_ch;               // sum, 256-aligned pieces
  __host__ __device__ FwdLayout(int C_, int DK_, int dv_, int ob_, bool chan,
                                bool bwd = false)
      : C(C_), DK(DK_), dv(dv_), ob(ob_) {
    NB = C / 16;
    NKD = (DK + 31) / 32;
    NKC = (C + 31) / 32;
    NDT = DK / 16;
    w = al(size_t(NB) * NKD * 512 * ob);
    k = al(size_t(NDT) * NKC * 512 * ob);
    p = al(size_t(NB) * NKC * 512 * ob);
    u = al(size_t(C) * dv * ob);
    q = chan ? w : 0;
    g = al(size_t(C + DK) * 4);
    kf = bwd ? w : 0;
    wt = bwd ? k : 0;
    pt = bwd ? p : 0;
    qt = bwd ? k : 0;
    per_ch = w + k + p + u + q + g + kf + wt + pt + qt;
  }
  __host__ __device__ static size_t al(size_t x) { return (x + 255) & ~size_t(255); }
};

struct FwdBuffers {
  char* base;     // per-chunk operand area
  size_t per_ch;
  size_t off_w, off_k, off_p, off_u, off_q, off_g;
  size_t off_kf, off_wt, off_pt, off_qt;
  __device__ char* at(int64_t ch, size_t off) const {
    return base + static_cast<size_t>(ch) * per_ch + off;
  }
};

inline FwdBuffers make_buffers(char* base, const FwdLayout& L) {
  FwdBuffers b;
  b.base = base;
  b.per_ch = L.per_ch;
  b.off_w = 0;
  b.off_k = b.off_w + L.w;
  b.off_p = b.off_k + L.k;
  b.off_u = b.off_p + L.p;
  b.off_q = b.off_u + L.u;
  b.off_g = b.off_q + L.q;
  b.off_kf = b.off_g + L.g;
  b.off_wt = b.off_kf + L.kf;
  b.off_pt = b.off_wt + L.wt;
  b.off_qt = b.off_pt + L.pt;
  return b;
}

// Host: bytes of the varlen chunk map (chunk table + first-chunk index, then
// the segment table + first-segment index when sequences are split).
inline size_t chunk_map_bytes(const Problem& p) {
  if (!p.varlen) return 0;
  size_t b = FwdLayout::al(size_t(p.nchunks) * 16) + FwdLayout::al(size_t(p.nseq + 1) * 4);
  if (p.seg > 0)
    b += FwdLayout::al(size_t(p.nsegs) * 16) + FwdLayout::al(size_t(p.nseq + 1) * 4);
  return b;
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

// ----------------------------------------------------------- segments ---
// The forward state pass splits each sequence into segments of at most L
// consecutive chunks so that short batches still fill the machine: the
// state entering segment j is  M_j = Phi_{j-1} M_{j-1} + M0_{j-1},  where
// Phi is the segment's transition (the product of its per-chunk maps
// M -> (gamma_c I - K~^T W) M) and M0 the state it produces from zero.
// L = 0 keeps one segment per sequence (slot = sequence).
struct SegMap {
  int L;                 // chunks per segment, 0 = whole sequences
  int varlen;
  int nt;                // dense: chunks per sequence
  int per_seq;           // dense: segments per sequence (>= 1)
  const int4* tab;       // varlen, L > 0: [nsegs] (seq, c0, c1, j); seq < 0 unused
  const int32_t* first;  // varlen, L > 0: [nseq + 1] first segment slot
};

struct SegInfo {
  int seq;     // < 0: unused slot
  int j;       // index of the segment within its sequence
  int c0, c1;  // chunk slots [c0, c1)
  bool last;   // last segment of its sequence
};

__device__ inline SegInfo seg_info(const SegMap& s, const ChunkMap& m, int slot) {
  SegInfo r;
  if (s.L == 0) {
    r.seq = slot;
    r.j = 0;
    seq_chunks(m, slot, &r.c0, &r.c1);
    r.last = true;
  } else if (!s.varlen) {
    r.seq = slot / s.per_seq;
    r.j = slot % s.per_seq;
    r.c0 = r.seq * s.nt + r.j * s.L;
    r.c1 = min(r.c0 + s.L, (r.seq + 1) * s.nt);
    r.last = r.j == s.per_seq - 1;
  } else {
    const int4 e = ld_table(s.tab, slot);
    r.seq = e.x;
    r.c0 = e.y;
    r.c1 = e.z;
    r.j = e.w;
    r.last = e.x >= 0 && slot + 1 == ld_table(s.first, e.x + 1);
  }
  return r;
}

// Segment slots of one sequence: [b, e).
__device__ inline void seq_segs(const SegMap& s, int seq, int* b, int* e) {
  if (s.L == 0) {
    *b = seq;
    *e = seq + 1;
  } else if (!s.varlen) {
    *b = seq * s.per_seq;
    *e = (seq + 1) * s.per_seq;
  } else {
    *b = ld_table(s.first, seq);
    *e = ld_table(s.first, seq + 1);
  }
}

// Host: a SegMap for segments of L chunks (L = 0 or p.seg) over the map at
// `map_base`.
inline SegMap make_seg_map(const Problem& p, char* map_base, int L) {
  SegMap s{};
  s.L = L;
  s.varlen = p.varlen ? 1 : 0;
  s.nt = (p.T + p.chunk - 1) / p.chunk;
  s.per_seq = L > 0 ? std::max(1, (s.nt + L - 1) / L) : 1;
  if (p.varlen && L > 0) {
    char* b = map_base + FwdLayout::al(size_t(p.nchunks) * 16) +
              FwdLayout::al(size_t(p.nseq + 1) * 4);
    s.tab = reinterpret_cast<const int4*>(b);
    s.first = reinterpret_cast<const int32_t*>(b + FwdLayout::al(size_t(p.nsegs) * 16));
  }
  return s;
}

// Device: build the varlen chunk map (one workgroup).  Lengths are clamped
// into [0, T] so malformed cu_seqlens cannot send later kernels out of
// bounds; chunks beyond the slot budget are dropped.  With p.seg > 0 it
// also fills the segment table.
hipError_t launch_chunk_map(const Problem& p, char* map_base, hipStream_t s);

}  // namespace gdn
