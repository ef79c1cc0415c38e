// Chunkwise backward of the gated delta rule.
//
// Gradients of L = <dO, o> + <dS_final, S_final> with respect to q, k, v,
// beta, log alpha and S_0.  The pages ("Gated Delta Networks: Improving
// Mamba2 with Delta Rule", paper review, "Method") define the forward only;
// this is the adjoint of the chunk form the forward kernels evaluate.  Per
// chunk, with M0 the state at the chunk start, dM1 the gradient of the state
// at the chunk end, and the forward's chunk quantities (T, W = T X with
// X = diag(b gamma) K, Y = diag(b) V, U = T Y, E = U - W M0, K~, Q~, P, D):
//
//   reverse recurrence   dE  = P^T dO + K~ dM1
//                        dM0 = D dM1 + Q~^T dO - W^T dE
//   per chunk            dQ~ = dO M0^T     dW = -dE M0^T     dK~ = E dM1^T
//                        dP  = dO E^T      dY = T^T dE       dX  = T^T dW
//                        dT  = dE Y^T + dW X^T,   dA = -T^T dT T^T (strict lower)
//   and then through the decays and K K^T / Q K^T into dq, dk, dbeta and the
//   per-token gate gradient dg, whose reverse cumulative sum inside the chunk
//   is d log alpha (the chunk-end decay D feeds the chunk's last row).
//
// Kernels, all on the caller's stream:
//   1. prep (a forward prep with BWD = true; the per-token gates take the
//      scalar-gate prep): the forward operands plus the reverse recurrence's
//      fragments K~, -W^T, P^T, Q~^T.
//   2. forward state pass in STATES mode: the state at every chunk start.
//   3. reverse state pass (bwd_scan_kernel): dM across chunks, one workgroup
//      per (sequence, head, 16-column slab of dv); stores dM at every chunk
//      end and writes dS_0.  As in the forward, a helper wave forms the
//      chain-free terms P^T dO and Q~^T dO one chunk ahead.
//   4. per-chunk gradients (bwd_grad_kernel), one workgroup per chunk-head,
//      value columns in slabs; no atomics, so the result is deterministic.

#include "gdn_fwd_kernels.hpp"

namespace gdn {

namespace {

// ------------------------------------------------------ reverse chain ---

template <int C, int DK, typename OP, int GATE>
struct RevOps {
  static constexpr int NB = C / 16, NKD = (DK + 31) / 32, NKC = (C + 31) / 32,
                       NDT = DK / 16;
  opvec<OP> Kf[NB][NKD];   // K~ rows i, k = dk (permuted)
  opvec<OP> Wt[NDT][NKC];  // -W^T rows dk, k = tokens (permuted)
  floatx4 gc[GATE == GDN_GATE_CHANNEL ? NDT : 1];
};

template <int C, int DK, typename OP, int GATE>
__device__ __forceinline__ void load_rev(RevOps<C, DK, OP, GATE>& x,
                                         const FwdBuffers& buf, int64_t ch,
                                         int lane, int lg) {
  using X = RevOps<C, DK, OP, GATE>;
  constexpr int ob = opstore<OP>::bytes;
  const char* pk = buf.at(ch, buf.off_kf);
  const char* pw = buf.at(ch, buf.off_wt);
  const float* pg = reinterpret_cast<const float*>(buf.at(ch, buf.off_g)) + C;
#pragma unroll
  for (int rt = 0; rt < X::NB; ++rt)
#pragma unroll
    for (int jb = 0; jb < X::NKD; ++jb)
      x.Kf[rt][jb] = *reinterpret_cast<const opvec<OP>*>(
          pk + ((size_t(rt) * X::NKD + jb) * 64 + lane) * 8 * ob);
#pragma unroll
  for (int a = 0; a < X::NDT; ++a)
#pragma unroll
    for (int jb = 0; jb < X::NKC; ++jb)
      x.Wt[a][jb] = *reinterpret_cast<const opvec<OP>*>(
          pw + ((size_t(a) * X::NKC + jb) * 64 + lane) * 8 * ob);
  if constexpr (GATE == GDN_GATE_CHANNEL) {
#pragma unroll
    for (int a = 0; a < X::NDT; ++a)
      x.gc[a] = *reinterpret_cast<const floatx4*>(pg + 16 * a + 4 * lg);
  } else if constexpr (GATE == GDN_GATE_SCALAR) {
    const float g = pg[0];
    x.gc[0] = floatx4{g, g, g, g};
  } else {
    x.gc[0] = floatx4{1.f, 1.f, 1.f, 1.f};
  }
}

template <int C, int DK, typename OP>
struct HelpOps {
  static constexpr int NB = C / 16, NKC = (C + 31) / 32, NDT = DK / 16;
  opvec<OP> Pt[NB][NKC];   // P^T rows i, k = r (permuted)
  opvec<OP> Qt[NDT][NKC];  // Q~^T rows dk, k = r (permuted)
};

template <int C, int DK, typename OP>
__device__ __forceinline__ void load_help(HelpOps<C, DK, OP>& x,
                                          const FwdBuffers& buf, int64_t ch,
                                          int lane) {
  using X = HelpOps<C, DK, OP>;
  constexpr int ob = opstore<OP>::bytes;
  const char* pp = buf.at(ch, buf.off_pt);
  const char* pq = buf.at(ch, buf.off_qt);
#pragma unroll
  for (int it = 0; it < X::NB; ++it)
#pragma unroll
    for (int jb = 0; jb < X::NKC; ++jb)
      if (32 * jb + 31 >= 16 * it)
        x.Pt[it][jb] = *reinterpret_cast<const opvec<OP>*>(
            pp + ((size_t(it) * X::NKC + jb) * 64 + lane) * 8 * ob);
#pragma unroll
  for (int a = 0; a < X::NDT; ++a)
#pragma unroll
    for (int jb = 0; jb < X::NKC; ++jb)
      x.Qt[a][jb] = *reinterpret_cast<const opvec<OP>*>(
          pq + ((size_t(a) * X::NKC + jb) * 64 + lane) * 8 * ob);
}

// Reverse state pass: wave 0 carries dM backwards over the chunks of one
// (segment, head, 16-column slab); wave 1 computes R = P^T dO and
// G = Q~^T dO for the chunk wave 0 takes next and hands them over in LDS.
// Over a segment the reverse map is affine, dM_start = Phi^T dM_end + b,
// with Phi the forward transition of the segment.  Two modes:
//   ZERO (segment maps): start from dM_end = 0, store nothing per chunk and
//     write dM_start = b into `seg_out` (segments j >= 1 only);
//   otherwise: start from dS_final (last segment of a sequence) or from
//     `seg_in` (the gradient entering the segment from the right), store dM
//     at every chunk end and write dS_0 from the first segment.
// One segment per sequence (sm.L = 0) is the plain reverse pass.
template <int C, int DK, typename IO, int GATE, bool ZERO = false>
__global__ __launch_bounds__(128) void bwd_scan_kernel(
    ChunkMap map, SegMap sm, int H, int dv, int64_t nchunks, const void* __restrict__ d_o,
    const float* __restrict__ ds_final, float* __restrict__ ds0,
    FwdBuffers buf, void* __restrict__ dstates, const float* __restrict__ seg_in,
    float* __restrict__ seg_out) {
  using OP = IO;
  using X = RevOps<C, DK, OP, GATE>;
  using Y = HelpOps<C, DK, OP>;
  using E = typename io<IO>::storage;
  constexpr int NB = X::NB, NKD = X::NKD, NKC = X::NKC, NDT = X::NDT;
  constexpr bool CH = GATE == GDN_GATE_CHANNEL;
  constexpr bool kPrefetch = io<IO>::bytes == 2;

  __shared__ floatx4 sR[2][NB][64];
  __shared__ floatx4 sG[2][NDT][64];
  __shared__ __attribute__((aligned(16))) E sDO[C][16];

  const int w = xcd_swizzle(blockIdx.x, gridDim.x);
  const int ndvt = dv / 16;
  const int vt = w % ndvt;
  const int chain = w / ndvt;
  const int h = chain % H;
  const int slot = chain / H;
  const SegInfo si = seg_info(sm, map, slot);
  if (si.seq < 0 || (ZERO && si.j == 0)) return;  // whole workgroup, before any barrier
  const int seq = si.seq;
  // wave index in a scalar register: branches on it are scalar branches,
  // never EXEC masks (matrix instructions ignore EXEC)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
  const int col = 16 * vt + l16;
  const int64_t sbase = (static_cast<int64_t>(seq) * H + h) * DK * dv;
  // segment buffers, accumulator layout [slot][H][dv/16][DK/16][64]
  const size_t sl = (static_cast<size_t>(slot) * H + h) * ndvt + vt;

  const int ce = si.c1;
  const int n = si.c1 - si.c0;
  const int64_t chl = static_cast<int64_t>(h) * nchunks + ce - 1;  // p = 0

  if (wave == 0) {
    floatx4 dM[NDT];
    if (ZERO) {
#pragma unroll
      for (int a = 0; a < NDT; ++a) dM[a] = floatx4{0.f, 0.f, 0.f, 0.f};
    } else if (si.last) {
      // the test on ds_final outside the loads, so that they issue together
      if (ds_final != nullptr) {
#pragma unroll
        for (int a = 0; a < NDT; ++a)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            dM[a][s] = ds_final[sbase + static_cast<int64_t>(16 * a + 4 * lg + s) * dv + col];
      } else {
#pragma unroll
        for (int a = 0; a < NDT; ++a) dM[a] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    } else {
      const floatx4* src = reinterpret_cast<const floatx4*>(seg_in) + sl * NDT * 64;
#pragma unroll
      for (int a = 0; a < NDT; ++a) dM[a] = src[a * 64 + lane];
    }

    auto step = [&](const X& cur, X& nxt, int p) {
      if (kPrefetch && p + 1 < n) load_rev<C, DK, OP, GATE>(nxt, buf, chl - p - 1, lane, lg);
      if constexpr (!ZERO) {
        const int64_t st = (chl - p) * static_cast<int64_t>(DK) * dv;
#pragma unroll
        for (int a = 0; a < NDT; ++a)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            io<IO>::store(dstates, st + static_cast<int64_t>(16 * a + 4 * lg + s) * dv + col,
                          dM[a][s]);
      }
      opvec<OP> Mb[NKD];
#pragma unroll
      for (int jb = 0; jb < NKD; ++jb) {
        const floatx4 z = {0.f, 0.f, 0.f, 0.f};
        Mb[jb] = pack2<OP>(dM[2 * jb], 2 * jb + 1 < NDT ? dM[2 * jb + 1] : z);
      }
      floatx4 dE[NB];
#pragma unroll
      for (int it = 0; it < NB; ++it) {
        dE[it] = sR[p & 1][it][lane];
#pragma unroll
        for (int jb = 0; jb < NKD; ++jb) dE[it] = mma32(cur.Kf[it][jb], Mb[jb], dE[it]);
      }
      opvec<OP> Eb[NKC];
#pragma unroll
      for (int jb = 0; jb < NKC; ++jb) {
        const floatx4 z = {0.f, 0.f, 0.f, 0.f};
        Eb[jb] = pack2<OP>(dE[2 * jb], 2 * jb + 1 < NB ? dE[2 * jb + 1] : z);
      }
#pragma unroll
      for (int a = 0; a < NDT; ++a) {
        dM[a] = dM[a] * cur.gc[CH ? a : 0] + sG[p & 1][a][lane];
#pragma unroll
        for (int jb = 0; jb < NKC; ++jb) dM[a] = mma32(cur.Wt[a][jb], Eb[jb], dM[a]);
      }
    };

    __syncthreads();  // iteration 0: wave 1 prepares p = 0
    if constexpr (kPrefetch) {
      X A, B;
      if (n > 0) load_rev<C, DK, OP, GATE>(A, buf, chl, lane, lg);
      for (int j = 1; j <= n; j += 2) {
        step(A, B, j - 1);
        __syncthreads();
        if (j + 1 <= n) {
          step(B, A, j);
          __syncthreads();
        }
      }
    } else {
      for (int j = 1; j <= n; ++j) {
        X A;
        load_rev<C, DK, OP, GATE>(A, buf, chl - (j - 1), lane, lg);
        step(A, A, j - 1);
        __syncthreads();
      }
    }
    if (ZERO) {
      floatx4* dst = reinterpret_cast<floatx4*>(seg_out) + sl * NDT * 64;
#pragma unroll
      for (int a = 0; a < NDT; ++a) dst[a * 64 + lane] = dM[a];
    } else if (ds0 && si.j == 0) {
#pragma unroll
      for (int a = 0; a < NDT; ++a)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          ds0[sbase + static_cast<int64_t>(16 * a + 4 * lg + s) * dv + col] = dM[a][s];
    }
  } else {
    // helper: R = P^T dO and G = Q~^T dO of chunk p into buffer p & 1
    auto step = [&](const Y& cur, int p) {
      const ChunkInfo ci = chunk_info(map, ce - 1 - p);
      constexpr int PPR = 16 * sizeof(E) / 16;  // 16-byte pieces per row
#pragma unroll
      for (int u = 0; u < (C * PPR + 63) / 64; ++u) {
        const int e = lane + 64 * u;
        const int r = e / PPR, piece = e % PPR;
        if (e < C * PPR) {
          uint4 val = make_uint4(0, 0, 0, 0);
          if (r < ci.len)
            val = *reinterpret_cast<const uint4*>(static_cast<const char*>(d_o) +
                (((ci.tok0 + r) * H + h) * dv + 16 * vt) * sizeof(E) + piece * 16);
          *reinterpret_cast<uint4*>(&sDO[r][piece * (16 / sizeof(E))]) = val;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      opvec<OP> Df[NKC];
#pragma unroll
      for (int jb = 0; jb < NKC; ++jb) {
        float x[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int r = 32 * jb + perm_k(lg, s);
          x[s] = r < C ? io<IO>::load(&sDO[0][0], r * 16 + l16) : 0.f;
        }
        Df[jb] = frag<OP>::from_floats(x);
      }
#pragma unroll
      for (int it = 0; it < NB; ++it) {
        floatx4 R = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jb = 0; jb < NKC; ++jb)
          if (32 * jb + 31 >= 16 * it) R = mma32(cur.Pt[it][jb], Df[jb], R);
        sR[p & 1][it][lane] = R;
      }
#pragma unroll
      for (int a = 0; a < NDT; ++a) {
        floatx4 G = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jb = 0; jb < NKC; ++jb) G = mma32(cur.Qt[a][jb], Df[jb], G);
        sG[p & 1][a][lane] = G;
      }
      __builtin_amdgcn_wave_barrier();
    };
    if constexpr (kPrefetch) {
      Y A, B;
      if (n > 0) load_help<C, DK, OP>(A, buf, chl, lane);
      for (int j = 0; j <= n; j += 2) {
        if (j < n) {
          if (j + 1 < n) load_help<C, DK, OP>(B, buf, chl - j - 1, lane);
          step(A, j);
        }
        __syncthreads();
        if (j + 1 <= n) {
          if (j + 1 < n) {
            if (j + 2 < n) load_help<C, DK, OP>(A, buf, chl - j - 2, lane);
            step(B, j + 1);
          }
          __syncthreads();
        }
      }
    } else {
      for (int j = 0; j <= n; ++j) {
        if (j < n) {
          Y A;
          load_help<C, DK, OP>(A, buf, chl - j, lane);
          step(A, j);
        }
        __syncthreads();
      }
    }
  }
}

// Reverse state pass for bf16 operands with the chunk operands shared in
// LDS: one workgroup per (segment, head, group of kRevSlabs 16-column slabs),
// one wave per slab.  The per-chunk operands (decays, K~, -W^T, P^T, Q~^T:
// one contiguous stretch of the chunk's workspace) are copied once per
// workgroup straight into LDS, double-buffered, together with the group's
// dO columns, instead of once per slab.  Each wave forms its slab's
// chain-free terms R = P^T dO and G = Q~^T dO from LDS in the same step as
// the chain, so no helper wave is needed.  Modes as bwd_scan_kernel.
constexpr int kRevSlabs = 4;

template <int C, int DK>
struct RevLds {
  static constexpr int NB = C / 16, NKD = (DK + 31) / 32, NKC = (C + 31) / 32, NDT = DK / 16;
  static constexpr size_t al(size_t x) { return (x + 255) & ~size_t(255); }
  // the workspace's [g | K~ | -W^T | P^T | Q~^T] stretch (bf16 fragments)
  static constexpr size_t oG = 0;
  static constexpr size_t oKF = al(size_t(C + DK) * 4);
  static constexpr size_t oWT = oKF + al(size_t(NB) * NKD * 1024);
  static constexpr size_t oPT = oWT + al(size_t(NDT) * NKC * 1024);
  static constexpr size_t oQT = oPT + al(size_t(NB) * NKC * 1024);
  static constexpr size_t REG = oQT + al(size_t(NDT) * NKC * 1024);
  // dO rows of the group's columns, [C][16 kRevSlabs] bf16
  static constexpr int DOP = 2 * kRevSlabs;  // 16-byte pieces per row
  static constexpr size_t oDO = REG;
  static constexpr size_t STAGE = oDO + size_t(C) * DOP * 16;
  static constexpr size_t total = 2 * STAGE;
  static_assert(REG % 16 == 0 && STAGE % 16 == 0, "16-byte pieces");
};

template <int C, int DK, int GATE, bool ZERO = false>
__global__ __launch_bounds__(64 * kRevSlabs) void bwd_scan_lds_kernel(
    ChunkMap map, SegMap sm, int H, int dv, int64_t nchunks, const void* __restrict__ d_o,
    const float* __restrict__ ds_final, float* __restrict__ ds0,
    FwdBuffers buf, void* __restrict__ dstates, const float* __restrict__ seg_in,
    float* __restrict__ seg_out) {
  using OP = bf16_t;
  using L = RevLds<C, DK>;
  constexpr int NB = L::NB, NKD = L::NKD, NKC = L::NKC, NDT = L::NDT;
  constexpr int NT = 64 * kRevSlabs;
  constexpr bool CH = GATE == GDN_GATE_CHANNEL;
  constexpr int NDO = (C * L::DOP + NT - 1) / NT;  // dO pieces per thread
  __shared__ __attribute__((aligned(16))) char smem[L::total];

  const int w = xcd_swizzle(blockIdx.x, gridDim.x);
  const int ndvt = dv / 16;
  const int ngrp = (ndvt + kRevSlabs - 1) / kRevSlabs;
  const int grp = w % ngrp;
  const int chain = w / ngrp;
  const int h = chain % H;
  const int slot = chain / H;
  const SegInfo si = seg_info(sm, map, slot);
  if (si.seq < 0 || (ZERO && si.j == 0)) return;  // whole workgroup, before any barrier
  const int seq = si.seq;
  const int tid = threadIdx.x;
  // wave index in a scalar register: branches on it are scalar branches,
  // never EXEC masks (matrix instructions ignore EXEC)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int vt = grp * kRevSlabs + wave;
  const bool active = vt < ndvt;  // wave-uniform
  const int col = 16 * vt + l16;
  const int c0 = 16 * grp * kRevSlabs;  // first column of the group
  const int64_t sbase = (static_cast<int64_t>(seq) * H + h) * DK * dv;
  const size_t sl = (static_cast<size_t>(slot) * H + h) * ndvt + vt;
  const int ce = si.c1;
  const int n = si.c1 - si.c0;
  const int64_t chl = static_cast<int64_t>(h) * nchunks + ce - 1;  // step 0

  floatx4 dM[NDT];
#pragma unroll
  for (int a = 0; a < NDT; ++a) dM[a] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (active && !ZERO) {
    if (si.last) {
      if (ds_final) {
#pragma unroll
        for (int a = 0; a < NDT; ++a)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            dM[a][s] = ds_final[sbase + static_cast<int64_t>(16 * a + 4 * lg + s) * dv + col];
      }
    } else {
      const floatx4* src = reinterpret_cast<const floatx4*>(seg_in) + sl * NDT * 64;
#pragma unroll
      for (int a = 0; a < NDT; ++a) dM[a] = src[a * 64 + lane];
    }
  }

  // operands of step j into stage buffer `lds`; the dO pieces travel in
  // registers and are written after the current step (rows past the chunk
  // and columns past dv are zero)
  uint4 dop[NDO];
  auto copy = [&](char* lds, int j) {
    lds_copy<NT, L::REG>(lds, buf.at(chl - j, buf.off_g), wave, lane);
    const ChunkInfo ci = chunk_info(map, ce - 1 - j);
#pragma unroll
    for (int u = 0; u < NDO; ++u) {
      const int e = tid + NT * u, r = e / L::DOP, pc = e % L::DOP;
      dop[u] = make_uint4(0, 0, 0, 0);
      if (e < C * L::DOP && r < ci.len && c0 + 8 * pc < dv)
        dop[u] = *reinterpret_cast<const uint4*>(
            static_cast<const char*>(d_o) + (((ci.tok0 + r) * H + h) * dv + c0 + 8 * pc) * 2);
    }
  };
  auto put_do = [&](char* lds) {
#pragma unroll
    for (int u = 0; u < NDO; ++u) {
      const int e = tid + NT * u;
      if (e < C * L::DOP) *reinterpret_cast<uint4*>(lds + L::oDO + size_t(e) * 16) = dop[u];
    }
  };
  auto lfrag = [&](const char* lds, size_t off, int f) {
    return *reinterpret_cast<const opvec<OP>*>(lds + off + (size_t(f) * 64 + lane) * 16);
  };

  auto step = [&](const char* lds, int j) {
    if (!active) return;
    // chain-free terms of this chunk: R = P^T dO, G = Q~^T dO
    opvec<OP> Df[NKC];
#pragma unroll
    for (int jb = 0; jb < NKC; ++jb) {
      float x[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int r = 32 * jb + perm_k(lg, s);
        x[s] = r < C ? static_cast<float>(reinterpret_cast<const __bf16*>(lds + L::oDO)[
                           r * 16 * kRevSlabs + 16 * wave + l16])
                     : 0.f;
      }
      Df[jb] = frag<OP>::from_floats(x);
    }
    floatx4 dE[NB], Gm[NDT];
#pragma unroll
    for (int it = 0; it < NB; ++it) {
      dE[it] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jb = 0; jb < NKC; ++jb)
        if (32 * jb + 31 >= 16 * it) dE[it] = mma32(lfrag(lds, L::oPT, it * NKC + jb), Df[jb], dE[it]);
    }
#pragma unroll
    for (int a = 0; a < NDT; ++a) {
      Gm[a] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jb = 0; jb < NKC; ++jb) Gm[a] = mma32(lfrag(lds, L::oQT, a * NKC + jb), Df[jb], Gm[a]);
    }
    // the gradient at the chunk end
    if constexpr (!ZERO) {
      const int64_t st = (chl - j) * static_cast<int64_t>(DK) * dv;
#pragma unroll
      for (int a = 0; a < NDT; ++a)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          io<OP>::store(dstates, st + static_cast<int64_t>(16 * a + 4 * lg + s) * dv + col,
                        dM[a][s]);
    }
    // dE = R + K~ dM1;  dM0 = D dM1 + G - W^T dE
    opvec<OP> Mb[NKD];
#pragma unroll
    for (int jb = 0; jb < NKD; ++jb) {
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      Mb[jb] = pack2<OP>(dM[2 * jb], 2 * jb + 1 < NDT ? dM[2 * jb + 1] : z);
    }
#pragma unroll
    for (int it = 0; it < NB; ++it)
#pragma unroll
      for (int jb = 0; jb < NKD; ++jb) dE[it] = mma32(lfrag(lds, L::oKF, it * NKD + jb), Mb[jb], dE[it]);
    opvec<OP> Eb[NKC];
#pragma unroll
    for (int jb = 0; jb < NKC; ++jb) {
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      Eb[jb] = pack2<OP>(dE[2 * jb], 2 * jb + 1 < NB ? dE[2 * jb + 1] : z);
    }
    const float* gam = reinterpret_cast<const float*>(lds + L::oG) + C;
#pragma unroll
    for (int a = 0; a < NDT; ++a) {
      floatx4 gc;
      if constexpr (CH) gc = *reinterpret_cast<const floatx4*>(gam + 16 * a + 4 * lg);
      else if constexpr (GATE == GDN_GATE_SCALAR) gc = floatx4{gam[0], gam[0], gam[0], gam[0]};
      else gc = floatx4{1.f, 1.f, 1.f, 1.f};
      dM[a] = dM[a] * gc + Gm[a];
#pragma unroll
      for (int jb = 0; jb < NKC; ++jb) dM[a] = mma32(lfrag(lds, L::oWT, a * NKC + jb), Eb[jb], dM[a]);
    }
  };

  char* sA = smem;
  char* sB = smem + L::STAGE;
  if (n > 0) {
    copy(sA, 0);
    put_do(sA);
  }
  wait_vmcnt<0>();
  __syncthreads();
  for (int j = 0; j < n; j += 2) {
    if (j + 1 < n) copy(sB, j + 1);
    step(sA, j);
    if (j + 1 < n) put_do(sB);
    wait_vmcnt<0>();
    __syncthreads();
    if (j + 1 < n) {
      if (j + 2 < n) copy(sA, j + 2);
      step(sB, j + 1);
      if (j + 2 < n) put_do(sA);
      wait_vmcnt<0>();
      __syncthreads();
    }
  }
  if (!active) return;
  if (ZERO) {
    floatx4* dst = reinterpret_cast<floatx4*>(seg_out) + sl * NDT * 64;
#pragma unroll
    for (int a = 0; a < NDT; ++a) dst[a * 64 + lane] = dM[a];
  } else if (ds0 && si.j == 0) {
#pragma unroll
    for (int a = 0; a < NDT; ++a)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        ds0[sbase + static_cast<int64_t>(16 * a + 4 * lg + s) * dv + col] = dM[a][s];
  }
}

// Reverse chain over the segments of one (sequence, head, 16-column slab):
// the gradient entering segment j from the right is g_j (g_last = dS_final),
// and g_{j-1} = Phi_j^T g_j + b_j with b_j the segment's ZERO-mode result.
// Phi_j is stored as operand fragments of its rows (the forward transition
// pass); its transpose's fragments are read back through LDS.  One wave.
template <int DK, typename IO>
__global__ __launch_bounds__(64) void bwd_combine_kernel(
    ChunkMap map, SegMap sm, int H, int dv, const float* __restrict__ ds_final,
    SegBuffers sb, const float* __restrict__ seg_b, float* __restrict__ seg_g) {
  using OP = IO;
  using E = typename io<IO>::storage;
  constexpr int NKD = (DK + 31) / 32, NDT = DK / 16, LP = DK + 16 / sizeof(E);
  __shared__ __attribute__((aligned(16))) E sPhi[DK * LP];
  (void)map;
  const int ndvt = dv / 16;
  const int nseq = static_cast<int>(gridDim.x) / (H * ndvt);
  const int wg = blockIdx.x;
  const int vt = wg % ndvt;
  const int seq = (wg / ndvt) % nseq;
  const int h = wg / ndvt / nseq;
  int sb0, se0;
  seq_segs(sm, seq, &sb0, &se0);
  if (se0 - sb0 <= 1) return;
  const int lane = threadIdx.x, l16 = lane & 15, lg = lane >> 4;
  const int col = 16 * vt + l16;
  const int64_t sbase = (static_cast<int64_t>(seq) * H + h) * DK * dv;

  floatx4 g[NDT];
  if (ds_final != nullptr) {
#pragma unroll
    for (int a = 0; a < NDT; ++a)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        g[a][s] = ds_final[sbase + static_cast<int64_t>(16 * a + 4 * lg + s) * dv + col];
  } else {
#pragma unroll
    for (int a = 0; a < NDT; ++a) g[a] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  for (int j = se0 - 1; j > sb0; --j) {
    const size_t sh = static_cast<size_t>(j) * H + h;
    // Phi_j rows into LDS, element (r, c) at r * LP + c
    const opvec<OP>* phi = reinterpret_cast<const opvec<OP>*>(sb.trp + sh * sb.trp_bytes);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int a = 0; a < NDT; ++a)
#pragma unroll
      for (int jb = 0; jb < NKD; ++jb) {
        float x[8];
        to_floats<OP>(phi[(a * NKD + jb) * 64 + lane], x);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int c = 32 * jb + perm_k(lg, s);
          if (c < DK) lds_st<IO>(reinterpret_cast<char*>(sPhi), size_t(16 * a + l16) * LP + c, x[s]);
        }
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes
    __builtin_amdgcn_wave_barrier();
    opvec<OP> gb[NKD];
#pragma unroll
    for (int jb = 0; jb < NKD; ++jb) {
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      gb[jb] = pack2<OP>(g[2 * jb], 2 * jb + 1 < NDT ? g[2 * jb + 1] : z);
    }
    const floatx4* bj = reinterpret_cast<const floatx4*>(seg_b) + (sh * ndvt + vt) * NDT * 64;
    floatx4* out = reinterpret_cast<floatx4*>(seg_g) + ((sh - H) * ndvt + vt) * NDT * 64;
#pragma unroll
    for (int a = 0; a < NDT; ++a) {
      floatx4 acc = bj[a * 64 + lane];
#pragma unroll
      for (int jb = 0; jb < NKD; ++jb) {
        // rows 16 a .. of Phi^T: Phi's columns, k = Phi's rows (permuted)
        float x[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int r = 32 * jb + perm_k(lg, s);
          x[s] = r < DK ? lds_ld<IO>(reinterpret_cast<const char*>(sPhi),
                                     size_t(r) * LP + 16 * a + l16) : 0.f;
        }
        acc = mma32(frag<OP>::from_floats(x), gb[jb], acc);
      }
      g[a] = acc;
      out[a * 64 + lane] = acc;  // entering gradient of segment j - 1
    }
  }
}

// ---------------------------------------------------- chunk gradients ---

// acc += sum_k A(m0 + row, k) B(k, n0 + col) for the 16x16 tile at (m0, n0);
// A and B are element readers (LDS), so any transposition is free.
template <typename OP, int KD, typename FA, typename FB>
__device__ __forceinline__ floatx4 tmma(FA A, FB B, int m0, int n0, int l16,
                                        int lg, floatx4 acc) {
#pragma unroll
  for (int kb = 0; kb < (KD + 31) / 32; ++kb) {
    float a[8], b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int kk = kb * 32 + 8 * lg + s;
      a[s] = kk < KD ? A(m0 + l16, kk) : 0.f;
      b[s] = kk < KD ? B(kk, n0 + l16) : 0.f;
    }
    acc = mma32(frag<OP>::from_floats(a), frag<OP>::from_floats(b), acc);
  }
  return acc;
}

// acc += A B for the 16x16 tile at (m0, n0) with both operands stored with
// the contraction index contiguous in the input dtype: A(m, k) = A[m][k],
// B(k, n) = B[n][k], rows ld elements apart (16-byte aligned).  Each lane's
// 8 K-slots are one 16-byte LDS read; slots past KD are zero.
template <typename IO, int KD>
__device__ __forceinline__ floatx4 rows_mma(const char* A, const char* B, int ld, int m0,
                                            int n0, int l16, int lg, floatx4 acc) {
#pragma unroll
  for (int kb = 0; kb < (KD + 31) / 32; ++kb) {
    const int k0 = kb * 32 + 8 * lg;
    opvec<IO> a = zero_vec<IO>(), b = zero_vec<IO>();
    if (k0 < KD) {
      a = lds_vec8<IO>(A, size_t(m0 + l16) * ld + k0);
      b = lds_vec8<IO>(B, size_t(n0 + l16) * ld + k0);
    }
    acc = mma32(a, b, acc);
  }
  return acc;
}

// Operand fragment of a 16-row block of a [rows][16] bf16 slab: lanes of K
// groups 0 and 1 take 8 consecutive columns of row l16 (one 16-byte LDS
// read), groups 2 and 3 the zero half of the 32-wide K block.
__device__ __forceinline__ opvec<bf16_t> slab_row16(const __bf16* base, int l16, int lg) {
  opvec<bf16_t> x = zero_vec<bf16_t>();
  if (lg < 2) x = *reinterpret_cast<const opvec<bf16_t>*>(base + l16 * 16 + 8 * lg);
  return x;
}

// 16x16 tile product over a 16-column value slab whose operands both keep
// the contraction index contiguous in fp32 LDS: A(m, j) = A[m * ld + j],
// B(j, n) = bs(n) * B[n * ld + j] (ld even).  Lanes of K groups 0 and 1 read
// their 8 columns as 8-byte pieces, groups 2 and 3 carry the zero half of
// the 32-wide K block; the product itself is unconditional.
template <typename OP>
__device__ __forceinline__ floatx4 slab_mma(const float* A, const float* B, int ld,
                                            float bs, int l16, int lg, floatx4 acc) {
  float a[8], b[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) a[s] = b[s] = 0.f;
  if (lg < 2) {
    const float* pa = A + l16 * ld + 8 * lg;
    const float* pb = B + l16 * ld + 8 * lg;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float2 x = *reinterpret_cast<const float2*>(pa + 2 * s);
      const float2 y = *reinterpret_cast<const float2*>(pb + 2 * s);
      a[2 * s] = x.x;
      a[2 * s + 1] = x.y;
      b[2 * s] = y.x * bs;
      b[2 * s + 1] = y.y * bs;
    }
  }
  return mma32(frag<OP>::from_floats(a), frag<OP>::from_floats(b), acc);
}

// Sum of a 16x16 accumulator tile over its 16 columns: lanes with
// l16 == 0 return the sums of rows 4 lg .. 4 lg + 3.
__device__ __forceinline__ floatx4 tile_rowsum(floatx4 x) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1)
#pragma unroll
    for (int s = 0; s < 4; ++s) x[s] += __shfl_xor(x[s], m, 64);
  return x;
}

// Sum of a 16x16 accumulator tile over its 16 rows: lanes with lg == 0
// return the sum of column l16.
__device__ __forceinline__ float tile_colsum(const floatx4& x) {
  float c = x[0] + x[1] + x[2] + x[3];
  c += __shfl_xor(c, 16, 64);
  c += __shfl_xor(c, 32, 64);
  return c;
}

// Per-element form of the two products of a C x C lower-triangular matrix G
// with a key-side matrix under the per-channel pairwise decay, for the 16x16
// output tile (mt, nt) in the MFMA accumulator layout (row 4 lg + s, column
// l16), used where a chunk's channel span is too wide to factor:
//   a(r, d) = sum_{i <= r} G[r][i] A(i, d) e^{g[r][d] - g[i][d]}
//   b(r, d) = sum_{i >= r} G[i][r] B(i, d) e^{g[i][d] - g[r][d]}
template <typename FA, typename FB>
__device__ inline void pair_decay_products(const float* G, int ldg, FA A, FB B, const float* g,
                                           int DK, int C, int mt, int nt, int l16, int lg,
                                           floatx4* a, floatx4* b) {
  const int d = 16 * nt + l16;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int r = 16 * mt + 4 * lg + s;
    const float gr = g[r * DK + d];
    float x = 0.f, y = 0.f;
    for (int i = 0; i <= r; ++i) x += G[r * ldg + i] * A(i, d) * fast_exp(gr - g[i * DK + d]);
    for (int i = r; i < C; ++i) y += G[i * ldg + r] * B(i, d) * fast_exp(g[i * DK + d] - gr);
    (*a)[s] = x;
    (*b)[s] = y;
  }
}

template <int C, int DK, typename IO, int GATE, int SW>
struct GradSmem {
  static constexpr int ib = io<IO>::bytes;
  static constexpr bool CH = GATE == GDN_GATE_CHANNEL;
  static constexpr int LDK = DK + 16 / ib;   // K, Q rows (elements)
  static constexpr int LDC = C + 1;          // fp32 C x C
  // fp32 slab rows: an even pitch lets the products over the slab's columns
  // read 8-byte pieces (conflict-free at 18); the per-channel gate keeps the
  // odd pitch, its LDS budget has no room for the extra column
  static constexpr int LDS_ = CH ? SW + 1 : SW + 2;
  static constexpr int LDD = DK + 1;         // fp32 C x DK (post phase)
  static constexpr int NB = C / 16, NDT = DK / 16;
  static constexpr size_t k_off = 0;
  static constexpr size_t q_off = k_off + size_t(C) * LDK * ib;
  static constexpr size_t t_off = q_off + size_t(C) * LDK * ib;
  static constexpr size_t p_off = t_off + size_t(C) * LDC * 4;
  static constexpr size_t kk_off = p_off + size_t(C) * LDC * 4;
  static constexpr size_t g_off = kk_off + size_t(C) * LDC * 4;
  static constexpr size_t mid_off = g_off + size_t(CH ? C * DK : C) * 4;
  static constexpr size_t beta_off = mid_off + size_t(CH ? DK : 1) * 4;
  static constexpr size_t db_off = beta_off + size_t(C) * 4;
  static constexpr size_t dd_off = db_off + size_t(C) * 4;
  // per-row decays gamma_r and e^{g_C - g_r} (per-token gates)
  static constexpr size_t eq_off = dd_off + size_t(DK) * 4;
  static constexpr size_t ek_off = eq_off + size_t(CH ? 0 : C) * 4;
  // tile partial sums: [0, NB*DK) column sums of dK~ (.) K~, then dA row
  // sums [NB][C], then dX row sums [NDT][C]; the slab phase uses [0, C)
  static constexpr size_t part_off = ek_off + size_t(CH ? 0 : C) * 4;
  static constexpr size_t part_a = size_t(NB) * DK;
  static constexpr size_t part_x = part_a + size_t(NB) * C;
  static constexpr size_t part_n = part_x + size_t(NDT) * C;
  static constexpr size_t r_off = (part_off + part_n * 4 + 15) / 16 * 16;  // 16-byte rows
  // slab phase: V, dO, Z, E, dE [C][SW+1]; M0, dM1 [DK][SW+1]
  // per-token gates also keep M0 and dM1 transposed in the input dtype
  // ([SW][LDK]), so that K M0 and K dM1 read both operands as 16-byte rows
  static constexpr size_t slabt_bytes = CH ? 0 : 2 * size_t(SW) * LDK * ib;
  // bf16 inputs with per-token gates also keep dO, diag(b) V, E, dE ([C][SW])
  // and M0, dM1 ([DK][SW]) as bf16 rows for the contractions over the slab
  static constexpr bool BROWS = !CH && ib == 2 && SW == 16;
  static constexpr size_t slabb_bytes = BROWS ? (4 * size_t(C) + 2 * size_t(DK)) * SW * 2 : 0;
  // bf16 inputs, 64-token chunks, 32-column slabs (16 for the per-channel
  // gate, whose cumulative gates take 32 KB of LDS): the slab lives only as
  // bf16 rows, each operand in the layout its products read as 16-byte
  // fragments (contraction index contiguous): V, dO, E, dE [C][PR]; M0, dM1
  // [DK][PD]; M0^T, dM1^T [SW][PT]; dO^T, Z^T, dE^T [SW][PC]
  static constexpr bool FAST = ib == 2 && C == 64 && SW == (CH ? 16 : 32);
  static constexpr int PR = SW + 8, PD = SW, PT = DK + 8, PC = C + 8;
  static constexpr size_t fast_bytes =
      (4 * size_t(C) * PR + 2 * size_t(DK) * PD + 2 * size_t(SW) * PT + 3 * size_t(SW) * PC) * 2;
  static constexpr size_t slab_bytes =
      FAST ? fast_bytes
           : (5 * size_t(C) + 2 * size_t(DK)) * LDS_ * 4 + slabt_bytes + slabb_bytes;
  // post phase: dW, then dT T^T, then the gate gradient, each [C][DK+1]
  static constexpr size_t post_bytes = size_t(C) * (LDD > LDC ? LDD : LDC) * 4;
  static constexpr size_t r_bytes = slab_bytes > post_bytes ? slab_bytes : post_bytes;
  static constexpr size_t total = r_off + r_bytes;
  static constexpr bool fits = total + 16 <= 160 * 1024;
};

template <int C, int DK, typename IO, int GATE, int SW, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_grad_kernel(
    ChunkMap map, int H, int dv, int64_t nchunks, const void* __restrict__ q,
    const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ beta, const void* __restrict__ la, bool gbf,
    const void* __restrict__ d_o, const void* __restrict__ states,
    const void* __restrict__ dstates, void* __restrict__ dq,
    void* __restrict__ dk, void* __restrict__ dvv, float* __restrict__ dbeta,
    float* __restrict__ dla) {
  using OP = IO;
  using S = GradSmem<C, DK, IO, GATE, SW>;
  static_assert(S::fits, "gradient LDS budget");
  constexpr bool CH = GATE == GDN_GATE_CHANNEL;
  constexpr bool SC = GATE == GDN_GATE_SCALAR;
  constexpr int ib = S::ib;
  constexpr int NB = C / 16, NDT = DK / 16;
  constexpr int LDK = S::LDK, LDC = S::LDC, LS = S::LDS_, LDD = S::LDD;
  constexpr int VW = 16 / ib;
  constexpr int VPR = DK / VW;
  constexpr int NT = 64 * NW;                         // threads
  constexpr int NCD = NB * NDT, NU = (NCD + NW - 1) / NW;   // C x DK tiles per wave
  constexpr int NCC = NB * NB, NUC = (NCC + NW - 1) / NW;   // C x C tiles per wave
  constexpr int NCS = NB * (SW / 16);                 // C x SW tiles

  __shared__ __attribute__((aligned(16))) char smem[S::total];
  __shared__ int s_span_bits;
  char* sK = smem + S::k_off;
  char* sQ = smem + S::q_off;
  float* sT = reinterpret_cast<float*>(smem + S::t_off);
  float* sP = reinterpret_cast<float*>(smem + S::p_off);
  float* sKK = reinterpret_cast<float*>(smem + S::kk_off);
  float* sg = reinterpret_cast<float*>(smem + S::g_off);
  float* smid = reinterpret_cast<float*>(smem + S::mid_off);
  float* sbeta = reinterpret_cast<float*>(smem + S::beta_off);
  float* sdb = reinterpret_cast<float*>(smem + S::db_off);
  float* sdD = reinterpret_cast<float*>(smem + S::dd_off);
  float* seq = reinterpret_cast<float*>(smem + S::eq_off);
  float* sek = reinterpret_cast<float*>(smem + S::ek_off);
  float* spart = reinterpret_cast<float*>(smem + S::part_off);
  float* sR = reinterpret_cast<float*>(smem + S::r_off);
  // slab phase views
  float* sV = sR;
  float* sDO = sV + C * LS;
  float* sZ = sDO + C * LS;
  float* sE = sZ + C * LS;
  float* sDE = sE + C * LS;
  float* sM0 = sDE + C * LS;
  float* sDM1 = sM0 + DK * LS;
  char* sM0t = reinterpret_cast<char*>(sDM1 + DK * LS);    // [SW][LDK], !CH
  char* sDM1t = sM0t + size_t(SW) * LDK * ib;
  // bf16 slab rows (S::BROWS)
  __bf16* sDOb = reinterpret_cast<__bf16*>(sDM1t + size_t(SW) * LDK * ib);
  __bf16* sYb = sDOb + C * SW;
  __bf16* sEb = sYb + C * SW;
  __bf16* sDEb = sEb + C * SW;
  __bf16* sM0b = sDEb + C * SW;
  __bf16* sDM1b = sM0b + DK * SW;
  // post phase views
  float* sDW = sR;

  const int L = blockIdx.x;
  const int c = static_cast<int>(L / H);
  const int h = L - c * H;
  const ChunkInfo ci = chunk_info(map, c);
  if (ci.seq < 0) return;
  const int len = ci.len;
  const int64_t tok0 = ci.tok0;
  const int tid = threadIdx.x;
  // wave index in a scalar register: branches on it are scalar branches,
  // never EXEC masks (matrix instructions ignore EXEC)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  // fast slab phase: the wave's row tile and, with two waves per row tile,
  // its half of the column / key / chunk tiles (constants with one wave)
  constexpr int HWG = S::FAST ? NW / NB : 1;
  const int frt = HWG == 1 ? wave : wave % NB;
  const int fhw = HWG == 1 ? 0 : wave / NB;
  const int64_t ch = static_cast<int64_t>(h) * nchunks + c;
  // chunk-start state and chunk-end state gradient, stored in the input dtype
  const int64_t m0 = ch * DK * dv;

  // ---- 0. gates, beta, K and Q rows ----------------------------------------
  if (tid == 0) s_span_bits = 0;
  if (tid < C) {
    sbeta[tid] = tid < len ? load_gate(beta, (tok0 + tid) * H + h, gbf) : 0.f;
    sdb[tid] = 0.f;
  }
  for (int d = tid; d < DK; d += NT) sdD[d] = 0.f;
  if constexpr (!CH) {
    if (wave == 0) {
      float x = 0.f;
      if constexpr (SC)
        if (lane < len) x = load_gate(la, (tok0 + lane) * H + h, gbf);
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
      }
      if (lane < C) sg[lane] = x;
    }
  } else {
    for (int e = tid; e < C * DK; e += NT) {
      const int r = e / DK, cc = e % DK;
      sg[e] = r < len ? load_gate(la, ((tok0 + r) * H + h) * DK + cc, gbf) : 0.f;
    }
  }
  auto load_kq = [&]() {
    for (int e = tid; e < C * VPR; e += NT) {
      const int r = e / VPR, cv = (e % VPR) * VW;
      uint4 rk = make_uint4(0, 0, 0, 0), rq = make_uint4(0, 0, 0, 0);
      if (r < len) {
        const int64_t off = (((tok0 + r) * H + h) * DK + cv) * ib;
        rk = *reinterpret_cast<const uint4*>(static_cast<const char*>(k) + off);
        rq = *reinterpret_cast<const uint4*>(static_cast<const char*>(q) + off);
      }
      *reinterpret_cast<uint4*>(sK + (size_t(r) * LDK + cv) * ib) = rk;
      *reinterpret_cast<uint4*>(sQ + (size_t(r) * LDK + cv) * ib) = rq;
    }
  };
  load_kq();
  __syncthreads();
  if constexpr (CH) {
    for (int cc = tid; cc < DK; cc += NT) {
      float x = 0.f, mx = -3.0e38f, mn = 3.0e38f;
      for (int r = 0; r < C; ++r) {
        x += sg[r * DK + cc];
        sg[r * DK + cc] = x;
        mx = fmaxf(mx, x);
        mn = fminf(mn, x);
      }
      smid[cc] = 0.5f * (mx + mn);
      atomicMax(&s_span_bits, __float_as_int(0.5f * (mx - mn)));
    }
  } else if constexpr (SC) {
    if (tid < C) {
      seq[tid] = fast_exp(sg[tid]);
      sek[tid] = fast_exp(sg[C - 1] - sg[tid]);
    }
  }
  __syncthreads();

  // element readers of the chunk's matrices
  auto Kr = [&](int r, int d) { return lds_ld<IO>(sK, size_t(r) * LDK + d); };
  auto Qr = [&](int r, int d) { return lds_ld<IO>(sQ, size_t(r) * LDK + d); };
  // decays: gamma_r (per row / per (row, channel)), chunk-end relative decay
  auto gq = [&](int r, int d) -> float {
    if constexpr (CH) return fast_exp(sg[r * DK + d]);
    else if constexpr (SC) return seq[r];
    else return 1.f;
  };
  auto gk = [&](int r, int d) -> float {
    if constexpr (CH) return fast_exp(sg[(C - 1) * DK + d] - sg[r * DK + d]);
    else if constexpr (SC) return sek[r];
    else return 1.f;
  };
  auto gl = [&](int d) -> float {
    if constexpr (CH) return fast_exp(sg[(C - 1) * DK + d]);
    else if constexpr (SC) return fast_exp(sg[C - 1]);
    else return 1.f;
  };
  // factored per-channel decays around the channel's midpoint
  auto up = [&](int r, int d) -> float {   // e^{g - mid}
    if constexpr (CH) return fast_exp(sg[r * DK + d] - smid[d]);
    else return 1.f;
  };
  auto dn = [&](int r, int d) -> float {   // e^{mid - g}
    if constexpr (CH) return fast_exp(smid[d] - sg[r * DK + d]);
    else return 1.f;
  };
  auto dec = [&](int r, int i) -> float {  // scalar pairwise decay, i <= r
    if constexpr (SC) return fast_exp(sg[r] - sg[i]);
    else return 1.f;
  };
  auto Xr = [&](int r, int d) { return Kr(r, d) * sbeta[r] * gq(r, d); };
  bool exact = false;
  if constexpr (CH) exact = __int_as_float(s_span_bits) > kChannelHalfSpan;

  // ---- 1. KK = decayed K K^T (strict lower) and P (lower) ------------------
  if (!exact) {
    for (int t = wave; t < NCC; t += NW) {
      const int mt = t / NB, nt = t % NB;
      if (nt > mt) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          sKK[(16 * mt + 4 * lg + s) * LDC + 16 * nt + l16] = 0.f;
          sP[(16 * mt + 4 * lg + s) * LDC + 16 * nt + l16] = 0.f;
        }
        continue;
      }
      floatx4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
      a = tmma<OP, DK>([&](int r, int d) { return Kr(r, d) * up(r, d); },
                       [&](int d, int i) { return Kr(i, d) * dn(i, d); },
                       16 * mt, 16 * nt, l16, lg, a);
      b = tmma<OP, DK>([&](int r, int d) { return Qr(r, d) * up(r, d); },
                       [&](int d, int i) { return Kr(i, d) * dn(i, d); },
                       16 * mt, 16 * nt, l16, lg, b);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 16 * mt + 4 * lg + s, i = 16 * nt + l16;
        sKK[r * LDC + i] = i < r ? a[s] * dec(r, i) : 0.f;
        sP[r * LDC + i] = i <= r ? b[s] * dec(r, i) : 0.f;
      }
    }
  } else if constexpr (CH) {
    for (int e = tid; e < C * C; e += NT) {
      const int r = e / C, i = e % C;
      float kv = 0.f, pv = 0.f;
      if (i <= r) {
        for (int d = 0; d < DK; ++d) {
          const float dd = fast_exp(sg[r * DK + d] - sg[i * DK + d]);
          const float ki = Kr(i, d) * dd;
          kv += Kr(r, d) * ki;
          pv += Qr(r, d) * ki;
        }
      }
      sKK[r * LDC + i] = i < r ? kv : 0.f;
      sP[r * LDC + i] = pv;
    }
  }
  __syncthreads();

  // ---- 2. T = (I + diag(beta) KK)^-1 ---------------------------------------
  float* sZb = sR;  // 4 x 16 x 16 scratch of the block inverse
  if (wave == 0) {
    const int b = lane >> 4, j = lane & 15;
    if (b < NB) {
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = 0.f;
        const float br = sbeta[16 * b + r];
#pragma unroll
        for (int i = 0; i < r; ++i) s += br * sKK[(16 * b + r) * LDC + 16 * b + i] * x[i];
        x[r] = (r == j) ? 1.f : (r < j ? 0.f : -s);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[(16 * b + r) * LDC + 16 * b + j] = x[r];
    }
  } else {
    for (int e = tid - 64; e < C * C; e += NT - 64) {
      const int r = e / C, i = e % C;
      if ((i >> 4) > (r >> 4)) sT[r * LDC + i] = 0.f;
    }
  }
  __syncthreads();
  for (int b = 1; b < NB; ++b) {
    if (wave < b) {
      const int a = wave;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = lane * 4 + u, r = e >> 4, cc = e & 15;
        const float br = sbeta[16 * b + r];
        float z = 0.f;
        for (int jj = a; jj < b; ++jj) {
#pragma unroll
          for (int s = 0; s < 16; ++s)
            z += br * sKK[(16 * b + r) * LDC + 16 * jj + s] * sT[(16 * jj + s) * LDC + 16 * a + cc];
        }
        sZb[(a * 16 + r) * 16 + cc] = z;
      }
    }
    __syncthreads();
    if (wave < b) {
      const int a = wave;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = lane * 4 + u, r = e >> 4, cc = e & 15;
        float t = 0.f;
#pragma unroll
        for (int s = 0; s < 16; ++s)
          t += sT[(16 * b + r) * LDC + 16 * b + s] * sZb[(a * 16 + s) * 16 + cc];
        sT[(16 * b + r) * LDC + 16 * a + cc] = -t;
      }
    }
    __syncthreads();
  }

  // ---- 3. value slabs: accumulate everything that contracts over dv -------
  floatx4 aQ[NU], aW[NU], aK[NU];   // dQ~, -dW, dK~   (C x DK tiles)
  floatx4 aP[NUC], aT[NUC];         // dP, dE Y^T      (C x C tiles)
#pragma unroll
  for (int u = 0; u < NU; ++u) aQ[u] = aW[u] = aK[u] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NUC; ++u) aP[u] = aT[u] = floatx4{0.f, 0.f, 0.f, 0.f};

  if constexpr (S::FAST) {
    // Wave w owns row tile w (C = 64 = 16 NW) of every product.  Per slab:
    // stage (16-byte global loads, the next slab's issued before this one is
    // processed), A: Z = diag(b) (V - diag(gamma) K M0) and dE = P^T dO
    // + diag(e^{g_C - g}) K dM1, B: E = T Z and dY = T^T dE (dv, dbeta),
    // C: the contractions over the slab's columns.  All operands are read as
    // 16-byte fragments except T, T^T and P^T, built from the fp32 matrices.
    // NW = NB: wave w owns row tile w of every product; NW = 2 NB: two
    // waves share a row tile and split its column tiles (phases A, B), its
    // key tiles and chunk tiles (phase C)
    static_assert(NW == NB || NW == 2 * NB, "one or two waves per row tile");
    constexpr int PR = S::PR, PD = S::PD, PT = S::PT, PC = S::PC;
    constexpr int NKDF = (DK + 31) / 32;
    constexpr int VP = SW / 8, NVP = (C * VP + NT - 1) / NT;   // bf16 pieces
    constexpr int MP = SW / 8, NMP = (DK * MP + NT - 1) / NT;  // state pieces
    __bf16* fV = reinterpret_cast<__bf16*>(sR);
    __bf16* fDO = fV + C * PR;
    __bf16* fE = fDO + C * PR;
    __bf16* fDE = fE + C * PR;
    __bf16* fM0 = fDE + C * PR;
    __bf16* fDM1 = fM0 + DK * PD;
    __bf16* fM0t = fDM1 + DK * PD;
    __bf16* fDM1t = fM0t + SW * PT;
    __bf16* fDOt = fDM1t + SW * PT;
    __bf16* fZt = fDOt + SW * PC;
    __bf16* fDEt = fZt + SW * PC;
    auto fr = [](const __bf16* base, int idx) {
      return lds_vec8<IO>(reinterpret_cast<const char*>(base), size_t(idx));
    };
    uint4 rv[NVP], rg[NVP], rm[NMP], rd[NMP];
    float ddacc[NMP];
#pragma unroll
    for (int u = 0; u < NMP; ++u) ddacc[u] = 0.f;
    auto load = [&](int s0) {
#pragma unroll
      for (int u = 0; u < NVP; ++u) {
        const int e = tid + NT * u, r = e / VP, col = s0 + 8 * (e % VP);
        rv[u] = rg[u] = make_uint4(0, 0, 0, 0);
        if (e < C * VP && r < len && col < dv) {
          const int64_t off = (((tok0 + r) * H + h) * dv + col) * 2;
          rv[u] = *reinterpret_cast<const uint4*>(static_cast<const char*>(v) + off);
          rg[u] = *reinterpret_cast<const uint4*>(static_cast<const char*>(d_o) + off);
        }
      }
#pragma unroll
      for (int u = 0; u < NMP; ++u) {
        const int e = tid + NT * u, d = e / MP, col = s0 + 8 * (e % MP);
        rm[u] = rd[u] = make_uint4(0, 0, 0, 0);
        if (e < DK * MP && col < dv) {
          const int64_t off = (m0 + static_cast<int64_t>(d) * dv + col) * 2;
          rm[u] = *reinterpret_cast<const uint4*>(static_cast<const char*>(states) + off);
          rd[u] = *reinterpret_cast<const uint4*>(static_cast<const char*>(dstates) + off);
        }
      }
    };
    auto stage = [&]() {
#pragma unroll
      for (int u = 0; u < NVP; ++u) {
        const int e = tid + NT * u;
        if (e >= C * VP) continue;
        const int r = e / VP, j0 = 8 * (e % VP);
        *reinterpret_cast<uint4*>(fV + r * PR + j0) = rv[u];
        *reinterpret_cast<uint4*>(fDO + r * PR + j0) = rg[u];
        const __bf16* g = reinterpret_cast<const __bf16*>(&rg[u]);
#pragma unroll
        for (int q = 0; q < 8; ++q) fDOt[(j0 + q) * PC + r] = g[q];
      }
#pragma unroll
      for (int u = 0; u < NMP; ++u) {
        const int e = tid + NT * u;
        if (e >= DK * MP) continue;
        const int d = e / MP, j0 = 8 * (e % MP);
        const __bf16* m = reinterpret_cast<const __bf16*>(&rm[u]);
        const __bf16* dm = reinterpret_cast<const __bf16*>(&rd[u]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          ddacc[u] += static_cast<float>(m[q]) * static_cast<float>(dm[q]);
          fM0t[(j0 + q) * PT + d] = m[q];
          fDM1t[(j0 + q) * PT + d] = dm[q];
        }
        *reinterpret_cast<uint4*>(fM0 + d * PD + j0) = rm[u];
        *reinterpret_cast<uint4*>(fDM1 + d * PD + j0) = rd[u];
      }
    };
    if constexpr (CH) {
      // the per-element decays of the two key operands, applied once per
      // chunk: X = K (.) e^{g} over Q's rows, K~ = K (.) e^{g_C - g} over
      // K's rows (K and Q are loaded again for the post phase)
      for (int e = tid; e < C * DK; e += NT) {
        const int r = e / DK, d = e % DK;
        const float kv = Kr(r, d), g = sg[r * DK + d];
        lds_st<IO>(sQ, size_t(r) * LDK + d, kv * fast_exp(g));
        lds_st<IO>(sK, size_t(r) * LDK + d, kv * fast_exp(sg[(C - 1) * DK + d] - g));
      }
      __syncthreads();
    }
    constexpr int HW = NW / NB;
    const int r0 = 16 * frt, hw = fhw;
    floatx4 dbacc = {0.f, 0.f, 0.f, 0.f};
    // the per-channel gate's registers do not leave room for the next
    // slab's loads in flight: it loads each slab just before staging it
    if constexpr (!CH) load(0);
    for (int s0 = 0; s0 < dv; s0 += SW) {
      if constexpr (CH) load(s0);
      stage();
      if (!CH && s0 + SW < dv) load(s0 + SW);
      __syncthreads();
      // A. Z (into Z^T) and dE (rows and dE^T).  Per-token gates scale the
      // rows of K M0 and K dM1; with the per-channel gate Q's rows hold
      // K (.) e^{g} and K's rows K (.) e^{g_C - g} during the slab phase
      opvec<OP> pt[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float a[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) a[q] = sP[(32 * kb + 8 * lg + q) * LDC + r0 + l16];
        pt[kb] = frag<OP>::from_floats(a);
      }
#pragma unroll
      for (int nt = hw; nt < SW / 16; nt += HW) {
        const int j = 16 * nt + l16;
        floatx4 xm = {0.f, 0.f, 0.f, 0.f}, a1 = xm, a2 = xm;
#pragma unroll
        for (int kb = 0; kb < NKDF; ++kb) {
          const int k0 = 32 * kb + 8 * lg;
          const bool in = k0 < DK;  // lanes past DK (DK = 16) carry zeros
          const size_t ko = size_t(r0 + l16) * LDK + k0;
          const opvec<OP> xf = in ? lds_vec8<IO>(CH ? sQ : sK, ko) : zero_vec<OP>();
          const opvec<OP> kt = in ? lds_vec8<IO>(sK, ko) : zero_vec<OP>();
          xm = mma32(xf, in ? fr(fM0t, j * PT + k0) : zero_vec<OP>(), xm);
          a2 = mma32(kt, in ? fr(fDM1t, j * PT + k0) : zero_vec<OP>(), a2);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) a1 = mma32(pt[kb], fr(fDOt, j * PC + 32 * kb + 8 * lg), a1);
        bf16x4 zb, eb;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = r0 + 4 * lg + q;
          const float vr = static_cast<float>(fV[r * PR + j]);
          const float sx = CH ? 1.f : gq(r, 0), sk = CH ? 1.f : gk(r, 0);
          zb[q] = static_cast<__bf16>(sbeta[r] * (vr - sx * xm[q]));
          eb[q] = static_cast<__bf16>(a1[q] + sk * a2[q]);
          fDE[r * PR + j] = eb[q];
        }
        *reinterpret_cast<bf16x4*>(fZt + j * PC + r0 + 4 * lg) = zb;
        *reinterpret_cast<bf16x4*>(fDEt + j * PC + r0 + 4 * lg) = eb;
      }
      __syncthreads();
      // B. E = T Z (rows) and dY = T^T dE: dv = b dY, dbeta += rowsum(dY V)
      opvec<OP> tf[2], ttf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float a[8], b[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int i = 32 * kb + 8 * lg + q;
          a[q] = sT[(r0 + l16) * LDC + i];
          b[q] = sT[i * LDC + r0 + l16];
        }
        tf[kb] = frag<OP>::from_floats(a);
        ttf[kb] = frag<OP>::from_floats(b);
      }
#pragma unroll
      for (int nt = hw; nt < SW / 16; nt += HW) {
        const int j = 16 * nt + l16;
        floatx4 ee = {0.f, 0.f, 0.f, 0.f}, yy = ee;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          ee = mma32(tf[kb], fr(fZt, j * PC + 32 * kb + 8 * lg), ee);
          yy = mma32(ttf[kb], fr(fDEt, j * PC + 32 * kb + 8 * lg), yy);
        }
        floatx4 pv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = r0 + 4 * lg + q;
          fE[i * PR + j] = static_cast<__bf16>(ee[q]);
          pv[q] = yy[q] * static_cast<float>(fV[i * PR + j]);
          if (i < len && s0 + j < dv)
            io<IO>::store(dvv, ((tok0 + i) * H + h) * dv + s0 + j, sbeta[i] * yy[q]);
        }
        dbacc += tile_rowsum(pv);
      }
      __syncthreads();
      // C. contractions over the slab's columns (one K block of 32; a
      // 16-column slab fills K groups 0 and 1, the others carry zeros);
      // this wave's key tiles hw NU .. and chunk tiles hw NUC ..
      const bool kin = 8 * lg < SW;
      auto fs = [&](const __bf16* base, int idx) { return kin ? fr(base, idx) : zero_vec<OP>(); };
      const opvec<OP> fdo = fs(fDO, (r0 + l16) * PR + 8 * lg);
      const opvec<OP> fde = fs(fDE, (r0 + l16) * PR + 8 * lg);
      const opvec<OP> fe = fs(fE, (r0 + l16) * PR + 8 * lg);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int kt = hw * NU + u;
        const opvec<OP> fm = fs(fM0, (16 * kt + l16) * PD + 8 * lg);
        const opvec<OP> fd = fs(fDM1, (16 * kt + l16) * PD + 8 * lg);
        aQ[u] = mma32(fdo, fm, aQ[u]);
        aW[u] = mma32(fde, fm, aW[u]);
        aK[u] = mma32(fe, fd, aK[u]);
      }
#pragma unroll
      for (int u = 0; u < NUC; ++u) {
        const int ct = hw * NUC + u;
        aP[u] = mma32(fdo, fs(fE, (16 * ct + l16) * PR + 8 * lg), aP[u]);
        aT[u] = mma32(fde, fs(fV, (16 * ct + l16) * PR + 8 * lg), aT[u]);
      }
      __syncthreads();
    }
    // Y = diag(b) V: the scale of aT's columns
#pragma unroll
    for (int u = 0; u < NUC; ++u) {
      const float bi = sbeta[16 * (hw * NUC + u) + l16];
#pragma unroll
      for (int q = 0; q < 4; ++q) aT[u][q] *= bi;
    }
    // dbeta's slab part: the column halves' row sums, added in a fixed order
    if (l16 == 0 && hw == HW - 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) sdb[r0 + 4 * lg + q] = dbacc[q];
    }
    if constexpr (HW == 2) {
      __syncthreads();
      if (l16 == 0 && hw == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) sdb[r0 + 4 * lg + q] = dbacc[q] + sdb[r0 + 4 * lg + q];
      }
    }
    // sum_j M0 (.) dM1 per key row: the MP lanes of a row are adjacent
#pragma unroll
    for (int u = 0; u < NMP; ++u) {
      float x = ddacc[u];
#pragma unroll
      for (int m = 1; m < MP; m <<= 1) x += __shfl_xor(x, m, 64);
      const int e = tid + NT * u;
      if (e < DK * MP && e % MP == 0) sdD[e / MP] = x;
    }
    if constexpr (CH) load_kq();
    __syncthreads();
  } else {
  // slab loads in registers: the next slab's are issued as soon as the
  // current one is in LDS, so they travel while the slab is processed
  constexpr int NVE = (C * SW + NT - 1) / NT, NME = (DK * SW + NT - 1) / NT;
  float vv[NVE], gg[NVE], mm[NME], dd[NME];
  auto load_slab = [&](int s0) {
#pragma unroll
    for (int u = 0; u < NVE; ++u) {
      const int e = tid + NT * u;
      const int r = e / SW, j = e % SW;
      vv[u] = gg[u] = 0.f;
      if (e < C * SW && r < len) {
        const int64_t off = ((tok0 + r) * H + h) * dv + s0 + j;
        vv[u] = io<IO>::load(v, off);
        gg[u] = io<IO>::load(d_o, off);
      }
    }
#pragma unroll
    for (int u = 0; u < NME; ++u) {
      const int e = tid + NT * u;
      const int d = e / SW, j = e % SW;
      mm[u] = dd[u] = 0.f;
      if (e < DK * SW) {
        mm[u] = io<IO>::load(states, m0 + static_cast<int64_t>(d) * dv + s0 + j);
        dd[u] = io<IO>::load(dstates, m0 + static_cast<int64_t>(d) * dv + s0 + j);
      }
    }
  };
  load_slab(0);
  for (int s0 = 0; s0 < dv; s0 += SW) {
    // stage V, dO (rows of the chunk) and M0, dM1 (rows dk) for this slab
    {
#pragma unroll
      for (int u = 0; u < NVE; ++u) {
        const int e = tid + NT * u;
        if (e < C * SW) {
          sV[(e / SW) * LS + e % SW] = vv[u];
          sDO[(e / SW) * LS + e % SW] = gg[u];
          if constexpr (S::BROWS) {
            sDOb[e] = static_cast<__bf16>(gg[u]);
            sYb[e] = static_cast<__bf16>(sbeta[e / SW] * vv[u]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NME; ++u) {
        const int e = tid + NT * u;
        if (e < DK * SW) {
          sM0[(e / SW) * LS + e % SW] = mm[u];
          if constexpr (S::BROWS) {
            sM0b[e] = static_cast<__bf16>(mm[u]);
            sDM1b[e] = static_cast<__bf16>(dd[u]);
          }
          sDM1[(e / SW) * LS + e % SW] = dd[u];
          if constexpr (!CH) {
            lds_st<IO>(sM0t, size_t(e % SW) * LDK + e / SW, mm[u]);
            lds_st<IO>(sDM1t, size_t(e % SW) * LDK + e / SW, dd[u]);
          }
        }
      }
    }
    if (s0 + SW < dv) load_slab(s0 + SW);
    __syncthreads();
    // Z = Y - X M0 (Y = diag(b) V),  dE = P^T dO + K~ dM1
    for (int t = wave; t < 2 * NCS; t += NW) {
      const int tt = t % NCS, mt = tt / (SW / 16), nt = tt % (SW / 16);
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      if (t < NCS) {
        if constexpr (!CH) {
          // X M0 = diag(b gamma) (K M0): the row scale goes on the result
          acc = rows_mma<IO, DK>(sK, sM0t, LDK, 16 * mt, 16 * nt, l16, lg, acc);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int r = 16 * mt + 4 * lg + s, j = 16 * nt + l16;
            sZ[r * LS + j] = sbeta[r] * (sV[r * LS + j] - gq(r, 0) * acc[s]);
          }
        } else {
          acc = tmma<OP, DK>(Xr, [&](int d, int j) { return sM0[d * LS + j]; },
                             16 * mt, 16 * nt, l16, lg, acc);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int r = 16 * mt + 4 * lg + s, j = 16 * nt + l16;
            sZ[r * LS + j] = sbeta[r] * sV[r * LS + j] - acc[s];
          }
        }
      } else {
        acc = tmma<OP, C>([&](int i, int r) { return sP[r * LDC + i]; },
                          [&](int r, int j) { return sDO[r * LS + j]; },
                          16 * mt, 16 * nt, l16, lg, acc);
        if constexpr (!CH) {
          // K~ dM1 = diag(e^{g_C - g}) (K dM1)
          floatx4 a2 = {0.f, 0.f, 0.f, 0.f};
          a2 = rows_mma<IO, DK>(sK, sDM1t, LDK, 16 * mt, 16 * nt, l16, lg, a2);
#pragma unroll
          for (int s = 0; s < 4; ++s) acc[s] += gk(16 * mt + 4 * lg + s, 0) * a2[s];
        } else {
          acc = tmma<OP, DK>([&](int i, int d) { return Kr(i, d) * gk(i, d); },
                             [&](int d, int j) { return sDM1[d * LS + j]; },
                             16 * mt, 16 * nt, l16, lg, acc);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
          sDE[(16 * mt + 4 * lg + s) * LS + 16 * nt + l16] = acc[s];
        if constexpr (S::BROWS) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            sDEb[(16 * mt + 4 * lg + s) * SW + 16 * nt + l16] = static_cast<__bf16>(acc[s]);
        }
      }
    }
    __syncthreads();
    // E = T Z;  dY = T^T dE -> dv = b dY and dbeta += rowsum(dY V)
    for (int t = wave; t < 2 * NCS; t += NW) {
      const int tt = t % NCS, mt = tt / (SW / 16), nt = tt % (SW / 16);
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      if (t < NCS) {
        acc = tmma<OP, C>([&](int r, int i) { return sT[r * LDC + i]; },
                          [&](int i, int j) { return sZ[i * LS + j]; },
                          16 * mt, 16 * nt, l16, lg, acc);
#pragma unroll
        for (int s = 0; s < 4; ++s)
          sE[(16 * mt + 4 * lg + s) * LS + 16 * nt + l16] = acc[s];
        if constexpr (S::BROWS) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            sEb[(16 * mt + 4 * lg + s) * SW + 16 * nt + l16] = static_cast<__bf16>(acc[s]);
        }
      } else {
        acc = tmma<OP, C>([&](int i, int r) { return sT[r * LDC + i]; },
                          [&](int r, int j) { return sDE[r * LS + j]; },
                          16 * mt, 16 * nt, l16, lg, acc);
        floatx4 pv;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int i = 16 * mt + 4 * lg + s, j = 16 * nt + l16;
          pv[s] = acc[s] * sV[i * LS + j];
          if (i < len)
            io<IO>::store(dvv, ((tok0 + i) * H + h) * dv + s0 + j, sbeta[i] * acc[s]);
        }
        pv = tile_rowsum(pv);
        // one column tile per slab when SW == 16: fixed owner, fixed order
        if (l16 == 0) {
#pragma unroll
          for (int s = 0; s < 4; ++s) spart[nt * C + 16 * mt + 4 * lg + s] = pv[s];
        }
      }
    }
    __syncthreads();
    if (tid < C) {
      float acc = sdb[tid];
      for (int nt = 0; nt < SW / 16; ++nt) acc += spart[nt * C + tid];
      sdb[tid] = acc;
    }
    for (int d = tid; d < DK; d += NT) {
      float acc = 0.f;
      for (int j = 0; j < SW; ++j) acc += sM0[d * LS + j] * sDM1[d * LS + j];
      sdD[d] += acc;
    }
    // register accumulators (contractions over the slab's columns)
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int t = wave + NW * u;
      if (t >= NCD) continue;
      const int mt = t / NDT, nt = t % NDT;
      if constexpr (S::BROWS) {
        const opvec<OP> fdo = slab_row16(sDOb + 16 * mt * SW, l16, lg);
        const opvec<OP> fde = slab_row16(sDEb + 16 * mt * SW, l16, lg);
        const opvec<OP> fe = slab_row16(sEb + 16 * mt * SW, l16, lg);
        const opvec<OP> fm = slab_row16(sM0b + 16 * nt * SW, l16, lg);
        const opvec<OP> fd = slab_row16(sDM1b + 16 * nt * SW, l16, lg);
        aQ[u] = mma32(fdo, fm, aQ[u]);
        aW[u] = mma32(fde, fm, aW[u]);
        aK[u] = mma32(fe, fd, aK[u]);
      } else if constexpr (LS % 2 == 0 && SW == 16) {
        aQ[u] = slab_mma<OP>(sDO + 16 * mt * LS, sM0 + 16 * nt * LS, LS, 1.f, l16, lg, aQ[u]);
        aW[u] = slab_mma<OP>(sDE + 16 * mt * LS, sM0 + 16 * nt * LS, LS, 1.f, l16, lg, aW[u]);
        aK[u] = slab_mma<OP>(sE + 16 * mt * LS, sDM1 + 16 * nt * LS, LS, 1.f, l16, lg, aK[u]);
      } else {
        auto M0t = [&](int j, int d) { return sM0[d * LS + j]; };
        aQ[u] = tmma<OP, SW>([&](int r, int j) { return sDO[r * LS + j]; }, M0t,
                             16 * mt, 16 * nt, l16, lg, aQ[u]);
        aW[u] = tmma<OP, SW>([&](int r, int j) { return sDE[r * LS + j]; }, M0t,
                             16 * mt, 16 * nt, l16, lg, aW[u]);
        aK[u] = tmma<OP, SW>([&](int r, int j) { return sE[r * LS + j]; },
                             [&](int j, int d) { return sDM1[d * LS + j]; },
                             16 * mt, 16 * nt, l16, lg, aK[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < NUC; ++u) {
      const int t = wave + NW * u;
      if (t >= NCC) continue;
      const int mt = t / NB, nt = t % NB;
      if constexpr (S::BROWS) {
        aP[u] = mma32(slab_row16(sDOb + 16 * mt * SW, l16, lg),
                      slab_row16(sEb + 16 * nt * SW, l16, lg), aP[u]);
        aT[u] = mma32(slab_row16(sDEb + 16 * mt * SW, l16, lg),
                      slab_row16(sYb + 16 * nt * SW, l16, lg), aT[u]);
      } else if constexpr (LS % 2 == 0 && SW == 16) {
        aP[u] = slab_mma<OP>(sDO + 16 * mt * LS, sE + 16 * nt * LS, LS, 1.f, l16, lg, aP[u]);
        aT[u] = slab_mma<OP>(sDE + 16 * mt * LS, sV + 16 * nt * LS, LS,
                             sbeta[16 * nt + l16], l16, lg, aT[u]);
      } else {
        aP[u] = tmma<OP, SW>([&](int r, int j) { return sDO[r * LS + j]; },
                             [&](int j, int i) { return sE[i * LS + j]; },
                             16 * mt, 16 * nt, l16, lg, aP[u]);
        aT[u] = tmma<OP, SW>([&](int r, int j) { return sDE[r * LS + j]; },
                             [&](int j, int i) { return sbeta[i] * sV[i * LS + j]; },
                             16 * mt, 16 * nt, l16, lg, aT[u]);
      }
    }
    __syncthreads();
  }
  }  // slab phase

  // ---- 4. post: through T, the decays and K K^T / Q K^T --------------------
  // tile u of this wave: C x DK tiles (mt, nt) and C x C tiles; the fast
  // slab phase gives wave w row tile w, the others deal tiles round robin
  auto tile_cd = [&](int u, int* mt, int* nt) -> bool {
    if constexpr (S::FAST) {
      *mt = frt;
      *nt = fhw * NU + u;
      return true;
    } else {
      const int t = wave + NW * u;
      *mt = t / NDT;
      *nt = t % NDT;
      return t < NCD;
    }
  };
  auto tile_cc = [&](int u, int* mt, int* nt) -> bool {
    if constexpr (S::FAST) {
      *mt = frt;
      *nt = fhw * NUC + u;
      return true;
    } else {
      const int t = wave + NW * u;
      *mt = t / NB;
      *nt = t % NB;
      return t < NCC;
    }
  };
  // dq = dQ~ (.) gamma + dq_P ; dk = dK~ (.) e^{g_C - g} + dX (.) b gamma + ...
  // dg collects the per-(row, channel) gate gradient.
  floatx4 oq[NU], ok[NU], og[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if constexpr (CH) __builtin_amdgcn_sched_barrier(0);  // tiles one at a time (registers)
    oq[u] = ok[u] = og[u] = floatx4{0.f, 0.f, 0.f, 0.f};
    int mt, nt;
    if (!tile_cd(u, &mt, &nt)) continue;
    floatx4 cs;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = 16 * mt + 4 * lg + s, d = 16 * nt + l16;
      const float eq = gq(r, d), ek = gk(r, d);
      oq[u][s] = aQ[u][s] * eq;
      ok[u][s] = aK[u][s] * ek;
      const float kt = aK[u][s] * Kr(r, d) * ek;  // dK~ (.) K~
      og[u][s] = aQ[u][s] * Qr(r, d) * eq - kt;
      cs[s] = kt;
    }
    // the chunk-end decay e^{g_C} of K~ sends sum_i dK~ (.) K~ to the last row
    const float colsum = tile_colsum(cs);
    if (lg == 0) spart[mt * DK + 16 * nt + l16] = colsum;
  }
  // dW into LDS (dW = -aW), dP decayed into sP (overwrites P)
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if constexpr (CH) __builtin_amdgcn_sched_barrier(0);  // tiles one at a time (registers)
    int mt, nt;
    if (!tile_cd(u, &mt, &nt)) continue;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      sDW[(16 * mt + 4 * lg + s) * LDD + 16 * nt + l16] = -aW[u][s];
  }
  __syncthreads();  // all P reads of the slab phase are done
#pragma unroll
  for (int u = 0; u < NUC; ++u) {
    if constexpr (CH) __builtin_amdgcn_sched_barrier(0);  // tiles one at a time (registers)
    int mt, nt;
    if (!tile_cc(u, &mt, &nt)) continue;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = 16 * mt + 4 * lg + s, i = 16 * nt + l16;
      sP[r * LDC + i] = i <= r ? aP[u][s] * dec(r, i) : 0.f;
    }
  }
  __syncthreads();
  // dX = T^T dW ;  dq_P, dk_P ;  dT = dE Y^T + dW X^T (kept in registers)
  floatx4 oX[NU];
#pragma unroll
  for (int u = 0; u < NUC; ++u) {
    if constexpr (CH) __builtin_amdgcn_sched_barrier(0);  // tiles one at a time (registers)
    int mt, nt;
    if (!tile_cc(u, &mt, &nt)) continue;
    aT[u] = tmma<OP, DK>([&](int r, int d) { return sDW[r * LDD + d]; },
                         [&](int d, int i) { return Xr(i, d); },
                         16 * mt, 16 * nt, l16, lg, aT[u]);
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if constexpr (CH) __builtin_amdgcn_sched_barrier(0);  // tiles one at a time (registers)
    oX[u] = floatx4{0.f, 0.f, 0.f, 0.f};
    int mt, nt;
    if (!tile_cd(u, &mt, &nt)) continue;
    oX[u] = tmma<OP, C>([&](int i, int r) { return sT[r * LDC + i]; },
                        [&](int r, int d) { return sDW[r * LDD + d]; },
                        16 * mt, 16 * nt, l16, lg, oX[u]);
    // dq_P = (dP o Gamma) K  (channel: factored around the midpoint)
    floatx4 tq = {0.f, 0.f, 0.f, 0.f}, tk = tq;
    if (exact) {  // channel spans beyond the factored range: per element
      pair_decay_products(sP, LDC, Kr, Qr, sg, DK, C, mt, nt, l16, lg, &tq, &tk);
    } else {
      tq = tmma<OP, C>([&](int r, int i) { return sP[r * LDC + i]; },
                       [&](int i, int d) { return Kr(i, d) * dn(i, d); },
                       16 * mt, 16 * nt, l16, lg, tq);
      // dk_P = (dP o Gamma)^T Q
      tk = tmma<OP, C>([&](int i, int r) { return sP[r * LDC + i]; },
                       [&](int r, int d) { return Qr(r, d) * up(r, d); },
                       16 * mt, 16 * nt, l16, lg, tk);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = 16 * mt + 4 * lg + s, d = 16 * nt + l16;
      const float vq = exact ? tq[s] : tq[s] * up(r, d);
      const float vk = exact ? tk[s] : tk[s] * dn(r, d);
      oq[u][s] += vq;
      ok[u][s] += vk;
      og[u][s] += Qr(r, d) * vq - Kr(r, d) * vk;
    }
  }
  __syncthreads();
  // dT into sP (dP is consumed)
  float* sDT = sP;
#pragma unroll
  for (int u = 0; u < NUC; ++u) {
    if constexpr (CH) __builtin_amdgcn_sched_barrier(0);  // tiles one at a time (registers)
    int mt, nt;
    if (!tile_cc(u, &mt, &nt)) continue;
#pragma unroll
    for (int s = 0; s < 4; ++s) sDT[(16 * mt + 4 * lg + s) * LDC + 16 * nt + l16] = aT[u][s];
  }
  __syncthreads();
  // Z2 = dT T^T into the dW bytes (dW is consumed)
  float* sZ2 = sR;
#pragma unroll
  for (int u = 0; u < NUC; ++u) {
    if constexpr (CH) __builtin_amdgcn_sched_barrier(0);  // tiles one at a time (registers)
    int mt, nt;
    if (!tile_cc(u, &mt, &nt)) continue;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tmma<OP, C>([&](int r, int cc) { return sDT[r * LDC + cc]; },
                      [&](int cc, int i) { return sT[i * LDC + cc]; },
                      16 * mt, 16 * nt, l16, lg, acc);
#pragma unroll
    for (int s = 0; s < 4; ++s) sZ2[(16 * mt + 4 * lg + s) * LDC + 16 * nt + l16] = acc[s];
  }
  __syncthreads();
  // dA = -T^T Z2 (strict lower); dbeta += rowsum(dA (.) KK); b (.) dA (scalar
  // gate: with the pairwise decay) replaces dT in sP
  float* sDA = sP;
#pragma unroll
  for (int u = 0; u < NUC; ++u) {
    if constexpr (CH) __builtin_amdgcn_sched_barrier(0);  // tiles one at a time (registers)
    int mt, nt;
    if (!tile_cc(u, &mt, &nt)) continue;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tmma<OP, C>([&](int a, int r) { return sT[r * LDC + a]; },
                      [&](int r, int b) { return sZ2[r * LDC + b]; },
                      16 * mt, 16 * nt, l16, lg, acc);
    aT[u] = acc;
  }
  __syncthreads();  // every read of dT is done before dA overwrites it
#pragma unroll
  for (int u = 0; u < NUC; ++u) {
    if constexpr (CH) __builtin_amdgcn_sched_barrier(0);  // tiles one at a time (registers)
    int mt, nt;
    if (!tile_cc(u, &mt, &nt)) continue;
    floatx4 pb;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int a = 16 * mt + 4 * lg + s, b = 16 * nt + l16;
      const float da = b < a ? -aT[u][s] : 0.f;
      pb[s] = da * sKK[a * LDC + b];
      sDA[a * LDC + b] = b < a ? da * sbeta[a] * dec(a, b) : 0.f;
    }
    pb = tile_rowsum(pb);
    if (l16 == 0) {
#pragma unroll
      for (int s = 0; s < 4; ++s) spart[S::part_a + nt * C + 16 * mt + 4 * lg + s] = pb[s];
    }
  }
  __syncthreads();
  // dk_A1 = (b dA o Gamma) K, dk_A2 = (b dA o Gamma)^T K, and the dX terms
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if constexpr (CH) __builtin_amdgcn_sched_barrier(0);  // tiles one at a time (registers)
    int mt, nt;
    if (!tile_cd(u, &mt, &nt)) continue;
    floatx4 t1 = {0.f, 0.f, 0.f, 0.f}, t2 = {0.f, 0.f, 0.f, 0.f};
    if (exact) {
      pair_decay_products(sDA, LDC, Kr, Kr, sg, DK, C, mt, nt, l16, lg, &t1, &t2);
    } else {
      t1 = tmma<OP, C>([&](int r, int i) { return sDA[r * LDC + i]; },
                       [&](int i, int d) { return Kr(i, d) * dn(i, d); },
                       16 * mt, 16 * nt, l16, lg, t1);
      t2 = tmma<OP, C>([&](int i, int r) { return sDA[r * LDC + i]; },
                       [&](int r, int d) { return Kr(r, d) * up(r, d); },
                       16 * mt, 16 * nt, l16, lg, t2);
    }
    floatx4 pb;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = 16 * mt + 4 * lg + s, d = 16 * nt + l16;
      const float v1 = exact ? t1[s] : t1[s] * up(r, d);
      const float v2 = exact ? t2[s] : t2[s] * dn(r, d);
      const float kr = Kr(r, d), eq = gq(r, d);
      ok[u][s] += v1 + v2 + oX[u][s] * sbeta[r] * eq;
      og[u][s] += kr * (v1 - v2) + oX[u][s] * sbeta[r] * eq * kr;
      pb[s] = oX[u][s] * kr * eq;
    }
    pb = tile_rowsum(pb);
    if (l16 == 0) {
#pragma unroll
      for (int s = 0; s < 4; ++s) spart[S::part_x + nt * C + 16 * mt + 4 * lg + s] = pb[s];
    }
  }
  __syncthreads();
  if (tid < C) {
    float acc = sdb[tid];
    for (int nt = 0; nt < NB; ++nt) acc += spart[S::part_a + nt * C + tid];
    for (int nt = 0; nt < NDT; ++nt) acc += spart[S::part_x + nt * C + tid];
    if (tid < len) dbeta[(tok0 + tid) * H + h] = acc;
  }
  // last row: sum_i dK~ (.) K~ and the chunk-end decay of the state
  float* sdg = sR;  // [C][DK+1] gate gradient per (row, channel)
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if constexpr (CH) __builtin_amdgcn_sched_barrier(0);  // tiles one at a time (registers)
    int mt, nt;
    if (!tile_cd(u, &mt, &nt)) continue;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = 16 * mt + 4 * lg + s, d = 16 * nt + l16;
      float x = og[u][s];
      if (r == C - 1) {
        float cs = 0.f;
        for (int b = 0; b < NB; ++b) cs += spart[b * DK + d];
        x += cs + gl(d) * sdD[d];
      }
      sdg[r * LDD + d] = x;
      if (r < len) {
        const int64_t off = ((tok0 + r) * H + h) * DK + d;
        io<IO>::store(dq, off, oq[u][s]);
        io<IO>::store(dk, off, ok[u][s]);
      }
    }
  }
  __syncthreads();
  // d log alpha = reverse cumulative sum of dg inside the chunk
  if constexpr (CH) {
    for (int d = tid; d < DK; d += NT) {
      float acc = 0.f;
      for (int r = C - 1; r >= 0; --r) {
        acc += sdg[r * LDD + d];
        if (r < len) dla[((tok0 + r) * H + h) * DK + d] = acc;
      }
    }
  } else if constexpr (SC) {
    if (tid < C) {
      float x = 0.f;
      for (int d = 0; d < DK; ++d) x += sdg[tid * LDD + d];
      spart[tid] = x;
    }
    __syncthreads();
    if (tid == 0) {
      float acc = 0.f;
      for (int r = C - 1; r >= 0; --r) {
        acc += spart[r];
        if (r < len) dla[(tok0 + r) * H + h] = acc;
      }
    }
  }
}

// ------------------------------------------------------------ dispatch ---

// Chunk-start states and chunk-end state gradients, one [dk][dv] matrix
// per chunk-head in the input dtype.
inline size_t bwd_states_bytes(const Problem& p) {
  return FwdLayout::al(size_t(p.nchunks) * p.H * p.dk * p.dv * (p.io == GDN_BF16 ? 2 : 4));
}

constexpr int kSlab = 16;  // value columns per slab of the gradient kernel
// waves of the gradient kernel (its LDS plan allows one workgroup per CU).
// Eight waves were measured against four on the 16k varlen batch: the same
// time with the scalar gate (2.50 against 2.52 ms) and slower with the
// per-channel gate (8.4 against 8.0 ms), whose accumulators then spill.
constexpr int kGradWaves = 4;

// waves of the gradient kernel: 8 on the fast slab phase with dk >= 32 (two
// waves per row tile), kGradWaves otherwise
template <int C, int DK, typename IO, int GATE>
constexpr int grad_waves();

// value columns per slab: 32 with bf16 inputs, per-token gates and 64-token
// chunks, kSlab otherwise (bf16 with the per-channel gate and 64-token
// chunks takes the same fast slab phase at kSlab columns)
template <int C, typename IO, int GATE>
constexpr int grad_slab() {
  return (io<IO>::bytes == 2 && GATE != GDN_GATE_CHANNEL && C == 64) ? 32 : kSlab;
}

template <int C, int DK, typename IO, int GATE>
constexpr int grad_waves() {
  return (GradSmem<C, DK, IO, GATE, grad_slab<C, IO, GATE>()>::FAST &&
          DK >= 32) ? 8 : kGradWaves;
}

template <int C, int DK, typename IO, int GATE>
hipError_t run_bwd(const Problem& p, const void* q, const void* k,
                   const void* v, const void* beta, const void* la,
                   const float* s0, const void* d_o, const float* ds_final,
                   void* dq, void* dk, void* dv, float* dbeta, float* dla,
                   float* ds0, char* ws, hipStream_t s) {
  constexpr int SW = grad_slab<C, IO, GATE>();
  if constexpr (!GradSmem<C, DK, IO, GATE, SW>::fits) {
    return hipErrorNotSupported;
  } else {
  const FwdLayout L(C, DK, p.dv, opstore<IO>::bytes, GATE == GDN_GATE_CHANNEL, true);
  char* map_base = ws;
  char* ops = ws + chunk_map_bytes(p);
  const FwdBuffers buf = make_buffers(ops, L);
  char* states = ops + size_t(p.nchunks) * p.H * L.per_ch;
  char* dstates = states + bwd_states_bytes(p);
  const ChunkMap map = make_chunk_map(p, map_base);
  const bool gbf = p.gdt == GDN_BF16;
  hipError_t e;
  if (p.varlen) {
    e = launch_chunk_map(p, map_base, s);
    if (e != hipSuccess) return e;
  }
  const SegMap sm = make_seg_map(p, map_base, p.seg);
  // the reverse pass has one workgroup per (chain, 16-column slab) already;
  // it is split into segments only while those leave the CUs short of work
  // (splitting adds a pass over all but the first segment)
  constexpr int64_t kRevSplitBelow = 512;
  const bool rseg = p.seg > 0 && static_cast<int64_t>(p.nseq) * p.H * (p.dv / 16) < kRevSplitBelow;
  const SegMap rsm = rseg ? sm : make_seg_map(p, map_base, 0);
  const int64_t nwork = (rseg ? p.nsegs : p.nseq) * p.H * (p.dv / 16);
  const SegBuffers sb = make_seg_buffers(p, dstates + bwd_states_bytes(p), opstore<IO>::bytes);
  if (p.nchunks > 0) {
    {
      StageScope scope(GDN_STAGE_FWD_PREP, s);
      if constexpr (GATE == GDN_GATE_CHANNEL)
        hipLaunchKernelGGL((fwd_prep_kernel<C, DK, IO, GATE, true, kPrepChWaves>),
                           dim3(static_cast<unsigned>(p.nchunks * p.H)), dim3(64 * kPrepChWaves), 0, s,
                           map, p.H, p.dv, p.nchunks, q, k, v, beta, la, gbf, buf, nullptr);
      else
        hipLaunchKernelGGL((fwd_prep_sg_kernel<C, DK, IO, GATE, true>),
                           dim3(static_cast<unsigned>(p.nchunks * p.H)),
                           dim3(64 * prep_waves(C)), 0, s, map, p.H, p.dv, p.nchunks, q, k, v,
                           beta, la, gbf, buf, 0, false, static_cast<const int32_t*>(nullptr),
                           static_cast<const void*>(nullptr));
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    {
      // the forward's state pass, storing every chunk-start state: split
      // into segments like the forward (per-segment maps, their chain,
      // then every segment from its entering state) when the plan says so
      StageScope scope(GDN_STAGE_BWD_STATES, s);
      const int ndvt = p.dv / 16;
      if (p.seg > 0) {
        const int64_t tgrp = (ndvt + DK / 16 + kTransGroup - 1) / kTransGroup;
        hipLaunchKernelGGL((fwd_trans_kernel<C, DK, IO, GATE>),
                           dim3(static_cast<unsigned>(p.nsegs * p.H * tgrp)),
                           dim3(64 * kTransWaves), 0, s, map, sm, p.H, p.dv, p.nchunks,
                           buf, sb, rseg);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((fwd_combine_kernel<DK, IO>),
                           dim3(static_cast<unsigned>(p.nseq * p.H * ndvt)),
                           dim3(64 * ((DK + 31) / 32)), 0, s, map, sm, p.H, p.dv, s0, sb);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      const int64_t ngrp = (ndvt + kScanGroup - 1) / kScanGroup;
      hipLaunchKernelGGL((fwd_scan_kernel<C, DK, IO, GATE, true>),
                         dim3(static_cast<unsigned>(p.nsegs * p.H * ngrp)),
                         dim3(64 * kScanWaves), 0, s, map,
                         sm, p.H, p.dv, p.nchunks, q, s0,
                         static_cast<void*>(nullptr), static_cast<float*>(nullptr),
                         buf, sb, states, 0);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  {
    // split like the state recomputation: each segment's reverse map from a
    // zero gradient (its M0 buffer is free again), the chain over segments
    // through the transposed transitions (into the entering-state buffer),
    // then every segment from its entering gradient
    StageScope scope(GDN_STAGE_BWD_SCAN, s);
    // bf16: the LDS-shared pass, kRevSlabs slabs per workgroup
    constexpr bool kLds = io<IO>::bytes == 2;
    const int64_t chains = (rseg ? p.nsegs : p.nseq) * p.H;
    const int64_t nlds = chains * ((p.dv / 16 + kRevSlabs - 1) / kRevSlabs);
    if constexpr (kLds) {
      if (RevLds<C, DK>::REG != L.g + L.kf + L.wt + L.pt + L.qt) return hipErrorInvalidValue;
    }
    if (rseg && p.nchunks > 0) {
      if constexpr (kLds)
        hipLaunchKernelGGL((bwd_scan_lds_kernel<C, DK, GATE, true>),
                           dim3(static_cast<unsigned>(nlds)), dim3(64 * kRevSlabs), 0, s, map,
                           rsm, p.H, p.dv, p.nchunks, d_o, ds_final, ds0, buf, dstates,
                           static_cast<const float*>(nullptr), sb.trm);
      else
        hipLaunchKernelGGL((bwd_scan_kernel<C, DK, IO, GATE, true>),
                           dim3(static_cast<unsigned>(nwork)), dim3(128), 0, s, map, rsm,
                           p.H, p.dv, p.nchunks, d_o, ds_final, ds0, buf, dstates,
                           static_cast<const float*>(nullptr), sb.trm);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((bwd_combine_kernel<DK, IO>),
                         dim3(static_cast<unsigned>(p.nseq * p.H * (p.dv / 16))), dim3(64),
                         0, s, map, rsm, p.H, p.dv, ds_final, sb,
                         static_cast<const float*>(sb.trm), sb.ss);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if constexpr (kLds)
      hipLaunchKernelGGL((bwd_scan_lds_kernel<C, DK, GATE>),
                         dim3(static_cast<unsigned>(nlds)), dim3(64 * kRevSlabs), 0, s, map, rsm,
                         p.H, p.dv, p.nchunks, d_o, ds_final, ds0, buf, dstates,
                         static_cast<const float*>(sb.ss), static_cast<float*>(nullptr));
    else
      hipLaunchKernelGGL((bwd_scan_kernel<C, DK, IO, GATE>),
                         dim3(static_cast<unsigned>(nwork)), dim3(128), 0, s, map, rsm,
                         p.H, p.dv, p.nchunks, d_o, ds_final, ds0, buf, dstates,
                         static_cast<const float*>(sb.ss), static_cast<float*>(nullptr));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.nchunks > 0) {
    StageScope scope(GDN_STAGE_BWD_GRAD, s);
    constexpr int NW = grad_waves<C, DK, IO, GATE>();
    hipLaunchKernelGGL((bwd_grad_kernel<C, DK, IO, GATE, SW, NW>),
                       dim3(static_cast<unsigned>(p.nchunks * p.H)), dim3(64 * NW), 0, s,
                       map, p.H, p.dv, p.nchunks, q, k, v, beta, la, gbf, d_o,
                       states, dstates, dq, dk, dv, dbeta, dla);
    e = hipGetLastError();
  }
  return e;
  }
}

template <int C, int DK, typename IO>
bool fits_gate(int gate) {
  switch (gate) {
    case GDN_GATE_NONE:
      return GradSmem<C, DK, IO, GDN_GATE_NONE, grad_slab<C, IO, GDN_GATE_NONE>()>::fits;
    case GDN_GATE_SCALAR:
      return GradSmem<C, DK, IO, GDN_GATE_SCALAR, grad_slab<C, IO, GDN_GATE_SCALAR>()>::fits;
    default:
      return GradSmem<C, DK, IO, GDN_GATE_CHANNEL, grad_slab<C, IO, GDN_GATE_CHANNEL>()>::fits;
  }
}

template <int C>
bool fits_dk(const Problem& p) {
  const bool bf = p.io == GDN_BF16;
  switch (p.dk) {
    case 16: return bf ? fits_gate<C, 16, bf16_t>(p.gate) : fits_gate<C, 16, f32_t>(p.gate);
    case 32: return bf ? fits_gate<C, 32, bf16_t>(p.gate) : fits_gate<C, 32, f32_t>(p.gate);
    case 64: return bf ? fits_gate<C, 64, bf16_t>(p.gate) : fits_gate<C, 64, f32_t>(p.gate);
    default: return bf ? fits_gate<C, 128, bf16_t>(p.gate) : fits_gate<C, 128, f32_t>(p.gate);
  }
}

template <int C, int DK, typename IO>
hipError_t bwd_gate(const Problem& p, const void* q, const void* k,
                    const void* v, const void* beta, const void* la,
                    const float* s0, const void* d_o, const float* dsf,
                    void* dq, void* dk, void* dv, float* db, float* dla,
                    float* ds0, char* ws, hipStream_t s) {
  switch (p.gate) {
    case GDN_GATE_NONE:
      return run_bwd<C, DK, IO, GDN_GATE_NONE>(p, q, k, v, beta, la, s0, d_o, dsf, dq, dk, dv, db, dla, ds0, ws, s);
    case GDN_GATE_SCALAR:
      return run_bwd<C, DK, IO, GDN_GATE_SCALAR>(p, q, k, v, beta, la, s0, d_o, dsf, dq, dk, dv, db, dla, ds0, ws, s);
    default:
      return run_bwd<C, DK, IO, GDN_GATE_CHANNEL>(p, q, k, v, beta, la, s0, d_o, dsf, dq, dk, dv, db, dla, ds0, ws, s);
  }
}

template <int C, int DK>
hipError_t bwd_types(const Problem& p, const void* q, const void* k,
                     const void* v, const void* beta, const void* la,
                     const float* s0, const void* d_o, const float* dsf,
                     void* dq, void* dk, void* dv, float* db, float* dla,
                     float* ds0, char* ws, hipStream_t s) {
  if (p.io == GDN_BF16)
    return bwd_gate<C, DK, bf16_t>(p, q, k, v, beta, la, s0, d_o, dsf, dq, dk, dv, db, dla, ds0, ws, s);
  return bwd_gate<C, DK, f32_t>(p, q, k, v, beta, la, s0, d_o, dsf, dq, dk, dv, db, dla, ds0, ws, s);
}

template <int C>
hipError_t bwd_dk(const Problem& p, const void* q, const void* k,
                  const void* v, const void* beta, const void* la,
                  const float* s0, const void* d_o, const float* dsf,
                  void* dq, void* dk, void* dv, float* db, float* dla,
                  float* ds0, char* ws, hipStream_t s) {
  switch (p.dk) {
    case 16: return bwd_types<C, 16>(p, q, k, v, beta, la, s0, d_o, dsf, dq, dk, dv, db, dla, ds0, ws, s);
    case 32: return bwd_types<C, 32>(p, q, k, v, beta, la, s0, d_o, dsf, dq, dk, dv, db, dla, ds0, ws, s);
    case 64: return bwd_types<C, 64>(p, q, k, v, beta, la, s0, d_o, dsf, dq, dk, dv, db, dla, ds0, ws, s);
    default: return bwd_types<C, 128>(p, q, k, v, beta, la, s0, d_o, dsf, dq, dk, dv, db, dla, ds0, ws, s);
  }
}

}  // namespace

bool bwd_supported(const Problem& p) {
  switch (p.chunk) {
    case 16: return fits_dk<16>(p);
    case 32: return fits_dk<32>(p);
    default: return fits_dk<64>(p);
  }
}

size_t bwd_workspace_bytes(const Problem& p) {
  const int ob = p.io == GDN_BF16 ? 2 : 4;
  const FwdLayout L(p.chunk, p.dk, p.dv, ob, p.gate == GDN_GATE_CHANNEL, true);
  return chunk_map_bytes(p) + size_t(p.nchunks) * p.H * L.per_ch +
         2 * bwd_states_bytes(p) + seg_buffer_bytes(p, ob);
}

hipError_t launch_bwd(const Problem& p, const void* q, const void* k,
                      const void* v, const void* beta, const void* la,
                      const float* s0, const void* d_o, const float* ds_final,
                      void* dq, void* dk, void* dv, float* dbeta, float* dla,
                      float* ds0, void* ws, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  switch (p.chunk) {
    case 16: return bwd_dk<16>(p, q, k, v, beta, la, s0, d_o, ds_final, dq, dk, dv, dbeta, dla, ds0, w, s);
    case 32: return bwd_dk<32>(p, q, k, v, beta, la, s0, d_o, ds_final, dq, dk, dv, dbeta, dla, ds0, w, s);
    default: return bwd_dk<64>(p, q, k, v, beta, la, s0, d_o, ds_final, dq, dk, dv, dbeta, dla, ds0, w, s);
  }
}

}  // namespace gdn
