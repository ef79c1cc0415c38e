// Forward kernels of the chunkwise gated delta rule, shared by the forward
// and (recomputation inside) the backward entry points.  See gdn_fwd.hip for
// the algorithm.
#pragma once

#include "gdn_chunk_common.hpp"

namespace gdn {
namespace {

// Half-span limit of the per-channel log-gate within one chunk for the
// factored products: each factor stays within exp(+-80), inside the fp32 and
// bf16 normal range.  Chunks beyond it take an exact per-element path.
constexpr float kChannelHalfSpan = 80.f;

// ------------------------------------------------------------ LDS plan ---

template <int C, int DK, typename IO, int GATE, bool BWD>
struct PrepSmem {
  static constexpr int ib = io<IO>::bytes;
  static constexpr int LDT = C + 16 / ib;           // K^T rows (elements)
  static constexpr int LDK = DK + 16 / ib;          // K rows (elements)
  static constexpr int LDC = C + 4;                 // fp32 C x C matrices
  static constexpr int LDV = C + 16 / ib;           // V^T rows (elements)
  static constexpr bool CH = GATE == GDN_GATE_CHANNEL;
  static constexpr int NG = CH ? C * DK : C;
  static constexpr size_t kt_off = 0;
  static constexpr size_t k_off = kt_off + size_t(DK) * LDT * ib;
  static constexpr size_t g_off = k_off + size_t(C) * LDK * ib;
  static constexpr size_t mid_off = g_off + size_t(NG) * 4;
  static constexpr size_t beta_off = mid_off + size_t(CH ? DK : 4) * 4;
  static constexpr size_t xs_off = beta_off + size_t(C) * 4;
  static constexpr size_t ks_off = xs_off + size_t(C) * 4;
  static constexpr size_t t_off = ks_off + size_t(C) * 4;
  static constexpr size_t z_off = t_off + size_t(C) * LDC * 4;
  // A lives until T is formed; then the same bytes hold V^T slabs (and, on
  // the exact per-channel path, P before that)
  static constexpr size_t a_off = z_off + 4 * 256 * 4;
  static constexpr size_t a_bytes = size_t(C) * LDC * 4;
  static constexpr size_t v_bytes = 64 * size_t(LDV) * ib;
  static constexpr size_t p_off = a_off + (a_bytes > v_bytes ? a_bytes : v_bytes);
  // per-channel gate, bf16 inputs: the decay factors e^{g - mid} and
  // e^{mid - g} of every (row, channel) as bf16 rows [C][LDE], formed once
  static constexpr bool EF = CH && ib == 2;
  static constexpr int LDE = DK + 8;
  static constexpr size_t eu_off = p_off + (CH ? size_t(C) * LDC * 4 : 0);
  static constexpr size_t total = eu_off + (EF ? 2 * size_t(C) * LDE * 2 : 0);
  static_assert(total <= 160 * 1024, "prep LDS budget");
};

template <typename IO>
__device__ inline float lds_ld(const char* base, size_t idx) {
  if constexpr (io<IO>::bytes == 2)
    return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(base)[idx]);
  else
    return reinterpret_cast<const float*>(base)[idx];
}

// 8 consecutive LDS elements of the input dtype, as floats.
template <typename IO>
__device__ inline void lds_ld8(const char* base, size_t idx, float* out) {
  if constexpr (io<IO>::bytes == 2) {
    const uint4 raw = *reinterpret_cast<const uint4*>(base + idx * 2);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      out[2 * s] = __uint_as_float(w[s] << 16);
      out[2 * s + 1] = __uint_as_float(w[s] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(base + idx * 4);
    const float4 a = p[0], b = p[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

// 8 consecutive LDS elements of the input dtype, as an operand vector.
template <typename IO>
__device__ inline opvec<IO> lds_vec8(const char* base, size_t idx) {
  return *reinterpret_cast<const opvec<IO>*>(base + idx * io<IO>::bytes);
}

// 4 consecutive LDS elements of the input dtype, as floats.
template <typename IO>
__device__ inline void lds_ld4(const char* base, size_t idx, float* out) {
  if constexpr (io<IO>::bytes == 2) {
    const uint2 raw = *reinterpret_cast<const uint2*>(base + idx * 2);
    out[0] = __uint_as_float(raw.x << 16);
    out[1] = __uint_as_float(raw.x & 0xffff0000u);
    out[2] = __uint_as_float(raw.y << 16);
    out[3] = __uint_as_float(raw.y & 0xffff0000u);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(base + idx * 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  }
}

__device__ inline void lds_f8(const float* p, float* out) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// A row fragment of an input tensor [tokens, H, DK]: row r of the chunk,
// K-slots k0 .. k0+7; zero past the chunk length or the key size.
template <typename IO, int DK>
__device__ inline opvec<IO> row_frag(const void* x, int64_t tok0, int H, int h,
                                     int r, int len, int k0) {
  if (r >= len || k0 >= DK) return zero_vec<IO>();
  return gload8<IO>(x, ((tok0 + r) * H + h) * DK + k0);
}

// 4 consecutive elements of an input tensor in global memory as floats
// (one 8-byte load in bf16, one 16-byte load in fp32; index a multiple of 4).
template <typename IO>
__device__ inline void gload4(const void* base, int64_t idx, float* out) {
  if constexpr (io<IO>::bytes == 2) {
    const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const char*>(base) + idx * 2);
    out[0] = __uint_as_float(raw.x << 16);
    out[1] = __uint_as_float(raw.x & 0xffff0000u);
    out[2] = __uint_as_float(raw.y << 16);
    out[3] = __uint_as_float(raw.y & 0xffff0000u);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const char*>(base) + idx * 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  }
}

// Decode 16 bytes of the input dtype into floats (8 bf16 or 4 fp32).
template <typename IO>
__device__ inline void unpack16(const uint4& raw, float* x) {
  if constexpr (io<IO>::bytes == 2) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      x[2 * s] = __uint_as_float(w[s] << 16);
      x[2 * s + 1] = __uint_as_float(w[s] & 0xffff0000u);
    }
  } else {
    x[0] = __uint_as_float(raw.x);
    x[1] = __uint_as_float(raw.y);
    x[2] = __uint_as_float(raw.z);
    x[3] = __uint_as_float(raw.w);
  }
}

// Encode floats as 16 bytes of the input dtype (8 bf16, rounded to nearest
// even, or 4 fp32); the inverse of unpack16.
template <typename IO>
__device__ inline uint4 pack16(const float* x) {
  if constexpr (io<IO>::bytes == 2) {
    uint32_t w[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x[2 * s]));
      const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x[2 * s + 1]));
      w[s] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                      __float_as_uint(x[3]));
  }
}

template <typename IO>
__device__ inline void lds_st(char* base, size_t idx, float x) {
  if constexpr (io<IO>::bytes == 2)
    reinterpret_cast<__bf16*>(base)[idx] = (__bf16)x;
  else
    reinterpret_cast<float*>(base)[idx] = x;
}

// --------------------------------------------------------- prep kernel ---

// Number of P^T fragments (it, jb) with some r >= i: 32 jb + 31 >= 16 it.
__host__ __device__ constexpr int num_pt_frags(int NB, int NKC) {
  int n = 0;
  for (int it = 0; it < NB; ++it)
    for (int jb = 0; jb < NKC; ++jb)
      if (32 * jb + 31 >= 16 * it) ++n;
  return n;
}

// e^x as one hardware base-2 exponential of x log2(e): relative error about
// 1e-7 for |x| <= 88, zero far below (the decays here are bounded so).
__device__ inline float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Waves of the per-channel prep: its LDS plan allows one workgroup per CU,
// so eight waves give every SIMD two to interleave.
constexpr int kPrepChWaves = 8;

template <int C, int DK, typename IO, int GATE, bool BWD = false, int NW = 4>
__global__ __launch_bounds__(64 * NW) void fwd_prep_kernel(
    ChunkMap map, int H, int dv, int64_t nchunks, const void* __restrict__ q,
    const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ beta, const void* __restrict__ la, bool gbf,
    FwdBuffers buf, const void* __restrict__ beta_w = nullptr) {
  using OP = IO;  // bf16 inputs multiply on bf16 MFMA, fp32 on fp32 MFMA
  using S = PrepSmem<C, DK, IO, GATE, BWD>;
  constexpr bool CH = GATE == GDN_GATE_CHANNEL;
  constexpr int ib = S::ib;
  constexpr int ob = opstore<OP>::bytes;
  constexpr int NB = C / 16;
  constexpr int NKD = (DK + 31) / 32;
  constexpr int NKC = (C + 31) / 32;
  constexpr int NDT = DK / 16;
  constexpr int LDT = S::LDT, LDK = S::LDK, LDC = S::LDC, LDV = S::LDV;
  constexpr int VW = 16 / ib;       // elements per 16-byte vector
  constexpr int VPR = DK / VW;      // vectors per K row
  constexpr int NT = 64 * NW;       // threads

  __shared__ __attribute__((aligned(16))) char smem[S::total];
  __shared__ int s_span_bits;
  char* sKt = smem + S::kt_off;
  char* sK = smem + S::k_off;
  float* sg = reinterpret_cast<float*>(smem + S::g_off);
  float* smid = reinterpret_cast<float*>(smem + S::mid_off);
  float* sbeta = reinterpret_cast<float*>(smem + S::beta_off);
  float* sxs = reinterpret_cast<float*>(smem + S::xs_off);
  float* sks = reinterpret_cast<float*>(smem + S::ks_off);
  float* sT = reinterpret_cast<float*>(smem + S::t_off);
  float* sZ = reinterpret_cast<float*>(smem + S::z_off);
  float* sA = reinterpret_cast<float*>(smem + S::a_off);
  char* sVt = smem + S::a_off;
  float* sP = reinterpret_cast<float*>(smem + S::p_off);
  __bf16* sEu = reinterpret_cast<__bf16*>(smem + S::eu_off);
  __bf16* sEd = sEu + C * S::LDE;
  // x[0..7] (channels k0 .. k0 + 7 of row r) times e^{g - mid} (up) or
  // e^{mid - g}: from the factor rows when they exist, else evaluated here
  auto chan = [&](float* x, bool up, int r, int k0) {
    if (k0 >= DK) return;  // DK is a multiple of 16: all 8 or none
    if constexpr (S::EF) {
      float e[8];
      to_floats<bf16_t>(*reinterpret_cast<const opvec<bf16_t>*>(
                            (up ? sEu : sEd) + r * S::LDE + k0), e);
#pragma unroll
      for (int s = 0; s < 8; ++s) x[s] *= e[s];
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float gm = sg[r * DK + k0 + s] - smid[k0 + s];
        x[s] *= fast_exp(up ? gm : -gm);
      }
    }
  };

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
  const int64_t ch = static_cast<int64_t>(h) * nchunks + c;

  // P jobs: fragment (rt, jb) of P for 32 jb <= 16 rt + 15, computed as P^T
  // tiles so the accumulators are already the permuted fragments the state
  // pass uses.  Their q rows are requested first so the loads overlap the
  // gate and key staging below.
  constexpr int NT2 = NB * (NB + 1) / 2;
  constexpr int NPF = NB == 1 ? 1 : (NB == 2 ? 2 : 6);
  constexpr int NPT = BWD ? num_pt_frags(NB, NKC) : 0;  // P^T fragments
  constexpr int JOBS = NT2 + NPF + NPT;
  constexpr int MAXJ = (JOBS + NW - 1) / NW;
  opvec<OP> qpre[MAXJ][NKD];
#pragma unroll
  for (int u = 0; u < MAXJ; ++u) {
    const int job = wave + NW * u;
    if (job >= NT2 && job < NT2 + NPF) {
      int f = job - NT2, rt = 0;
      for (rt = 0; rt < NB; ++rt) {
        const int nj = (16 * rt + 15) / 32 + 1;
        if (f < nj) break;
        f -= nj;
      }
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb)
        qpre[u][kb] = row_frag<IO, DK>(q, tok0, H, h, 16 * rt + l16, len, kb * 32 + lg * 8);
    }
  }

  // ---- 1. beta, cumulative log-gate, K and K^T ----------------------------
  if (tid == 0) s_span_bits = 0;
  if (tid < C) sbeta[tid] = tid < len ? load_gate(beta, (tok0 + tid) * H + h, gbf) : 0.f;
  // decoupled erase / write: beta (erase) scales A and W, the write strength
  // U; it replaces beta in LDS once A and W's scales are formed (step 3)
  float bw = 0.f;
  if (beta_w != nullptr && tid < len) bw = load_gate(beta_w, (tok0 + tid) * H + h, gbf);
  if constexpr (!CH) {
    if (wave == 0) {
      float x = 0.f;
      if constexpr (GATE == GDN_GATE_SCALAR)
        if (lane < len) x = load_gate(la, (tok0 + lane) * H + h, gbf);
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
      }
      if (lane < C) sg[lane] = x;
    }
  }
  // K rows, and the per-channel log gates, as 16-byte pieces: every load is
  // issued before the first LDS store, so the loads travel together
  constexpr int NKP = (C * VPR + NT - 1) / NT;
  uint4 kraw[NKP];
#pragma unroll
  for (int u = 0; u < NKP; ++u) {
    const int e = tid + NT * u;
    const int r = e / VPR, cv = (e % VPR) * VW;
    kraw[u] = make_uint4(0, 0, 0, 0);
    if (e < C * VPR && r < len)
      kraw[u] = *reinterpret_cast<const uint4*>(
          static_cast<const char*>(k) + (((tok0 + r) * H + h) * DK + cv) * ib);
  }
  if constexpr (CH) {
    constexpr int NGP = (C * DK / 4 + NT - 1) / NT;  // pieces per thread (fp32 gates)
    const int per = gbf ? 8 : 4;                    // gate elements per piece
    const int np = C * DK / per;
    uint4 graw[NGP];
#pragma unroll
    for (int u = 0; u < NGP; ++u) {
      const int e = tid + NT * u;
      const int r = (e * per) / DK, col = (e * per) % DK;
      graw[u] = make_uint4(0, 0, 0, 0);
      if (e < np && r < len)
        graw[u] = *reinterpret_cast<const uint4*>(
            static_cast<const char*>(la) + (((tok0 + r) * H + h) * DK + col) * (gbf ? 2 : 4));
    }
#pragma unroll
    for (int u = 0; u < NGP; ++u) {
      const int e = tid + NT * u;
      if (e < np) {
        float x[8];
        if (gbf) unpack16<bf16_t>(graw[u], x);
        else unpack16<f32_t>(graw[u], x);
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
          if (s2 < per) sg[e * per + s2] = x[s2];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NKP; ++u) {
    const int e = tid + NT * u;
    if (e >= C * VPR) continue;
    const int r = e / VPR, cv = (e % VPR) * VW;
    *reinterpret_cast<uint4*>(sK + (size_t(r) * LDK + cv) * ib) = kraw[u];
    float x[8];
    unpack16<IO>(kraw[u], x);
#pragma unroll
    for (int s = 0; s < VW; ++s) lds_st<IO>(sKt, size_t(cv + s) * LDT + r, x[s]);
  }
  __syncthreads();
  if constexpr (CH) {
    for (int col = tid; col < DK; col += NT) {
      float x = 0.f, mx = -3.0e38f, mn = 3.0e38f;
      for (int r = 0; r < C; ++r) {
        x += sg[r * DK + col];
        sg[r * DK + col] = x;
        mx = fmaxf(mx, x);
        mn = fminf(mn, x);
      }
      smid[col] = 0.5f * (mx + mn);
      atomicMax(&s_span_bits, __float_as_int(0.5f * (mx - mn)));
    }
  }
  if (tid < C) {
    if constexpr (GATE == GDN_GATE_SCALAR) {
      sxs[tid] = sbeta[tid] * fast_exp(sg[tid]);
      sks[tid] = fast_exp(sg[C - 1] - sg[tid]);
    } else {
      sxs[tid] = sbeta[tid];
      sks[tid] = 1.f;
    }
  }
  __syncthreads();

  // ---- 2. A = decayed beta K K^T (LDS) and P fragments (workspace) --------
  bool exact = false;
  if constexpr (CH) exact = __int_as_float(s_span_bits) > kChannelHalfSpan;
  if constexpr (S::EF) {
    if (!exact) {  // the same for the whole workgroup
      for (int e = tid; e < C * DK; e += NT) {
        const int r = e / DK, d = e % DK;
        const float gm = sg[e] - smid[d];
        sEu[r * S::LDE + d] = static_cast<__bf16>(fast_exp(gm));
        sEd[r * S::LDE + d] = static_cast<__bf16>(fast_exp(-gm));
      }
      __syncthreads();
    }
  }
  char* dP = buf.at(ch, buf.off_p);
  if (!exact) {
#pragma unroll
    for (int u = 0; u < MAXJ; ++u) {
      const int job = wave + NW * u;
      if (job >= JOBS) continue;
      if (job < NT2) {
        int t = job, rt = 0;
        while (t > rt) { t -= rt + 1; ++rt; }
        const int it = t;
        const int ra = 16 * rt + l16, rb = 16 * it + l16;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) {
          const int k0 = kb * 32 + lg * 8;
          opvec<OP> af = zero_vec<OP>(), bf = zero_vec<OP>();
          if (k0 < DK) {
            af = lds_vec8<IO>(sK, size_t(ra) * LDK + k0);
            bf = lds_vec8<IO>(sK, size_t(rb) * LDK + k0);
          }
          if constexpr (CH) {
            float x[8], y[8];
            to_floats<OP>(af, x);
            to_floats<OP>(bf, y);
            chan(x, true, ra, k0);
            chan(y, false, rb, k0);
            af = frag<OP>::from_floats(x);
            bf = frag<OP>::from_floats(y);
          }
          acc = mma32(af, bf, acc);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int r = 16 * rt + 4 * lg + s;
          const int i = 16 * it + l16;
          float val = 0.f;
          if (i < r) {
            val = acc[s] * sbeta[r];
            if constexpr (GATE == GDN_GATE_SCALAR) val *= fast_exp(sg[r] - sg[i]);
          }
          sA[r * LDC + i] = val;
        }
      } else if (BWD && job >= NT2 + NPF) {
        // fragment (it, jb) of P^T: rows i of tile it, k = r in the
        // permuted order; the accumulators of P tiles (2jb, it), (2jb+1, it)
        int f = job - NT2 - NPF, it = 0, jb = 0;
        for (it = 0; it < NB; ++it) {
          int nj = 0;
          for (int b2 = 0; b2 < NKC; ++b2) nj += (32 * b2 + 31 >= 16 * it) ? 1 : 0;
          if (f < nj) { jb = NKC - nj + f; break; }
          f -= nj;
        }
        const int ri = 16 * it + l16;
        float out[8];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int rt = 2 * jb + half;
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          if (rt >= it && rt < NB) {
            const int rr = 16 * rt + l16;
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb) {
              const int k0 = kb * 32 + lg * 8;
              opvec<OP> af = zero_vec<OP>(), bf = zero_vec<OP>();
              af = row_frag<IO, DK>(q, tok0, H, h, rr, len, k0);
              if (k0 < DK) bf = lds_vec8<IO>(sK, size_t(ri) * LDK + k0);
              if constexpr (CH) {
                float x[8], y[8];
                to_floats<OP>(af, x);
                to_floats<OP>(bf, y);
                chan(x, true, rr, k0);
                chan(y, false, ri, k0);
                af = frag<OP>::from_floats(x);
                bf = frag<OP>::from_floats(y);
              }
              acc = mma32(af, bf, acc);
            }
          }
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int r = 16 * rt + 4 * lg + s;
            const int i = 16 * it + l16;
            float val = 0.f;
            if (rt >= it && rt < NB && i <= r) {
              val = acc[s];
              if constexpr (GATE == GDN_GATE_SCALAR) val *= fast_exp(sg[r] - sg[i]);
            }
            out[4 * half + s] = val;
          }
        }
        *reinterpret_cast<opvec<OP>*>(
            buf.at(ch, buf.off_pt) + ((size_t(it) * NKC + jb) * 64 + lane) * 8 * ob) =
            frag<OP>::from_floats(out);
      } else {
        int f = job - NT2, rt = 0, jb = 0;
        for (rt = 0; rt < NB; ++rt) {
          const int nj = (16 * rt + 15) / 32 + 1;
          if (f < nj) { jb = f; break; }
          f -= nj;
        }
        const int r = 16 * rt + l16;
        opvec<OP> qf[NKD];
#pragma unroll
        for (int kb = 0; kb < NKD; ++kb) {
          qf[kb] = qpre[u][kb];
          if constexpr (CH) {
            float x[8];
            to_floats<OP>(qf[kb], x);
            chan(x, true, r, kb * 32 + lg * 8);
            qf[kb] = frag<OP>::from_floats(x);
          }
        }
        float out[8];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int it = 2 * jb + half;
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          if (it <= rt && it < NB) {
            const int ri = 16 * it + l16;
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb) {
              const int k0 = kb * 32 + lg * 8;
              opvec<OP> kf = zero_vec<OP>();
              if (k0 < DK) kf = lds_vec8<IO>(sK, size_t(ri) * LDK + k0);
              if constexpr (CH) {
                float x[8];
                to_floats<OP>(kf, x);
                chan(x, false, ri, k0);
                kf = frag<OP>::from_floats(x);
              }
              acc = mma32(kf, qf[kb], acc);
            }
          }
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int i = 16 * it + 4 * lg + s;
            float val = 0.f;
            if (it <= rt && i <= r) {
              val = acc[s];
              if constexpr (GATE == GDN_GATE_SCALAR) val *= fast_exp(sg[r] - sg[i]);
            }
            out[4 * half + s] = val;
          }
        }
        *reinterpret_cast<opvec<OP>*>(
            dP + ((size_t(rt) * NKC + jb) * 64 + lane) * 8 * ob) =
            frag<OP>::from_floats(out);
      }
    }
  } else if constexpr (CH) {
    // exact per-element path for extreme per-channel decay spans
    for (int e = tid; e < C * C; e += NT) {
      const int r = e / C, i = e % C;
      float pv = 0.f, av = 0.f;
      if (i <= r && r < len) {
        for (int kk = 0; kk < DK; ++kk) {
          const float d = fast_exp(sg[r * DK + kk] - sg[i * DK + kk]);
          const float ki = lds_ld<IO>(sKt, size_t(kk) * LDT + i) * d;
          pv += io<IO>::load(q, ((tok0 + r) * H + h) * DK + kk) * ki;
          av += lds_ld<IO>(sKt, size_t(kk) * LDT + r) * ki;
        }
      }
      sP[r * LDC + i] = pv;
      sA[r * LDC + i] = (i < r) ? av * sbeta[r] : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < NB * NKC * 64; e += NT) {
      const int ln = e & 63, fr = e >> 6;
      const int rt = fr / NKC, jb = fr % NKC;
      if (32 * jb > 16 * rt + 15) continue;
      const int r = 16 * rt + (ln & 15), g = ln >> 4;
      float vals[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int i = 32 * jb + perm_k(g, s);
        vals[s] = (i < C && i <= r) ? sP[r * LDC + i] : 0.f;
      }
      *reinterpret_cast<opvec<OP>*>(dP + (size_t(fr) * 64 + ln) * 8 * ob) =
          frag<OP>::from_floats(vals);
    }
    if constexpr (BWD) {
      for (int e = tid; e < NB * NKC * 64; e += NT) {
        const int ln = e & 63, fr = e >> 6;
        const int it = fr / NKC, jb = fr % NKC;
        if (32 * jb + 31 < 16 * it) continue;
        const int i = 16 * it + (ln & 15), g = ln >> 4;
        float vals[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int r = 32 * jb + perm_k(g, s);
          vals[s] = (r < C && i <= r) ? sP[r * LDC + i] : 0.f;
        }
        *reinterpret_cast<opvec<OP>*>(buf.at(ch, buf.off_pt) + (size_t(fr) * 64 + ln) * 8 * ob) =
            frag<OP>::from_floats(vals);
      }
    }
  }
  __syncthreads();
  if (beta_w != nullptr && tid < C) sbeta[tid] = bw;  // last read of beta was A's

  // ---- 3. diagonal blocks of T (wave 0) beside the T-free outputs ---------
  if (wave == 0) {
    const int b = lane >> 4, j = lane & 15;
    if (b < NB) {
      float x[16];
      const float* Ab = sA + (16 * b) * LDC + 16 * b;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) s += Ab[r * LDC + i] * x[i];
        x[r] = (r == j) ? 1.f : (r < j ? 0.f : -s);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[(16 * b + r) * LDC + 16 * b + j] = x[r];
    }
  } else {
    const int t3 = tid - 64;
    for (int e = t3; e < C * C; e += NT - 64) {
      const int r = e / C, i = e % C;
      if ((i >> 4) > (r >> 4)) sT[r * LDC + i] = 0.f;
    }
    // K~^T fragments: rows dk, tokens in the permuted order
    char* dk_ = buf.at(ch, buf.off_k);
    for (int e = t3; e < NDT * NKC * 64; e += NT - 64) {
      const int ln = e & 63, fr = e >> 6;
      const int a = fr / NKC, jb = fr % NKC;
      const int m = ln & 15, g = ln >> 4;
      const int dk = 16 * a + m;
      float vals[8];
      const int i0 = 32 * jb + 4 * g, i1 = 32 * jb + 16 + 4 * g;
      if (i0 < C) lds_ld4<IO>(sKt, size_t(dk) * LDT + i0, vals);
      else vals[0] = vals[1] = vals[2] = vals[3] = 0.f;
      if (i1 < C) lds_ld4<IO>(sKt, size_t(dk) * LDT + i1, vals + 4);
      else vals[4] = vals[5] = vals[6] = vals[7] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int i = 32 * jb + perm_k(g, s);
        if (i < C) {
          if constexpr (CH) vals[s] *= fast_exp(sg[(C - 1) * DK + dk] - sg[i * DK + dk]);
          else vals[s] *= sks[i];
        }
      }
      *reinterpret_cast<opvec<OP>*>(dk_ + (size_t(fr) * 64 + ln) * 8 * ob) =
          frag<OP>::from_floats(vals);
    }
    if constexpr (CH) {
      char* dq = buf.at(ch, buf.off_q);
      // slots 0..3 and 4..7 of a lane are channels 32 jb + 4 g .. + 3 and
      // 16 further on: two 4-element loads, all issued before any use
      constexpr int NQF = NB * NKD * 64, NQI = (NQF + NT - 65) / (NT - 64);
      float qv[NQI][8];
#pragma unroll
      for (int u = 0; u < NQI; ++u) {
        const int e = t3 + (NT - 64) * u;
        const int ln = e & 63, fr = e >> 6;
        const int rt = fr / NKD, jb = fr % NKD;
        const int r = 16 * rt + (ln & 15), dk0 = 32 * jb + 4 * (ln >> 4);
#pragma unroll
        for (int s = 0; s < 8; ++s) qv[u][s] = 0.f;
        if (e < NQF && r < len && dk0 < DK) {
          const int64_t base = ((tok0 + r) * H + h) * DK;
          gload4<IO>(q, base + dk0, qv[u]);
          if (dk0 + 16 < DK) gload4<IO>(q, base + dk0 + 16, qv[u] + 4);
        }
      }
#pragma unroll
      for (int u = 0; u < NQI; ++u) {
        const int e = t3 + (NT - 64) * u;
        if (e >= NQF) continue;
        const int ln = e & 63, fr = e >> 6;
        const int rt = fr / NKD, jb = fr % NKD;
        const int g = ln >> 4;
        const int r = 16 * rt + (ln & 15);
        float vals[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int dk = 32 * jb + perm_k(g, s);
          vals[s] = dk < DK ? qv[u][s] * fast_exp(sg[r * DK + dk]) : 0.f;
        }
        *reinterpret_cast<opvec<OP>*>(dq + (size_t(fr) * 64 + ln) * 8 * ob) =
            frag<OP>::from_floats(vals);
      }
    }
    if constexpr (BWD) {
      // K~ fragments (rows i, k = dk permuted) and Q~^T fragments (rows dk,
      // k = r permuted) for the reverse recurrence
      char* dkf = buf.at(ch, buf.off_kf);
      for (int e = t3; e < NB * NKD * 64; e += NT - 64) {
        const int ln = e & 63, fr = e >> 6;
        const int rt = fr / NKD, jb = fr % NKD;
        const int m = ln & 15, g = ln >> 4;
        const int i = 16 * rt + m;
        float vals[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int dk = 32 * jb + perm_k(g, s);
          float x = 0.f;
          if (dk < DK) {
            x = lds_ld<IO>(sK, size_t(i) * LDK + dk);
            if constexpr (CH) x *= fast_exp(sg[(C - 1) * DK + dk] - sg[i * DK + dk]);
            else x *= sks[i];
          }
          vals[s] = x;
        }
        *reinterpret_cast<opvec<OP>*>(dkf + (size_t(fr) * 64 + ln) * 8 * ob) =
            frag<OP>::from_floats(vals);
      }
      char* dqt = buf.at(ch, buf.off_qt);
      for (int e = t3; e < NDT * NKC * 64; e += NT - 64) {
        const int ln = e & 63, fr = e >> 6;
        const int a = fr / NKC, jb = fr % NKC;
        const int m = ln & 15, g = ln >> 4;
        const int dk = 16 * a + m;
        float vals[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int r = 32 * jb + perm_k(g, s);
          float x = 0.f;
          if (r < len) {
            x = io<IO>::load(q, ((tok0 + r) * H + h) * DK + dk);
            if constexpr (CH) x *= fast_exp(sg[r * DK + dk]);
            else if constexpr (GATE == GDN_GATE_SCALAR) x *= fast_exp(sg[r]);
          }
          vals[s] = x;
        }
        *reinterpret_cast<opvec<OP>*>(dqt + (size_t(fr) * 64 + ln) * 8 * ob) =
            frag<OP>::from_floats(vals);
      }
    }
    float* gam = reinterpret_cast<float*>(buf.at(ch, buf.off_g));
    if (t3 < C) {
      float x = 1.f;
      if constexpr (GATE == GDN_GATE_SCALAR) x = fast_exp(sg[t3]);
      gam[t3] = x;
    }
    for (int d = t3; d < DK; d += NT - 64) {
      float x = 1.f;
      if constexpr (GATE == GDN_GATE_SCALAR) x = fast_exp(sg[C - 1]);
      if constexpr (CH) x = fast_exp(sg[(C - 1) * DK + d]);
      gam[C + d] = x;
    }
  }
  __syncthreads();

  // ---- 4. blocks below the diagonal, one diagonal d = b - a at a time, on
  //      fp32 MFMA:  T_ba = -T_bb sum_{a <= j < b} A_bj T_ja
  for (int d = 1; d < NB; ++d) {
    const int a = wave, b = wave + d;  // wave-uniform: never under an EXEC mask
    if (b < NB) {
      floatx4 z = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 16 * a; k0 < 16 * b; k0 += 4)
        z = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * b + l16) * LDC + k0 + lg],
                                                 sT[(k0 + lg) * LDC + 16 * a + l16], z, 0, 0, 0);
      float* zw = sZ + wave * 256;
#pragma unroll
      for (int e = 0; e < 4; ++e) zw[(4 * lg + e) * 16 + l16] = z[e];
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes
      __builtin_amdgcn_wave_barrier();
      floatx4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4)
        t = __builtin_amdgcn_mfma_f32_16x16x4f32(sT[(16 * b + l16) * LDC + 16 * b + k0 + lg],
                                                 zw[(k0 + lg) * 16 + l16], t, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[(16 * b + 4 * lg + e) * LDC + 16 * a + l16] = -t[e];
    }
    __syncthreads();
  }

  // ---- 5. -W fragments: W^T = X^T T^T with X = diag(b gamma) K ------------
  {
    char* dst = buf.at(ch, buf.off_w);
    for (int job = wave; job < NKD * NB; job += NW) {
      const int jb = job / NB, rt = job % NB;
      floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      const int r = 16 * rt + l16;
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) {
        if (32 * kb > 16 * rt + 15) continue;  // T is lower triangular
        const int i0 = 32 * kb + 8 * lg;
        float tv[8], xs[8];
        if (i0 < C) {
          lds_f8(sT + r * LDC + i0, tv);
          lds_f8(sxs + i0, xs);
        } else {
#pragma unroll
          for (int s = 0; s < 8; ++s) tv[s] = xs[s] = 0.f;
        }
        const auto bf = frag<OP>::from_floats(tv);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int a = 2 * jb + half;
          if (16 * a >= DK) continue;
          const int dk = 16 * a + l16;
          float av[8];
          if (i0 < C) {
            lds_ld8<IO>(sKt, size_t(dk) * LDT + i0, av);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              av[s] *= xs[s];
              if constexpr (CH) av[s] *= fast_exp(sg[(i0 + s) * DK + dk]);
            }
          } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) av[s] = 0.f;
          }
          if (half == 0) acc0 = mma32(frag<OP>::from_floats(av), bf, acc0);
          else acc1 = mma32(frag<OP>::from_floats(av), bf, acc1);
        }
      }
      float out[8];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        out[s] = -acc0[s];
        out[4 + s] = -acc1[s];
      }
      *reinterpret_cast<opvec<OP>*>(dst + ((size_t(rt) * NKD + jb) * 64 + lane) * 8 * ob) =
          frag<OP>::from_floats(out);
    }
  }

  if constexpr (BWD) {
    // -W^T fragments (rows dk, k = tokens permuted) from W = T X tiles
    char* dst = buf.at(ch, buf.off_wt);
    for (int job = wave; job < NDT * NKC; job += NW) {
      const int a = job / NKC, jb = job % NKC;
      const int dk = 16 * a + l16;
      float out[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int rt = 2 * jb + half;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        if (rt < NB) {
          const int r = 16 * rt + l16;
#pragma unroll
          for (int kb = 0; kb < NKC; ++kb) {
            if (32 * kb > 16 * rt + 15) continue;
            const int i0 = 32 * kb + 8 * lg;
            float tv[8], xv[8], xs[8];
            if (i0 < C) {
              lds_f8(sT + r * LDC + i0, tv);
              lds_f8(sxs + i0, xs);
              lds_ld8<IO>(sKt, size_t(dk) * LDT + i0, xv);
#pragma unroll
              for (int s = 0; s < 8; ++s) {
                xv[s] *= xs[s];
                if constexpr (CH) xv[s] *= fast_exp(sg[(i0 + s) * DK + dk]);
              }
            } else {
#pragma unroll
              for (int s = 0; s < 8; ++s) tv[s] = xv[s] = 0.f;
            }
            acc = mma32(frag<OP>::from_floats(tv), frag<OP>::from_floats(xv), acc);
          }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) out[4 * half + s] = -acc[s];
      }
      *reinterpret_cast<opvec<OP>*>(dst + ((size_t(a) * NKC + jb) * 64 + lane) * 8 * ob) =
          frag<OP>::from_floats(out);
    }
  }

  // ---- 6. U = T diag(b) V, 64 value columns at a time (V^T over A) --------
  {
    char* U = buf.at(ch, buf.off_u);
    const int ndt = dv / 16;
    constexpr int SV = 64 / VW;  // 16-byte vectors per slab row
    // the next slab's V pieces are loaded while the current one is used
    constexpr int NVS = (C * SV + NT - 1) / NT;
    uint4 vraw[NVS];
    auto load_v = [&](int slab) {
      const int ncol = min(64, dv - slab);
#pragma unroll
      for (int u = 0; u < NVS; ++u) {
        const int e = tid + NT * u;
        const int i = e / SV, cv = (e % SV) * VW;
        vraw[u] = make_uint4(0, 0, 0, 0);
        if (e < C * SV && i < len && cv < ncol)
          vraw[u] = *reinterpret_cast<const uint4*>(
              static_cast<const char*>(v) + (((tok0 + i) * H + h) * dv + slab + cv) * ib);
      }
    };
    load_v(0);
    for (int slab = 0; slab < dv; slab += 64) {
      const int ncol = min(64, dv - slab);
#pragma unroll
      for (int u = 0; u < NVS; ++u) {
        const int e = tid + NT * u;
        if (e >= C * SV) continue;
        const int i = e / SV, cv = (e % SV) * VW;
        float x[8];
        unpack16<IO>(vraw[u], x);
#pragma unroll
        for (int s = 0; s < VW; ++s) lds_st<IO>(sVt, size_t(cv + s) * LDV + i, x[s]);
      }
      if (slab + 64 < dv) load_v(slab + 64);
      __syncthreads();
      const int nvt = ncol / 16;
      for (int job = wave; job < NB * nvt; job += NW) {
        const int rt = job / nvt, vt = job % nvt;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        const int r = 16 * rt + l16;
        const int col = 16 * vt + l16;
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) {
          if (32 * kb > 16 * rt + 15) continue;
          const int i0 = 32 * kb + 8 * lg;
          float av[8], bv[8], bt[8];
          if (i0 < C) {
            lds_f8(sT + r * LDC + i0, av);
            lds_ld8<IO>(sVt, size_t(col) * LDV + i0, bv);
            lds_f8(sbeta + i0, bt);
#pragma unroll
            for (int s = 0; s < 8; ++s) bv[s] *= bt[s];
          } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) av[s] = bv[s] = 0.f;
          }
          acc = mma32(frag<OP>::from_floats(av), frag<OP>::from_floats(bv), acc);
        }
        const int vtg = slab / 16 + vt;
        *reinterpret_cast<typename acc4<OP>::type*>(
            U + ((size_t(rt) * ndt + vtg) * 64 + lane) * 4 * ob) = from_f4<OP>(acc);
      }
      __syncthreads();  // the slab buffer is rewritten next
    }
  }
}

// ---------------------------------------- prep for per-token gates ---
// Prep of one (chunk, head) for the scalar gate or no gate, with the same
// outputs as fwd_prep_kernel, organised around the matrix cores:
//   - K and V rows are staged in LDS once as 16-byte pieces; the operands
//     that contract over tokens (X^T = (diag(b gamma) K)^T, K~^T and
//     Y = diag(b) V) are gathered from their columns, the A and P tiles use
//     row fragments;
//   - T = (I + A)^-1 has its 16 x 16 diagonal blocks solved by substitution
//     (one wave, all blocks at once) and the blocks below filled diagonal by
//     diagonal on fp32 MFMA:  T_ba = -T_bb sum_{a <= j < b} A_bj T_ja;
//   - W^T = X^T T^T and U = T Y on the matrix cores in the operand type;
//   - decays as exp2 of base-2 cumulative log gates.
// waves of the per-token-gate prep: a 16- or 32-token chunk has too few
// tiles for eight waves, and smaller workgroups keep more chunks in flight
constexpr int prep_waves(int C) { return C == 16 ? 2 : (C == 32 ? 4 : 8); }

template <int C, int DK, typename IO, bool CONV = false>
struct PrepSgSmem {
  static constexpr int ib = io<IO>::bytes;
  static constexpr int LDKB = DK * ib + 16;        // K row pitch (bytes)
  static constexpr int VCOLS = 128;                // V columns staged at a time
  static constexpr int LDVB = VCOLS * ib + 16;     // V row pitch
  static constexpr int LDC = C + 4;                // fp32 C x C matrices
  static constexpr int LDZ = 17;                   // 16 x 16 scratch tiles
  static constexpr size_t k_off = 0;
  static constexpr size_t v_off = k_off + size_t(C) * LDKB;
  static constexpr size_t a_off = v_off + size_t(C) * LDVB;
  static constexpr size_t t_off = a_off + size_t(C) * LDC * 4;
  static constexpr size_t z_off = t_off + size_t(C) * LDC * 4;
  static constexpr size_t beta_off = z_off + size_t(4) * 16 * LDZ * 4;
  static constexpr size_t g_off = beta_off + size_t(C) * 4;
  static constexpr size_t xs_off = g_off + size_t(C) * 4;
  static constexpr size_t ks_off = xs_off + size_t(C) * 4;
  static constexpr size_t qn_off = ks_off + size_t(C) * 4;   // 1 / |q_r|
  static constexpr size_t anc_off = qn_off + size_t(C) * 4;  // tree ancestor sets
  // fused convolution taps (widths up to 8): over the A and T matrices'
  // bytes (free while K and V are staged) when they fit, else their own
  static constexpr size_t tap_bytes = CONV ? size_t(DK + VCOLS) * 8 * 4 : 0;
  static constexpr bool tap_in_at = 2 * size_t(C) * LDC * 4 >= tap_bytes;
  static constexpr size_t tap_off = tap_in_at ? a_off : anc_off + size_t(C) * 8;
  static constexpr size_t total = tap_in_at ? anc_off + size_t(C) * 8 : tap_off + tap_bytes;
  static_assert(total <= 160 * 1024, "prep LDS budget");
};

// lnh > 0 (Householder products, 2^lnh delta steps per token): rows are
// steps; q and log alpha are per token, the gate acts on a token's first
// step and q on its last (the other steps' outputs are never stored).
// qkn: q and k rows are used divided by their L2 norms (an all-zero row stays
// zero).  K rows are normalised as they enter LDS (then rounded to the input
// dtype); q rows keep their values and the factor 1 / |q_r| goes to the P
// rows (in fp32, after the product) and into gamma_r for the scan, whose
// state term multiplies the raw q product by gamma_r.
// parent != nullptr (draft trees, one tree per chunk): row r continues the
// state of row parent[tok0 + r] (-1: the chunk's entering state) instead of
// row r - 1.  The cumulative log gate is summed along root paths and the A
// and P entries are kept only where i is an ancestor of r (P: or r itself);
// everything else is the chunk form unchanged, since an entry of
// T = (I + A)^-1 only ever chains ancestors.  The state carried past the
// chunk is not meaningful for a tree: its decays are set to zero.  Parent
// entries outside [-1, r) are read as -1.
// CONV (fused short convolution, width cw): K and V rows are staged as the causal
// depthwise convolution of k and v over the cw tokens ending at the row (taps
// ctk, ctv [H, d, cw]; no tokens before the sequence start) through SiLU, and
// K rows are then L2-normalised; q arrives already processed.
//
// BWD (backward recomputation): also the reverse recurrence's operands, the
// K~ rows, -W^T, P^T and Q~^T fragments (the layouts of the general prep).
template <int C, int DK, typename IO, int GATE, bool BWD = false, bool CONV = false>
__global__ __launch_bounds__(64 * prep_waves(C)) void fwd_prep_sg_kernel(
    ChunkMap map, int H, int dv, int64_t nchunks, const void* __restrict__ q,
    const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ beta, const void* __restrict__ la, bool gbf,
    FwdBuffers buf, int lnh, bool qkn, const int32_t* __restrict__ parent,
    const void* __restrict__ beta_w, int cw = 0, const float* __restrict__ ctk = nullptr,
    const float* __restrict__ ctv = nullptr) {
  static_assert(GATE != GDN_GATE_CHANNEL, "per-token gates only");
  using OP = IO;
  using S = PrepSgSmem<C, DK, IO, CONV>;
  constexpr int ib = S::ib;
  constexpr int ob = opstore<OP>::bytes;
  constexpr int NB = C / 16, NKD = (DK + 31) / 32, NKC = (C + 31) / 32, NDT = DK / 16;
  constexpr int LDC = S::LDC, LDZ = S::LDZ, LDKB = S::LDKB, LDVB = S::LDVB;
  constexpr float kLog2e = 1.4426950408889634f;
  (void)NDT;

  __shared__ __attribute__((aligned(16))) char smem[S::total];
  char* sK = smem + S::k_off;
  char* sV = smem + S::v_off;
  float* sA = reinterpret_cast<float*>(smem + S::a_off);
  float* sT = reinterpret_cast<float*>(smem + S::t_off);
  float* sZ = reinterpret_cast<float*>(smem + S::z_off);
  float* sbeta = reinterpret_cast<float*>(smem + S::beta_off);
  float* sg2 = reinterpret_cast<float*>(smem + S::g_off);
  float* sxs = reinterpret_cast<float*>(smem + S::xs_off);
  float* sks = reinterpret_cast<float*>(smem + S::ks_off);
  float* sqn = reinterpret_cast<float*>(smem + S::qn_off);
  uint64_t* sanc = reinterpret_cast<uint64_t*>(smem + S::anc_off);
  const bool tree = parent != nullptr;

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
  const int64_t ch = static_cast<int64_t>(h) * nchunks + c;

  // jobs: the NT2 lower tiles of A (diagonal included), then the P
  // fragments (rt, jb) with 32 jb <= 16 rt + 15
  constexpr int NT2 = NB * (NB + 1) / 2;
  constexpr int NPF = NB == 1 ? 1 : (NB == 2 ? 2 : 6);
  constexpr int JOBS = NT2 + NPF;
  constexpr int PW = prep_waves(C), NT = 64 * PW;
  static_assert(PW >= C / 16 - 1 && NT >= C, "prep waves per chunk size");
  constexpr int MAXJ = (JOBS + PW - 1) / PW;
  auto p_job = [&](int job, int* rt, int* jb) {
    int f = job - NT2;
    for (*rt = 0; *rt < NB; ++*rt) {
      const int nj = (16 * *rt + 15) / 32 + 1;
      if (f < nj) { *jb = f; return; }
      f -= nj;
    }
  };
  const int nhm = (1 << lnh) - 1;
  // The staging loads are raw buffer loads over this chunk and head (rows
  // past the chunk, or given the out-of-range offset, read as zero): with no
  // branch around them, each wait for data sits at its first use.
  // q row of step r: the token's q on its last step, zero elsewhere
  const int64_t qt0 = tok0 >> lnh;
  const uint32_t krow = static_cast<uint32_t>(H) * DK * ib;  // bytes between tokens
  const auto rq = make_rsrc(static_cast<const char*>(q) + (qt0 * H + h) * DK * ib,
                            static_cast<uint32_t>(((tok0 + len - 1) >> lnh) - qt0) * krow +
                                DK * ib);
  auto q_row_frag = [&](int r, int k0, bool want) -> opvec<OP> {
    const int64_t t = tok0 + r;
    const bool on = want && r < len && k0 < DK && (t & nhm) == nhm;
    return bload8<OP>(rq, on ? static_cast<uint32_t>((t >> lnh) - qt0) * krow + k0 * ib : kOob);
  };
  opvec<OP> qpre[MAXJ][NKD];

  // ---- 0. K rows into LDS; beta and base-2 cumulative log gate.  The
  //      loads go out in the order their data is needed: the gate values,
  //      K (LDS, before step 1), the P jobs' q rows (step 1, after the A
  //      tiles), then the first V columns, which are only written to LDS
  //      after step 2, so that neither q nor V holds up the K stores.
  constexpr int KP = DK * ib / 16;             // 16-byte pieces per K row
  constexpr int VPM = S::VCOLS * ib / 16;      // pieces per staged V row
  constexpr int NKL = (C * KP + NT - 1) / NT;   // K pieces per thread
  constexpr int NVL = (C * VPM + NT - 1) / NT;  // V pieces per thread (max)
  // fused convolution: the 16-byte piece of row r at element column col0 of
  // x ([tokens, H, D]) convolved with its taps over the rows r, r - 1, ..
  // back to the sequence start, through SiLU
  int64_t sstart = 0;
  if constexpr (CONV)
    sstart = map.varlen ? chunk_info(map, ld_table(map.first, ci.seq)).tok0
                        : static_cast<int64_t>(ci.seq) * map.T;
  // taps of this head in LDS, tap-major ([cw][columns]: a piece's channels
  // are adjacent); over the A and T bytes they are written before step 1 and
  // again in step 6, where both are dead: K's columns, then V's staged ones
  float* stk = reinterpret_cast<float*>(smem + S::tap_off);
  float* stv = stk + (CONV ? DK * cw : 0);
  auto stage_taps = [&](float* dst, const float* taps, int D, int c0,
                        int nc) __attribute__((always_inline)) {
    for (int e = tid; e < nc * cw; e += NT) {
      const int c = e / cw, j = e - (e / cw) * cw;
      dst[j * nc + c] = taps[(static_cast<int64_t>(h) * D + c0 + c) * cw + j];
    }
  };
  // the piece of row r at columns col .. col + 16 / ib of x ([tokens, H, D])
  // convolved over rows r, r - 1, .. (not before the sequence start) with
  // the LDS taps st ([cw][nc], column col - c0), through SiLU
  auto conv_piece = [&](const void* x, const float* st, int nc, int D, int col, int c0, int r,
                        float* acc) __attribute__((always_inline)) {
    constexpr int VE = 16 / ib;
#pragma unroll
    for (int s2 = 0; s2 < VE; ++s2) acc[s2] = 0.f;
    const int64_t t = tok0 + r;
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // widths up to 8; all loads issued together
      if (j < cw && t - j >= sstart) {
        float xv[VE];
        unpack16<IO>(*reinterpret_cast<const uint4*>(
                         static_cast<const char*>(x) + (((t - j) * H + h) * D + col) * ib),
                     xv);
        const float* tj = st + j * nc + (col - c0);
#pragma unroll
        for (int s2 = 0; s2 < VE; ++s2) acc[s2] += tj[s2] * xv[s2];
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < VE; ++s2) acc[s2] = acc[s2] / (1.f + expf(-acc[s2]));
  };
  // columns [c0, c0 + VCOLS) of V into registers; pieces past dv or the
  // chunk are zero.  The staging lambdas are always inlined: stage_v, with
  // the convolution and two call sites, was compiled as a call, which put
  // every array it reaches (the K, V and q pieces) in scratch memory and
  // doubled the convolution prep's time (headline shape: 113 -> 56 us)
  auto load_v = [&](int c0, uint4* raw) __attribute__((always_inline)) {
    const int VP = min(S::VCOLS, dv - c0) * ib / 16;
    const int nvc = min(S::VCOLS, dv - c0);
    if constexpr (CONV) {
      if (c0 > 0) {  // the taps of these columns (A and T are dead by now)
        stage_taps(stv, ctv, dv, c0, nvc);
        __syncthreads();
      }
    }
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
      const int e = tid + NT * u;
      const int r = e / VPM, pc = e % VPM;
      if constexpr (CONV) {
        raw[u] = make_uint4(0, 0, 0, 0);
        if (e < C * VPM && r < len && pc < VP) {
          float x[16 / ib];
          conv_piece(v, stv, nvc, dv, c0 + pc * (16 / ib), c0, r, x);
          raw[u] = pack16<IO>(x);
        }
      } else {
        const uint32_t vrow = static_cast<uint32_t>(H) * dv * ib;
        const auto rv = make_rsrc(
            static_cast<const char*>(v) + ((tok0 * H + h) * static_cast<int64_t>(dv) + c0) * ib,
            (len - 1) * vrow + (dv - c0) * ib);
        raw[u] = bload16(rv, e < C * VPM && pc < VP ? r * vrow + pc * 16 : kOob);
      }
    }
  };
  auto store_v = [&](const uint4* raw) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
      const int e = tid + NT * u;
      if (e < C * VPM) *reinterpret_cast<uint4*>(sV + (e / VPM) * LDVB + (e % VPM) * 16) = raw[u];
    }
  };
  auto stage_v = [&](int c0) __attribute__((always_inline)) {
    uint4 raw[NVL];
    load_v(c0, raw);
    store_v(raw);
  };
  if constexpr (CONV) {
    stage_taps(stk, ctk, DK, 0, DK);
    stage_taps(stv, ctv, dv, 0, min(S::VCOLS, dv));
    __syncthreads();
  }
  // wave 0, lane = row: beta, the write strength (decoupled erase / write;
  // U only) and the base-2 log gate
  // (every wave requests them, so that no branch separates the requests
  // from wave 0's use)
  RawGate rgb{}, rgw{}, rgx{};
  {
    const int gsz = gbf ? 2 : 4;
    const uint32_t n = static_cast<uint32_t>(len - 1) * H + 1;
    const int64_t at = (tok0 * H + h) * gsz;
    rgb = gate_issue(static_cast<const char*>(beta) + at, n, lane * H, gbf);
    rgw = gate_issue(static_cast<const char*>(beta_w != nullptr ? beta_w : beta) + at,
                     beta_w != nullptr ? n : 0, lane * H, gbf);
    if constexpr (GATE == GDN_GATE_SCALAR) {
      // the decay acts on a token's first step
      const int64_t t = tok0 + lane;
      const uint32_t nx = static_cast<uint32_t>(((tok0 + len - 1) >> lnh) - qt0) * H + 1;
      rgx = gate_issue(static_cast<const char*>(la) + (qt0 * H + h) * gsz, nx,
                       lane < len && (t & nhm) == 0 ? static_cast<uint32_t>((t >> lnh) - qt0) * H
                                                    : nx,
                       gbf);
    }
  }
  uint4 vraw[NVL];  // the first V columns (not with the fused convolution)
  {
    uint4 raw[NKL];
    float kc[CONV ? NKL : 1][16 / ib];  // convolved K pieces, unrounded until normalised
#pragma unroll
    for (int u = 0; u < NKL; ++u) {
      const int e = tid + NT * u;
      const int r = e / KP, pc = e % KP;
      raw[u] = make_uint4(0, 0, 0, 0);
      if constexpr (CONV) {
#pragma unroll
        for (int s2 = 0; s2 < 16 / ib; ++s2) kc[u][s2] = 0.f;
        if (e < C * KP && r < len) conv_piece(k, stk, DK, DK, pc * (16 / ib), 0, r, kc[u]);
      } else {
        const auto rk = make_rsrc(static_cast<const char*>(k) + (tok0 * H + h) * DK * ib,
                                  (len - 1) * krow + DK * ib);
        raw[u] = bload16(rk, e < C * KP ? r * krow + pc * 16 : kOob);
      }
    }
    // every slot is requested (slots of A jobs out of range), so that the
    // K stores wait for K alone on every wave
#pragma unroll
    for (int u = 0; u < MAXJ; ++u) {
      const int job = wave + PW * u;
      const bool pj = job >= NT2 && job < JOBS;
      int rt = 0, jb = 0;
      p_job(pj ? job : NT2, &rt, &jb);
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb)
        qpre[u][kb] = q_row_frag(16 * rt + l16, kb * 32 + lg * 8, pj);
    }
    if constexpr (CONV)
      stage_v(0);
    else
      load_v(0, vraw);
    if (qkn || CONV) {
      // the KP pieces of a row sit in KP aligned consecutive lanes
      static_assert(KP <= 64 && (KP & (KP - 1)) == 0, "K row pieces per wave");
#pragma unroll
      for (int u = 0; u < NKL; ++u) {
        float x[16 / ib];
        if constexpr (CONV) {
#pragma unroll
          for (int s2 = 0; s2 < 16 / ib; ++s2) x[s2] = kc[u][s2];
        } else {
          unpack16<IO>(raw[u], x);
        }
        float ss = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 16 / ib; ++s2) ss += x[s2] * x[s2];
#pragma unroll
        for (int m = 1; m < KP; m <<= 1) ss += __shfl_xor(ss, m, 64);
        const float sc = ss > 0.f ? rsqrtf(ss) : 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 16 / ib; ++s2) x[s2] *= sc;
        raw[u] = pack16<IO>(x);
      }
    }
#pragma unroll
    for (int u = 0; u < NKL; ++u) {
      const int e = tid + NT * u;
      if (e < C * KP) *reinterpret_cast<uint4*>(sK + (e / KP) * LDKB + (e % KP) * 16) = raw[u];
    }
  }
  if (qkn) {
    // 1 / |q_r| of every row from the P jobs' q rows (row tile rt has the
    // job jb = 0); a row's lanes l16, l16 + 16, .. hold its 32-slot pieces
#pragma unroll
    for (int u = 0; u < MAXJ; ++u) {
      const int job = wave + PW * u;
      if (job < NT2 || job >= JOBS) continue;
      int rt = 0, jb = 0;
      p_job(job, &rt, &jb);
      if (jb != 0) continue;
      float ss = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) {
        float x[8];
        to_floats<OP>(qpre[u][kb], x);
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) ss += x[s2] * x[s2];
      }
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      if (lg == 0) sqn[16 * rt + l16] = ss > 0.f ? rsqrtf(ss) : 0.f;
    }
  }
  float bw = 0.f;  // decoupled erase / write: the write strength (U only)
  if (wave == 0) {
    float x = 0.f;
    const float b = gate_value(rgb, gbf);
    bw = gate_value(rgw, gbf);  // zero without a write strength
    if constexpr (GATE == GDN_GATE_SCALAR) x = gate_value(rgx, gbf) * kLog2e;
    if (!tree) {
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
      }
    } else {
      // pointer jumping over parents: after round j, x sums the log gates of
      // the 2^j nearest nodes of the root path (the row itself included),
      // anc holds the 2^j nearest strict ancestors and nx the next node up
      int nx = -1;
      if (lane < len) {
        nx = parent[tok0 + lane];
        if (nx < -1 || nx >= lane) nx = -1;
      }
      uint64_t anc = nx >= 0 ? (uint64_t(1) << nx) : 0;
#pragma unroll
      for (int j = 0; j < 6; ++j) {  // 2^6 = 64 >= any path in a chunk
        const int src = nx >= 0 ? nx : lane;
        const float xs = __shfl(x, src, 64);
        const uint32_t alo = __shfl(static_cast<uint32_t>(anc), src, 64);
        const uint32_t ahi = __shfl(static_cast<uint32_t>(anc >> 32), src, 64);
        const int ns = __shfl(nx, src, 64);
        if (nx >= 0) {
          x += xs;
          anc |= (static_cast<uint64_t>(ahi) << 32) | alo;
          nx = ns;
        }
      }
      if (lane < C) sanc[lane] = anc;
    }
    const float gend = __shfl(x, C - 1, 64);
    if (lane < C) {
      sbeta[lane] = b;
      sg2[lane] = x;
      if constexpr (GATE == GDN_GATE_SCALAR) {
        sxs[lane] = b * __builtin_amdgcn_exp2f(x);
        sks[lane] = tree ? 0.f : __builtin_amdgcn_exp2f(gend - x);
      } else {
        sxs[lane] = b;
        sks[lane] = tree ? 0.f : 1.f;
      }
    }
  }
  __syncthreads();

  // ---- 1. A tiles (LDS, fp32) and P fragments (workspace) ---------------
  char* dP = buf.at(ch, buf.off_p);
#pragma unroll
  for (int u = 0; u < MAXJ; ++u) {
    const int job = wave + PW * u;
    if (job >= JOBS) continue;
    if (job < NT2) {
      int t = job, rt = 0;
      while (t > rt) { t -= rt + 1; ++rt; }
      const int it = t;
      const int ra = 16 * rt + l16, rb = 16 * it + l16;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) {
        // K slots past DK (DK = 16) hold zero; the product itself is never
        // behind a per-lane condition
        const int k0 = kb * 32 + lg * 8;
        opvec<OP> af = zero_vec<OP>(), bf = zero_vec<OP>();
        if (k0 < DK) {
          af = *reinterpret_cast<const opvec<OP>*>(sK + ra * LDKB + k0 * ib);
          bf = *reinterpret_cast<const opvec<OP>*>(sK + rb * LDKB + k0 * ib);
        }
        acc = mma32(af, bf, acc);
      }
      const int i = 16 * it + l16;
      const float gi = sg2[i];
      const floatx4 br = *reinterpret_cast<const floatx4*>(sbeta + 16 * rt + 4 * lg);
      const floatx4 gr = *reinterpret_cast<const floatx4*>(sg2 + 16 * rt + 4 * lg);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * lg + e;
        float val = acc[e] * br[e];
        if constexpr (GATE == GDN_GATE_SCALAR) val *= __builtin_amdgcn_exp2f(gr[e] - gi);
        const bool keep = i < r && (!tree || ((sanc[r] >> i) & 1));
        sA[r * LDC + i] = keep ? val : 0.f;
      }
    } else {
      int rt = 0, jb = 0;
      p_job(job, &rt, &jb);
      const int r = 16 * rt + l16;
      const float grr = sg2[r];
      const float qs = qkn ? sqn[r] : 1.f;
      // columns kept in row r: all i <= r, or the ancestors of r and r itself
      const uint64_t keep = tree ? (sanc[r] | (uint64_t(1) << r)) : ~uint64_t(0);
      float out[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int it = 2 * jb + half;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f}, acct = acc;
        const floatx4 gi4 = it < NB ? *reinterpret_cast<const floatx4*>(sg2 + 16 * it + 4 * lg)
                                    : floatx4{0.f, 0.f, 0.f, 0.f};
        if (it <= rt && it < NB) {
          const int ri = 16 * it + l16;
#pragma unroll
          for (int kb = 0; kb < NKD; ++kb) {
            const int k0 = kb * 32 + lg * 8;
            opvec<OP> kf = zero_vec<OP>();
            if (k0 < DK) kf = *reinterpret_cast<const opvec<OP>*>(sK + ri * LDKB + k0 * ib);
            acc = mma32(kf, qpre[u][kb], acc);
            if constexpr (BWD) acct = mma32(qpre[u][kb], kf, acct);
          }
        }
        if constexpr (BWD) {
          // P^T fragment (it, rt / 2): row i = 16 it + l16, slots 4 (rt & 1)
          // .. + 3 are the rows r = 16 rt + 4 lg + e (zero above the
          // diagonal); with an odd tile count the missing half is zero
          if (it < NB) {
            const int i = 16 * it + l16;
            const float gi = sg2[i];
            const floatx4 gr4 = *reinterpret_cast<const floatx4*>(sg2 + 16 * rt + 4 * lg);
            floatx4 pt;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int rr = 16 * rt + 4 * lg + e;
              float val = acct[e];
              if constexpr (GATE == GDN_GATE_SCALAR) val *= __builtin_amdgcn_exp2f(gr4[e] - gi);
              pt[e] = (it <= rt && i <= rr) ? val : 0.f;
            }
            char* dst = buf.at(ch, buf.off_pt) + ((size_t(it) * NKC + (rt >> 1)) * 64 + lane) * 8 * ob;
            *reinterpret_cast<typename acc4<OP>::type*>(dst + (rt & 1) * 4 * ob) = from_f4<OP>(pt);
            if ((NB & 1) && rt == NB - 1)
              *reinterpret_cast<typename acc4<OP>::type*>(dst + 4 * ob) =
                  from_f4<OP>(floatx4{0.f, 0.f, 0.f, 0.f});
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * it + 4 * lg + e;
          float val = acc[e] * qs;
          if constexpr (GATE == GDN_GATE_SCALAR) val *= __builtin_amdgcn_exp2f(grr - gi4[e]);
          out[4 * half + e] =
              (it <= rt && it < NB && i <= r && ((keep >> i) & 1)) ? val : 0.f;
        }
      }
      *reinterpret_cast<opvec<OP>*>(dP + ((size_t(rt) * NKC + jb) * 64 + lane) * 8 * ob) =
          frag<OP>::from_floats(out);
    }
  }
  // strictly upper blocks of T are zero; decays for the state pass
  for (int e = tid; e < C * C; e += NT) {
    const int r = e / C, i = e % C;
    if ((i >> 4) > (r >> 4)) sT[r * LDC + i] = 0.f;
  }
  {
    float* gam = reinterpret_cast<float*>(buf.at(ch, buf.off_g));
    if (tid < C)
      gam[tid] = (GATE == GDN_GATE_SCALAR ? __builtin_amdgcn_exp2f(sg2[tid]) : 1.f) *
                 (qkn ? sqn[tid] : 1.f);
    for (int d = tid; d < DK; d += NT)
      gam[C + d] = tree ? 0.f : (GATE == GDN_GATE_SCALAR ? __builtin_amdgcn_exp2f(sg2[C - 1]) : 1.f);
  }
  __syncthreads();

  // ---- 2. diagonal blocks of T: lane 16 b + j solves column j of block b
  // (beta's last reader was A in step 1: U takes the write strength)
  if (wave == 0 && beta_w != nullptr && lane < C) sbeta[lane] = bw;
  if (wave == 0) {
    const int b = lane >> 4, j = lane & 15;
    if (b < NB) {
      float x[16];
      const float* Ab = sA + (16 * b) * LDC + 16 * b;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) s += Ab[r * LDC + i] * x[i];
        x[r] = (r == j) ? 1.f : (r < j ? 0.f : -s);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[(16 * b + r) * LDC + 16 * b + j] = x[r];
    }
  }
  __syncthreads();

  if constexpr (!CONV) {
    // the first V columns; step 6 reads them behind step 3's barriers
    store_v(vraw);
    if constexpr (NB < 2) __syncthreads();
  }

  // ---- 3. blocks below the diagonal, one diagonal d = b - a at a time ---
  for (int d = 1; d < NB; ++d) {
    const int a = wave, b = wave + d;
    if (b < NB) {
      floatx4 z = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 16 * a; k0 < 16 * b; k0 += 4)
        z = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * b + l16) * LDC + k0 + lg],
                                                 sT[(k0 + lg) * LDC + 16 * a + l16], z, 0, 0, 0);
      float* zw = sZ + wave * 16 * LDZ;
#pragma unroll
      for (int e = 0; e < 4; ++e) zw[(4 * lg + e) * LDZ + l16] = z[e];
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes
      __builtin_amdgcn_wave_barrier();
      floatx4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4)
        t = __builtin_amdgcn_mfma_f32_16x16x4f32(sT[(16 * b + l16) * LDC + 16 * b + k0 + lg],
                                                 zw[(k0 + lg) * LDZ + l16], t, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[(16 * b + 4 * lg + e) * LDC + 16 * a + l16] = -t[e];
    }
    __syncthreads();
  }

  // ---- 4. T fragments: row r of tile rt, tokens 32 kb + perm_k ---------
  opvec<OP> tf[NB][NKC];
#pragma unroll
  for (int rt = 0; rt < NB; ++rt)
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) {
      if (32 * kb > 16 * rt + 15) continue;  // T is lower triangular
      const float* row = sT + (16 * rt + l16) * LDC + 32 * kb + 4 * lg;
      float x[8];
      const floatx4 lo = *reinterpret_cast<const floatx4*>(row);
      floatx4 hi = {0.f, 0.f, 0.f, 0.f};
      if (32 * kb + 16 < C) hi = *reinterpret_cast<const floatx4*>(row + 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) { x[e] = lo[e]; x[4 + e] = hi[e]; }
      tf[rt][kb] = frag<OP>::from_floats(x);
    }

  // ---- 5. K~^T fragments and -W fragments: job (jb, half) takes key tile
  //      a = 2 jb + half, the K~^T fragments of that tile and half of the
  //      -W fragments of key block jb (token order perm_k in both, so one
  //      gather of K's columns serves both)
  for (int job = wave; job < 2 * NKD; job += PW) {
    const int jb = job >> 1, half = job & 1, a = 2 * jb + half;
    opvec<OP> xf[NKC];
#pragma unroll
    for (int kb = 0; kb < NKC; ++kb) {
      float kt[8], xt[8];
      const int dk = 16 * a + l16;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int i = 32 * kb + perm_k(lg, s);
        float x = 0.f;
        if (16 * a < DK && i < C) x = lds_ld<IO>(sK + i * LDKB, dk);
        kt[s] = i < C ? x * sks[i] : 0.f;
        xt[s] = i < C ? x * sxs[i] : 0.f;
      }
      xf[kb] = frag<OP>::from_floats(xt);
      if (16 * a < DK)
        *reinterpret_cast<opvec<OP>*>(
            buf.at(ch, buf.off_k) + ((size_t(a) * NKC + kb) * 64 + lane) * 8 * ob) =
            frag<OP>::from_floats(kt);
    }
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f}, acct = acc;
      if (16 * a < DK) {
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) {
          if (32 * kb > 16 * rt + 15) continue;
          acc = mma32(xf[kb], tf[rt][kb], acc);
          if constexpr (BWD) acct = mma32(tf[rt][kb], xf[kb], acct);
        }
      }
      // slots 4 half .. +3 of the lane's fragment (zero past DK)
      *reinterpret_cast<typename acc4<OP>::type*>(
          buf.at(ch, buf.off_w) + ((size_t(rt) * NKD + jb) * 64 + lane) * 8 * ob + half * 4 * ob) =
          from_f4<OP>(-acc);
      if constexpr (BWD) {
        // -W^T fragment (a, rt / 2): row dk = 16 a + l16, slots 4 (rt & 1)
        // .. + 3 are the tokens 16 rt + 4 lg + e
        if (16 * a < DK) {
          char* dst = buf.at(ch, buf.off_wt) + ((size_t(a) * NKC + (rt >> 1)) * 64 + lane) * 8 * ob;
          *reinterpret_cast<typename acc4<OP>::type*>(dst + (rt & 1) * 4 * ob) = from_f4<OP>(-acct);
          if ((NB & 1) && rt == NB - 1)
            *reinterpret_cast<typename acc4<OP>::type*>(dst + 4 * ob) =
                from_f4<OP>(floatx4{0.f, 0.f, 0.f, 0.f});
        }
      }
    }
  }
  if constexpr (BWD) {
    // K~ fragments: rows i, slots dk = 32 jb + perm_k (zero past DK)
    char* dkf = buf.at(ch, buf.off_kf);
    for (int e = tid; e < NB * NKD * 64; e += NT) {
      const int ln = e & 63, fr = e >> 6;
      const int rt = fr / NKD, jb = fr % NKD;
      const int i = 16 * rt + (ln & 15), g = ln >> 4;
      float vals[8];
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        const int d = 32 * jb + perm_k(g, s2);
        vals[s2] = d < DK ? lds_ld<IO>(sK + i * LDKB, d) * sks[i] : 0.f;
      }
      *reinterpret_cast<opvec<OP>*>(dkf + (size_t(fr) * 64 + ln) * 8 * ob) =
          frag<OP>::from_floats(vals);
    }
  }

  // ---- 6. U = T Y, Y = diag(b) V: wave w takes value tiles w, w + PW, ..
  //      of each VCOLS-column pass --------------------------------------
  for (int c0 = 0; c0 < dv; c0 += S::VCOLS) {
    if (c0 > 0) {
      __syncthreads();  // every wave is done with the previous columns
      stage_v(c0);
      __syncthreads();
    }
    char* U = buf.at(ch, buf.off_u);
    const int ndvt = dv / 16;
    // in a scalar register, so the loop below never runs under an EXEC mask
    const int nvt = __builtin_amdgcn_readfirstlane(min(S::VCOLS, dv - c0) / 16);
    for (int vl = wave; vl < nvt; vl += PW) {
      const int vt = c0 / 16 + vl;
      opvec<OP> yf[NKC];
      const int col = 16 * vl + l16;
#pragma unroll
      for (int kb = 0; kb < NKC; ++kb) {
        float y[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int i = 32 * kb + perm_k(lg, s);
          y[s] = i < C ? lds_ld<IO>(sV + i * LDVB, col) * sbeta[i] : 0.f;
        }
        yf[kb] = frag<OP>::from_floats(y);
      }
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb) {
          if (32 * kb > 16 * rt + 15) continue;
          acc = mma32(tf[rt][kb], yf[kb], acc);
        }
        *reinterpret_cast<typename acc4<OP>::type*>(
            U + ((size_t(rt) * ndvt + vt) * 64 + lane) * 4 * ob) = from_f4<OP>(acc);
      }
    }
  }

  if constexpr (BWD) {
    // ---- 7. Q~^T fragments (rows dk, slots tokens 32 jb + perm_k): the q
    //      rows go through the V staging area (zero past the chunk)
    constexpr int LDQB = DK * ib + 16;
    static_assert(LDQB <= LDVB, "q rows fit the V staging rows");
    __syncthreads();  // every wave is done with V
    for (int e = tid; e < C * KP; e += NT) {
      const int r = e / KP, pc = e % KP;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (r < len)
        x = *reinterpret_cast<const uint4*>(
            static_cast<const char*>(q) + ((tok0 + r) * H + h) * DK * ib + pc * 16);
      *reinterpret_cast<uint4*>(sV + r * LDQB + pc * 16) = x;
    }
    __syncthreads();
    char* dqt = buf.at(ch, buf.off_qt);
    for (int e = tid; e < NDT * NKC * 64; e += NT) {
      const int ln = e & 63, fr = e >> 6;
      const int a = fr / NKC, jb = fr % NKC;
      const int d = 16 * a + (ln & 15), g = ln >> 4;
      float vals[8];
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        const int r = 32 * jb + perm_k(g, s2);
        float x = 0.f;
        if (r < C) {
          x = lds_ld<IO>(sV + r * LDQB, d);
          if constexpr (GATE == GDN_GATE_SCALAR) x *= __builtin_amdgcn_exp2f(sg2[r]);
        }
        vals[s2] = x;
      }
      *reinterpret_cast<opvec<OP>*>(dqt + (size_t(fr) * 64 + ln) * 8 * ob) =
          frag<OP>::from_floats(vals);
    }
  }
}

// Segment buffers of the split state pass (per segment slot and head):
//   trm : state the segment produces from zero, fp32 accumulator layout
//         [dv/16][DK/16][64 lanes][4]
//   trp : the segment's transition Phi (DK x DK) as operand fragments
//         [DK/16][NKD][64][8] in the operand type (permuted K)
//   ss  : state entering the segment, same layout as trm (segments j >= 1)
struct SegBuffers {
  float* trm;
  char* trp;
  float* ss;
  size_t trp_bytes;  // per (slot, head)
};

// Host: segment buffers at `base` (p.seg > 0; empty otherwise) and their size.
inline SegBuffers make_seg_buffers(const Problem& p, char* base, int ob) {
  SegBuffers sb{};
  if (p.seg == 0) return sb;
  const int NKD = (p.dk + 31) / 32, NDT = p.dk / 16;
  const size_t n = static_cast<size_t>(p.nsegs) * p.H;
  const size_t st = FwdLayout::al(size_t(p.dk) * p.dv * 4);
  sb.trp_bytes = FwdLayout::al(size_t(NDT) * NKD * 512 * ob);
  sb.trm = reinterpret_cast<float*>(base);
  sb.trp = base + n * st;
  sb.ss = reinterpret_cast<float*>(base + n * (st + sb.trp_bytes));
  return sb;
}

inline size_t seg_buffer_bytes(const Problem& p, int ob) {
  if (p.seg == 0) return 0;
  const int NKD = (p.dk + 31) / 32, NDT = p.dk / 16;
  const size_t st = FwdLayout::al(size_t(p.dk) * p.dv * 4);
  const size_t tp = FwdLayout::al(size_t(NDT) * NKD * 512 * ob);
  return static_cast<size_t>(p.nsegs) * p.H * (2 * st + tp);
}

// ---------------------------------------------------- state pass kernels ---
// The state recurrence runs per (segment, head) and 16-column slab of the
// value dimension.  A workgroup of NW waves owns NW * SPW slabs of one
// (segment, head); all of them read the same per-chunk operands (W, K~ and,
// for the outputs, Q and P), so the workgroup copies each chunk's operands
// once into LDS and every wave reads the fragments it needs from there.  The
// copies go straight from global memory into LDS (global_load_lds, 16 bytes
// per lane) into one buffer while the waves compute from the other (bf16;
// fp32 operands are twice the size and use one buffer).

constexpr int kScanWaves = 8;   // scan: waves per workgroup (two per SIMD)
constexpr int kScanSlabs = 1;   // scan: slabs per wave, 8 slabs per workgroup
constexpr int kTransWaves = 8;  // transitions: waves per workgroup
constexpr int kTransSlabs = 2;  // transitions: slabs per wave, [M0 | Phi] of 128 + 128
constexpr int kScanGroup = kScanWaves * kScanSlabs;
constexpr int kTransGroup = kTransWaves * kTransSlabs;

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Wait until at most N vector memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Copy MAXB bytes (a multiple of 16; only the first `bytes` when given) from
// global `src` to LDS `dst` with all NTH threads: lane l of a wave moves the
// 16 bytes at the wave's base + 16 l, and the LDS address of a wave's piece
// is its base + 16 * lane.  The uniform base stays in scalar registers and
// each lane adds a 32-bit offset.
template <int NTH, int MAXB>
__device__ __forceinline__ void lds_copy(char* dst, const char* src, int wave, int lane,
                                         int bytes = MAXB) {
  constexpr int STEP = NTH * 16;
  // a region that is not whole 1 KiB wave pieces needs the per-lane bound
  constexpr bool WHOLE = MAXB % 1024 == 0;
#pragma unroll
  for (int it = 0; it < (MAXB + STEP - 1) / STEP; ++it) {
    const int b = it * STEP + wave * 1024;  // uniform
    if (MAXB % STEP == 0 || b < MAXB) {
      const uint32_t off = static_cast<uint32_t>(lane * 16);
      if ((WHOLE && bytes == MAXB) || b + static_cast<int>(off) < bytes)
        __builtin_amdgcn_global_load_lds(src + b + off, (lds_void_ptr)(dst + b), 16, 0, 0);
    }
  }
}

// LDS image of one chunk's operands.  Q holds the Q~ fragments (per-channel
// gate) or the raw q rows of the chunk with their 16-byte pieces permuted
// within each row (piece c of row r sits at c ^ swz(r)), so that the 16 rows
// a fragment read touches fall on different banks.
template <int C, int DK, typename OP, bool OUT, bool RAWQ, int GS>
struct LdsChunk {
  static constexpr int ob = opstore<OP>::bytes;
  static constexpr int NB = C / 16, NKD = (DK + 31) / 32, NKC = (C + 31) / 32,
                       NDT = DK / 16;
  static constexpr int W = NB * NKD * 512 * ob;            // -W fragments
  static constexpr int K = NDT * NKC * 512 * ob;           // K~^T fragments
  static constexpr int P = OUT ? NB * NKC * 512 * ob : 0;  // P fragments
  static constexpr int Q = OUT ? (RAWQ ? C * DK * ob : NB * NKD * 512 * ob) : 0;
  static constexpr int G = (C + DK) * 4;                   // gamma_r, chunk decays
  static constexpr int U = NB * GS * 256 * ob;             // U tiles of the group
  static constexpr int oW = 0, oK = W, oP = W + K, oQ = W + K + P, oG = W + K + P + Q,
                       oU = W + K + P + Q + G;
  static constexpr int BYTES = oU + U;
  static constexpr int PR = DK * ob / 16;                  // 16-byte pieces per q row
  __device__ static int swz(int r) { return r & ((PR < 16 ? PR : 16) - 1); }
};

// Per-lane byte offsets, within a chunk's q rows, of the raw-q pieces a lane
// copies (row i / PR, piece (i % PR) ^ swz(row)) for a full chunk.
template <int C, int DK, typename OP, int NTH>
struct QPieces {
  static constexpr int PR = DK * opstore<OP>::bytes / 16;
  static constexpr int NIT = (C * PR + NTH - 1) / NTH;
  uint32_t off[NIT];
  __device__ __forceinline__ int piece(int it, int wave, int lane) const {
    return it * NTH + wave * 64 + lane;
  }
  // LDS row r holds the q row of step r, the row of token r >> lnh of the
  // chunk (chunks start on a token boundary)
  __device__ __forceinline__ static uint32_t offset(int r, int i, int H, int lnh) {
    const int c = (i % PR) ^ (r & ((PR < 16 ? PR : 16) - 1));
    return static_cast<uint32_t>(r >> lnh) * static_cast<uint32_t>(H * DK * opstore<OP>::bytes) +
           static_cast<uint32_t>(c * 16);
  }
  __device__ __forceinline__ void init(int H, int lnh, int wave, int lane) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int i = piece(it, wave, lane);
      off[it] = offset(i / PR, i, H, lnh);
    }
  }
};

// Issue the copies of chunk slot ch (chunk info ci) into LDS buffer `lds`:
// [W | K~ | P] (contiguous in the workspace: every piece is a multiple of 256
// bytes), Q, the decays and the U tiles of the group's slabs [u0, u0 + nu).
template <int C, int DK, typename OP, int GATE, bool OUT, int NTH, int GS>
__device__ __forceinline__ void copy_chunk(char* lds, const FwdBuffers& buf, int64_t ch,
                                           const ChunkInfo& ci, const void* q,
                                           const QPieces<C, DK, OP, NTH>& qp, int H,
                                           int h, int ndvt, int u0, int nu, int wave,
                                           int lane, int lnh = 0) {
  constexpr bool RAWQ = OUT && GATE != GDN_GATE_CHANNEL;
  using L = LdsChunk<C, DK, OP, OUT, RAWQ, GS>;
  using QP = QPieces<C, DK, OP, NTH>;
  constexpr int ob = L::ob;
  lds_copy<NTH, L::W + L::K + L::P>(lds, buf.at(ch, buf.off_w), wave, lane);
  if constexpr (OUT) {
    if constexpr (!RAWQ) {
      lds_copy<NTH, L::Q>(lds + L::oQ, buf.at(ch, buf.off_q), wave, lane);
    } else {
      // rows past the chunk repeat its last row (they only feed outputs that
      // are not stored)
      const char* qb = static_cast<const char*>(q) + ((ci.tok0 >> lnh) * H + h) * DK * ob;
      const bool full = ci.len == C;
#pragma unroll
      for (int it = 0; it < QP::NIT; ++it) {
        const int b = it * NTH + wave * 64;  // uniform
        if (!((C * QP::PR) % NTH == 0 || b < C * QP::PR)) continue;
        const int i = b + lane;
        if ((C * QP::PR) % 64 != 0 && i >= C * QP::PR) continue;  // past the rows
        const uint32_t off =
            full ? qp.off[it] : QP::offset(min(i / QP::PR, ci.len - 1), i, H, lnh);
        __builtin_amdgcn_global_load_lds(qb + off, (lds_void_ptr)(lds + L::oQ + b * 16),
                                         16, 0, 0);
      }
    }
  }
  lds_copy<NTH, L::G>(lds + L::oG, buf.at(ch, buf.off_g), wave, lane);
  if (nu > 0) {
    const char* pu = buf.at(ch, buf.off_u);
#pragma unroll
    for (int rt = 0; rt < L::NB; ++rt)
      lds_copy<NTH, GS * 256 * ob>(lds + L::oU + rt * GS * 256 * ob,
                                           pu + (static_cast<size_t>(rt) * ndvt + u0) * 256 * ob,
                                           wave, lane, nu * 256 * ob);
  }
}

// One chunk of the chain for the wave's slabs, operands in LDS `ops`:
//   E = U - W M  (U only where has_u),  M <- gamma_c M + K~^T E.
// Slab s of the wave is slab us[s] of the LDS U tiles.  Returns the operand
// fragments of M (chunk start) and E in Mb / Eb.  Every slab is computed,
// also one past the problem's columns (its values are never stored), so the
// matrix work carries no branches.
template <int C, int DK, typename OP, int GATE, int SPW, bool OUT, bool RAWQ, int GS>
__device__ __forceinline__ void chain_lds(
    const char* ops, floatx4 (&M)[SPW][DK / 16],
    const bool (&has_u)[SPW], const int (&us)[SPW],
    opvec<OP> (&Mb)[SPW][(DK + 31) / 32], opvec<OP> (&Eb)[SPW][(C + 31) / 32],
    int lane, int lg) {
  using L = LdsChunk<C, DK, OP, OUT, RAWQ, GS>;
  constexpr int NB = L::NB, NKD = L::NKD, NKC = L::NKC, NDT = L::NDT;
  constexpr bool CH = GATE == GDN_GATE_CHANNEL;
  using A4 = typename acc4<OP>::type;
  const opvec<OP>* sW = reinterpret_cast<const opvec<OP>*>(ops + L::oW);
  const opvec<OP>* sK = reinterpret_cast<const opvec<OP>*>(ops + L::oK);
  const A4* sU = reinterpret_cast<const A4*>(ops + L::oU);
  const float* sg = reinterpret_cast<const float*>(ops + L::oG) + C;
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int jb = 0; jb < NKD; ++jb)
      Mb[s][jb] = pack2<OP>(M[s][2 * jb], 2 * jb + 1 < NDT ? M[s][2 * jb + 1] : z);
  floatx4 E[SPW][NB];
#pragma unroll
  for (int rt = 0; rt < NB; ++rt) {
    opvec<OP> wf[NKD];
#pragma unroll
    for (int jb = 0; jb < NKD; ++jb) wf[jb] = sW[(rt * NKD + jb) * 64 + lane];
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const floatx4 u = to_f4(sU[(rt * GS + us[s]) * 64 + lane]);
      E[s][rt] = has_u[s] ? u : z;
#pragma unroll
      for (int jb = 0; jb < NKD; ++jb) E[s][rt] = mma32(wf[jb], Mb[s][jb], E[s][rt]);
    }
  }
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int jb = 0; jb < NKC; ++jb)
      Eb[s][jb] = pack2<OP>(E[s][2 * jb], 2 * jb + 1 < NB ? E[s][2 * jb + 1] : z);
#pragma unroll
  for (int a = 0; a < NDT; ++a) {
    opvec<OP> kf[NKC];
#pragma unroll
    for (int jb = 0; jb < NKC; ++jb) kf[jb] = sK[(a * NKC + jb) * 64 + lane];
    floatx4 gc;
    if constexpr (CH) gc = *reinterpret_cast<const floatx4*>(sg + 16 * a + 4 * lg);
    else if constexpr (GATE == GDN_GATE_SCALAR) gc = floatx4{sg[0], sg[0], sg[0], sg[0]};
    else gc = floatx4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      M[s][a] *= gc;
#pragma unroll
      for (int jb = 0; jb < NKC; ++jb) M[s][a] = mma32(kf[jb], Eb[s][jb], M[s][a]);
    }
  }
}

// Segment transitions.  Slabs run over the [dv | DK] columns of [M0 | Phi]:
// the chain over the segment's chunks from M = 0 with U (columns of M0) or
// from the identity columns without U (columns of Phi; the map from the
// entering to the leaving state is affine, M_end = Phi M_start + M0).  The
// forward's chain never needs the last segment of a sequence; the backward's
// reverse chain needs every segment's Phi but the first's (with_last).
template <int C, int DK, typename IO, int GATE>
__global__ __launch_bounds__(64 * kTransWaves)
void fwd_trans_kernel(
    ChunkMap map, SegMap sm, int H, int dv, int64_t nchunks, FwdBuffers buf,
    SegBuffers sb, bool with_last) {
  using OP = IO;
  constexpr int NW = kTransWaves, SPW = kTransSlabs, NTH = 64 * NW, GS = kTransGroup;
  using L = LdsChunk<C, DK, OP, false, false, GS>;
  constexpr int NKD = L::NKD, NKC = L::NKC, NDT = L::NDT;
  constexpr bool DB = opstore<OP>::bytes == 2;  // double-buffered
  __shared__ __attribute__((aligned(16))) char sA[L::BYTES];
  __shared__ __attribute__((aligned(16))) char sB[DB ? L::BYTES : 16];

  const int ndvt = dv / 16, ncol = ndvt + NDT;
  const int ngrp = (ncol + GS - 1) / GS;
  // head-major: a head's segments (and their maps) stay on one XCD
  const int nslot = static_cast<int>(gridDim.x) / (ngrp * H);
  const int w = xcd_swizzle(blockIdx.x, gridDim.x);
  const int grp = w % ngrp;
  const int slot = (w / ngrp) % nslot;
  const int h = w / ngrp / nslot;
  const SegInfo si = seg_info(sm, map, slot);
  if (si.seq < 0 || (si.last && !with_last)) return;  // whole workgroup, before any barrier
  const int tid = threadIdx.x;
  // wave index in a scalar register: branches on it are scalar branches,
  // never EXEC masks (matrix instructions ignore EXEC)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int g0 = grp * GS;                                // first column slab of the group
  const int u0 = g0, nu = max(0, min(GS, ndvt - g0));      // its M0 slabs
  const int vt0 = g0 + wave * SPW;
  bool own[SPW], phi[SPW], has_u[SPW];
  int us[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    own[s] = vt0 + s < ncol;
    phi[s] = vt0 + s >= ndvt;
    has_u[s] = own[s] && !phi[s];
    us[s] = wave * SPW + s;
  }

  floatx4 M[SPW][NDT];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int pc = 16 * (vt0 + s - ndvt) + l16;  // Phi column of this lane
#pragma unroll
    for (int a = 0; a < NDT; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        M[s][a][e] = (phi[s] && 16 * a + 4 * lg + e == pc) ? 1.f : 0.f;
  }

  const int n = si.c1 - si.c0;
  const int64_t ch0 = static_cast<int64_t>(h) * nchunks + si.c0;
  const ChunkInfo ci{};
  opvec<OP> Mb[SPW][NKD], Eb[SPW][NKC];
  QPieces<C, DK, OP, NTH> qp;  // unused without outputs
  auto copy = [&](char* lds, int j) {
    copy_chunk<C, DK, OP, GATE, false, NTH, GS>(lds, buf, ch0 + j, ci, nullptr, qp, H, h,
                                                ndvt, u0, nu, wave, lane);
  };
  auto step = [&](const char* lds) {
    chain_lds<C, DK, OP, GATE, SPW, false, false, GS>(lds, M, has_u, us, Mb, Eb, lane, lg);
  };
  if constexpr (DB) {
    if (n > 0) copy(sA, 0);
    wait_vmcnt<0>();
    __syncthreads();
    for (int j = 0; j < n; j += 2) {
      if (j + 1 < n) copy(sB, j + 1);
      step(sA);
      wait_vmcnt<0>();
      __syncthreads();
      if (j + 1 < n) {
        if (j + 2 < n) copy(sA, j + 2);
        step(sB);
        wait_vmcnt<0>();
        __syncthreads();
      }
    }
  } else {
    for (int j = 0; j < n; ++j) {
      if (j > 0) __syncthreads();  // every wave is done with chunk j - 1
      copy(sA, j);
      wait_vmcnt<0>();
      __syncthreads();
      step(sA);
    }
  }

  const size_t sh = static_cast<size_t>(slot) * H + h;
  // Phi leaves as operand fragments: lane holds Phi(16a + 4lg + e, pc), and
  // operand fragment (a, jb) lane L' slot t stands for
  // Phi(16a + L'%16, 32jb + perm_k(L'/16, t)), so a slab fills one half
  // (slots 4 half ..) of every lane of the fragments (a, jb).  The wave
  // scatters its values into an LDS image of the fragments and reads back
  // the halves it owns, lane L' its own 8 bytes (bf16), which go out as one
  // store per fragment instead of 32 two-byte stores per lane (the other half
  // may belong to a slab of another wave or workgroup).  A wave's LDS
  // accesses complete in order, so no barrier separates its writes from its
  // reads; the one before keeps the image clear of the chunk buffers still
  // being read.
  using E = typename io<IO>::storage;
  constexpr int FB = 8 * static_cast<int>(sizeof(E));  // bytes per fragment lane
  constexpr bool STAGE = NDT * NKD * 64 * FB <= L::BYTES;
  if constexpr (STAGE) __syncthreads();
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    if (!own[s]) continue;
    if (!phi[s]) {
      floatx4* dst = reinterpret_cast<floatx4*>(sb.trm) + (sh * ndvt + vt0 + s) * NDT * 64;
#pragma unroll
      for (int a = 0; a < NDT; ++a) dst[a * 64 + lane] = M[s][a];
    } else {
      char* dst = sb.trp + sh * sb.trp_bytes;
      E* img = reinterpret_cast<E*>(STAGE ? sA : dst);
      const int cp = vt0 + s - ndvt, jb = cp >> 1, half = cp & 1;
      const int t = (l16 & 3) + 4 * half;
#pragma unroll
      for (int a = 0; a < NDT; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int Lp = 4 * lg + e + 16 * (l16 >> 2);
          const size_t off = ((static_cast<size_t>(a) * NKD + jb) * 64 + Lp) * 8;
          io<IO>::store(img, off + t, M[s][a][e]);
          if (DK == 16) io<IO>::store(img, off + t + 4, 0.f);  // K slots past DK
        }
      if constexpr (STAGE) {
        // the lanes read what other lanes wrote: keep the compiler from
        // moving a lane's reads above its own writes
        __builtin_amdgcn_wave_barrier();
        // lane's own half (both halves when DK = 16: the second is zero)
        constexpr int HB = DK == 16 ? FB : FB / 2;
        const int hoff = DK == 16 ? 0 : half * (FB / 2);
#pragma unroll
        for (int a = 0; a < NDT; ++a) {
          const size_t off = ((static_cast<size_t>(a) * NKD + jb) * 64 + lane) * FB + hoff;
          if constexpr (HB == 8) {
            *reinterpret_cast<uint2*>(dst + off) = *reinterpret_cast<const uint2*>(sA + off);
          } else {
            *reinterpret_cast<uint4*>(dst + off) = *reinterpret_cast<const uint4*>(sA + off);
            if constexpr (HB == 32)
              *reinterpret_cast<uint4*>(dst + off + 16) =
                  *reinterpret_cast<const uint4*>(sA + off + 16);
          }
        }
      }
    }
  }
}

// Q fragment (row tile rt, K block jb) of raw q rows staged in LDS: lane
// holds row 16 rt + l%16, the runs of 4 columns at 32 jb + 4 (l/16) and 16
// further (zero past DK).
template <int C, int DK, typename OP>
__device__ __forceinline__ opvec<OP> q_frag_raw(const char* sq, int rt, int jb, int l16, int lg) {
  using L = LdsChunk<C, DK, OP, true, true, kScanGroup>;
  const int r = 16 * rt + l16;
  const int d0 = 32 * jb + 4 * lg;
  const char* row = sq + r * L::PR * 16;
  if constexpr (opstore<OP>::bytes == 2) {
    const int c0 = d0 >> 3, in = (d0 & 7) * 2;
    const u32x2 x = *reinterpret_cast<const u32x2*>(row + ((c0 ^ L::swz(r)) * 16) + in);
    u32x2 y = {0u, 0u};
    if (d0 + 16 < DK)
      y = *reinterpret_cast<const u32x2*>(row + (((c0 + 2) ^ L::swz(r)) * 16) + in);
    return __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], y[0], y[1]});
  } else {
    const int c0 = d0 >> 2;
    const floatx4 x = *reinterpret_cast<const floatx4*>(row + ((c0 ^ L::swz(r)) * 16));
    floatx4 y = {0.f, 0.f, 0.f, 0.f};
    if (d0 + 16 < DK) y = *reinterpret_cast<const floatx4*>(row + (((c0 + 4) ^ L::swz(r)) * 16));
    return floatx8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  }
}

// State pass over one segment with the outputs.  Each wave carries the fp32
// state of its slabs from the segment's entering state (s0, or the combine
// result) and per chunk forms
//   E = U - W M,   M <- gamma_C M + K~^T E,
//   O^T = M^T Q~^T + E^T P^T   (Q~ = gamma (.) Q for the scalar gate),
// the outputs transposed so that each lane ends up with 4 consecutive
// columns of one token row (one 8-byte store in bf16).  The operands of the
// transposed products are the same register fragments with the roles of A
// and B swapped.  A chunk's stores are issued at the start of the next
// step, so they have the whole step to complete before the wait at its end.
//
// STATES = true (backward recomputation): no outputs; every chunk-start
// state is stored into `states` ([chunk-head][DK][dv]) in the input dtype
// (the chain itself stays fp32; the gradient kernel multiplies the stored
// states on the matrix cores in that dtype).
template <int C, int DK, typename IO, int GATE, bool STATES = false>
__global__ __launch_bounds__(64 * kScanWaves)
void fwd_scan_kernel(
    ChunkMap map, SegMap sm, int H, int dv, int64_t nchunks,
    const void* __restrict__ q, const float* __restrict__ s0,
    void* __restrict__ o, float* __restrict__ s_final, FwdBuffers buf,
    SegBuffers sb, void* __restrict__ states, int lnh) {
  using OP = IO;
  constexpr bool OUT = !STATES;
  constexpr bool RAWQ = OUT && GATE != GDN_GATE_CHANNEL;
  constexpr int NW = kScanWaves, SPW = kScanSlabs, NTH = 64 * NW, GS = kScanGroup;
  using L = LdsChunk<C, DK, OP, OUT, RAWQ, GS>;
  constexpr int NB = L::NB, NKD = L::NKD, NKC = L::NKC, NDT = L::NDT;
  constexpr bool DB = opstore<OP>::bytes == 2;  // double-buffered
  using E = typename io<IO>::storage;
  __shared__ __attribute__((aligned(16))) char sA[L::BYTES];
  __shared__ __attribute__((aligned(16))) char sB[DB ? L::BYTES : 16];
  // bf16 chunk-start states: each wave's [DK][16] slab image, so that the
  // states leave as 16-byte row pieces
  constexpr bool STG = STATES && DB;
  __shared__ __attribute__((aligned(16))) __bf16 sStg[STG ? NW * DK * 16 : 8];

  const int ndvt = dv / 16;
  const int ngrp = (ndvt + GS - 1) / GS;
  const int nslot = static_cast<int>(gridDim.x) / (ngrp * H);
  const int w = xcd_swizzle(blockIdx.x, gridDim.x);
  const int grp = w % ngrp;
  const int slot = (w / ngrp) % nslot;
  const int h = w / ngrp / nslot;
  const SegInfo si = seg_info(sm, map, slot);
  if (si.seq < 0) return;  // whole workgroup, before any barrier
  const int seq = si.seq;
  const int tid = threadIdx.x;
  // wave index in a scalar register: branches on it are scalar branches,
  // never EXEC masks (matrix instructions ignore EXEC)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int g0 = grp * GS;
  const int nu = max(0, min(GS, ndvt - g0));
  const int vt0 = g0 + wave * SPW;
  const int nown = max(0, min(SPW, ndvt - vt0));  // slabs of this wave
  bool own[SPW], has_u[SPW];
  int us[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    own[s] = s < nown;
    has_u[s] = true;
    us[s] = wave * SPW + s;
  }
  const int64_t sbase = (static_cast<int64_t>(seq) * H + h) * DK * dv;

  floatx4 M[SPW][NDT];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int col = 16 * (vt0 + s) + l16;
    if (si.j == 0) {
#pragma unroll
      for (int a = 0; a < NDT; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          M[s][a][e] = (s0 && own[s])
              ? s0[sbase + static_cast<int64_t>(16 * a + 4 * lg + e) * dv + col] : 0.f;
    } else {
      const size_t sh = static_cast<size_t>(slot) * H + h;
      const floatx4* src = reinterpret_cast<const floatx4*>(sb.ss) + (sh * ndvt + vt0 + s) * NDT * 64;
#pragma unroll
      for (int a = 0; a < NDT; ++a) M[s][a] = own[s] ? src[a * 64 + lane] : floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }

  const int n = si.c1 - si.c0;
  const int64_t ch0 = static_cast<int64_t>(h) * nchunks + si.c0;

  // outputs of the previous chunk, held for their stores
  using O4 = typename acc4<OP>::type;
  O4 Ov[SPW][NB];
  int64_t o_tok0 = 0;
  int o_len = 0;
  // lane part of an output address: row l16 of a row tile, columns 4 lg ..;
  // with 2^lnh steps per token only a token's last step is an output row,
  // stored at the token's row
  const int nhm = (1 << lnh) - 1;
  const bool o_row = (l16 & nhm) == nhm;
  const uint32_t o_lane =
      static_cast<uint32_t>(((l16 >> lnh) * H * dv + 16 * vt0 + 4 * lg) * sizeof(E));
  auto store_out = [&]() {
    if constexpr (OUT) {
      char* ob = static_cast<char*>(o) +
                 ((o_tok0 >> lnh) * H + h) * dv * static_cast<int64_t>(sizeof(E));
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const int r = 16 * rt + l16;
        if (r >= o_len || !o_row) continue;
        char* dst = ob + static_cast<int64_t>((16 * rt) >> lnh) * H * dv * sizeof(E) + o_lane;
#pragma unroll
        for (int s = 0; s < SPW; ++s)
          if (own[s]) *reinterpret_cast<O4*>(dst + 16 * s * sizeof(E)) = Ov[s][rt];
      }
    }
  };

  QPieces<C, DK, OP, NTH> qp;
  if constexpr (RAWQ) qp.init(H, lnh, wave, lane);
  auto copy = [&](char* lds, int j) {
    const ChunkInfo ci = OUT ? chunk_info(map, si.c0 + j) : ChunkInfo{};
    copy_chunk<C, DK, OP, GATE, OUT, NTH, GS>(lds, buf, ch0 + j, ci, q, qp, H, h, ndvt, g0,
                                              nu, wave, lane, lnh);
  };
  // The next chunk's copies (into buffer nxt, chunk jn >= 0) are issued
  // between the chain and the output products: issued before the chain,
  // the waves' copy instructions held up its start (the chain is the
  // step's critical part); after it they overlap the output products, which
  // read only this chunk's operands (headline: 27.5 -> 25.2 us).  Without
  // outputs nothing follows the chain, so the copies go first.
  auto step = [&](const char* ops, int j, char* nxt, int jn) {
    if (!OUT && jn >= 0) copy(nxt, jn);
    if constexpr (STATES) {
      const int64_t st0 = (ch0 + j) * static_cast<int64_t>(DK) * dv;
#pragma unroll
      for (int s = 0; s < SPW; ++s) {
        if (!own[s]) continue;
        if constexpr (STG) {
          // the slab through the wave's LDS image: a lane holds 4 rows of
          // one column per row tile, a store wants 8 columns of one row
          // (32 two-byte stores per lane and chunk before: the state pass of
          // the 16k backward batch 271 -> 246 us)
          __bf16* img = sStg + wave * DK * 16;
#pragma unroll
          for (int a = 0; a < NDT; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              img[(16 * a + 4 * lg + e) * 16 + l16] = static_cast<__bf16>(M[s][a][e]);
          // the lanes read what other lanes of the wave wrote (a wave's LDS
          // accesses complete in order; this keeps the compiler's order too)
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int it = 0; it < (2 * DK + 63) / 64; ++it) {
            const int pc = 64 * it + lane, r = pc >> 1, hh = pc & 1;
            if (pc < 2 * DK)
              *reinterpret_cast<uint4*>(static_cast<char*>(states) +
                                        (st0 + static_cast<int64_t>(r) * dv + 16 * (vt0 + s) +
                                         8 * hh) * 2) =
                  *reinterpret_cast<const uint4*>(img + r * 16 + 8 * hh);
          }
          __builtin_amdgcn_wave_barrier();
        } else {
          const int col = 16 * (vt0 + s) + l16;
#pragma unroll
          for (int a = 0; a < NDT; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              io<IO>::store(states, st0 + static_cast<int64_t>(16 * a + 4 * lg + e) * dv + col,
                            M[s][a][e]);
        }
      }
    }
    opvec<OP> Mb[SPW][NKD], Eb[SPW][NKC];
    chain_lds<C, DK, OP, GATE, SPW, OUT, RAWQ, GS>(ops, M, has_u, us, Mb, Eb, lane, lg);
    if (OUT && jn >= 0) copy(nxt, jn);
    if constexpr (OUT) {
      const ChunkInfo ci = chunk_info(map, si.c0 + j);
      const opvec<OP>* sQ = reinterpret_cast<const opvec<OP>*>(ops + L::oQ);
      const opvec<OP>* sP = reinterpret_cast<const opvec<OP>*>(ops + L::oP);
      const float* sg = reinterpret_cast<const float*>(ops + L::oG);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        opvec<OP> qf[NKD], pf[NKC];
#pragma unroll
        for (int jb = 0; jb < NKD; ++jb) {
          if constexpr (RAWQ) qf[jb] = q_frag_raw<C, DK, OP>(ops + L::oQ, rt, jb, l16, lg);
          else qf[jb] = sQ[(rt * NKD + jb) * 64 + lane];
        }
#pragma unroll
        for (int jb = 0; jb < NKC; ++jb)
          if (32 * jb <= 16 * rt + 15) pf[jb] = sP[(rt * NKC + jb) * 64 + lane];
        // gamma_r (the decay, times 1 / |q_r| when q is normalised)
        const float gr = RAWQ ? sg[16 * rt + l16] : 1.f;
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
          floatx4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int jb = 0; jb < NKD; ++jb) O = mma32(Mb[s][jb], qf[jb], O);
          if constexpr (RAWQ) O *= gr;
#pragma unroll
          for (int jb = 0; jb < NKC; ++jb)
            if (32 * jb <= 16 * rt + 15) O = mma32(Eb[s][jb], pf[jb], O);
          Ov[s][rt] = from_f4<OP>(O);
        }
      }
      o_tok0 = ci.tok0;
      o_len = ci.len;
    }
  };

  if constexpr (DB) {
    if (n > 0) copy(sA, 0);
    wait_vmcnt<0>();
    __syncthreads();
    for (int j = 0; j < n; j += 2) {
      store_out();
      step(sA, j, sB, j + 1 < n ? j + 1 : -1);
      wait_vmcnt<0>();
      __syncthreads();
      if (j + 1 < n) {
        store_out();
        step(sB, j + 1, sA, j + 2 < n ? j + 2 : -1);
        wait_vmcnt<0>();
        __syncthreads();
      }
    }
  } else {
    for (int j = 0; j < n; ++j) {
      store_out();
      if (j > 0) __syncthreads();  // every wave is done with chunk j - 1
      copy(sA, j);
      wait_vmcnt<0>();
      __syncthreads();
      step(sA, j, nullptr, -1);
    }
  }
  store_out();
  if (s_final && si.last) {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      if (!own[s]) continue;
      const int col = 16 * (vt0 + s) + l16;
#pragma unroll
      for (int a = 0; a < NDT; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s_final[sbase + static_cast<int64_t>(16 * a + 4 * lg + e) * dv + col] = M[s][a][e];
    }
  }
}

// Sequential combine over the segments of each sequence:
//   M_{j+1} = Phi_j M_j + M0_j,  M_0 = s0.
// One workgroup per (sequence, head, 16-column slab).  Wave w computes the
// row tiles 2w, 2w+1 of the slab, which together are the w-th 32-row K block
// of the next product: after each step every wave publishes that block's
// operand fragment in LDS and reads the others'.  Phi_j's rows and M0_j's
// tiles do not depend on the recurrence and are loaded D steps ahead.
template <int DK, typename IO>
__global__ __launch_bounds__(64 * ((DK + 31) / 32)) void fwd_combine_kernel(
    ChunkMap map, SegMap sm, int H, int dv, const float* __restrict__ s0,
    SegBuffers sb) {
  using OP = IO;
  constexpr int NKD = (DK + 31) / 32, NDT = DK / 16;
  constexpr int NT = NDT >= 2 ? 2 : 1;                 // row tiles per wave
  constexpr int D = opstore<OP>::bytes == 2 ? 4 : 2;   // steps loaded ahead
  __shared__ opvec<OP> sMb[2][NKD][64];
  (void)map;

  const int ndvt = dv / 16;
  const int nseq = static_cast<int>(gridDim.x) / (H * ndvt);
  // head-major and XCD-aware, like the transition kernel that wrote the
  // segment maps, so a head's maps are read from the L2 they were written to
  const int wg = xcd_swizzle(blockIdx.x, gridDim.x);
  const int vt = wg % ndvt;
  const int seq = (wg / ndvt) % nseq;
  const int h = wg / ndvt / nseq;
  int sb0, se0;
  seq_segs(sm, seq, &sb0, &se0);
  const int nsteps = se0 - sb0 - 1;
  if (nsteps <= 0) return;  // whole workgroup, before any barrier
  // wave index in a scalar register: branches on it are scalar branches,
  // never EXEC masks (matrix instructions ignore EXEC)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
  const int t0 = NT * wave;
  const int col = 16 * vt + l16;
  const int64_t sbase = (static_cast<int64_t>(seq) * H + h) * DK * dv;

  // the test on s0 outside the loads, so that they are issued together
  // (a select per element made the compiler wait on each load in turn)
  floatx4 M[NT];
  if (s0 != nullptr) {
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        M[u][e] = s0[sbase + static_cast<int64_t>(16 * (t0 + u) + 4 * lg + e) * dv + col];
  } else {
#pragma unroll
    for (int u = 0; u < NT; ++u) M[u] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  struct Ahead {
    opvec<OP> phi[NT][NKD];
    floatx4 m0[NT];
  };
  Ahead ah[D];
  auto fetch = [&](Ahead& a, int j) {
    const size_t sh = static_cast<size_t>(sb0 + j) * H + h;
    const opvec<OP>* phi = reinterpret_cast<const opvec<OP>*>(sb.trp + sh * sb.trp_bytes);
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int jb = 0; jb < NKD; ++jb) a.phi[u][jb] = phi[((t0 + u) * NKD + jb) * 64 + lane];
    const floatx4* m0 = reinterpret_cast<const floatx4*>(sb.trm) + (sh * ndvt + vt) * NDT * 64;
#pragma unroll
    for (int u = 0; u < NT; ++u) a.m0[u] = m0[(t0 + u) * 64 + lane];
  };
  auto publish = [&](int b) {
    const floatx4 z = {0.f, 0.f, 0.f, 0.f};
    sMb[b][wave][lane] = pack2<OP>(M[0], NT > 1 ? M[NT - 1] : z);
  };

  // The step count is padded to a multiple of D and every step fetches and
  // stores unconditionally, so the body is straight-line code and the
  // compiler's waits let D steps of loads stay in flight.  Padded steps
  // re-read the last segment's map and write to the sequence's first slot,
  // which holds no entering state (the first segment starts from s0).
  const int npad = (nsteps + D - 1) / D * D;
#pragma unroll
  for (int d = 0; d < D; ++d) fetch(ah[d], min(d, nsteps - 1));
  publish(0);
  __syncthreads();
  for (int j = 0; j < npad; j += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int jj = j + d;
      opvec<OP> Mb[NKD];
#pragma unroll
      for (int jb = 0; jb < NKD; ++jb) Mb[jb] = sMb[jj & 1][jb][lane];
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        floatx4 acc = ah[d].m0[u];
#pragma unroll
        for (int jb = 0; jb < NKD; ++jb) acc = mma32(ah[d].phi[u][jb], Mb[jb], acc);
        M[u] = acc;
      }
      fetch(ah[d], min(jj + D, nsteps - 1));
      const int slot = jj < nsteps ? sb0 + jj + 1 : sb0;
      const size_t sh = static_cast<size_t>(slot) * H + h;
      floatx4* dst = reinterpret_cast<floatx4*>(sb.ss) + (sh * ndvt + vt) * NDT * 64;
#pragma unroll
      for (int u = 0; u < NT; ++u) dst[(t0 + u) * 64 + lane] = M[u];
      publish((jj + 1) & 1);
      __syncthreads();
    }
  }
}

}  // namespace

}  // namespace gdn
