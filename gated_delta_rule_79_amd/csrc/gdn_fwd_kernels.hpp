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
  static constexpr size_t total = p_off + (CH ? size_t(C) * LDC * 4 : 0);
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

template <int C, int DK, typename IO, int GATE, bool BWD = false>
__global__ __launch_bounds__(256) void fwd_prep_kernel(
    ChunkMap map, int H, int dv, int64_t nchunks, const void* __restrict__ q,
    const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ beta, const void* __restrict__ la, bool gbf,
    FwdBuffers buf) {
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

  const int L = blockIdx.x;
  const int c = static_cast<int>(L / H);
  const int h = L - c * H;
  const ChunkInfo ci = chunk_info(map, c);
  if (ci.seq < 0) return;
  const int len = ci.len;
  const int64_t tok0 = ci.tok0;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int64_t ch = static_cast<int64_t>(h) * nchunks + c;

  // P jobs: fragment (rt, jb) of P for 32 jb <= 16 rt + 15, computed as P^T
  // tiles so the accumulators are already the permuted fragments the state
  // pass uses.  Their q rows are requested first so the loads overlap the
  // gate and key staging below.
  constexpr int NT2 = NB * (NB + 1) / 2;
  constexpr int NPF = NB == 1 ? 1 : (NB == 2 ? 2 : 6);
  constexpr int NPT = BWD ? num_pt_frags(NB, NKC) : 0;  // P^T fragments
  constexpr int JOBS = NT2 + NPF + NPT;
  constexpr int MAXJ = (JOBS + 3) / 4;
  opvec<OP> qpre[MAXJ][NKD];
#pragma unroll
  for (int u = 0; u < MAXJ; ++u) {
    const int job = wave + 4 * u;
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
  } else {
    for (int e = tid; e < C * DK; e += 256) {
      const int r = e / DK, col = e % DK;
      sg[e] = r < len ? load_gate(la, ((tok0 + r) * H + h) * DK + col, gbf) : 0.f;
    }
  }
  for (int e = tid; e < C * VPR; e += 256) {
    const int r = e / VPR, cv = (e % VPR) * VW;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (r < len)
      raw = *reinterpret_cast<const uint4*>(
          static_cast<const char*>(k) + (((tok0 + r) * H + h) * DK + cv) * ib);
    *reinterpret_cast<uint4*>(sK + (size_t(r) * LDK + cv) * ib) = raw;
    float x[8];
    unpack16<IO>(raw, x);
#pragma unroll
    for (int s = 0; s < VW; ++s) lds_st<IO>(sKt, size_t(cv + s) * LDT + r, x[s]);
  }
  __syncthreads();
  if constexpr (CH) {
    for (int col = tid; col < DK; col += 256) {
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
      sxs[tid] = sbeta[tid] * expf(sg[tid]);
      sks[tid] = expf(sg[C - 1] - sg[tid]);
    } else {
      sxs[tid] = sbeta[tid];
      sks[tid] = 1.f;
    }
  }
  __syncthreads();

  // ---- 2. A = decayed beta K K^T (LDS) and P fragments (workspace) --------
  bool exact = false;
  if constexpr (CH) exact = __int_as_float(s_span_bits) > kChannelHalfSpan;
  char* dP = buf.at(ch, buf.off_p);
  if (!exact) {
#pragma unroll
    for (int u = 0; u < MAXJ; ++u) {
      const int job = wave + 4 * u;
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
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const int kk = k0 + s;
              if (kk < DK) {
                x[s] *= expf(sg[ra * DK + kk] - smid[kk]);
                y[s] *= expf(smid[kk] - sg[rb * DK + kk]);
              }
            }
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
            if constexpr (GATE == GDN_GATE_SCALAR) val *= expf(sg[r] - sg[i]);
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
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                  const int kk = k0 + s;
                  if (kk < DK) {
                    x[s] *= expf(sg[rr * DK + kk] - smid[kk]);
                    y[s] *= expf(smid[kk] - sg[ri * DK + kk]);
                  }
                }
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
              if constexpr (GATE == GDN_GATE_SCALAR) val *= expf(sg[r] - sg[i]);
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
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const int kk = kb * 32 + lg * 8 + s;
              if (kk < DK) x[s] *= expf(sg[r * DK + kk] - smid[kk]);
            }
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
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                  const int kk = k0 + s;
                  if (kk < DK) x[s] *= expf(smid[kk] - sg[ri * DK + kk]);
                }
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
              if constexpr (GATE == GDN_GATE_SCALAR) val *= expf(sg[r] - sg[i]);
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
    for (int e = tid; e < C * C; e += 256) {
      const int r = e / C, i = e % C;
      float pv = 0.f, av = 0.f;
      if (i <= r && r < len) {
        for (int kk = 0; kk < DK; ++kk) {
          const float d = expf(sg[r * DK + kk] - sg[i * DK + kk]);
          const float ki = lds_ld<IO>(sKt, size_t(kk) * LDT + i) * d;
          pv += io<IO>::load(q, ((tok0 + r) * H + h) * DK + kk) * ki;
          av += lds_ld<IO>(sKt, size_t(kk) * LDT + r) * ki;
        }
      }
      sP[r * LDC + i] = pv;
      sA[r * LDC + i] = (i < r) ? av * sbeta[r] : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < NB * NKC * 64; e += 256) {
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
      for (int e = tid; e < NB * NKC * 64; e += 256) {
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
    for (int e = t3; e < C * C; e += 192) {
      const int r = e / C, i = e % C;
      if ((i >> 4) > (r >> 4)) sT[r * LDC + i] = 0.f;
    }
    // K~^T fragments: rows dk, tokens in the permuted order
    char* dk_ = buf.at(ch, buf.off_k);
    for (int e = t3; e < NDT * NKC * 64; e += 192) {
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
          if constexpr (CH) vals[s] *= expf(sg[(C - 1) * DK + dk] - sg[i * DK + dk]);
          else vals[s] *= sks[i];
        }
      }
      *reinterpret_cast<opvec<OP>*>(dk_ + (size_t(fr) * 64 + ln) * 8 * ob) =
          frag<OP>::from_floats(vals);
    }
    if constexpr (CH) {
      char* dq = buf.at(ch, buf.off_q);
      for (int e = t3; e < NB * NKD * 64; e += 192) {
        const int ln = e & 63, fr = e >> 6;
        const int rt = fr / NKD, jb = fr % NKD;
        const int m = ln & 15, g = ln >> 4;
        const int r = 16 * rt + m;
        float vals[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int dk = 32 * jb + perm_k(g, s);
          float x = 0.f;
          if (dk < DK && r < len)
            x = io<IO>::load(q, ((tok0 + r) * H + h) * DK + dk) * expf(sg[r * DK + dk]);
          vals[s] = x;
        }
        *reinterpret_cast<opvec<OP>*>(dq + (size_t(fr) * 64 + ln) * 8 * ob) =
            frag<OP>::from_floats(vals);
      }
    }
    if constexpr (BWD) {
      // K~ fragments (rows i, k = dk permuted) and Q~^T fragments (rows dk,
      // k = r permuted) for the reverse recurrence
      char* dkf = buf.at(ch, buf.off_kf);
      for (int e = t3; e < NB * NKD * 64; e += 192) {
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
            if constexpr (CH) x *= expf(sg[(C - 1) * DK + dk] - sg[i * DK + dk]);
            else x *= sks[i];
          }
          vals[s] = x;
        }
        *reinterpret_cast<opvec<OP>*>(dkf + (size_t(fr) * 64 + ln) * 8 * ob) =
            frag<OP>::from_floats(vals);
      }
      char* dqt = buf.at(ch, buf.off_qt);
      for (int e = t3; e < NDT * NKC * 64; e += 192) {
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
            if constexpr (CH) x *= expf(sg[r * DK + dk]);
            else if constexpr (GATE == GDN_GATE_SCALAR) x *= expf(sg[r]);
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
      if constexpr (GATE == GDN_GATE_SCALAR) x = expf(sg[t3]);
      gam[t3] = x;
    }
    for (int d = t3; d < DK; d += 192) {
      float x = 1.f;
      if constexpr (GATE == GDN_GATE_SCALAR) x = expf(sg[C - 1]);
      if constexpr (CH) x = expf(sg[(C - 1) * DK + d]);
      gam[C + d] = x;
    }
  }
  __syncthreads();

  // ---- 4. off-diagonal blocks of T, block row by block row ----------------
  for (int b = 1; b < NB; ++b) {
    if (wave < b) {
      const int a = wave;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = lane * 4 + u, r = e >> 4, cc = e & 15;
        float z = 0.f;
        for (int jj = a; jj < b; ++jj) {
#pragma unroll
          for (int s = 0; s < 16; ++s)
            z += sA[(16 * b + r) * LDC + 16 * jj + s] *
                 sT[(16 * jj + s) * LDC + 16 * a + cc];
        }
        sZ[(a * 16 + r) * 16 + cc] = z;
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
          t += sT[(16 * b + r) * LDC + 16 * b + s] * sZ[(a * 16 + s) * 16 + cc];
        sT[(16 * b + r) * LDC + 16 * a + cc] = -t;
      }
    }
    __syncthreads();
  }

  // ---- 5. -W fragments: W^T = X^T T^T with X = diag(b gamma) K ------------
  {
    char* dst = buf.at(ch, buf.off_w);
    for (int job = wave; job < NKD * NB; job += 4) {
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
              if constexpr (CH) av[s] *= expf(sg[(i0 + s) * DK + dk]);
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
    for (int job = wave; job < NDT * NKC; job += 4) {
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
                if constexpr (CH) xv[s] *= expf(sg[(i0 + s) * DK + dk]);
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
    for (int slab = 0; slab < dv; slab += 64) {
      const int ncol = min(64, dv - slab);
      for (int e = tid; e < C * SV; e += 256) {
        const int i = e / SV, cv = (e % SV) * VW;
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (i < len && cv < ncol)
          raw = *reinterpret_cast<const uint4*>(
              static_cast<const char*>(v) + (((tok0 + i) * H + h) * dv + slab + cv) * ib);
        float x[8];
        unpack16<IO>(raw, x);
#pragma unroll
        for (int s = 0; s < VW; ++s) lds_st<IO>(sVt, size_t(cv + s) * LDV + i, x[s]);
      }
      __syncthreads();
      const int nvt = ncol / 16;
      for (int job = wave; job < NB * nvt; job += 4) {
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

// --------------------------------------------------------- scan kernel ---

// Per-chunk operands of the state recurrence.
template <int C, int DK, typename OP, int GATE>
struct ChainOps {
  static constexpr int NB = C / 16, NKD = (DK + 31) / 32, NKC = (C + 31) / 32,
                       NDT = DK / 16;
  opvec<OP> W[NB][NKD];
  opvec<OP> K[NDT][NKC];
  typename acc4<OP>::type U[NB];
  floatx4 gc[GATE == GDN_GATE_CHANNEL ? NDT : 1];
};

template <int C, int DK, typename OP, int GATE>
__device__ __forceinline__ void load_chain(ChainOps<C, DK, OP, GATE>& x,
                                           const FwdBuffers& buf, int64_t ch,
                                           int vt, int ndvt, int lane, int lg) {
  using X = ChainOps<C, DK, OP, GATE>;
  constexpr int ob = opstore<OP>::bytes;
  const char* pw = buf.at(ch, buf.off_w);
  const char* pk = buf.at(ch, buf.off_k);
  const char* pu = buf.at(ch, buf.off_u);
  const float* pg = reinterpret_cast<const float*>(buf.at(ch, buf.off_g)) + C;
#pragma unroll
  for (int rt = 0; rt < X::NB; ++rt)
#pragma unroll
    for (int jb = 0; jb < X::NKD; ++jb)
      x.W[rt][jb] = *reinterpret_cast<const opvec<OP>*>(
          pw + ((size_t(rt) * X::NKD + jb) * 64 + lane) * 8 * ob);
#pragma unroll
  for (int rt = 0; rt < X::NB; ++rt)
    x.U[rt] = *reinterpret_cast<const typename acc4<OP>::type*>(
        pu + ((size_t(rt) * ndvt + vt) * 64 + lane) * 4 * ob);
#pragma unroll
  for (int a = 0; a < X::NDT; ++a)
#pragma unroll
    for (int jb = 0; jb < X::NKC; ++jb)
      x.K[a][jb] = *reinterpret_cast<const opvec<OP>*>(
          pk + ((size_t(a) * X::NKC + jb) * 64 + lane) * 8 * ob);
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

// Operands of one chunk's outputs.
template <int C, int DK, typename OP, int GATE>
struct OutOps {
  static constexpr int NB = C / 16, NKD = (DK + 31) / 32, NKC = (C + 31) / 32;
  opvec<OP> Q[NB][NKD];
  opvec<OP> P[NB][NKC];
  floatx4 gr[GATE == GDN_GATE_SCALAR ? NB : 1];
};

template <int C, int DK, typename OP, int GATE>
__device__ __forceinline__ void load_out(OutOps<C, DK, OP, GATE>& x,
                                         const FwdBuffers& buf, int64_t ch,
                                         const ChunkInfo& ci,
                                         const void* __restrict__ q,
                                         __amdgpu_buffer_rsrc_t qr, bool qbuf,
                                         int H, int h, int lane, int l16, int lg) {
  using X = OutOps<C, DK, OP, GATE>;
  constexpr int ob = opstore<OP>::bytes;
  const char* pp = buf.at(ch, buf.off_p);
#pragma unroll
  for (int rt = 0; rt < X::NB; ++rt) {
    const int r = 16 * rt + l16;
    // byte offset of q row r (rows past the chunk only feed output rows
    // that are never stored; past the tensor the buffer returns zero)
    const uint32_t qrow = static_cast<uint32_t>(((ci.tok0 + r) * H + h) * DK * ob);
#pragma unroll
    for (int jb = 0; jb < X::NKD; ++jb) {
      if constexpr (GATE == GDN_GATE_CHANNEL) {
        x.Q[rt][jb] = *reinterpret_cast<const opvec<OP>*>(
            buf.at(ch, buf.off_q) + ((size_t(rt) * X::NKD + jb) * 64 + lane) * 8 * ob);
      } else {
        // raw q rows; the scalar decay is applied to the product's rows
        const int d0 = 32 * jb + 4 * lg;
        if (d0 >= DK) {
          x.Q[rt][jb] = zero_vec<OP>();
        } else if (qbuf) {
          x.Q[rt][jb] = bload4x2<OP>(qr, qrow + d0 * ob, qrow + (d0 + 16) * ob);
        } else if (r < ci.len) {
          const int64_t base = ((ci.tok0 + r) * H + h) * DK;
          x.Q[rt][jb] = gload4x2<OP>(q, base + d0, base + d0 + 16);
        } else {
          x.Q[rt][jb] = zero_vec<OP>();
        }
      }
    }
#pragma unroll
    for (int jb = 0; jb < X::NKC; ++jb)
      if (32 * jb <= 16 * rt + 15)
        x.P[rt][jb] = *reinterpret_cast<const opvec<OP>*>(
            pp + ((size_t(rt) * X::NKC + jb) * 64 + lane) * 8 * ob);
    if constexpr (GATE == GDN_GATE_SCALAR)
      x.gr[rt] = *reinterpret_cast<const floatx4*>(
          reinterpret_cast<const float*>(buf.at(ch, buf.off_g)) + 16 * rt + 4 * lg);
  }
}

// State pass.  A workgroup is two waves working on one (sequence, head,
// 16-column slab of dv):
//   wave 0 carries the chain  E = U - W M,  M <- gamma_C M + K~^T E  and
//          hands the bf16 fragments of M (chunk start) and E to wave 1
//          through a double buffer in LDS;
//   wave 1 forms the outputs  O = gamma (.) (Q M) + P E  one chunk behind.
// One barrier per chunk keeps the two waves a chunk apart.  With bf16
// operands each wave loads the next chunk's operands while it computes the
// current one.
//
// STATES = true (backward recomputation): wave 0 also stores the fp32 state
// at the start of every chunk into `states` ([chunk-head][DK][dv]) and no
// outputs are formed.
template <int C, int DK, typename IO, int GATE, bool STATES = false>
__global__ __launch_bounds__(128) void fwd_scan_kernel(
    ChunkMap map, int H, int dv, int64_t nchunks, const void* __restrict__ q,
    uint32_t q_bytes, const float* __restrict__ s0, void* __restrict__ o,
    float* __restrict__ s_final, FwdBuffers buf, float* __restrict__ states) {
  using OP = IO;
  using X = ChainOps<C, DK, OP, GATE>;
  using Y = OutOps<C, DK, OP, GATE>;
  constexpr int NB = X::NB, NKD = X::NKD, NKC = X::NKC, NDT = X::NDT;
  constexpr bool CH = GATE == GDN_GATE_CHANNEL;
  constexpr bool kPrefetch = io<IO>::bytes == 2;

  __shared__ opvec<OP> sMb[2][NKD][64];
  __shared__ opvec<OP> sEb[2][NKC][64];
  // output staging: the chunk's [C rows][16 cols] slab in the output dtype
  __shared__ __attribute__((aligned(16))) typename opstore<OP>::vec sO[C][2];

  const int w = xcd_swizzle(blockIdx.x, gridDim.x);
  const int ndvt = dv / 16;
  const int vt = w % ndvt;
  const int chain = w / ndvt;
  const int h = chain % H;
  const int seq = chain / H;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
  const int col = 16 * vt + l16;
  const int64_t sbase = (static_cast<int64_t>(seq) * H + h) * DK * dv;

  int cb, ce;
  seq_chunks(map, seq, &cb, &ce);
  const int n = ce - cb;
  const int64_t ch0 = static_cast<int64_t>(h) * nchunks + cb;

  if (wave == 0) {
    floatx4 M[NDT];
#pragma unroll
    for (int a = 0; a < NDT; ++a)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        M[a][s] = s0 ? s0[sbase + static_cast<int64_t>(16 * a + 4 * lg + s) * dv + col] : 0.f;

    auto step = [&](const X& cur, X& nxt, int j) {
      if (kPrefetch && j + 1 < n)
        load_chain<C, DK, OP, GATE>(nxt, buf, ch0 + j + 1, vt, ndvt, lane, lg);
      if constexpr (STATES) {
        float* st = states + (ch0 + j) * static_cast<int64_t>(DK) * dv;
#pragma unroll
        for (int a = 0; a < NDT; ++a)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            st[static_cast<int64_t>(16 * a + 4 * lg + s) * dv + col] = M[a][s];
      }
      opvec<OP> Mb[NKD];
#pragma unroll
      for (int jb = 0; jb < NKD; ++jb) {
        const floatx4 z = {0.f, 0.f, 0.f, 0.f};
        Mb[jb] = pack2<OP>(M[2 * jb], 2 * jb + 1 < NDT ? M[2 * jb + 1] : z);
        sMb[j & 1][jb][lane] = Mb[jb];
      }
      floatx4 E[NB];
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        E[rt] = to_f4(cur.U[rt]);
#pragma unroll
        for (int jb = 0; jb < NKD; ++jb) E[rt] = mma32(cur.W[rt][jb], Mb[jb], E[rt]);
      }
      opvec<OP> Eb[NKC];
#pragma unroll
      for (int jb = 0; jb < NKC; ++jb) {
        const floatx4 z = {0.f, 0.f, 0.f, 0.f};
        Eb[jb] = pack2<OP>(E[2 * jb], 2 * jb + 1 < NB ? E[2 * jb + 1] : z);
        sEb[j & 1][jb][lane] = Eb[jb];
      }
#pragma unroll
      for (int a = 0; a < NDT; ++a) {
        M[a] *= cur.gc[CH ? a : 0];
#pragma unroll
        for (int jb = 0; jb < NKC; ++jb) M[a] = mma32(cur.K[a][jb], Eb[jb], M[a]);
      }
    };

    if constexpr (kPrefetch) {
      X A, B;
      if (n > 0) load_chain<C, DK, OP, GATE>(A, buf, ch0, vt, ndvt, lane, lg);
      for (int j = 0; j <= n; j += 2) {
        if (j < n) step(A, B, j);
        __syncthreads();
        if (j + 1 <= n) {
          if (j + 1 < n) step(B, A, j + 1);
          __syncthreads();
        }
      }
    } else {
      for (int j = 0; j <= n; ++j) {
        if (j < n) {
          X A;
          load_chain<C, DK, OP, GATE>(A, buf, ch0 + j, vt, ndvt, lane, lg);
          step(A, A, j);
        }
        __syncthreads();
      }
    }
    if (s_final) {
#pragma unroll
      for (int a = 0; a < NDT; ++a)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          s_final[sbase + static_cast<int64_t>(16 * a + 4 * lg + s) * dv + col] = M[a][s];
    }
  } else {
    const bool qbuf = q_bytes > 0;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(q, q_bytes);
    auto step = [&](const Y& cur, int jj) {
      if constexpr (STATES) return;
      const ChunkInfo ci = chunk_info(map, cb + jj);
      opvec<OP> Mb[NKD], Eb[NKC];
#pragma unroll
      for (int jb = 0; jb < NKD; ++jb) Mb[jb] = sMb[jj & 1][jb][lane];
#pragma unroll
      for (int jb = 0; jb < NKC; ++jb) Eb[jb] = sEb[jj & 1][jb][lane];
      // O tile rt lands in LDS as rows of the output dtype; each lane then
      // writes whole 16-byte pieces of one row
      using E = typename io<IO>::storage;
      E* so = reinterpret_cast<E*>(&sO[0][0]);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        floatx4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jb = 0; jb < NKD; ++jb) O = mma32(cur.Q[rt][jb], Mb[jb], O);
        if constexpr (GATE == GDN_GATE_SCALAR) O *= cur.gr[rt];
#pragma unroll
        for (int jb = 0; jb < NKC; ++jb)
          if (32 * jb <= 16 * rt + 15) O = mma32(cur.P[rt][jb], Eb[jb], O);
#pragma unroll
        for (int s = 0; s < 4; ++s) io<IO>::store(so, (16 * rt + 4 * lg + s) * 16 + l16, O[s]);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes
      __builtin_amdgcn_wave_barrier();
      constexpr int PPR = 16 * sizeof(E) / 16;  // 16-byte pieces per row
#pragma unroll
      for (int u = 0; u < (C * PPR + 63) / 64; ++u) {
        const int e = lane + 64 * u;
        const int r = e / PPR, piece = e % PPR;
        if (e < C * PPR && r < ci.len) {
          const uint4 val = *reinterpret_cast<const uint4*>(so + r * 16 + piece * (16 / sizeof(E)));
          *reinterpret_cast<uint4*>(static_cast<char*>(o) +
              (((ci.tok0 + r) * H + h) * dv + 16 * vt) * sizeof(E) + piece * 16) = val;
        }
      }
      __builtin_amdgcn_wave_barrier();
    };
    auto load = [&](Y& x, int jj) {
      if constexpr (STATES) return;
      const ChunkInfo ci = chunk_info(map, cb + jj);
      load_out<C, DK, OP, GATE>(x, buf, ch0 + jj, ci, q, qr, qbuf, H, h, lane, l16, lg);
    };

    if constexpr (kPrefetch) {
      Y A, B;
      if (n > 0) load(A, 0);
      __syncthreads();
      for (int j = 1; j <= n; j += 2) {
        if (j < n) load(B, j);
        step(A, j - 1);
        __syncthreads();
        if (j + 1 <= n) {
          if (j + 1 < n) load(A, j + 1);
          step(B, j);
          __syncthreads();
        }
      }
    } else {
      __syncthreads();
      for (int j = 1; j <= n; ++j) {
        Y A;
        load(A, j - 1);
        step(A, j - 1);
        __syncthreads();
      }
    }
  }
}

}  // namespace

}  // namespace gdn
