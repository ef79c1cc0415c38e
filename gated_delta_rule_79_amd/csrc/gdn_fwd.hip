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

#include "gdn_chunk_common.hpp"

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
  hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(256), 0, s, p.cu_seqlens,
                     p.nseq, p.T, p.chunk, p.nchunks,
                     const_cast<int4*>(m.tab), const_cast<int32_t*>(m.first));
  return hipGetLastError();
}

namespace {

// ------------------------------------------------------------- helpers ---

// 8 consecutive values of row `row` starting at column k0 of an LDS matrix
// stored in the input dtype with row stride ld (elements); zeros past `lim`.
template <typename IO>
__device__ inline void lds_row8(const char* base, int ld, int row, int k0,
                                int lim, float* out) {
  if (k0 >= lim) {
#pragma unroll
    for (int s = 0; s < 8; ++s) out[s] = 0.f;
    return;
  }
  if constexpr (io<IO>::bytes == 2) {
    const uint4 raw = *reinterpret_cast<const uint4*>(
        base + (static_cast<size_t>(row) * ld + k0) * 2);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      out[2 * s] = __uint_as_float(w[s] << 16);
      out[2 * s + 1] = __uint_as_float(w[s] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(
        base + (static_cast<size_t>(row) * ld + k0) * 4);
    const float4 a = p[0], b = p[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

template <typename IO>
__device__ inline float lds_at(const char* base, int ld, int row, int col) {
  if constexpr (io<IO>::bytes == 2) {
    const uint16_t u = *reinterpret_cast<const uint16_t*>(
        base + (static_cast<size_t>(row) * ld + col) * 2);
    return bf16_bits_to_float(u);
  } else {
    return *reinterpret_cast<const float*>(
        base + (static_cast<size_t>(row) * ld + col) * 4);
  }
}

template <typename OP>
__device__ inline void store_frag(char* dst, const float* v) {
  using V = typename opstore<OP>::vec;
  *reinterpret_cast<V*>(dst) = frag<OP>::from_floats(v);
}

template <typename OP>
__device__ inline typename opstore<OP>::vec load_frag(const char* src) {
  using V = typename opstore<OP>::vec;
  return *reinterpret_cast<const V*>(src);
}

// Pack two stacked accumulator tiles into one operand fragment (permuted K).
template <typename OP>
__device__ inline typename opstore<OP>::vec pack2(const floatx4& lo,
                                                  const floatx4& hi) {
  float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return frag<OP>::from_floats(v);
}

// Half-span limit of the per-channel log-gate within one chunk for the
// factored products: each factor stays within exp(+-80), inside the fp32 and
// bf16 normal range.
constexpr float kChannelHalfSpan = 80.f;

// ------------------------------------------------------------ LDS plan ---

template <int C, int DK, typename IO, int GATE>
struct PrepSmem {
  static constexpr int ib = io<IO>::bytes;
  static constexpr int LDK = DK + 16 / ib;          // K, Q rows (elements)
  static constexpr int LDC = C + 4;                 // fp32 C x C matrices
  static constexpr int LDV = C + 16 / ib;           // V^T rows (elements)
  static constexpr int NG = GATE == GDN_GATE_CHANNEL ? C * DK : C;
  static constexpr size_t k_off = 0;
  static constexpr size_t q_off = k_off + size_t(C) * LDK * ib;
  static constexpr size_t g_off = q_off + size_t(C) * LDK * ib;
  static constexpr size_t mid_off = g_off + size_t(NG) * 4;
  static constexpr size_t beta_off = mid_off + size_t(GATE == GDN_GATE_CHANNEL ? DK : 4) * 4;
  static constexpr size_t a_off = beta_off + size_t(C) * 4;
  static constexpr size_t t_off = a_off + size_t(C) * LDC * 4;
  static constexpr size_t r_off = t_off + size_t(C) * LDC * 4;
  static constexpr size_t r_p = size_t(C) * LDC * 4;
  static constexpr size_t r_z = 4 * 256 * 4;
  static constexpr size_t r_v = 64 * size_t(LDV) * ib;
  static constexpr size_t r_bytes = r_p > r_z ? (r_p > r_v ? r_p : r_v) : (r_z > r_v ? r_z : r_v);
  static constexpr size_t total = r_off + r_bytes + 16;
  static_assert(total <= 160 * 1024, "prep LDS budget");
};

// --------------------------------------------------------- prep kernel ---

template <int C, int DK, typename IO, typename GT, int GATE>
__global__ __launch_bounds__(256) void fwd_prep_kernel(
    ChunkMap map, int H, int dv, int64_t nchunks, const void* __restrict__ q,
    const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ beta, const void* __restrict__ la,
    FwdBuffers buf) {
  using OP = IO;  // bf16 inputs multiply on bf16 MFMA, fp32 on fp32 MFMA
  using S = PrepSmem<C, DK, IO, GATE>;
  constexpr int ib = S::ib;
  constexpr int ob = opstore<OP>::bytes;
  constexpr int NB = C / 16;
  constexpr int NKD = (DK + 31) / 32;
  constexpr int NKC = (C + 31) / 32;
  constexpr int LDK = S::LDK, LDC = S::LDC, LDV = S::LDV;

  __shared__ __attribute__((aligned(16))) char smem[S::total];
  __shared__ int s_span_bits;
  char* sK = smem + S::k_off;
  char* sQ = smem + S::q_off;
  float* sg = reinterpret_cast<float*>(smem + S::g_off);
  float* smid = reinterpret_cast<float*>(smem + S::mid_off);
  float* sbeta = reinterpret_cast<float*>(smem + S::beta_off);
  float* sA = reinterpret_cast<float*>(smem + S::a_off);
  float* sT = reinterpret_cast<float*>(smem + S::t_off);
  char* sR = smem + S::r_off;
  float* sP = reinterpret_cast<float*>(sR);
  float* sZ = reinterpret_cast<float*>(sR);
  char* sVt = sR;

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

  // ---- 1. gates and beta -------------------------------------------------
  if (tid == 0) s_span_bits = 0;
  if (tid < C) {
    float b = 0.f;
    if (tid < len) b = io<GT>::load(beta, (tok0 + tid) * H + h);
    sbeta[tid] = b;
  }
  if constexpr (GATE != GDN_GATE_CHANNEL) {
    if (wave == 0) {
      float x = 0.f;
      if constexpr (GATE == GDN_GATE_SCALAR)
        if (lane < len) x = io<GT>::load(la, (tok0 + lane) * H + h);
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
      }
      if (lane < C) sg[lane] = x;
    }
  }
  __syncthreads();  // s_span_bits initialised before the atomics below
  if constexpr (GATE == GDN_GATE_CHANNEL) {
    // raw per-channel log-gates (zero past the sequence end), then a running
    // sum down each channel in LDS
    for (int e = tid; e < C * DK; e += 256) {
      const int r = e / DK, col = e % DK;
      sg[e] = r < len ? io<GT>::load(la, ((tok0 + r) * H + h) * DK + col) : 0.f;
    }
    __syncthreads();
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
  // K and Q rows of the chunk (zero past the sequence end)
  {
    constexpr int VW = 16 / ib;  // elements per 16-byte vector
    constexpr int VPR = DK / VW;
    for (int e = tid; e < C * VPR; e += 256) {
      const int r = e / VPR, cv = (e % VPR) * VW;
      uint4 kv = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
      if (r < len) {
        const int64_t off = ((tok0 + r) * H + h) * DK + cv;
        kv = *reinterpret_cast<const uint4*>(static_cast<const char*>(k) + off * ib);
        qv = *reinterpret_cast<const uint4*>(static_cast<const char*>(q) + off * ib);
      }
      *reinterpret_cast<uint4*>(sK + (size_t(r) * LDK + cv) * ib) = kv;
      *reinterpret_cast<uint4*>(sQ + (size_t(r) * LDK + cv) * ib) = qv;
    }
  }
  __syncthreads();

  // ---- 2. P = decayed Q K^T (i <= r) and A = decayed b K K^T (i < r) -------
  bool exact = false;
  if constexpr (GATE == GDN_GATE_CHANNEL)
    exact = __int_as_float(s_span_bits) > kChannelHalfSpan;
  if (!exact) {
    constexpr int NT2 = NB * (NB + 1) / 2;
    for (int job = wave; job < 2 * NT2; job += 4) {
      const bool isP = job < NT2;
      int t = isP ? job : job - NT2;
      int tr = 0;
      while (t > tr) { t -= tr + 1; ++tr; }
      const int ti = t;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      const int ra = 16 * tr + l16;  // row of the A operand (token r)
      const int rb = 16 * ti + l16;  // row of the B operand (token i)
#pragma unroll
      for (int kb = 0; kb < NKD; ++kb) {
        const int k0 = kb * 32 + lg * 8;
        float av[8], bv[8];
        lds_row8<IO>(isP ? sQ : sK, LDK, ra, k0, DK, av);
        lds_row8<IO>(sK, LDK, rb, k0, DK, bv);
        if constexpr (GATE == GDN_GATE_CHANNEL) {
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const int kk = k0 + s;
            if (kk < DK) {
              av[s] *= expf(sg[ra * DK + kk] - smid[kk]);
              bv[s] *= expf(smid[kk] - sg[rb * DK + kk]);
            }
          }
        }
        acc = mma32(frag<OP>::from_floats(av), frag<OP>::from_floats(bv), acc);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 16 * tr + 4 * lg + s;
        const int i = 16 * ti + l16;
        float val = acc[s];
        if constexpr (GATE == GDN_GATE_SCALAR) val *= expf(sg[r] - sg[i]);
        if (isP) {
          sP[r * LDC + i] = (i <= r) ? val : 0.f;
        } else {
          sA[r * LDC + i] = (i < r) ? val * sbeta[r] : 0.f;
        }
      }
    }
  } else {
    // exact per-element path for extreme per-channel decay spans
    for (int e = tid; e < C * C; e += 256) {
      const int r = e / C, i = e % C;
      float pv = 0.f, av = 0.f;
      if (i <= r) {
        for (int kk = 0; kk < DK; ++kk) {
          const float d = expf(sg[r * DK + kk] - sg[i * DK + kk]);
          const float ki = lds_at<IO>(sK, LDK, i, kk) * d;
          pv += lds_at<IO>(sQ, LDK, r, kk) * ki;
          av += lds_at<IO>(sK, LDK, r, kk) * ki;
        }
      }
      sP[r * LDC + i] = pv;
      sA[r * LDC + i] = (i < r) ? av * sbeta[r] : 0.f;
    }
  }
  __syncthreads();

  // ---- 3. P fragments -----------------------------------------------------
  {
    char* dst = buf.at(ch, buf.off_p);
    for (int e = tid; e < NB * NKC * 64; e += 256) {
      const int ln = e & 63, fr = e >> 6;
      const int rt = fr / NKC, jb = fr % NKC;
      const int m = ln & 15, g = ln >> 4;
      const int r = 16 * rt + m;
      float vals[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int i = 32 * jb + perm_k(g, s);
        vals[s] = (i < C && i <= r) ? sP[r * LDC + i] : 0.f;
      }
      store_frag<OP>(dst + (size_t(fr) * 64 + ln) * 8 * ob, vals);
    }
  }
  // zero the strictly upper blocks of T
  for (int e = tid; e < C * C; e += 256) {
    const int r = e / C, i = e % C;
    if ((i >> 4) > (r >> 4)) sT[r * LDC + i] = 0.f;
  }
  __syncthreads();

  // ---- 4. T = (I + A)^-1 ---------------------------------------------------
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
        for (int s = 0; s <= r; ++s)
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
      const int kbmax = (16 * rt + 15) / 32;
      const int r = 16 * rt + l16;
      for (int kb = 0; kb <= kbmax; ++kb) {
        float bv[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int i = 32 * kb + 8 * lg + s;
          bv[s] = (i < C) ? sT[r * LDC + i] : 0.f;
        }
        const auto bf = frag<OP>::from_floats(bv);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int a = 2 * jb + half;
          if (16 * a >= DK) continue;
          const int dk = 16 * a + l16;
          float av[8];
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const int i = 32 * kb + 8 * lg + s;
            float x = 0.f;
            if (i < C) {
              x = lds_at<IO>(sK, LDK, i, dk) * sbeta[i];
              if constexpr (GATE == GDN_GATE_SCALAR) x *= expf(sg[i]);
              if constexpr (GATE == GDN_GATE_CHANNEL) x *= expf(sg[i * DK + dk]);
            }
            av[s] = x;
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
      store_frag<OP>(dst + ((size_t(rt) * NKD + jb) * 64 + lane) * 8 * ob, out);
    }
  }

  // ---- 6. Q~ and K~^T fragments, chunk decay of the state rows ------------
  {
    char* dq = buf.at(ch, buf.off_q);
    for (int e = tid; e < NB * NKD * 64; e += 256) {
      const int ln = e & 63, fr = e >> 6;
      const int rt = fr / NKD, jb = fr % NKD;
      const int m = ln & 15, g = ln >> 4;
      const int r = 16 * rt + m;
      float vals[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int dk = 32 * jb + perm_k(g, s);
        float x = 0.f;
        if (dk < DK) {
          x = lds_at<IO>(sQ, LDK, r, dk);
          if constexpr (GATE == GDN_GATE_SCALAR) x *= expf(sg[r]);
          if constexpr (GATE == GDN_GATE_CHANNEL) x *= expf(sg[r * DK + dk]);
        }
        vals[s] = x;
      }
      store_frag<OP>(dq + (size_t(fr) * 64 + ln) * 8 * ob, vals);
    }
    char* dk_ = buf.at(ch, buf.off_k);
    for (int e = tid; e < (DK / 16) * NKC * 64; e += 256) {
      const int ln = e & 63, fr = e >> 6;
      const int a = fr / NKC, jb = fr % NKC;
      const int m = ln & 15, g = ln >> 4;
      const int dk = 16 * a + m;
      float vals[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int i = 32 * jb + perm_k(g, s);
        float x = 0.f;
        if (i < C) {
          x = lds_at<IO>(sK, LDK, i, dk);
          if constexpr (GATE == GDN_GATE_SCALAR) x *= expf(sg[C - 1] - sg[i]);
          if constexpr (GATE == GDN_GATE_CHANNEL)
            x *= expf(sg[(C - 1) * DK + dk] - sg[i * DK + dk]);
        }
        vals[s] = x;
      }
      store_frag<OP>(dk_ + (size_t(fr) * 64 + ln) * 8 * ob, vals);
    }
    float* gam = reinterpret_cast<float*>(buf.at(ch, buf.off_g));
    for (int d = tid; d < DK; d += 256) {
      float x = 1.f;
      if constexpr (GATE == GDN_GATE_SCALAR) x = expf(sg[C - 1]);
      if constexpr (GATE == GDN_GATE_CHANNEL) x = expf(sg[(C - 1) * DK + d]);
      gam[d] = x;
    }
  }

  // ---- 7. U = T diag(b) V, 64 value columns at a time ---------------------
  {
    float* U = reinterpret_cast<float*>(buf.at(ch, buf.off_u));
    const int ndt = dv / 16;
    for (int slab = 0; slab < dv; slab += 64) {
      __syncthreads();  // the region is free (T done / previous slab done)
      for (int e = tid; e < C * 64; e += 256) {
        const int i = e >> 6, col = e & 63;
        float x = 0.f;
        if (i < len && slab + col < dv)
          x = io<IO>::load(v, ((tok0 + i) * H + h) * dv + slab + col);
        if constexpr (ib == 2) {
          reinterpret_cast<__bf16*>(sVt)[col * LDV + i] = (__bf16)x;
        } else {
          reinterpret_cast<float*>(sVt)[col * LDV + i] = x;
        }
      }
      __syncthreads();
      const int nvt = min(4, (dv - slab) / 16);
      for (int job = wave; job < NB * nvt; job += 4) {
        const int rt = job / nvt, vt = job % nvt;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        const int kbmax = (16 * rt + 15) / 32;
        const int r = 16 * rt + l16;
        const int col = 16 * vt + l16;
        for (int kb = 0; kb <= kbmax; ++kb) {
          float av[8], bv[8];
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const int i = 32 * kb + 8 * lg + s;
            av[s] = (i < C) ? sT[r * LDC + i] : 0.f;
            bv[s] = (i < C) ? sbeta[i] * lds_at<IO>(sVt, LDV, col, i) : 0.f;
          }
          acc = mma32(frag<OP>::from_floats(av), frag<OP>::from_floats(bv), acc);
        }
        const int vtg = slab / 16 + vt;
        *reinterpret_cast<floatx4*>(U + ((size_t(rt) * ndt + vtg) * 64 + lane) * 4) = acc;
      }
    }
  }
}

// --------------------------------------------------------- scan kernel ---

template <int C, int DK, typename IO>
__global__ __launch_bounds__(64) void fwd_scan_kernel(
    ChunkMap map, int H, int dv, int64_t nchunks, const float* __restrict__ s0,
    void* __restrict__ o, float* __restrict__ s_final, FwdBuffers buf) {
  using OP = IO;
  using V = typename opstore<OP>::vec;
  constexpr int ob = opstore<OP>::bytes;
  constexpr int NB = C / 16;
  constexpr int NKD = (DK + 31) / 32;
  constexpr int NKC = (C + 31) / 32;
  constexpr int NDT = DK / 16;

  const int w = xcd_swizzle(blockIdx.x, gridDim.x);
  const int ndvt = dv / 16;
  const int vt = w % ndvt;
  const int chain = w / ndvt;
  const int h = chain % H;
  const int seq = chain / H;
  const int lane = threadIdx.x, l16 = lane & 15, lg = lane >> 4;
  const int col = 16 * vt + l16;

  floatx4 M[NDT];
  const int64_t sbase = (static_cast<int64_t>(seq) * H + h) * DK * dv;
#pragma unroll
  for (int a = 0; a < NDT; ++a)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      M[a][s] = s0 ? s0[sbase + static_cast<int64_t>(16 * a + 4 * lg + s) * dv + col] : 0.f;

  int cb, ce;
  seq_chunks(map, seq, &cb, &ce);
  for (int c = cb; c < ce; ++c) {
    const ChunkInfo ci = chunk_info(map, c);
    const int64_t ch = static_cast<int64_t>(h) * nchunks + c;
    const char* pw = buf.at(ch, buf.off_w);
    const char* pq = buf.at(ch, buf.off_q);
    const char* pk = buf.at(ch, buf.off_k);
    const char* pp = buf.at(ch, buf.off_p);
    const float* pu = reinterpret_cast<const float*>(buf.at(ch, buf.off_u));
    const float* pg = reinterpret_cast<const float*>(buf.at(ch, buf.off_g));

    // E = U - W M
    floatx4 E[NB];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
      E[rt] = *reinterpret_cast<const floatx4*>(pu + ((size_t(rt) * ndvt + vt) * 64 + lane) * 4);
    V Mb[NKD];
#pragma unroll
    for (int jb = 0; jb < NKD; ++jb) {
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      Mb[jb] = pack2<OP>(M[2 * jb], 2 * jb + 1 < NDT ? M[2 * jb + 1] : z);
    }
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int jb = 0; jb < NKD; ++jb)
        E[rt] = mma32(load_frag<OP>(pw + ((size_t(rt) * NKD + jb) * 64 + lane) * 8 * ob),
                      Mb[jb], E[rt]);
    // O = Q~ M + P E
    floatx4 O[NB];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      O[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jb = 0; jb < NKD; ++jb)
        O[rt] = mma32(load_frag<OP>(pq + ((size_t(rt) * NKD + jb) * 64 + lane) * 8 * ob),
                      Mb[jb], O[rt]);
    }
    V Eb[NKC];
#pragma unroll
    for (int jb = 0; jb < NKC; ++jb) {
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      Eb[jb] = pack2<OP>(E[2 * jb], 2 * jb + 1 < NB ? E[2 * jb + 1] : z);
    }
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int jb = 0; jb < NKC; ++jb)
        if (32 * jb <= 16 * rt + 15)
          O[rt] = mma32(load_frag<OP>(pp + ((size_t(rt) * NKC + jb) * 64 + lane) * 8 * ob),
                        Eb[jb], O[rt]);
    // M <- gamma_c M + K~^T E
#pragma unroll
    for (int a = 0; a < NDT; ++a) {
      const floatx4 gm = *reinterpret_cast<const floatx4*>(pg + 16 * a + 4 * lg);
      M[a] *= gm;
#pragma unroll
      for (int jb = 0; jb < NKC; ++jb)
        M[a] = mma32(load_frag<OP>(pk + ((size_t(a) * NKC + jb) * 64 + lane) * 8 * ob),
                     Eb[jb], M[a]);
    }
    // outputs of the chunk's valid rows
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 16 * rt + 4 * lg + s;
        if (r < ci.len)
          io<IO>::store(o, ((ci.tok0 + r) * H + h) * dv + col, O[rt][s]);
      }
  }
  if (s_final) {
#pragma unroll
    for (int a = 0; a < NDT; ++a)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        s_final[sbase + static_cast<int64_t>(16 * a + 4 * lg + s) * dv + col] = M[a][s];
  }
}

// ------------------------------------------------------------ dispatch ---

template <int C, int DK, typename IO, typename GT, int GATE>
hipError_t run_fwd(const Problem& p, const void* q, const void* k,
                   const void* v, const void* beta, const void* la,
                   const float* s0, void* o, float* s_final, char* ws,
                   hipStream_t s) {
  const FwdLayout L(C, DK, p.dv, opstore<IO>::bytes);
  char* map_base = ws;
  char* ops = ws + chunk_map_bytes(p);
  const FwdBuffers buf = make_buffers(ops, L);
  const ChunkMap map = make_chunk_map(p, map_base);
  if (p.varlen) {
    hipError_t e = launch_chunk_map(p, map_base, s);
    if (e != hipSuccess) return e;
  }
  if (p.nchunks > 0) {
    hipLaunchKernelGGL((fwd_prep_kernel<C, DK, IO, GT, GATE>),
                       dim3(static_cast<unsigned>(p.nchunks * p.H)), dim3(256),
                       0, s, map, p.H, p.dv, p.nchunks, q, k, v, beta, la, buf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nwork = static_cast<int64_t>(p.nseq) * p.H * (p.dv / 16);
  hipLaunchKernelGGL((fwd_scan_kernel<C, DK, IO>),
                     dim3(static_cast<unsigned>(nwork)), dim3(64), 0, s, map,
                     p.H, p.dv, p.nchunks, s0, o, s_final, buf);
  return hipGetLastError();
}

template <int C, int DK, typename IO, typename GT>
hipError_t fwd_gate(const Problem& p, const void* q, const void* k,
                    const void* v, const void* beta, const void* la,
                    const float* s0, void* o, float* sf, char* ws,
                    hipStream_t s) {
  switch (p.gate) {
    case GDN_GATE_NONE:
      return run_fwd<C, DK, IO, GT, GDN_GATE_NONE>(p, q, k, v, beta, la, s0, o, sf, ws, s);
    case GDN_GATE_SCALAR:
      return run_fwd<C, DK, IO, GT, GDN_GATE_SCALAR>(p, q, k, v, beta, la, s0, o, sf, ws, s);
    default:
      return run_fwd<C, DK, IO, GT, GDN_GATE_CHANNEL>(p, q, k, v, beta, la, s0, o, sf, ws, s);
  }
}

template <int C, int DK>
hipError_t fwd_types(const Problem& p, const void* q, const void* k,
                     const void* v, const void* beta, const void* la,
                     const float* s0, void* o, float* sf, char* ws,
                     hipStream_t s) {
  if (p.io == GDN_BF16) {
    if (p.gdt == GDN_BF16)
      return fwd_gate<C, DK, bf16_t, bf16_t>(p, q, k, v, beta, la, s0, o, sf, ws, s);
    return fwd_gate<C, DK, bf16_t, f32_t>(p, q, k, v, beta, la, s0, o, sf, ws, s);
  }
  if (p.gdt == GDN_BF16)
    return fwd_gate<C, DK, f32_t, bf16_t>(p, q, k, v, beta, la, s0, o, sf, ws, s);
  return fwd_gate<C, DK, f32_t, f32_t>(p, q, k, v, beta, la, s0, o, sf, ws, s);
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
  const FwdLayout L(p.chunk, p.dk, p.dv, p.io == GDN_BF16 ? 2 : 4);
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
