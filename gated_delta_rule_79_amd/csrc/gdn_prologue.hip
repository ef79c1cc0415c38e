// Prologue of the q, k, v paths in front of the recurrence.
//
// "Gated Delta Networks: Improving Mamba2 with Delta Rule" (paper review),
// "Method": in the block design q and k pass through a projection, a short
// convolution and SiLU before an L2 normalisation; v takes the same path
// without the normalisation.  The projection stays with the caller.  Here,
// for one projection x [tokens, H, D] and caller taps [H, D, W]:
//
//   y[t, h, c] = silu( sum_{j<W} taps[h, c, j] x[t - j, h, c] )    (conv)
//   y[t, h, :] = y[t, h, :] / |y[t, h, :]|                         (normalize)
//
// with no history before a sequence's first token (dense rows or packed
// varlen sequences) and an all-zero row kept zero.  Without `conv` the
// input row is only normalised (the L2 prologue of the per-channel gate).
// The result is written in the input dtype for the chunked forward.
//
// One workgroup holds rows of one head: a row is D / 8 consecutive lanes,
// each with 8 channels read and written as 16-byte pieces, so the row's sum
// of squares is a few shuffles (D / 8 is a power of two that divides 64
// whenever the row is normalised).  The head's taps sit in LDS tap-major.
// The pass is a stream over x and y; each input row is read W times, from
// L2 after the first.

#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {

constexpr int kMaxWidth = 8;
constexpr int kMaxD = 256;

// 8 channels starting at element i of a row (16-byte aligned pieces).
template <typename IO>
__device__ inline void load8(const void* p, int64_t i, float* x) {
  if constexpr (io<IO>::bytes == 2) {
    const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const char*>(p) + i * 2);
    const __bf16* b = reinterpret_cast<const __bf16*>(&r);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(b[e]);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

template <typename IO>
__device__ inline void store8(void* p, int64_t i, const float* x) {
  if constexpr (io<IO>::bytes == 2) {
    uint4 r;
    __bf16* b = reinterpret_cast<__bf16*>(&r);
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = static_cast<__bf16>(x[e]);
    *reinterpret_cast<uint4*>(static_cast<char*>(p) + i * 2) = r;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(static_cast<float*>(p) + i + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
}

// First token of the sequence holding token t.
__device__ inline int64_t seq_start(int64_t t, int T, const int32_t* cu, int nseq) {
  if (cu == nullptr) return t - t % T;
  int lo = 0, hi = nseq;  // largest n with cu[n] <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(cu[mid]) <= t) lo = mid;
    else hi = mid;
  }
  return max(static_cast<int64_t>(cu[lo]), int64_t(0));
}

template <typename IO>
__global__ __launch_bounds__(256) void prologue_kernel(
    int64_t ntok, int T, int H, int D, int W, const int32_t* __restrict__ cu, int nseq,
    const void* __restrict__ x, const float* __restrict__ taps, bool conv, bool normalize,
    void* __restrict__ y) {
  // this head's taps, tap-major ([W][D]): a lane's 8 channels are adjacent
  __shared__ __attribute__((aligned(16))) float st[kMaxWidth * kMaxD];
  const int G = D / 8;             // 8-channel groups per row
  const int rows = 256 / G;        // rows per workgroup
  const int tid = threadIdx.x;
  const int r = tid / G, g = tid - (tid / G) * G;
  const int h = blockIdx.y;
  if (conv) {  // uniform
    for (int e = tid; e < D * W; e += 256) {
      const int c = e / W, j = e - (e / W) * W;
      st[j * D + c] = taps[(static_cast<int64_t>(h) * D + c) * W + j];
    }
    __syncthreads();
  }
  const int64_t t = static_cast<int64_t>(blockIdx.x) * rows + r;
  const bool act = r < rows && t < ntok;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (act) {
    const int64_t col = static_cast<int64_t>(h) * D + 8 * g;
    if (conv) {
      const int64_t s0 = seq_start(t, T, cu, nseq);
#pragma unroll
      for (int j = 0; j < kMaxWidth; ++j) {  // all loads issued together
        if (j < W && t - j >= s0) {
          float xv[8];
          load8<IO>(x, (t - j) * H * D + col, xv);
          const float* tj = st + j * D + 8 * g;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += tj[e] * xv[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] / (1.f + expf(-acc[e]));
    } else {
      load8<IO>(x, t * H * D + col, acc);
    }
  }
  if (normalize) {  // uniform: every lane takes part in the shuffles
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += acc[e] * acc[e];
    for (int m = 1; m < G; m <<= 1) ss += __shfl_xor(ss, m, 64);
    const float sc = ss > 0.f ? rsqrtf(ss) : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= sc;
  }
  if (act) store8<IO>(y, t * H * D + static_cast<int64_t>(h) * D + 8 * g, acc);
}

// ------------------------------------------------------------ backward ---
// Adjoint of the path above (the chain rule of the forward, in reverse):
//   y = a / |a|:        da = (dy - y (y . dy)) / |a|   (an all-zero row: 0)
//   a = z sigmoid(z):   dz = da (s + a (1 - s)),  s = sigmoid(z)
//   z[t] = sum_j taps[., j] x[t - j]:
//                       dx[t] = sum_j taps[., j] dz[t + j]   (inside the sequence)
//                       dtaps[., j] = sum_t dz[t] x[t - j]
// Three passes: dz per row (the forward recomputed, the row's two sums by
// shuffles), then dx and per-block partial tap gradients with one thread per
// channel walking a run of tokens, then the partials summed over the blocks
// in a fixed order (no atomics: the result does not depend on scheduling).

template <typename IO>
__global__ __launch_bounds__(256) void prologue_bwd_dz_kernel(
    int64_t ntok, int T, int H, int D, int W, const int32_t* __restrict__ cu, int nseq,
    const void* __restrict__ x, const float* __restrict__ taps, bool normalize,
    const void* __restrict__ dy, float* __restrict__ dz) {
  __shared__ __attribute__((aligned(16))) float st[kMaxWidth * kMaxD];
  const int G = D / 8;
  const int rows = 256 / G;
  const int tid = threadIdx.x;
  const int r = tid / G, g = tid - (tid / G) * G;
  const int h = blockIdx.y;
  for (int e = tid; e < D * W; e += 256) {
    const int c = e / W, j = e - (e / W) * W;
    st[j * D + c] = taps[(static_cast<int64_t>(h) * D + c) * W + j];
  }
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * rows + r;
  const bool act = r < rows && t < ntok;
  const int64_t col = static_cast<int64_t>(h) * D + 8 * g;
  float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float gy[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (act) {
    const int64_t s0 = seq_start(t, T, cu, nseq);
#pragma unroll
    for (int j = 0; j < kMaxWidth; ++j) {
      if (j < W && t - j >= s0) {
        float xv[8];
        load8<IO>(x, (t - j) * H * D + col, xv);
        const float* tj = st + j * D + 8 * g;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] += tj[e] * xv[e];
      }
    }
    load8<IO>(dy, t * H * D + col, gy);
  }
  float s[8], a[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s[e] = 1.f / (1.f + expf(-z[e]));
    a[e] = z[e] * s[e];
  }
  if (normalize) {  // uniform: every lane takes part in the shuffles
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += a[e] * a[e];
    for (int m = 1; m < G; m <<= 1) ss += __shfl_xor(ss, m, 64);
    const float inv = ss > 0.f ? rsqrtf(ss) : 0.f;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot += a[e] * inv * gy[e];
    for (int m = 1; m < G; m <<= 1) dot += __shfl_xor(dot, m, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) gy[e] = (gy[e] - a[e] * inv * dot) * inv;
  }
  if (act) {
    float d[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = gy[e] * (s[e] + a[e] * (1.f - s[e]));
    float* o = dz + t * H * D + col;
    *reinterpret_cast<float4*>(o) = make_float4(d[0], d[1], d[2], d[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(d[4], d[5], d[6], d[7]);
  }
}

constexpr int kRun = 64;  // tokens a thread of the dx / tap pass walks

// Sequence [start, end) holding token t (dense rows of T, or packed by cu).
__device__ inline void seq_bounds(int64_t t, int T, const int32_t* cu, int nseq, int64_t* a,
                                  int64_t* b) {
  if (cu == nullptr) {
    *a = t - t % T;
    *b = *a + T;
    return;
  }
  int lo = 0, hi = nseq;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(cu[mid]) <= t) lo = mid;
    else hi = mid;
  }
  *a = cu[lo];
  *b = cu[lo + 1];
}

// Thread (run, channel c) walks kRun tokens: dx[t, c] from the dz of the
// next W tokens, and the run's tap-gradient partial sums, reduced over the
// workgroup's runs into part[block][h][c][j].
template <typename IO>
__global__ __launch_bounds__(256) void prologue_bwd_dx_kernel(
    int64_t ntok, int T, int H, int D, int W, const int32_t* __restrict__ cu, int nseq,
    const void* __restrict__ x, const float* __restrict__ taps, const float* __restrict__ dz,
    void* __restrict__ dx, float* __restrict__ part) {
  __shared__ float red[256 * kMaxWidth];
  const int S = 256 / D;  // runs per workgroup
  const int tid = threadIdx.x;
  const int c = tid % D, run = tid / D;
  const int h = blockIdx.y;
  const bool act = run < S;
  float acc[kMaxWidth], wc[kMaxWidth];
#pragma unroll
  for (int j = 0; j < kMaxWidth; ++j) {
    acc[j] = 0.f;
    wc[j] = (act && j < W) ? taps[(static_cast<int64_t>(h) * D + c) * W + j] : 0.f;
  }
  const int64_t t0 = (static_cast<int64_t>(blockIdx.x) * S + run) * kRun;
  if (act && t0 < ntok) {
    const int64_t t1 = min(t0 + kRun, ntok);
    const int64_t stride = static_cast<int64_t>(H) * D;
    const int64_t off = static_cast<int64_t>(h) * D + c;
    int64_t sa, sb;
    seq_bounds(t0, T, cu, nseq, &sa, &sb);
    // at the top of step t, xw[j] = x[t - 1 - j] (zero before the sequence
    // start); the step shifts it to xw[j] = x[t - j]
    float xw[kMaxWidth];
#pragma unroll
    for (int j = 0; j < kMaxWidth; ++j)
      xw[j] = (j < W - 1 && t0 - 1 - j >= sa) ? io<IO>::load(x, (t0 - 1 - j) * stride + off)
                                               : 0.f;
    for (int64_t t = t0; t < t1; ++t) {
      if (t >= sb) {  // next sequence: no history
        seq_bounds(t, T, cu, nseq, &sa, &sb);
#pragma unroll
        for (int j = 0; j < kMaxWidth; ++j) xw[j] = 0.f;
      }
#pragma unroll
      for (int j = kMaxWidth - 1; j > 0; --j) xw[j] = xw[j - 1];
      xw[0] = io<IO>::load(x, t * stride + off);
      const float d = dz[t * stride + off];
      float g = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxWidth; ++j) {
        acc[j] += d * xw[j];  // zero before the sequence start; j >= W never read
        if (j < W && t + j < sb) g += wc[j] * (j == 0 ? d : dz[(t + j) * stride + off]);
      }
      io<IO>::store(dx, t * stride + off, g);
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxWidth; ++j) red[(run * D + c) * kMaxWidth + j] = act ? acc[j] : 0.f;
  __syncthreads();
  for (int e = tid; e < D * W; e += 256) {
    const int cc = e / W, j = e - (e / W) * W;
    float sum = 0.f;
    for (int q = 0; q < S; ++q) sum += red[(q * D + cc) * kMaxWidth + j];
    part[(static_cast<int64_t>(blockIdx.x) * H + h) * D * W + e] = sum;
  }
}

// dtaps[h][c][j] = sum over blocks of part[block][h][c][j], in block order.
__global__ __launch_bounds__(256) void prologue_bwd_taps_kernel(int nblk, int H, int DW,
                                                                const float* __restrict__ part,
                                                                float* __restrict__ dtaps) {
  const int h = blockIdx.x;
  for (int e = threadIdx.x; e < DW; e += 256) {
    float sum = 0.f;
    for (int b = 0; b < nblk; ++b) sum += part[(static_cast<int64_t>(b) * H + h) * DW + e];
    dtaps[static_cast<int64_t>(h) * DW + e] = sum;
  }
}

}  // namespace

size_t prologue_bwd_workspace_bytes(const Problem& p, int D, int W) {
  const int64_t ntok = static_cast<int64_t>(p.B) * p.T;
  const int64_t per = static_cast<int64_t>(256 / D) * kRun;
  const int64_t nblk = (ntok + per - 1) / per;
  const size_t dz = (static_cast<size_t>(ntok) * p.H * D * 4 + 255) / 256 * 256;
  return dz + static_cast<size_t>(nblk) * p.H * D * W * 4;
}

hipError_t launch_prologue_bwd(const Problem& p, int D, int W, const void* x, const float* taps,
                               bool normalize, const void* dy, void* dx, float* dtaps, void* ws,
                               hipStream_t s) {
  const int64_t ntok = static_cast<int64_t>(p.B) * p.T;
  const int32_t* cu = p.varlen ? p.cu_seqlens : nullptr;
  StageScope scope(GDN_STAGE_PROLOGUE, s);
  if (ntok == 0) {  // no tokens: zero tap gradient
    hipLaunchKernelGGL(prologue_bwd_taps_kernel, dim3(p.H), dim3(256), 0, s, 0, p.H, D * W,
                       static_cast<const float*>(nullptr), dtaps);
    return hipGetLastError();
  }
  float* dz = static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(
      static_cast<char*>(ws) + (static_cast<size_t>(ntok) * p.H * D * 4 + 255) / 256 * 256);
  const int rows = 256 / (D / 8);
  const dim3 g1(static_cast<unsigned>((ntok + rows - 1) / rows), static_cast<unsigned>(p.H));
  const int64_t per = static_cast<int64_t>(256 / D) * kRun;
  const int nblk = static_cast<int>((ntok + per - 1) / per);
  const dim3 g2(static_cast<unsigned>(nblk), static_cast<unsigned>(p.H));
  if (p.io == GDN_BF16) {
    hipLaunchKernelGGL((prologue_bwd_dz_kernel<bf16_t>), g1, dim3(256), 0, s, ntok, p.T, p.H, D,
                       W, cu, p.nseq, x, taps, normalize, dy, dz);
    hipLaunchKernelGGL((prologue_bwd_dx_kernel<bf16_t>), g2, dim3(256), 0, s, ntok, p.T, p.H, D,
                       W, cu, p.nseq, x, taps, dz, dx, part);
  } else {
    hipLaunchKernelGGL((prologue_bwd_dz_kernel<f32_t>), g1, dim3(256), 0, s, ntok, p.T, p.H, D,
                       W, cu, p.nseq, x, taps, normalize, dy, dz);
    hipLaunchKernelGGL((prologue_bwd_dx_kernel<f32_t>), g2, dim3(256), 0, s, ntok, p.T, p.H, D,
                       W, cu, p.nseq, x, taps, dz, dx, part);
  }
  hipLaunchKernelGGL(prologue_bwd_taps_kernel, dim3(p.H), dim3(256), 0, s, nblk, p.H, D * W,
                     part, dtaps);
  return hipGetLastError();
}

hipError_t launch_prologue(const Problem& p, int D, int W, const void* x, const float* taps,
                           bool normalize, void* y, hipStream_t s) {
  const int64_t ntok = static_cast<int64_t>(p.B) * p.T;
  if (ntok == 0) return hipSuccess;
  const int rows = 256 / (D / 8);
  const dim3 grid(static_cast<unsigned>((ntok + rows - 1) / rows), static_cast<unsigned>(p.H));
  const bool conv = taps != nullptr;
  StageScope scope(GDN_STAGE_PROLOGUE, s);
  if (p.io == GDN_BF16)
    hipLaunchKernelGGL((prologue_kernel<bf16_t>), grid, dim3(256), 0, s, ntok, p.T, p.H, D, W,
                       p.varlen ? p.cu_seqlens : nullptr, p.nseq, x, taps, conv, normalize, y);
  else
    hipLaunchKernelGGL((prologue_kernel<f32_t>), grid, dim3(256), 0, s, ntok, p.T, p.H, D, W,
                       p.varlen ? p.cu_seqlens : nullptr, p.nseq, x, taps, conv, normalize, y);
  return hipGetLastError();
}

}  // namespace gdn
