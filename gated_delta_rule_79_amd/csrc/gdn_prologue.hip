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

}  // namespace

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
