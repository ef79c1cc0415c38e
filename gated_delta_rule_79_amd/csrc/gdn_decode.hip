// Single-token decode of the gated delta rule, state updated in place.
//
// "Gated Delta Networks: Improving Mamba2 with Delta Rule" (paper review),
// "Background": recurrent inference carries a fixed-size matrix state, so a
// decode step costs O(dk * dv) per head regardless of context length.  The
// step, in the stored orientation M = S^T ([dk, dv] row-major fp32):
//     Mt = a (.) M        (a = exp(log alpha): one value, or one per dk row)
//     u = Mt^T k,  w = Mt^T q,  e = beta (v - u)
//     o = w + (k . q) e   (= M_new^T q),   M_new = Mt + k e^T
//
// The step is a pure stream over the state: 8 bytes of HBM traffic (one fp32
// read, one fp32 write) per 6 flops, so HBM bandwidth bounds it.  Each
// workgroup owns one (sequence, head) and a 64-column slab of the state; a
// thread holds DK/16 rows x 4 columns in registers between the reduction and
// the write-back, so every state element crosses HBM exactly once each way.
// Loads are 16-byte and a wave covers four 256-byte row segments.

#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kSlab = 64;  // state columns per workgroup

// beta_w: write strength of the decoupled erase / write rule (then beta is
// the erase strength, e = beta_w v - beta Mt^T k); nullptr: beta does both.
template <int DK, typename IO, typename GT, int GATE>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    int H, int dv, const void* __restrict__ q, const void* __restrict__ k,
    const void* __restrict__ v, const void* __restrict__ beta,
    const void* __restrict__ la, float* __restrict__ state,
    void* __restrict__ o, const void* __restrict__ beta_w) {
  constexpr int RPT = DK / 16;  // rows per thread
  // the slabs of one head are consecutive workgroups, so the two halves of
  // every state row are streamed at about the same time
  const int nslab = (dv + kSlab - 1) / kSlab;
  const int nh = blockIdx.x / nslab;  // n * H + h
  const int slab = blockIdx.x - nh * nslab;
  const int t = threadIdx.x;
  const int cg = t & 15;        // column group: 4 consecutive columns
  const int rg = t >> 4;        // row group 0..15: rows rg + 16 j
  const int col = slab * kSlab + cg * 4;
  const bool active = col < dv;  // dv is a multiple of 16, so all-or-none

  const int64_t vec_off = static_cast<int64_t>(nh) * DK;
  float* M = state + static_cast<int64_t>(nh) * DK * dv;

  // per-row key, query and decay for the rows this thread owns
  float kr[RPT], qr[RPT], ar[RPT];
  float a_scalar = 1.0f;
  if constexpr (GATE == GDN_GATE_SCALAR) a_scalar = expf(io<GT>::load(la, nh));
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int r = rg + 16 * j;
    kr[j] = io<IO>::load(k, vec_off + r);
    qr[j] = io<IO>::load(q, vec_off + r);
    if constexpr (GATE == GDN_GATE_CHANNEL)
      ar[j] = expf(io<GT>::load(la, vec_off + r));
    else
      ar[j] = a_scalar;
  }

  // load and decay the state slab; partial reductions over this thread's rows
  floatx4 m[RPT];
  floatx4 u = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
  float kq = 0.f;
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int r = rg + 16 * j;
    if (active) {
      m[j] = __builtin_nontemporal_load(
          reinterpret_cast<const floatx4*>(M + static_cast<int64_t>(r) * dv + col));
    } else {
      m[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    m[j] *= ar[j];
    u += m[j] * kr[j];
    w += m[j] * qr[j];
    kq += kr[j] * qr[j];
  }

  // reduce over the 16 row groups: 4 per wave (lanes 16 and 32 apart), then
  // across the 4 waves through LDS
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u[c] = wave_sum_xor(u[c], 48);
    w[c] = wave_sum_xor(w[c], 48);
  }
  kq = wave_sum_xor(kq, 48);
  __shared__ floatx4 su[4][16], sw[4][16];
  __shared__ float skq[4];
  const int wave = t >> 6;
  const int lane = t & 63;
  if (lane < 16) {
    su[wave][lane] = u;
    sw[wave][lane] = w;
  }
  if (lane == 0) skq[wave] = kq;
  __syncthreads();
  u = su[0][cg] + su[1][cg] + su[2][cg] + su[3][cg];
  w = sw[0][cg] + sw[1][cg] + sw[2][cg] + sw[3][cg];
  kq = skq[0] + skq[1] + skq[2] + skq[3];

  if (!active) return;
  const float b = io<GT>::load(beta, nh);
  const int64_t vo = static_cast<int64_t>(nh) * dv + col;
  floatx4 e;
  if (beta_w == nullptr) {
#pragma unroll
    for (int c = 0; c < 4; ++c) e[c] = b * (io<IO>::load(v, vo + c) - u[c]);
  } else {
    const float bw = io<GT>::load(beta_w, nh);
#pragma unroll
    for (int c = 0; c < 4; ++c) e[c] = bw * io<IO>::load(v, vo + c) - b * u[c];
  }

  if (rg == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) io<IO>::store(o, vo + c, w[c] + kq * e[c]);
  }
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int r = rg + 16 * j;
    floatx4 mn = m[j] + kr[j] * e;
    __builtin_nontemporal_store(
        mn, reinterpret_cast<floatx4*>(M + static_cast<int64_t>(r) * dv + col));
  }
}

// Decode with Householder-product transitions: nh (k, v, beta) triples per
// token, one decay, nh delta steps in order, the output read after the last.
// One wave per (sequence, head, 64-column slab): lane (rg, cg) keeps rows
// rg, rg + 4, .. (DK / 4 of them) of columns 4 cg .. 4 cg + 3 in registers,
// each step's k-projection is reduced over the four row groups with two
// shuffles, so the nh steps need no LDS and no barrier and the state still
// crosses HBM once each way.
template <int DK, typename IO, typename GT, int GATE>
__global__ __launch_bounds__(64) void decode_product_kernel(
    int H, int dv, int nh, const void* __restrict__ q, const void* __restrict__ k,
    const void* __restrict__ v, const void* __restrict__ beta,
    const void* __restrict__ la, float* __restrict__ state, void* __restrict__ o) {
  constexpr int RPT = DK / 4;
  const int nslab = (dv + kSlab - 1) / kSlab;
  const int nhd = blockIdx.x / nslab;  // n * H + h
  const int slab = blockIdx.x - nhd * nslab;
  const int n = nhd / H, h = nhd - n * H;
  const int lane = threadIdx.x;
  const int cg = lane & 15, rg = lane >> 4;
  const int col = slab * kSlab + cg * 4;
  const bool active = col < dv;  // dv is a multiple of 16: whole lane groups
  float* M = state + static_cast<int64_t>(nhd) * DK * dv;
  floatx4 mm[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j)
    mm[j] = active ? __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(
                         M + static_cast<int64_t>(rg + 4 * j) * dv + col))
                   : floatx4{0.f, 0.f, 0.f, 0.f};
  if constexpr (GATE == GDN_GATE_SCALAR) {
    const float a = expf(io<GT>::load(la, nhd));
#pragma unroll
    for (int j = 0; j < RPT; ++j) mm[j] *= a;
  }
  for (int st = 0; st < nh; ++st) {
    const int64_t sh = (static_cast<int64_t>(n) * nh + st) * H + h;  // [N, nh, H]
    float kr[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) kr[j] = io<IO>::load(k, sh * DK + rg + 4 * j);
    const float b = io<GT>::load(beta, sh);
    floatx4 vv = {0.f, 0.f, 0.f, 0.f};
    if (active) {
#pragma unroll
      for (int c = 0; c < 4; ++c) vv[c] = io<IO>::load(v, sh * dv + col + c);
    }
    floatx4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RPT; ++j) u += mm[j] * kr[j];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u[c] += __shfl_xor(u[c], 16, 64);
      u[c] += __shfl_xor(u[c], 32, 64);
    }
    const floatx4 e = b * (vv - u);
#pragma unroll
    for (int j = 0; j < RPT; ++j) mm[j] += kr[j] * e;
  }
  // o = M^T q after the last step
  floatx4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < RPT; ++j)
    w += mm[j] * io<IO>::load(q, static_cast<int64_t>(nhd) * DK + rg + 4 * j);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    w[c] += __shfl_xor(w[c], 16, 64);
    w[c] += __shfl_xor(w[c], 32, 64);
  }
  if (!active) return;
  if (rg == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) io<IO>::store(o, static_cast<int64_t>(nhd) * dv + col + c, w[c]);
  }
#pragma unroll
  for (int j = 0; j < RPT; ++j)
    __builtin_nontemporal_store(
        mm[j], reinterpret_cast<floatx4*>(M + static_cast<int64_t>(rg + 4 * j) * dv + col));
}

template <int DK, typename IO, typename GT>
hipError_t dispatch_product(const Problem& p, int nh, const void* q, const void* k,
                            const void* v, const void* beta, const void* la,
                            float* state, void* o, hipStream_t s) {
  StageScope scope(GDN_STAGE_DECODE, s);
  const dim3 grid(static_cast<unsigned>(int64_t(p.B) * p.H * ((p.dv + kSlab - 1) / kSlab)));
  if (p.gate == GDN_GATE_SCALAR)
    hipLaunchKernelGGL((decode_product_kernel<DK, IO, GT, GDN_GATE_SCALAR>), grid, dim3(64),
                       0, s, p.H, p.dv, nh, q, k, v, beta, la, state, o);
  else
    hipLaunchKernelGGL((decode_product_kernel<DK, IO, GT, GDN_GATE_NONE>), grid, dim3(64),
                       0, s, p.H, p.dv, nh, q, k, v, beta, la, state, o);
  return hipGetLastError();
}

template <int DK, typename IO>
hipError_t product_gdt(const Problem& p, int nh, const void* q, const void* k,
                       const void* v, const void* beta, const void* la, float* state,
                       void* o, hipStream_t s) {
  if (p.gdt == GDN_BF16)
    return dispatch_product<DK, IO, bf16_t>(p, nh, q, k, v, beta, la, state, o, s);
  return dispatch_product<DK, IO, f32_t>(p, nh, q, k, v, beta, la, state, o, s);
}

template <int DK>
hipError_t product_io(const Problem& p, int nh, const void* q, const void* k,
                      const void* v, const void* beta, const void* la, float* state,
                      void* o, hipStream_t s) {
  if (p.io == GDN_BF16)
    return product_gdt<DK, bf16_t>(p, nh, q, k, v, beta, la, state, o, s);
  return product_gdt<DK, f32_t>(p, nh, q, k, v, beta, la, state, o, s);
}

template <int DK, typename IO, typename GT>
hipError_t dispatch_gate(const Problem& p, dim3 grid, const void* q,
                         const void* k, const void* v, const void* beta,
                         const void* la, float* state, void* o, hipStream_t s) {
  StageScope scope(GDN_STAGE_DECODE, s);
  switch (p.gate) {
    case GDN_GATE_NONE:
      hipLaunchKernelGGL((decode_kernel<DK, IO, GT, GDN_GATE_NONE>), grid,
                         dim3(kThreads), 0, s, p.H, p.dv, q, k, v, beta, la,
                         state, o, p.beta_w);
      break;
    case GDN_GATE_SCALAR:
      hipLaunchKernelGGL((decode_kernel<DK, IO, GT, GDN_GATE_SCALAR>), grid,
                         dim3(kThreads), 0, s, p.H, p.dv, q, k, v, beta, la,
                         state, o, p.beta_w);
      break;
    default:
      hipLaunchKernelGGL((decode_kernel<DK, IO, GT, GDN_GATE_CHANNEL>), grid,
                         dim3(kThreads), 0, s, p.H, p.dv, q, k, v, beta, la,
                         state, o, p.beta_w);
      break;
  }
  return hipGetLastError();
}

template <int DK, typename IO>
hipError_t dispatch_gdt(const Problem& p, dim3 grid, const void* q,
                        const void* k, const void* v, const void* beta,
                        const void* la, float* state, void* o, hipStream_t s) {
  if (p.gdt == GDN_BF16)
    return dispatch_gate<DK, IO, bf16_t>(p, grid, q, k, v, beta, la, state, o, s);
  return dispatch_gate<DK, IO, f32_t>(p, grid, q, k, v, beta, la, state, o, s);
}

template <int DK>
hipError_t dispatch_io(const Problem& p, dim3 grid, const void* q,
                       const void* k, const void* v, const void* beta,
                       const void* la, float* state, void* o, hipStream_t s) {
  if (p.io == GDN_BF16)
    return dispatch_gdt<DK, bf16_t>(p, grid, q, k, v, beta, la, state, o, s);
  return dispatch_gdt<DK, f32_t>(p, grid, q, k, v, beta, la, state, o, s);
}

}  // namespace

hipError_t launch_decode_product(const Problem& p, int nh, const void* q, const void* k,
                                 const void* v, const void* beta, const void* la,
                                 float* state, void* o, hipStream_t s) {
  switch (p.dk) {
    case 16: return product_io<16>(p, nh, q, k, v, beta, la, state, o, s);
    case 32: return product_io<32>(p, nh, q, k, v, beta, la, state, o, s);
    case 64: return product_io<64>(p, nh, q, k, v, beta, la, state, o, s);
    default: return product_io<128>(p, nh, q, k, v, beta, la, state, o, s);
  }
}

hipError_t launch_decode(const Problem& p, const void* q, const void* k,
                         const void* v, const void* beta, const void* la,
                         float* state, void* o, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(int64_t(p.B) * p.H * ((p.dv + kSlab - 1) / kSlab)));
  switch (p.dk) {
    case 16: return dispatch_io<16>(p, grid, q, k, v, beta, la, state, o, s);
    case 32: return dispatch_io<32>(p, grid, q, k, v, beta, la, state, o, s);
    case 64: return dispatch_io<64>(p, grid, q, k, v, beta, la, state, o, s);
    default: return dispatch_io<128>(p, grid, q, k, v, beta, la, state, o, s);
  }
}

}  // namespace gdn
