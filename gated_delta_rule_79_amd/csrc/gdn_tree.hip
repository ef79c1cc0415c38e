// Commit of draft trees: the accepted node's state rebuilt from its root path.
//
// "TreeWY: Speculative Verification for Gated DeltaNet Hybrids" (summary in
// the list of related papers): verification scores every node of a draft
// tree without a state per node, and the commit reconstructs only the state
// of the node that was accepted.  Node i of a tree continues the state of
// its parent (parent[i] < i, -1 for the committed state) with one step of
// the gated delta rule on its own token, so the accepted node's state is the
// committed state run through the tokens of its root path, in order.
//
// One wave per (tree, head, 64-column slab of the state).  Lane (rg, cg)
// holds rows rg, rg + 4, .. (DK / 4 of them) of columns 4 cg .. 4 cg + 3 in
// registers; per path node the decayed state's k-projection is reduced over
// the four row groups with two shuffles, and the rank-1 correction is applied
// in place.  The state crosses HBM once each way whatever the path length.
// The path itself comes from the tree's parent array in one wave: pointer
// jumping gives every node's ancestor set, and since parents precede their
// children, the accepted node's ancestors in increasing index order are its
// root path.

#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {

constexpr int kCommitCols = 64;  // state columns per wave

template <int DK, typename IO, int GATE>
__global__ __launch_bounds__(64) void tree_commit_kernel(
    int H, int dv, int n, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ parent, const int32_t* __restrict__ accepted,
    const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ beta, const void* __restrict__ la, bool gbf,
    float* __restrict__ state) {
  constexpr int RPT = DK / 4;  // rows per lane
  // the column slabs of one (tree, head) are consecutive workgroups
  const int nslab = (dv + kCommitCols - 1) / kCommitCols;
  const int mh = blockIdx.x / nslab;  // tree * H + head
  const int slab = blockIdx.x - mh * nslab;
  const int m = mh / H, h = mh - m * H;
  const int lane = threadIdx.x;
  const int64_t t0 = cu ? static_cast<int64_t>(cu[m]) : static_cast<int64_t>(m) * n;
  const int len = cu ? cu[m + 1] - cu[m] : n;
  const int a = accepted[m];
  // nothing accepted (or an index outside the tree): the state stays
  if (a < 0 || a >= len || a >= 64) return;

  int nx = -1;
  if (lane < len) {
    nx = parent[t0 + lane];
    if (nx < -1 || nx >= lane) nx = -1;
  }
  uint64_t anc = nx >= 0 ? (uint64_t(1) << nx) : 0;
#pragma unroll
  for (int j = 0; j < 6; ++j) {  // 2^6 = 64 >= any path in a 64-node tree
    const int src = nx >= 0 ? nx : lane;
    const uint32_t alo = __shfl(static_cast<uint32_t>(anc), src, 64);
    const uint32_t ahi = __shfl(static_cast<uint32_t>(anc >> 32), src, 64);
    const int ns = __shfl(nx, src, 64);
    if (nx >= 0) {
      anc |= (static_cast<uint64_t>(ahi) << 32) | alo;
      nx = ns;
    }
  }
  const uint64_t path =
      ((static_cast<uint64_t>(__shfl(static_cast<uint32_t>(anc >> 32), a, 64)) << 32) |
       __shfl(static_cast<uint32_t>(anc), a, 64)) |
      (uint64_t(1) << a);

  const int cg = lane & 15, rg = lane >> 4;
  const int col = slab * kCommitCols + cg * 4;
  const bool active = col < dv;  // dv is a multiple of 16: whole lane groups
  float* M = state + static_cast<int64_t>(mh) * DK * dv;
  floatx4 mm[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j)
    mm[j] = active ? *reinterpret_cast<const floatx4*>(M + static_cast<int64_t>(rg + 4 * j) * dv + col)
                   : floatx4{0.f, 0.f, 0.f, 0.f};

  uint64_t rest = path;
  while (rest != 0) {  // the same path in every lane: a uniform loop
    const int i = __builtin_ctzll(rest);
    rest &= rest - 1;
    const int64_t th = (t0 + i) * H + h;
    float kr[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) kr[j] = io<IO>::load(k, th * DK + rg + 4 * j);
    const float b = load_gate(beta, th, gbf);
    float dec = 1.f;
    if constexpr (GATE == GDN_GATE_SCALAR) dec = expf(load_gate(la, th, gbf));
    floatx4 vv = {0.f, 0.f, 0.f, 0.f};
    if (active) {
#pragma unroll
      for (int c = 0; c < 4; ++c) vv[c] = io<IO>::load(v, th * dv + col + c);
    }
    floatx4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      mm[j] *= dec;
      u += mm[j] * kr[j];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u[c] += __shfl_xor(u[c], 16, 64);
      u[c] += __shfl_xor(u[c], 32, 64);
    }
    const floatx4 e = b * (vv - u);
#pragma unroll
    for (int j = 0; j < RPT; ++j) mm[j] += kr[j] * e;
  }
  if (!active) return;
#pragma unroll
  for (int j = 0; j < RPT; ++j)
    *reinterpret_cast<floatx4*>(M + static_cast<int64_t>(rg + 4 * j) * dv + col) = mm[j];
}

template <int DK, typename IO>
hipError_t commit_gate(const Problem& p, dim3 grid, const int32_t* parent,
                       const int32_t* accepted, const void* k, const void* v,
                       const void* beta, const void* la, float* state, hipStream_t s) {
  const int n = p.varlen ? 0 : p.T;
  const int32_t* cu = p.varlen ? p.cu_seqlens : nullptr;
  const bool gbf = p.gdt == GDN_BF16;
  if (p.gate == GDN_GATE_SCALAR)
    hipLaunchKernelGGL((tree_commit_kernel<DK, IO, GDN_GATE_SCALAR>), grid, dim3(64), 0, s,
                       p.H, p.dv, n, cu, parent, accepted, k, v, beta, la, gbf, state);
  else
    hipLaunchKernelGGL((tree_commit_kernel<DK, IO, GDN_GATE_NONE>), grid, dim3(64), 0, s,
                       p.H, p.dv, n, cu, parent, accepted, k, v, beta, la, gbf, state);
  return hipGetLastError();
}

template <int DK>
hipError_t commit_io(const Problem& p, dim3 grid, const int32_t* parent,
                     const int32_t* accepted, const void* k, const void* v,
                     const void* beta, const void* la, float* state, hipStream_t s) {
  if (p.io == GDN_BF16)
    return commit_gate<DK, bf16_t>(p, grid, parent, accepted, k, v, beta, la, state, s);
  return commit_gate<DK, f32_t>(p, grid, parent, accepted, k, v, beta, la, state, s);
}

}  // namespace

hipError_t launch_tree_commit(const Problem& p, const int32_t* parent,
                              const int32_t* accepted, const void* k, const void* v,
                              const void* beta, const void* la, float* state,
                              hipStream_t s) {
  if (p.nseq == 0) return hipSuccess;
  StageScope scope(GDN_STAGE_TREE_COMMIT, s);
  const dim3 grid(static_cast<unsigned>(int64_t(p.nseq) * p.H *
                                        ((p.dv + kCommitCols - 1) / kCommitCols)));
  switch (p.dk) {
    case 16: return commit_io<16>(p, grid, parent, accepted, k, v, beta, la, state, s);
    case 32: return commit_io<32>(p, grid, parent, accepted, k, v, beta, la, state, s);
    case 64: return commit_io<64>(p, grid, parent, accepted, k, v, beta, la, state, s);
    default: return commit_io<128>(p, grid, parent, accepted, k, v, beta, la, state, s);
  }
}

}  // namespace gdn
