// C ABI of libgdn: argument validation, workspace sizing and dispatch.
// Every check runs on the host before anything is enqueued, so a non-OK
// status means no work was launched.  No exception crosses the ABI.

#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <exception>
#include <mutex>
#include <vector>

#include "gdn.h"
#include "gdn_internal.hpp"

namespace {

std::atomic<int> g_fail_launch{0};
std::atomic<int> g_seg_chunks{0};  // gdn_set_segment_chunks

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// A pointer that must be present when its tensor has elements.
gdn_status need(const void* p, int64_t elems) {
  if (elems == 0) return GDN_OK;
  if (p == nullptr) return GDN_ERR_NULL;
  if (!aligned16(p)) return GDN_ERR_ALIGN;
  return GDN_OK;
}

// An optional pointer: NULL is fine, otherwise it must be aligned.
gdn_status opt(const void* p) {
  if (p != nullptr && !aligned16(p)) return GDN_ERR_ALIGN;
  return GDN_OK;
}

#define GDN_TRY(expr)                 \
  do {                                \
    gdn_status _s = (expr);           \
    if (_s != GDN_OK) return _s;      \
  } while (0)

bool dk_ok(int dk) { return dk == 16 || dk == 32 || dk == 64 || dk == 128; }
bool dv_ok(int dv) { return dv >= 16 && dv <= 256 && dv % 16 == 0; }
bool dtype_ok(int d) { return d == GDN_F32 || d == GDN_BF16; }

// Shared checks of the chunked entry points; fills *out.  lnh > 0: each
// token takes 2^lnh delta steps (k, v, beta per step), out->T counts steps.
gdn_status check_chunk_problem(const gdn_problem* p, gdn::Problem* out, int lnh = 0) {
  if (p == nullptr) return GDN_ERR_NULL;
  if (!dtype_ok(p->io_dtype) || !dtype_ok(p->gate_dtype)) return GDN_ERR_DTYPE;
  if (p->gate < GDN_GATE_NONE || p->gate > GDN_GATE_CHANNEL)
    return GDN_ERR_UNSUPPORTED;
  if (p->B < 1 || p->H < 1 || p->T < 0 || p->nseq < 0) return GDN_ERR_SHAPE;
  if (!dk_ok(p->dk) || !dv_ok(p->dv)) return GDN_ERR_UNSUPPORTED;
  if (p->chunk != 16 && p->chunk != 32 && p->chunk != 64)
    return GDN_ERR_UNSUPPORTED;
  if (p->nseq > 0) {
    if (p->B != 1) return GDN_ERR_SHAPE;
    if (p->cu_seqlens == nullptr) return GDN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(p->cu_seqlens) & 3u) != 0)
      return GDN_ERR_ALIGN;
  } else if (p->cu_seqlens != nullptr) {
    return GDN_ERR_SHAPE;
  }
  // element counts must stay far inside int64 and the grid limits
  const int64_t tok = (static_cast<int64_t>(p->B) * p->T) << lnh;
  if (tok * p->H * 256 > (int64_t(1) << 46)) return GDN_ERR_SHAPE;
  if ((static_cast<int64_t>(p->T) << lnh) > (int64_t(1) << 30)) return GDN_ERR_SHAPE;
  out->B = p->B;
  out->T = p->T << lnh;
  out->lnh = lnh;
  out->qknorm = false;
  out->parent = nullptr;
  out->H = p->H;
  out->dk = p->dk;
  out->dv = p->dv;
  out->chunk = p->chunk;
  out->varlen = p->nseq > 0;
  out->nseq = out->varlen ? p->nseq : p->B;
  out->cu_seqlens = p->cu_seqlens;
  out->io = p->io_dtype;
  out->gdt = p->gate_dtype;
  out->gate = p->gate;
  const int64_t per_seq = (static_cast<int64_t>(out->T) + p->chunk - 1) / p->chunk;
  out->nchunks = out->varlen ? per_seq + p->nseq : per_seq * p->B;
  if (out->nchunks * p->H > (int64_t(1) << 31) - 1) return GDN_ERR_SHAPE;
  out->seg = gdn::plan_segments(*out);
  out->nsegs = gdn::seg_slots_host(*out);
  if (out->nsegs * p->H * 32 > (int64_t(1) << 31) - 1) return GDN_ERR_SHAPE;
  return GDN_OK;
}

gdn_status check_fwd_pointers(const gdn::Problem& p, const void* q,
                              const void* k, const void* v, const void* beta,
                              const void* la, const float* s0, const void* o,
                              const float* s_final) {
  const int64_t tok = static_cast<int64_t>(p.B) * p.T * p.H;  // steps
  const int64_t tq = tok >> p.lnh;                             // tokens
  GDN_TRY(need(q, tq * p.dk));
  GDN_TRY(need(k, tok * p.dk));
  GDN_TRY(need(v, tok * p.dv));
  GDN_TRY(need(beta, tok));
  if (p.gate != GDN_GATE_NONE) GDN_TRY(need(la, tq));
  else GDN_TRY(opt(la));
  GDN_TRY(need(o, tq * p.dv));
  GDN_TRY(opt(s0));
  GDN_TRY(opt(s_final));
  return GDN_OK;
}

gdn_status launched(hipError_t e) {
  return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// ------------------------------------------------------- stage timing ---

struct ProfRecord {
  int stage;
  hipEvent_t begin, end;
};

struct Profiler {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<ProfRecord> done;
  std::vector<hipEvent_t> pool;
  std::vector<std::pair<int, hipEvent_t>> open;  // stage, begin event

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

Profiler& prof() {
  static Profiler* p = new Profiler();  // never destroyed: events outlive exit
  return *p;
}

}  // namespace

namespace gdn {

void prof_begin(int stage, hipStream_t s) {
  Profiler& P = prof();
  if (!P.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(P.mu);
  hipEvent_t e = P.get();
  if (e == nullptr) return;
  if (hipEventRecord(e, s) != hipSuccess) {
    P.pool.push_back(e);
    return;
  }
  P.open.emplace_back(stage, e);
}

void prof_end(int stage, hipStream_t s) {
  Profiler& P = prof();
  if (!P.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(P.mu);
  for (size_t i = P.open.size(); i-- > 0;) {
    if (P.open[i].first != stage) continue;
    hipEvent_t b = P.open[i].second;
    P.open.erase(P.open.begin() + static_cast<long>(i));
    hipEvent_t e = P.get();
    if (e == nullptr || hipEventRecord(e, s) != hipSuccess) {
      P.pool.push_back(b);
      if (e) P.pool.push_back(e);
      return;
    }
    P.done.push_back({stage, b, e});
    return;
  }
}

int plan_segments(const Problem& p) {
  const int set = g_seg_chunks.load();
  if (set < 0 || p.nseq == 0) return 0;
  if (set > 0) return std::min(set, 1 << 20);
  // automatic: a state-pass workgroup takes one (sequence, head) and 8 value
  // slabs and walks its chunks in order, so with few (sequence, head) pairs
  // most CUs idle.  Segments of L chunks give groups * n / L workgroups;
  // take L so that they about fill the 256 CUs once, but not below
  // ~sqrt(n / 2.56) chunks (each segment costs a step of the sequential
  // combine and its own transition columns).  No split when the pairs alone
  // fill the CUs or the chains are short.
  constexpr double kCUs = 256.0;
  const int64_t groups = static_cast<int64_t>(p.nseq) * p.H * ((p.dv / 16 + 7) / 8);
  const double n = static_cast<double>(p.nchunks - (p.varlen ? p.nseq : 0)) / p.nseq;
  if (n < 8.0) return 0;
  const int fill = static_cast<int>(std::ceil(n * static_cast<double>(groups) / kCUs));
  const int lo = std::max(2, static_cast<int>(std::ceil(std::sqrt(n / 2.56))));
  const int L = std::max(fill, lo);
  return L >= n ? 0 : L;
}

int64_t seg_slots_host(const Problem& p) {
  if (p.seg == 0) return p.nseq;
  if (!p.varlen) {
    const int64_t nt = (static_cast<int64_t>(p.T) + p.chunk - 1) / p.chunk;
    return static_cast<int64_t>(p.nseq) * std::max<int64_t>(1, (nt + p.seg - 1) / p.seg);
  }
  // sum over sequences of max(1, ceil(n_s / L)) <= nchunks / L + nseq
  return p.nchunks / p.seg + p.nseq;
}

}  // namespace gdn

extern "C" {

void gdn_profile_enable(int enable) {
  Profiler& P = prof();
  std::lock_guard<std::mutex> lk(P.mu);
  P.on.store(enable != 0);
}

gdn_status gdn_profile_read(double* total_ms, int32_t* count) {
  try {
    if (total_ms == nullptr || count == nullptr) return GDN_ERR_NULL;
    for (int i = 0; i < GDN_STAGE_COUNT; ++i) {
      total_ms[i] = 0.0;
      count[i] = 0;
    }
    Profiler& P = prof();
    std::lock_guard<std::mutex> lk(P.mu);
    gdn_status st = GDN_OK;
    for (const ProfRecord& r : P.done) {
      float ms = 0.f;
      if (hipEventSynchronize(r.end) != hipSuccess ||
          hipEventElapsedTime(&ms, r.begin, r.end) != hipSuccess) {
        st = GDN_ERR_HIP;
      } else if (r.stage >= 0 && r.stage < GDN_STAGE_COUNT) {
        total_ms[r.stage] += ms;
        count[r.stage] += 1;
      }
      P.pool.push_back(r.begin);
      P.pool.push_back(r.end);
    }
    P.done.clear();
    return st;
  } catch (...) {
    return GDN_ERR_HIP;
  }
}


int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_str(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: size out of range or inconsistent";
    case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: unknown dtype code";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: outside the supported sizes or modes";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: pointer not 16-byte aligned";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: HIP runtime refused the launch";
  }
  return "GDN_ERR_UNKNOWN";
}

void gdn_test_set_fail_launch(int enable) { g_fail_launch.store(enable != 0); }

void gdn_set_segment_chunks(int n) { g_seg_chunks.store(n); }

gdn_status gdn_chunk_fwd_workspace(const gdn_problem* p, size_t* bytes) {
  try {
    if (bytes == nullptr) return GDN_ERR_NULL;
    gdn::Problem pp;
    GDN_TRY(check_chunk_problem(p, &pp));
    *bytes = gdn::fwd_workspace_bytes(pp);
    return GDN_OK;
  } catch (...) {
    return GDN_ERR_HIP;
  }
}

gdn_status gdn_chunk_fwd(const gdn_problem* p, const void* q, const void* k,
                         const void* v, const void* beta,
                         const void* log_alpha, const float* s0, void* o,
                         float* s_final, void* ws, size_t ws_bytes,
                         void* stream) {
  try {
    gdn::Problem pp;
    GDN_TRY(check_chunk_problem(p, &pp));
    GDN_TRY(check_fwd_pointers(pp, q, k, v, beta, log_alpha, s0, o, s_final));
    const size_t need_ws = gdn::fwd_workspace_bytes(pp);
    if (need_ws > 0 && (ws == nullptr || ws_bytes < need_ws))
      return GDN_ERR_WORKSPACE;
    GDN_TRY(opt(ws));
    if (g_fail_launch.load()) return GDN_ERR_HIP;
    return launched(gdn::launch_fwd(pp, q, k, v, beta, log_alpha, s0, o,
                                    s_final, ws,
                                    static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_ERR_HIP;
  }
}

// q and k rows L2-normalised inside the forward; per-token gates only.
gdn_status gdn_chunk_fwd_qknorm(const gdn_problem* p, const void* q, const void* k,
                                const void* v, const void* beta,
                                const void* log_alpha, const float* s0, void* o,
                                float* s_final, void* ws, size_t ws_bytes,
                                void* stream) {
  try {
    if (p == nullptr) return GDN_ERR_NULL;
    if (p->gate == GDN_GATE_CHANNEL) return GDN_ERR_UNSUPPORTED;
    gdn::Problem pp;
    GDN_TRY(check_chunk_problem(p, &pp));
    GDN_TRY(check_fwd_pointers(pp, q, k, v, beta, log_alpha, s0, o, s_final));
    const size_t need_ws = gdn::fwd_workspace_bytes(pp);
    if (need_ws > 0 && (ws == nullptr || ws_bytes < need_ws))
      return GDN_ERR_WORKSPACE;
    GDN_TRY(opt(ws));
    if (g_fail_launch.load()) return GDN_ERR_HIP;
    pp.qknorm = true;
    return launched(gdn::launch_fwd(pp, q, k, v, beta, log_alpha, s0, o,
                                    s_final, ws,
                                    static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_ERR_HIP;
  }
}

// Draft trees: one tree per chunk, no segment split, per-token gates only.
static gdn_status check_tree(const gdn_problem* p, gdn::Problem* out) {
  if (p == nullptr) return GDN_ERR_NULL;
  if (p->gate == GDN_GATE_CHANNEL) return GDN_ERR_UNSUPPORTED;
  GDN_TRY(check_chunk_problem(p, out));
  if (!out->varlen && p->T > p->chunk) return GDN_ERR_SHAPE;
  out->seg = 0;
  out->nsegs = out->nseq;
  return GDN_OK;
}

gdn_status gdn_tree_verify_workspace(const gdn_problem* p, size_t* bytes) {
  try {
    if (bytes == nullptr) return GDN_ERR_NULL;
    gdn::Problem pp;
    GDN_TRY(check_tree(p, &pp));
    *bytes = gdn::fwd_workspace_bytes(pp);
    return GDN_OK;
  } catch (...) {
    return GDN_ERR_HIP;
  }
}

gdn_status gdn_tree_verify(const gdn_problem* p, const int32_t* parent, const void* q,
                           const void* k, const void* v, const void* beta,
                           const void* log_alpha, const float* state, void* o,
                           void* ws, size_t ws_bytes, void* stream) {
  try {
    gdn::Problem pp;
    GDN_TRY(check_tree(p, &pp));
    GDN_TRY(check_fwd_pointers(pp, q, k, v, beta, log_alpha, state, o, nullptr));
    GDN_TRY(need(parent, static_cast<int64_t>(pp.B) * pp.T));
    if ((reinterpret_cast<uintptr_t>(parent) & 3u) != 0) return GDN_ERR_ALIGN;
    const size_t need_ws = gdn::fwd_workspace_bytes(pp);
    if (need_ws > 0 && (ws == nullptr || ws_bytes < need_ws))
      return GDN_ERR_WORKSPACE;
    GDN_TRY(opt(ws));
    if (g_fail_launch.load()) return GDN_ERR_HIP;
    pp.parent = parent;
    return launched(gdn::launch_fwd(pp, q, k, v, beta, log_alpha, state, o, nullptr, ws,
                                    static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_ERR_HIP;
  }
}

gdn_status gdn_tree_commit(const gdn_problem* p, const int32_t* parent,
                           const int32_t* accepted, const void* k, const void* v,
                           const void* beta, const void* log_alpha, float* state,
                           void* stream) {
  try {
    gdn::Problem pp;
    GDN_TRY(check_tree(p, &pp));
    const int64_t tok = static_cast<int64_t>(pp.B) * pp.T * pp.H;
    GDN_TRY(need(k, tok * pp.dk));
    GDN_TRY(need(v, tok * pp.dv));
    GDN_TRY(need(beta, tok));
    if (pp.gate != GDN_GATE_NONE) GDN_TRY(need(log_alpha, tok));
    else GDN_TRY(opt(log_alpha));
    GDN_TRY(need(parent, static_cast<int64_t>(pp.B) * pp.T));
    GDN_TRY(need(accepted, pp.nseq));
    GDN_TRY(need(state, static_cast<int64_t>(pp.nseq) * pp.H * pp.dk * pp.dv));
    if ((reinterpret_cast<uintptr_t>(parent) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(accepted) & 3u) != 0)
      return GDN_ERR_ALIGN;
    if (g_fail_launch.load()) return GDN_ERR_HIP;
    return launched(gdn::launch_tree_commit(pp, parent, accepted, k, v, beta, log_alpha,
                                            state, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_ERR_HIP;
  }
}

// Householder-product transitions: nh in {1, 2, 4} delta steps per token,
// per-token gates only.
static gdn_status check_product(const gdn_problem* p, int32_t nh, gdn::Problem* out) {
  if (p == nullptr) return GDN_ERR_NULL;
  if (nh != 1 && nh != 2 && nh != 4) return GDN_ERR_UNSUPPORTED;
  if (p->gate == GDN_GATE_CHANNEL) return GDN_ERR_UNSUPPORTED;
  return check_chunk_problem(p, out, nh == 1 ? 0 : (nh == 2 ? 1 : 2));
}

gdn_status gdn_chunk_fwd_product_workspace(const gdn_problem* p, int32_t nh,
                                           size_t* bytes) {
  try {
    if (bytes == nullptr) return GDN_ERR_NULL;
    gdn::Problem pp;
    GDN_TRY(check_product(p, nh, &pp));
    *bytes = gdn::fwd_workspace_bytes(pp);
    return GDN_OK;
  } catch (...) {
    return GDN_ERR_HIP;
  }
}

gdn_status gdn_chunk_fwd_product(const gdn_problem* p, int32_t nh, const void* q,
                                 const void* k, const void* v, const void* beta,
                                 const void* log_alpha, const float* s0, void* o,
                                 float* s_final, void* ws, size_t ws_bytes,
                                 void* stream) {
  try {
    gdn::Problem pp;
    GDN_TRY(check_product(p, nh, &pp));
    GDN_TRY(check_fwd_pointers(pp, q, k, v, beta, log_alpha, s0, o, s_final));
    const size_t need_ws = gdn::fwd_workspace_bytes(pp);
    if (need_ws > 0 && (ws == nullptr || ws_bytes < need_ws))
      return GDN_ERR_WORKSPACE;
    GDN_TRY(opt(ws));
    if (g_fail_launch.load()) return GDN_ERR_HIP;
    return launched(gdn::launch_fwd(pp, q, k, v, beta, log_alpha, s0, o,
                                    s_final, ws,
                                    static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_ERR_HIP;
  }
}

gdn_status gdn_chunk_bwd_workspace(const gdn_problem* p, size_t* bytes) {
  try {
    if (bytes == nullptr) return GDN_ERR_NULL;
    gdn::Problem pp;
    GDN_TRY(check_chunk_problem(p, &pp));
    if (!gdn::bwd_supported(pp)) return GDN_ERR_UNSUPPORTED;
    *bytes = gdn::bwd_workspace_bytes(pp);
    return GDN_OK;
  } catch (...) {
    return GDN_ERR_HIP;
  }
}

gdn_status gdn_chunk_bwd(const gdn_problem* p, const void* q, const void* k,
                         const void* v, const void* beta,
                         const void* log_alpha, const float* s0,
                         const void* d_o, const float* ds_final, void* dq,
                         void* dk, void* dv, float* dbeta, float* dlog_alpha,
                         float* ds0, void* ws, size_t ws_bytes, void* stream) {
  try {
    gdn::Problem pp;
    GDN_TRY(check_chunk_problem(p, &pp));
    if (!gdn::bwd_supported(pp)) return GDN_ERR_UNSUPPORTED;
    const int64_t tok = static_cast<int64_t>(pp.B) * pp.T * pp.H;
    GDN_TRY(need(q, tok * pp.dk));
    GDN_TRY(need(k, tok * pp.dk));
    GDN_TRY(need(v, tok * pp.dv));
    GDN_TRY(need(beta, tok));
    GDN_TRY(need(d_o, tok * pp.dv));
    GDN_TRY(need(dq, tok * pp.dk));
    GDN_TRY(need(dk, tok * pp.dk));
    GDN_TRY(need(dv, tok * pp.dv));
    GDN_TRY(need(dbeta, tok));
    if (pp.gate != GDN_GATE_NONE) {
      GDN_TRY(need(log_alpha, tok));
      GDN_TRY(need(dlog_alpha, tok));
    } else {
      GDN_TRY(opt(log_alpha));
      GDN_TRY(opt(dlog_alpha));
    }
    GDN_TRY(opt(s0));
    GDN_TRY(opt(ds_final));
    GDN_TRY(opt(ds0));
    const size_t need_ws = gdn::bwd_workspace_bytes(pp);
    if (need_ws > 0 && (ws == nullptr || ws_bytes < need_ws))
      return GDN_ERR_WORKSPACE;
    GDN_TRY(opt(ws));
    if (g_fail_launch.load()) return GDN_ERR_HIP;
    return launched(gdn::launch_bwd(pp, q, k, v, beta, log_alpha, s0, d_o,
                                    ds_final, dq, dk, dv, dbeta, dlog_alpha,
                                    ds0, ws, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_ERR_HIP;
  }
}

gdn_status gdn_decode_step(const gdn_problem* p, const void* q, const void* k,
                           const void* v, const void* beta,
                           const void* log_alpha, float* state, void* o,
                           void* stream) {
  try {
    if (p == nullptr) return GDN_ERR_NULL;
    if (!dtype_ok(p->io_dtype) || !dtype_ok(p->gate_dtype)) return GDN_ERR_DTYPE;
    if (p->gate < GDN_GATE_NONE || p->gate > GDN_GATE_CHANNEL)
      return GDN_ERR_UNSUPPORTED;
    if (p->B < 1 || p->H < 1) return GDN_ERR_SHAPE;
    if (!dk_ok(p->dk) || !dv_ok(p->dv)) return GDN_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(p->B) * p->H > (int64_t(1) << 31) - 1)
      return GDN_ERR_SHAPE;
    gdn::Problem pp{};
    pp.B = p->B;
    pp.T = 1;
    pp.H = p->H;
    pp.dk = p->dk;
    pp.dv = p->dv;
    pp.nseq = p->B;
    pp.io = p->io_dtype;
    pp.gdt = p->gate_dtype;
    pp.gate = p->gate;
    const int64_t nh = static_cast<int64_t>(p->B) * p->H;
    GDN_TRY(need(q, nh * p->dk));
    GDN_TRY(need(k, nh * p->dk));
    GDN_TRY(need(v, nh * p->dv));
    GDN_TRY(need(beta, nh));
    if (pp.gate != GDN_GATE_NONE) GDN_TRY(need(log_alpha, nh));
    else GDN_TRY(opt(log_alpha));
    GDN_TRY(need(state, nh * p->dk * p->dv));
    GDN_TRY(need(o, nh * p->dv));
    if (g_fail_launch.load()) return GDN_ERR_HIP;
    return launched(gdn::launch_decode(pp, q, k, v, beta, log_alpha, state, o,
                                       static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_ERR_HIP;
  }
}

gdn_status gdn_decode_step_product(const gdn_problem* p, int32_t nh, const void* q,
                                   const void* k, const void* v, const void* beta,
                                   const void* log_alpha, float* state, void* o,
                                   void* stream) {
  try {
    if (p == nullptr) return GDN_ERR_NULL;
    if (!dtype_ok(p->io_dtype) || !dtype_ok(p->gate_dtype)) return GDN_ERR_DTYPE;
    if (p->gate != GDN_GATE_NONE && p->gate != GDN_GATE_SCALAR) return GDN_ERR_UNSUPPORTED;
    if (nh != 1 && nh != 2 && nh != 4) return GDN_ERR_UNSUPPORTED;
    if (p->B < 1 || p->H < 1) return GDN_ERR_SHAPE;
    if (!dk_ok(p->dk) || !dv_ok(p->dv)) return GDN_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(p->B) * p->H > (int64_t(1) << 31) - 1) return GDN_ERR_SHAPE;
    gdn::Problem pp{};
    pp.B = p->B;
    pp.T = 1;
    pp.H = p->H;
    pp.dk = p->dk;
    pp.dv = p->dv;
    pp.nseq = p->B;
    pp.io = p->io_dtype;
    pp.gdt = p->gate_dtype;
    pp.gate = p->gate;
    const int64_t nhd = static_cast<int64_t>(p->B) * p->H;
    GDN_TRY(need(q, nhd * p->dk));
    GDN_TRY(need(k, nhd * nh * p->dk));
    GDN_TRY(need(v, nhd * nh * p->dv));
    GDN_TRY(need(beta, nhd * nh));
    if (pp.gate != GDN_GATE_NONE) GDN_TRY(need(log_alpha, nhd));
    else GDN_TRY(opt(log_alpha));
    GDN_TRY(need(state, nhd * p->dk * p->dv));
    GDN_TRY(need(o, nhd * p->dv));
    if (g_fail_launch.load()) return GDN_ERR_HIP;
    return launched(gdn::launch_decode_product(pp, nh, q, k, v, beta, log_alpha, state, o,
                                               static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_ERR_HIP;
  }
}

}  // extern "C"
