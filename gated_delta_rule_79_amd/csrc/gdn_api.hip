// C ABI of libgdn: argument validation, workspace sizing and dispatch.
// Every check runs on the host before anything is enqueued, so a non-OK
// status means no work was launched.  No exception crosses the ABI.

#include <stdint.h>
#include <stdio.h>
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

std::atomic<int> g_fail_launch{0};  // gdn_test_set_fail_launch

// ------------------------------------------------------------ diagnostics ---
// With GDN_LOG set (non-empty, not "0") every refused call writes one line
// to stderr naming the entry point, the status and the check's source line,
// and every launch writes the resolved problem and the dispatch choices.
// The variable is read at each call; the library is silent otherwise.

thread_local const char* t_entry = "gdn";

struct EntryScope {  // names the running entry point for the log lines
  const char* prev;
  explicit EntryScope(const char* name) : prev(t_entry) { t_entry = name; }
  ~EntryScope() { t_entry = prev; }
};

bool log_on() {
  const char* e = getenv("GDN_LOG");
  return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
}

gdn_status fail_at(gdn_status s, int line) {
  if (log_on())
    fprintf(stderr, "gdn: %s: %s (check at gdn_api.hip:%d)\n", t_entry, gdn_status_str(s),
            line);
  return s;
}

#define GDN_ENTRY() EntryScope gdn_entry_scope_(__func__)
#define GDN_FAIL(s) fail_at((s), __LINE__)

const char* dtype_name(int d) { return d == GDN_BF16 ? "bf16" : "f32"; }

const char* gate_name(int g) {
  return g == GDN_GATE_NONE ? "none" : g == GDN_GATE_SCALAR ? "scalar" : "channel";
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// A pointer that must be present when its tensor has elements.
gdn_status need(const void* p, int64_t elems) {
  if (elems == 0) return GDN_OK;
  if (p == nullptr) return GDN_FAIL(GDN_ERR_NULL);
  if (!aligned16(p)) return GDN_FAIL(GDN_ERR_ALIGN);
  return GDN_OK;
}

// An optional pointer: NULL is fine, otherwise it must be aligned.
gdn_status opt(const void* p) {
  if (p != nullptr && !aligned16(p)) return GDN_FAIL(GDN_ERR_ALIGN);
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
  if (p == nullptr) return GDN_FAIL(GDN_ERR_NULL);
  if (!dtype_ok(p->io_dtype) || !dtype_ok(p->gate_dtype)) return GDN_FAIL(GDN_ERR_DTYPE);
  if (p->gate < GDN_GATE_NONE || p->gate > GDN_GATE_CHANNEL)
    return GDN_FAIL(GDN_ERR_UNSUPPORTED);
  if (p->B < 1 || p->H < 1 || p->T < 0 || p->nseq < 0) return GDN_FAIL(GDN_ERR_SHAPE);
  if (!dk_ok(p->dk) || !dv_ok(p->dv)) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
  if (p->chunk != 16 && p->chunk != 32 && p->chunk != 64)
    return GDN_FAIL(GDN_ERR_UNSUPPORTED);
  if (p->nseq > 0) {
    if (p->B != 1) return GDN_FAIL(GDN_ERR_SHAPE);
    if (p->cu_seqlens == nullptr) return GDN_FAIL(GDN_ERR_NULL);
    if ((reinterpret_cast<uintptr_t>(p->cu_seqlens) & 3u) != 0)
      return GDN_FAIL(GDN_ERR_ALIGN);
  } else if (p->cu_seqlens != nullptr) {
    return GDN_FAIL(GDN_ERR_SHAPE);
  }
  // element counts must stay far inside int64 and the grid limits
  const int64_t tok = (static_cast<int64_t>(p->B) * p->T) << lnh;
  if (tok * p->H * 256 > (int64_t(1) << 46)) return GDN_FAIL(GDN_ERR_SHAPE);
  if ((static_cast<int64_t>(p->T) << lnh) > (int64_t(1) << 30)) return GDN_FAIL(GDN_ERR_SHAPE);
  out->B = p->B;
  out->T = p->T << lnh;
  out->lnh = lnh;
  out->qknorm = false;
  out->parent = nullptr;
  out->beta_w = nullptr;
  out->conv_w = 0;
  out->conv_tk = nullptr;
  out->conv_tv = nullptr;
  out->H = p->H;
  out->dk = p->dk;
  out->dv = p->dv;
  out->chunk = p->chunk;
  out->varlen = p->nseq > 0;
  out->nseq = out->varlen ? p->nseq : p->B;
  out->cu_seqlens = p->cu_seqlens;
  out->seg_req = p->seg_chunks;
  out->io = p->io_dtype;
  out->gdt = p->gate_dtype;
  out->gate = p->gate;
  const int64_t per_seq = (static_cast<int64_t>(out->T) + p->chunk - 1) / p->chunk;
  out->nchunks = out->varlen ? per_seq + p->nseq : per_seq * p->B;
  if (out->nchunks * p->H > (int64_t(1) << 31) - 1) return GDN_FAIL(GDN_ERR_SHAPE);
  out->seg = gdn::plan_segments(*out);
  out->nsegs = gdn::seg_slots_host(*out);
  if (out->nsegs * p->H * 32 > (int64_t(1) << 31) - 1) return GDN_FAIL(GDN_ERR_SHAPE);
  return GDN_OK;
}

// The backward's problem.  The gradient kernel's LDS plan for fp32 rows with
// the per-channel gate at dk = 128 does not fit a 64-token chunk; the
// gradients are those of the recurrence whatever the chunk length (only the
// order of rounding differs), so that case runs on 32-token chunks, with a
// fixed segment length kept at the same number of tokens.
gdn_status check_bwd_problem(const gdn_problem* p, gdn::Problem* out) {
  GDN_TRY(check_chunk_problem(p, out));
  if (gdn::bwd_supported(*out)) return GDN_OK;
  if (p->chunk != 64) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
  gdn_problem half = *p;
  half.chunk = 32;
  if (half.seg_chunks > 0) half.seg_chunks = half.seg_chunks > (1 << 29) ? (1 << 30) : 2 * half.seg_chunks;
  GDN_TRY(check_chunk_problem(&half, out));
  if (!gdn::bwd_supported(*out)) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
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

// Status of a launch; with GDN_LOG the resolved problem and its dispatch.
gdn_status launched(const gdn::Problem& p, hipError_t e) {
  if (log_on()) {
    fprintf(stderr,
            "gdn: %s: B=%d T=%d H=%d dk=%d dv=%d chunk=%d io=%s gate=%s/%s nseq=%d%s "
            "chunks=%lld segment_chunks=%d segments=%lld steps_per_token=%d%s%s conv_width=%d "
            "-> %s\n",
            t_entry, p.B, p.T, p.H, p.dk, p.dv, p.chunk, dtype_name(p.io), gate_name(p.gate),
            dtype_name(p.gdt), p.nseq, p.varlen ? " (varlen)" : "",
            static_cast<long long>(p.nchunks), p.seg, static_cast<long long>(p.nsegs),
            1 << p.lnh, p.qknorm ? " qk_l2norm" : "", p.beta_w ? " write_strength" : "",
            p.conv_w, hipGetErrorName(e));
  }
  return e == hipSuccess ? GDN_OK : GDN_FAIL(GDN_ERR_HIP);
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
  const int set = p.seg_req;
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
  GDN_ENTRY();
  try {
    if (total_ms == nullptr || count == nullptr) return GDN_FAIL(GDN_ERR_NULL);
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
    return GDN_FAIL(GDN_ERR_HIP);
  }
}


int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_str(int s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: size out of range or inconsistent";
    case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: unknown dtype code";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: outside the supported sizes or modes";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: pointer not 16-byte aligned";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: HIP runtime refused the launch";
    case GDN_ERR_SCRATCH:
      return "GDN_ERR_SCRATCH: problem needs more workspace than the library's static "
             "scratch buffer holds (GDN_NOALLOC_SCRATCH_BYTES)";
  }
  return "GDN_ERR_UNKNOWN";
}

void gdn_test_set_fail_launch(int enable) { g_fail_launch.store(enable != 0); }

gdn_status gdn_chunk_fwd_workspace(const gdn_problem* p, size_t* bytes) {
  GDN_ENTRY();
  try {
    if (bytes == nullptr) return GDN_FAIL(GDN_ERR_NULL);
    gdn::Problem pp;
    GDN_TRY(check_chunk_problem(p, &pp));
    *bytes = gdn::fwd_workspace_bytes(pp);
    return GDN_OK;
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

gdn_status gdn_chunk_fwd(const gdn_problem* p, const void* q, const void* k,
                         const void* v, const void* beta,
                         const void* log_alpha, const float* s0, void* o,
                         float* s_final, void* ws, size_t ws_bytes,
                         void* stream) {
  GDN_ENTRY();
  try {
    gdn::Problem pp;
    GDN_TRY(check_chunk_problem(p, &pp));
    GDN_TRY(check_fwd_pointers(pp, q, k, v, beta, log_alpha, s0, o, s_final));
    const size_t need_ws = gdn::fwd_workspace_bytes(pp);
    if (need_ws > 0 && (ws == nullptr || ws_bytes < need_ws))
      return GDN_FAIL(GDN_ERR_WORKSPACE);
    GDN_TRY(opt(ws));
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    return launched(pp, gdn::launch_fwd(pp, q, k, v, beta, log_alpha, s0, o,
                                    s_final, ws,
                                    static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

// ---------------------------------------------- forward without a workspace ---
// The workspace lives in a file-scope device array of fixed size: every GPU
// the library runs on holds its own copy until the process ends.  Host code
// never uses the array's name as an address (on the host it is only a
// stand-in for the symbol): the device address is looked up once per device
// with hipGetSymbolAddress, with that device current, and kept here.

}  // extern "C"

namespace {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on first use).
hipError_t scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_fwd_noalloc(const gdn_problem* p, const void* q, const void* k,
                                 const void* v, const void* beta,
                                 const void* log_alpha, const float* s0, void* o,
                                 float* s_final, void* stream) {
  GDN_ENTRY();
  try {
    gdn::Problem pp;
    GDN_TRY(check_chunk_problem(p, &pp));
    GDN_TRY(check_fwd_pointers(pp, q, k, v, beta, log_alpha, s0, o, s_final));
    if (gdn::fwd_workspace_bytes(pp) > GDN_NOALLOC_SCRATCH_BYTES) return GDN_FAIL(GDN_ERR_SCRATCH);
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = -1;
    if ((st != nullptr ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev)) != hipSuccess)
      return GDN_FAIL(GDN_ERR_HIP);
    void* ws = nullptr;
    if (scratch_on(dev, &ws) != hipSuccess) return GDN_FAIL(GDN_ERR_HIP);
    return launched(pp, gdn::launch_fwd(pp, q, k, v, beta, log_alpha, s0, o, s_final, ws, st));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

}  // extern "C"

namespace {

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

// Bytes of one [B * T, H, D] tensor in the problem's io dtype, 256-aligned.
size_t rows_bytes(const gdn::Problem& p, int D) {
  return al256(static_cast<size_t>(p.B) * p.T * p.H * D * (p.io == GDN_BF16 ? 2 : 4));
}

// The normalising forward: per-token gates normalise inside the forward's
// kernels; the per-channel gate takes normalised q, k rows from a prologue.
size_t qknorm_workspace_bytes(const gdn::Problem& p) {
  const size_t pro = p.gate == GDN_GATE_CHANNEL ? 2 * rows_bytes(p, p.dk) : 0;
  return pro + gdn::fwd_workspace_bytes(p);
}

// Per-token gates: the prep convolves k and v itself, q takes one prologue
// pass; the per-channel gate's prep takes all three rows processed.
size_t conv_workspace_bytes(const gdn::Problem& p) {
  const size_t pro = p.gate == GDN_GATE_CHANNEL
                         ? 2 * rows_bytes(p, p.dk) + rows_bytes(p, p.dv) : rows_bytes(p, p.dk);
  return pro + gdn::fwd_workspace_bytes(p);
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_fwd_qknorm_workspace(const gdn_problem* p, size_t* bytes) {
  GDN_ENTRY();
  try {
    if (bytes == nullptr) return GDN_FAIL(GDN_ERR_NULL);
    gdn::Problem pp;
    GDN_TRY(check_chunk_problem(p, &pp));
    *bytes = qknorm_workspace_bytes(pp);
    return GDN_OK;
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

// q and k rows L2-normalised inside the forward.
gdn_status gdn_chunk_fwd_qknorm(const gdn_problem* p, const void* q, const void* k,
                                const void* v, const void* beta,
                                const void* log_alpha, const float* s0, void* o,
                                float* s_final, void* ws, size_t ws_bytes,
                                void* stream) {
  GDN_ENTRY();
  try {
    gdn::Problem pp;
    GDN_TRY(check_chunk_problem(p, &pp));
    GDN_TRY(check_fwd_pointers(pp, q, k, v, beta, log_alpha, s0, o, s_final));
    const size_t need_ws = qknorm_workspace_bytes(pp);
    if (need_ws > 0 && (ws == nullptr || ws_bytes < need_ws))
      return GDN_FAIL(GDN_ERR_WORKSPACE);
    GDN_TRY(opt(ws));
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (pp.gate == GDN_GATE_CHANNEL) {
      char* w = static_cast<char*>(ws);
      char* qn = w;
      char* kn = w + rows_bytes(pp, pp.dk);
      char* fw = kn + rows_bytes(pp, pp.dk);
      hipError_t e = gdn::launch_prologue(pp, pp.dk, 0, q, nullptr, true, qn, st);
      if (e == hipSuccess) e = gdn::launch_prologue(pp, pp.dk, 0, k, nullptr, true, kn, st);
      if (e != hipSuccess) return GDN_FAIL(GDN_ERR_HIP);
      return launched(pp, gdn::launch_fwd(pp, qn, kn, v, beta, log_alpha, s0, o, s_final, fw, st));
    }
    pp.qknorm = true;
    return launched(pp, gdn::launch_fwd(pp, q, k, v, beta, log_alpha, s0, o, s_final, ws, st));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

gdn_status gdn_chunk_fwd_conv_workspace(const gdn_problem* p, int32_t width, size_t* bytes) {
  GDN_ENTRY();
  try {
    if (bytes == nullptr) return GDN_FAIL(GDN_ERR_NULL);
    if (width < 1 || width > 8) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
    gdn::Problem pp;
    GDN_TRY(check_chunk_problem(p, &pp));
    *bytes = conv_workspace_bytes(pp);
    return GDN_OK;
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

// Short convolution + SiLU on q, k, v (q and k then L2-normalised), then the
// forward.
gdn_status gdn_chunk_fwd_conv(const gdn_problem* p, int32_t width, const void* xq,
                              const void* xk, const void* xv, const float* wq,
                              const float* wk, const float* wv, const void* beta,
                              const void* log_alpha, const float* s0, void* o,
                              float* s_final, void* ws, size_t ws_bytes, void* stream) {
  GDN_ENTRY();
  try {
    if (width < 1 || width > 8) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
    gdn::Problem pp;
    GDN_TRY(check_chunk_problem(p, &pp));
    GDN_TRY(check_fwd_pointers(pp, xq, xk, xv, beta, log_alpha, s0, o, s_final));
    GDN_TRY(need(wq, static_cast<int64_t>(pp.H) * pp.dk * width));
    GDN_TRY(need(wk, static_cast<int64_t>(pp.H) * pp.dk * width));
    GDN_TRY(need(wv, static_cast<int64_t>(pp.H) * pp.dv * width));
    const size_t need_ws = conv_workspace_bytes(pp);
    if (ws == nullptr || ws_bytes < need_ws) return GDN_FAIL(GDN_ERR_WORKSPACE);
    GDN_TRY(opt(ws));
    if (pp.gate != GDN_GATE_CHANNEL) {  // the prep convolves k and v
      pp.conv_w = width;
      pp.conv_tk = wk;
      pp.conv_tv = wv;
    }
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* qn = static_cast<char*>(ws);
    if (pp.conv_w > 0) {
      // q through the prologue pass; k and v convolved in the prep's staging
      char* fw = qn + rows_bytes(pp, pp.dk);
      if (gdn::launch_prologue(pp, pp.dk, width, xq, wq, true, qn, st) != hipSuccess)
        return GDN_FAIL(GDN_ERR_HIP);
      return launched(pp, gdn::launch_fwd(pp, qn, xk, xv, beta, log_alpha, s0, o, s_final, fw,
                                          st));
    }
    char* kn = qn + rows_bytes(pp, pp.dk);
    char* vn = kn + rows_bytes(pp, pp.dk);
    char* fw = vn + rows_bytes(pp, pp.dv);
    hipError_t e = gdn::launch_prologue(pp, pp.dk, width, xq, wq, true, qn, st);
    if (e == hipSuccess) e = gdn::launch_prologue(pp, pp.dk, width, xk, wk, true, kn, st);
    if (e == hipSuccess) e = gdn::launch_prologue(pp, pp.dv, width, xv, wv, false, vn, st);
    if (e != hipSuccess) return GDN_FAIL(GDN_ERR_HIP);
    return launched(pp, gdn::launch_fwd(pp, qn, kn, vn, beta, log_alpha, s0, o, s_final, fw, st));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

// Draft trees: one tree per chunk, no segment split, per-token gates only.
// The prologue entry points: d is the problem's dk or dv, widths 1 .. 8;
// the normalised path needs d in {16, 32, 64, 128} (a row's lanes reduce by
// shuffles).
static gdn_status check_prologue(const gdn_problem* p, int32_t d, int32_t width,
                                 int32_t normalize, gdn::Problem* out) {
  GDN_TRY(check_chunk_problem(p, out));
  if (d != out->dk && d != out->dv) return GDN_FAIL(GDN_ERR_SHAPE);
  if (width < 1 || width > 8) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
  if (normalize && !dk_ok(d)) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
  return GDN_OK;
}

gdn_status gdn_prologue_fwd(const gdn_problem* p, int32_t d, int32_t width, int32_t normalize,
                            const void* x, const float* taps, void* y, void* stream) {
  GDN_ENTRY();
  try {
    gdn::Problem pp;
    GDN_TRY(check_prologue(p, d, width, normalize, &pp));
    const int64_t rows = static_cast<int64_t>(pp.B) * pp.T * pp.H;
    GDN_TRY(need(x, rows * d));
    GDN_TRY(need(y, rows * d));
    GDN_TRY(need(taps, static_cast<int64_t>(pp.H) * d * width));
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    return launched(pp, gdn::launch_prologue(pp, d, width, x, taps, normalize != 0, y,
                                             static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

gdn_status gdn_prologue_bwd_workspace(const gdn_problem* p, int32_t d, int32_t width,
                                      size_t* bytes) {
  GDN_ENTRY();
  try {
    if (bytes == nullptr) return GDN_FAIL(GDN_ERR_NULL);
    gdn::Problem pp;
    GDN_TRY(check_prologue(p, d, width, 0, &pp));
    *bytes = gdn::prologue_bwd_workspace_bytes(pp, d, width);
    return GDN_OK;
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

gdn_status gdn_prologue_bwd(const gdn_problem* p, int32_t d, int32_t width, int32_t normalize,
                            const void* x, const float* taps, const void* dy, void* dx,
                            float* dtaps, void* ws, size_t ws_bytes, void* stream) {
  GDN_ENTRY();
  try {
    gdn::Problem pp;
    GDN_TRY(check_prologue(p, d, width, normalize, &pp));
    const int64_t rows = static_cast<int64_t>(pp.B) * pp.T * pp.H;
    GDN_TRY(need(x, rows * d));
    GDN_TRY(need(dy, rows * d));
    GDN_TRY(need(dx, rows * d));
    GDN_TRY(need(taps, static_cast<int64_t>(pp.H) * d * width));
    if (dtaps == nullptr) return GDN_FAIL(GDN_ERR_NULL);
    GDN_TRY(opt(dtaps));
    const size_t need_ws = gdn::prologue_bwd_workspace_bytes(pp, d, width);
    if (ws == nullptr || ws_bytes < need_ws) return GDN_FAIL(GDN_ERR_WORKSPACE);
    GDN_TRY(opt(ws));
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    return launched(pp, gdn::launch_prologue_bwd(pp, d, width, x, taps, normalize != 0, dy, dx,
                                                 dtaps, ws, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

static gdn_status check_tree(const gdn_problem* p, gdn::Problem* out) {
  if (p == nullptr) return GDN_FAIL(GDN_ERR_NULL);
  if (p->gate == GDN_GATE_CHANNEL) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
  GDN_TRY(check_chunk_problem(p, out));
  if (!out->varlen && p->T > p->chunk) return GDN_FAIL(GDN_ERR_SHAPE);
  out->seg = 0;
  out->nsegs = out->nseq;
  return GDN_OK;
}

gdn_status gdn_tree_verify_workspace(const gdn_problem* p, size_t* bytes) {
  GDN_ENTRY();
  try {
    if (bytes == nullptr) return GDN_FAIL(GDN_ERR_NULL);
    gdn::Problem pp;
    GDN_TRY(check_tree(p, &pp));
    *bytes = gdn::fwd_workspace_bytes(pp);
    return GDN_OK;
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

gdn_status gdn_tree_verify(const gdn_problem* p, const int32_t* parent, const void* q,
                           const void* k, const void* v, const void* beta,
                           const void* log_alpha, const float* state, void* o,
                           void* ws, size_t ws_bytes, void* stream) {
  GDN_ENTRY();
  try {
    gdn::Problem pp;
    GDN_TRY(check_tree(p, &pp));
    GDN_TRY(check_fwd_pointers(pp, q, k, v, beta, log_alpha, state, o, nullptr));
    GDN_TRY(need(parent, static_cast<int64_t>(pp.B) * pp.T));
    if ((reinterpret_cast<uintptr_t>(parent) & 3u) != 0) return GDN_FAIL(GDN_ERR_ALIGN);
    const size_t need_ws = gdn::fwd_workspace_bytes(pp);
    if (need_ws > 0 && (ws == nullptr || ws_bytes < need_ws))
      return GDN_FAIL(GDN_ERR_WORKSPACE);
    GDN_TRY(opt(ws));
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    pp.parent = parent;
    return launched(pp, gdn::launch_fwd(pp, q, k, v, beta, log_alpha, state, o, nullptr, ws,
                                    static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

gdn_status gdn_tree_commit(const gdn_problem* p, const int32_t* parent,
                           const int32_t* accepted, const void* k, const void* v,
                           const void* beta, const void* log_alpha, float* state,
                           void* stream) {
  GDN_ENTRY();
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
      return GDN_FAIL(GDN_ERR_ALIGN);
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    return launched(pp, gdn::launch_tree_commit(pp, parent, accepted, k, v, beta, log_alpha,
                                            state, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

// Householder-product transitions: nh in {1, 2, 4} delta steps per token,
// per-token gates only.
static gdn_status check_product(const gdn_problem* p, int32_t nh, gdn::Problem* out) {
  if (p == nullptr) return GDN_FAIL(GDN_ERR_NULL);
  if (nh != 1 && nh != 2 && nh != 4) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
  if (p->gate == GDN_GATE_CHANNEL) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
  return check_chunk_problem(p, out, nh == 1 ? 0 : (nh == 2 ? 1 : 2));
}

gdn_status gdn_chunk_fwd_product_workspace(const gdn_problem* p, int32_t nh,
                                           size_t* bytes) {
  GDN_ENTRY();
  try {
    if (bytes == nullptr) return GDN_FAIL(GDN_ERR_NULL);
    gdn::Problem pp;
    GDN_TRY(check_product(p, nh, &pp));
    *bytes = gdn::fwd_workspace_bytes(pp);
    return GDN_OK;
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

gdn_status gdn_chunk_fwd_product(const gdn_problem* p, int32_t nh, const void* q,
                                 const void* k, const void* v, const void* beta,
                                 const void* log_alpha, const float* s0, void* o,
                                 float* s_final, void* ws, size_t ws_bytes,
                                 void* stream) {
  GDN_ENTRY();
  try {
    gdn::Problem pp;
    GDN_TRY(check_product(p, nh, &pp));
    GDN_TRY(check_fwd_pointers(pp, q, k, v, beta, log_alpha, s0, o, s_final));
    const size_t need_ws = gdn::fwd_workspace_bytes(pp);
    if (need_ws > 0 && (ws == nullptr || ws_bytes < need_ws))
      return GDN_FAIL(GDN_ERR_WORKSPACE);
    GDN_TRY(opt(ws));
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    return launched(pp, gdn::launch_fwd(pp, q, k, v, beta, log_alpha, s0, o,
                                    s_final, ws,
                                    static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

gdn_status gdn_chunk_bwd_workspace(const gdn_problem* p, size_t* bytes) {
  GDN_ENTRY();
  try {
    if (bytes == nullptr) return GDN_FAIL(GDN_ERR_NULL);
    gdn::Problem pp;
    GDN_TRY(check_bwd_problem(p, &pp));
    *bytes = gdn::bwd_workspace_bytes(pp);
    return GDN_OK;
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

gdn_status gdn_chunk_bwd(const gdn_problem* p, const void* q, const void* k,
                         const void* v, const void* beta,
                         const void* log_alpha, const float* s0,
                         const void* d_o, const float* ds_final, void* dq,
                         void* dk, void* dv, float* dbeta, float* dlog_alpha,
                         float* ds0, void* ws, size_t ws_bytes, void* stream) {
  GDN_ENTRY();
  try {
    gdn::Problem pp;
    GDN_TRY(check_bwd_problem(p, &pp));
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
      return GDN_FAIL(GDN_ERR_WORKSPACE);
    GDN_TRY(opt(ws));
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    return launched(pp, gdn::launch_bwd(pp, q, k, v, beta, log_alpha, s0, d_o,
                                    ds_final, dq, dk, dv, dbeta, dlog_alpha,
                                    ds0, ws, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

}  // extern "C"

namespace {

// Shared validation of the decode entry points; fills *pp.
gdn_status check_decode(const gdn_problem* p, const void* q, const void* k, const void* v,
                        const void* beta, const void* log_alpha, const float* state,
                        const void* o, gdn::Problem* pp) {
  if (p == nullptr) return GDN_FAIL(GDN_ERR_NULL);
  if (!dtype_ok(p->io_dtype) || !dtype_ok(p->gate_dtype)) return GDN_FAIL(GDN_ERR_DTYPE);
  if (p->gate < GDN_GATE_NONE || p->gate > GDN_GATE_CHANNEL)
    return GDN_FAIL(GDN_ERR_UNSUPPORTED);
  if (p->B < 1 || p->H < 1) return GDN_FAIL(GDN_ERR_SHAPE);
  if (!dk_ok(p->dk) || !dv_ok(p->dv)) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
  // one workgroup per (sequence, head, 64-column slab): within the grid limit
  if (static_cast<int64_t>(p->B) * p->H * ((p->dv + 63) / 64) > (int64_t(1) << 31) - 1)
    return GDN_FAIL(GDN_ERR_SHAPE);
  *pp = gdn::Problem{};
  pp->B = p->B;
  pp->T = 1;
  pp->H = p->H;
  pp->dk = p->dk;
  pp->dv = p->dv;
  pp->nseq = p->B;
  pp->io = p->io_dtype;
  pp->gdt = p->gate_dtype;
  pp->gate = p->gate;
  const int64_t nh = static_cast<int64_t>(p->B) * p->H;
  GDN_TRY(need(q, nh * p->dk));
  GDN_TRY(need(k, nh * p->dk));
  GDN_TRY(need(v, nh * p->dv));
  GDN_TRY(need(beta, nh));
  if (pp->gate != GDN_GATE_NONE) GDN_TRY(need(log_alpha, nh));
  else GDN_TRY(opt(log_alpha));
  GDN_TRY(need(state, nh * p->dk * p->dv));
  GDN_TRY(need(o, nh * p->dv));
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_decode_step(const gdn_problem* p, const void* q, const void* k,
                           const void* v, const void* beta,
                           const void* log_alpha, float* state, void* o,
                           void* stream) {
  GDN_ENTRY();
  try {
    gdn::Problem pp;
    GDN_TRY(check_decode(p, q, k, v, beta, log_alpha, state, o, &pp));
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    return launched(pp, gdn::launch_decode(pp, q, k, v, beta, log_alpha, state, o,
                                       static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

// Gated DeltaNet-2: separate erase and write strengths.
gdn_status gdn2_chunk_fwd(const gdn_problem* p, const void* q, const void* k,
                          const void* v, const void* erase, const void* write,
                          const void* log_alpha, const float* s0, void* o,
                          float* s_final, void* ws, size_t ws_bytes, void* stream) {
  GDN_ENTRY();
  try {
    gdn::Problem pp;
    GDN_TRY(check_chunk_problem(p, &pp));
    GDN_TRY(check_fwd_pointers(pp, q, k, v, erase, log_alpha, s0, o, s_final));
    GDN_TRY(need(write, static_cast<int64_t>(pp.B) * pp.T * pp.H));
    const size_t need_ws = gdn::fwd_workspace_bytes(pp);
    if (need_ws > 0 && (ws == nullptr || ws_bytes < need_ws))
      return GDN_FAIL(GDN_ERR_WORKSPACE);
    GDN_TRY(opt(ws));
    pp.beta_w = write;
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    return launched(pp, gdn::launch_fwd(pp, q, k, v, erase, log_alpha, s0, o, s_final, ws,
                                    static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

gdn_status gdn2_decode_step(const gdn_problem* p, const void* q, const void* k,
                            const void* v, const void* erase, const void* write,
                            const void* log_alpha, float* state, void* o, void* stream) {
  GDN_ENTRY();
  try {
    gdn::Problem pp;
    GDN_TRY(check_decode(p, q, k, v, erase, log_alpha, state, o, &pp));
    GDN_TRY(need(write, static_cast<int64_t>(pp.B) * pp.H));
    pp.beta_w = write;
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    return launched(pp, gdn::launch_decode(pp, q, k, v, erase, log_alpha, state, o,
                                       static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

gdn_status gdn_decode_step_product(const gdn_problem* p, int32_t nh, const void* q,
                                   const void* k, const void* v, const void* beta,
                                   const void* log_alpha, float* state, void* o,
                                   void* stream) {
  GDN_ENTRY();
  try {
    if (p == nullptr) return GDN_FAIL(GDN_ERR_NULL);
    if (!dtype_ok(p->io_dtype) || !dtype_ok(p->gate_dtype)) return GDN_FAIL(GDN_ERR_DTYPE);
    if (p->gate != GDN_GATE_NONE && p->gate != GDN_GATE_SCALAR) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
    if (nh != 1 && nh != 2 && nh != 4) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
    if (p->B < 1 || p->H < 1) return GDN_FAIL(GDN_ERR_SHAPE);
    if (!dk_ok(p->dk) || !dv_ok(p->dv)) return GDN_FAIL(GDN_ERR_UNSUPPORTED);
    if (static_cast<int64_t>(p->B) * p->H * ((p->dv + 63) / 64) > (int64_t(1) << 31) - 1)
      return GDN_FAIL(GDN_ERR_SHAPE);
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
    if (g_fail_launch.load()) return launched(pp, hipErrorLaunchFailure);  // test hook
    return launched(pp, gdn::launch_decode_product(pp, nh, q, k, v, beta, log_alpha, state, o,
                                               static_cast<hipStream_t>(stream)));
  } catch (...) {
    return GDN_FAIL(GDN_ERR_HIP);
  }
}

}  // extern "C"
