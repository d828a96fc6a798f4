// Host runtime behind the C ABI in include/fwpkm.h: configuration and
// argument validation, aliasing rules, the device workspace and the launch
// sequence of one chunk on the caller's stream.

#include "fwpkm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Byte sizes of the workspace regions for `units` units of `tokens` tokens.
struct WsLayout {
  size_t half_o, half_i, qnorm, sel_w, g, keys, coef, ent_row, ent_tw, kinds, check;
  size_t addr_s, addr_dk, addr_tok, addr_ell, total;
};

WsLayout ws_layout(const fwpkm_config& c, int64_t units, int64_t tokens) {
  const int64_t nblk = (c.sqrt_slots + fwpkm::kKeyBlock - 1) / fwpkm::kKeyBlock;
  const int64_t P = tokens * c.topk;
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes); return at; };
  L.half_o = take(sizeof(float) * units * tokens * 2 * nblk * c.topk);
  L.half_i = take(sizeof(int) * units * tokens * 2 * nblk * c.topk);
  L.qnorm = take(sizeof(float) * units * tokens * 2);
  L.sel_w = take(sizeof(float) * units * P);
  L.g = take(sizeof(float) * units * tokens * c.dim_v);
  L.keys = take(sizeof(int) * 3 * units * P);
  L.coef = take(sizeof(float) * 2 * units * P);
  L.ent_row = take(sizeof(int) * 3 * units * P);
  L.ent_tw = take(sizeof(int2) * 3 * units * P);
  // regions per list shrink as units grow: 3 * units * regions <= max(256, 3 * units)
  L.kinds = take(sizeof(int4) * std::max<int64_t>(256, 3 * units));
  L.check = take(sizeof(unsigned int));     // device-check word (checked builds)
  // addressing loss (only with addr_weight != 0): every token's score over
  // every sub-key (then its dL/ds coefficient), and the key gradient
  const bool addr = c.addr_weight != 0.0f;
  const int64_t n = c.sqrt_slots, half = c.dim_qk / 2;
  const int64_t np = (n + fwpkm::kAddrPad - 1) / fwpkm::kAddrPad * fwpkm::kAddrPad;
  L.addr_s = take(addr ? sizeof(float) * units * 2 * tokens * np : 0);
  L.addr_dk = take(addr ? sizeof(float) * units * 2 * n * half : 0);
  L.addr_tok = take(addr ? sizeof(float) * units * 2 * tokens * 2 : 0);
  L.addr_ell = take(addr ? sizeof(float) * units * 2 * n : 0);
  L.total = off;
  return L;
}

// Byte offsets of the sequence call's caller-provided workspace.
struct SeqLayout {
  size_t q, y, tw, total;
};

SeqLayout seq_layout(const fwpkm_config& c, int64_t batch, int64_t seq) {
  SeqLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes); return at; };
  const int64_t H = c.num_heads;
  L.q = take(sizeof(float) * batch * seq * H * c.dim_qk);     // chunk-major queries
  L.y = take(sizeof(float) * batch * seq * H * c.dim_v);      // chunk-major lookahead targets
  L.tw = take(sizeof(float) * batch * std::min<int64_t>(seq, c.chunk_size) * H);   // last chunk's weights
  L.total = off;
  return L;
}

int check_config(const fwpkm_config* c) {
  if (!c) return fail(FWPKM_ERR_INVALID_ARG, "config is NULL");
  if (c->sqrt_slots < 1) return fail(FWPKM_ERR_INVALID_ARG, "sqrt_slots must be >= 1 (got %d)", c->sqrt_slots);
  if (c->dim_qk < 2 || (c->dim_qk & 1)) return fail(FWPKM_ERR_INVALID_ARG, "dim_qk must be even and >= 2 (got %d)", c->dim_qk);
  if (c->dim_v < 1) return fail(FWPKM_ERR_INVALID_ARG, "dim_v must be >= 1 (got %d)", c->dim_v);
  const int64_t N = (int64_t)c->sqrt_slots * c->sqrt_slots;
  if (c->topk < 1 || c->topk > c->sqrt_slots || c->topk > N)
    return fail(FWPKM_ERR_INVALID_ARG, "topk must lie in [1, sqrt_slots] (got %d)", c->topk);
  if (c->chunk_size < 1) return fail(FWPKM_ERR_INVALID_ARG, "chunk_size must be >= 1 (got %d)", c->chunk_size);
  if (c->num_heads < 1) return fail(FWPKM_ERR_INVALID_ARG, "num_heads must be >= 1 (got %d)", c->num_heads);
  if (c->max_batch < 1) return fail(FWPKM_ERR_INVALID_ARG, "max_batch must be >= 1 (got %d)", c->max_batch);
  if (!std::isfinite(c->eps) || !(c->eps > 0.f)) return fail(FWPKM_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (c->score_mode != FWPKM_SCORE_IDW && c->score_mode != FWPKM_SCORE_DOT)
    return fail(FWPKM_ERR_INVALID_ARG, "unknown score_mode %d", c->score_mode);
  if (!std::isfinite(c->addr_weight)) return fail(FWPKM_ERR_INVALID_ARG, "addr_weight must be finite");
  // kernel limits
  const int half = c->dim_qk / 2;
  if (c->sqrt_slots > FWPKM_MAX_SQRT_SLOTS) return fail(FWPKM_ERR_UNSUPPORTED, "sqrt_slots > %d", FWPKM_MAX_SQRT_SLOTS);
  if (half % 4 != 0 || half > FWPKM_MAX_HALF) return fail(FWPKM_ERR_UNSUPPORTED, "dim_qk/2 must be a multiple of 4 and <= %d", FWPKM_MAX_HALF);
  if (c->dim_v % 4 != 0 || c->dim_v > FWPKM_MAX_DIM_V) return fail(FWPKM_ERR_UNSUPPORTED, "dim_v must be a multiple of 4 and <= %d", FWPKM_MAX_DIM_V);
  if (c->topk > FWPKM_MAX_TOPK) return fail(FWPKM_ERR_UNSUPPORTED, "topk > %d", FWPKM_MAX_TOPK);
  if (c->chunk_size > FWPKM_MAX_CHUNK) return fail(FWPKM_ERR_UNSUPPORTED, "chunk_size > %d", FWPKM_MAX_CHUNK);
  if ((int64_t)c->chunk_size * c->topk > fwpkm::kSortMaxPairs)
    return fail(FWPKM_ERR_UNSUPPORTED, "chunk_size * topk > %d", fwpkm::kSortMaxPairs);
  const int64_t units = (int64_t)c->max_batch * c->num_heads;
  if (3 * units > fwpkm::kUpdMaxLists)
    return fail(FWPKM_ERR_UNSUPPORTED, "max_batch * num_heads > %d", fwpkm::kUpdMaxLists / 3);
  return FWPKM_OK;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range table_range(const float* p, int64_t stride, int64_t size, int batch) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  const int64_t extent = (int64_t)(batch - 1) * stride + size;
  return {lo, lo + (uintptr_t)extent * sizeof(float)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

}  // namespace

// The workspace of fwpkm_forward_chunk_noalloc: a fixed array in the code
// object's zero-initialised device data, so each GPU the library runs on
// holds one copy from load until the process ends and no call allocates.
// On the host the name is a stand-in, not a device address: host code uses
// only the address hipGetSymbolAddress reports for the current device.
static __device__ __align__(256) unsigned char scratch[FWPKM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch[kMaxDevices] = {};   // device address of `scratch`, per device

// Device address of `scratch` on device `dev` (the current device), looked
// up once per device.
int scratch_of_device(int dev, char** out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FWPKM_ERR_UNSUPPORTED, "device %d: the fixed workspace serves devices 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(FWPKM_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    }
    g_scratch[dev] = static_cast<char*>(p);
  }
  *out = g_scratch[dev];
  return FWPKM_OK;
}

}  // namespace

struct fwpkm_handle {
  fwpkm_config cfg;
  int device = -1;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  // per-kernel timing
  struct Mark { hipEvent_t beg, end; int kernel; };
  bool prof = false;
  std::vector<Mark> marks;             // recorded, not yet read
  std::vector<hipEvent_t> spare;       // reusable events
  double ms[FWPKM_NUM_TIMED] = {};
  int64_t launches[FWPKM_NUM_TIMED] = {};
};

namespace {

hipEvent_t take_event(fwpkm_handle* h) {
  if (!h->spare.empty()) {
    hipEvent_t e = h->spare.back();
    h->spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Run `fn(timing)`: with profiling on, `timing` carries a start/stop event
// pair that the launch stamps (kernels: from the dispatch itself).
template <typename F>
hipError_t timed(fwpkm_handle* h, bool on, int kernel, F&& fn) {
  if (!on) return fn(nullptr);
  fwpkm::LaunchTiming tm;
  tm.beg = take_event(h);
  tm.end = take_event(h);
  if (!tm.beg || !tm.end) return hipErrorOutOfMemory;
  hipError_t r = fn(&tm);
  if (r != hipSuccess) return r;
  h->marks.push_back({tm.beg, tm.end, kernel});
  return hipSuccess;
}

const char* const kKernelNames[FWPKM_NUM_TIMED] = {"score", "read", "sort", "update", "copy",
                                                   "addr_stats", "addr_grad", "addr_apply",
                                                   "project", "gate"};

}  // namespace

extern "C" {

const char* fwpkm_last_error(void) { return g_err; }

size_t fwpkm_workspace_bytes(const fwpkm_config* cfg) {
  if (check_config(cfg) != FWPKM_OK) return 0;
  return ws_layout(*cfg, (int64_t)cfg->max_batch * cfg->num_heads, cfg->chunk_size).total;
}

int fwpkm_create(const fwpkm_config* cfg, fwpkm_handle** out) {
  if (!out) return fail(FWPKM_ERR_INVALID_ARG, "out is NULL");
  const int rc = check_config(cfg);
  if (rc != FWPKM_OK) return rc;
  fwpkm_handle* h = new (std::nothrow) fwpkm_handle();
  if (!h) return fail(FWPKM_ERR_OOM, "cannot allocate the handle");
  h->cfg = *cfg;
  h->ws_bytes = ws_layout(*cfg, (int64_t)cfg->max_batch * cfg->num_heads, cfg->chunk_size).total;
  *out = h;
  g_err[0] = '\0';
  return FWPKM_OK;
}

// validation and enqueue shared by both chunk entry points (below)
static int forward_impl(fwpkm_handle* h, const float* queries, const float* targets,
                        const float* token_weights, int32_t batch, int32_t tokens, float lr,
                        const fwpkm_state* past, const fwpkm_state* next,
                        float* retrieved, int32_t* out_slots, float* out_weights,
                        int64_t out_rows_b, hipStream_t stream, bool dry_run = false,
                        bool noalloc = false);

int fwpkm_forward_chunk(fwpkm_handle* h, const float* queries, const float* targets,
                        int32_t batch, int32_t tokens, float lr,
                        const fwpkm_state* past, const fwpkm_state* next,
                        float* retrieved, int32_t* out_slots, float* out_weights,
                        hipStream_t stream) {
  return forward_impl(h, queries, targets, nullptr, batch, tokens, lr, past, next, retrieved,
                      out_slots, out_weights, 0, stream);
}

int fwpkm_forward_chunk_weighted(fwpkm_handle* h, const float* queries, const float* targets,
                                 const float* token_weights, int32_t batch, int32_t tokens,
                                 float lr, const fwpkm_state* past, const fwpkm_state* next,
                                 float* retrieved, int32_t* out_slots, float* out_weights,
                                 hipStream_t stream) {
  return forward_impl(h, queries, targets, token_weights, batch, tokens, lr, past, next, retrieved,
                      out_slots, out_weights, 0, stream);
}

int fwpkm_forward_chunk_noalloc(fwpkm_handle* h, const float* queries, const float* targets,
                                int32_t batch, int32_t tokens, float lr,
                                const fwpkm_state* past, const fwpkm_state* next,
                                float* retrieved, int32_t* out_slots, float* out_weights,
                                hipStream_t stream) {
  return forward_impl(h, queries, targets, nullptr, batch, tokens, lr, past, next, retrieved,
                      out_slots, out_weights, 0, stream, /*dry_run=*/false, /*noalloc=*/true);
}

size_t fwpkm_sequence_workspace_bytes(const fwpkm_config* cfg, int32_t batch, int32_t seq) {
  if (check_config(cfg) != FWPKM_OK) return 0;
  if (batch < 1 || seq < 1) {
    fail(FWPKM_ERR_INVALID_ARG, "batch and seq must be >= 1 (got %d, %d)", batch, seq);
    return 0;
  }
  return seq_layout(*cfg, batch, seq).total;
}

int fwpkm_forward_sequence(fwpkm_handle* h, const float* x, const float* w_in,
                           const float* w_gate, const float* b_gate, int32_t batch, int32_t seq,
                           float lr, const fwpkm_state* past, const fwpkm_state* next, float* out,
                           int32_t* out_slots, float* out_weights, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  // ---------------------------------------------------------- validation
  if (!h) return fail(FWPKM_ERR_INVALID_ARG, "handle is NULL");
  const fwpkm_config& c = h->cfg;
  if (!x || !w_in || !w_gate || !out) return fail(FWPKM_ERR_INVALID_ARG, "x, w_in, w_gate and out must be non-NULL");
  if (!workspace) return fail(FWPKM_ERR_INVALID_ARG, "workspace is NULL");
  if (!past || !next) return fail(FWPKM_ERR_INVALID_ARG, "past_state and next_state must be non-NULL");
  if (batch < 1 || batch > c.max_batch) return fail(FWPKM_ERR_INVALID_ARG, "batch %d outside [1, %d]", batch, c.max_batch);
  if (seq < 1) return fail(FWPKM_ERR_INVALID_ARG, "seq must be >= 1 (got %d)", seq);
  const int H = c.num_heads, C = c.chunk_size, k = c.topk;
  const int64_t D = (int64_t)H * c.dim_v, M = (int64_t)batch * seq;
  const int64_t Nrows = (int64_t)H * (c.dim_qk + c.dim_v);
  if (M > ((int64_t)1 << 30))
    return fail(FWPKM_ERR_UNSUPPORTED, "batch * seq = %lld tokens is more than 2^30", (long long)M);
  const SeqLayout L = seq_layout(c, batch, seq);
  if (workspace_bytes < L.total)
    return fail(FWPKM_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);

  char* ws = static_cast<char*>(workspace);
  float* q_all = reinterpret_cast<float*>(ws + L.q);
  float* y_all = reinterpret_cast<float*>(ws + L.y);
  float* tw_last = reinterpret_cast<float*>(ws + L.tw);
  auto rng = [](const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, p ? a + (uintptr_t)bytes : a};
  };
  const Range rx = rng(x, 4 * M * D), rwi = rng(w_in, 4 * Nrows * D), rwg = rng(w_gate, 4 * (int64_t)H * D);
  const Range rbg = rng(b_gate, 4 * (int64_t)H), rout = rng(out, 4 * M * D), rws = rng(workspace, (int64_t)L.total);
  const Range rsl = rng(out_slots, 4 * M * H * k), rwt = rng(out_weights, 4 * M * H * k);
  const int n = c.sqrt_slots, half = c.dim_qk / 2;
  const int64_t sk = (int64_t)H * n * half, sv = (int64_t)H * n * n * c.dim_v;
  const Range tables[6] = {table_range(past->k1, past->batch_stride_k, sk, batch),
                           table_range(past->k2, past->batch_stride_k, sk, batch),
                           table_range(past->v, past->batch_stride_v, sv, batch),
                           table_range(next->k1, next->batch_stride_k, sk, batch),
                           table_range(next->k2, next->batch_stride_k, sk, batch),
                           table_range(next->v, next->batch_stride_v, sv, batch)};
  // everything the call writes (out, the selections, the workspace, next_state)
  // must stay clear of what it reads afterwards (x, the weights, the state)
  for (const Range& a : {rx, rwi, rwg, rbg}) {
    if (a.lo == a.hi) continue;
    for (const Range& b : {rout, rws, rsl, rwt, tables[3], tables[4], tables[5]})
      if (b.lo != b.hi && overlap(a, b)) return fail(FWPKM_ERR_ALIAS, "an output or the workspace overlaps x or a weight");
  }
  for (const Range& b : {rout, rsl, rwt}) {
    if (b.lo == b.hi) continue;
    if (overlap(b, rws)) return fail(FWPKM_ERR_ALIAS, "an output overlaps the workspace");
  }
  for (const Range& t : tables)
    if (overlap(t, rws)) return fail(FWPKM_ERR_ALIAS, "the workspace overlaps a state table");

  const int nchunks = (seq + C - 1) / C;
  auto chunk_call = [&](int ci, bool dry) {
    const int c0 = ci * C, cc = std::min(C, seq - c0);
    const int64_t rows0 = (int64_t)batch * c0 * H;     // rows of the chunks before this one
    return forward_impl(h, q_all + rows0 * c.dim_qk, y_all + rows0 * c.dim_v,
                        ci == nchunks - 1 ? tw_last : nullptr, batch, cc, lr,
                        ci == 0 ? past : next, next, out + (int64_t)c0 * D,
                        out_slots ? out_slots + (int64_t)c0 * H * k : nullptr,
                        out_weights ? out_weights + (int64_t)c0 * H * k : nullptr,
                        (int64_t)seq * H, stream, dry);
  };
  // the first and the last chunk calls cover every pointer and size the loop uses
  int rc = chunk_call(0, true);
  if (rc == FWPKM_OK && nchunks > 1) rc = chunk_call(nchunks - 1, true);
  if (rc != FWPKM_OK) return rc;

  // ---------------------------------------------------------- enqueue
  fwpkm::SeqArgs sa{};
  sa.x = x;
  sa.w_in = w_in;
  sa.w_gate = w_gate;
  sa.b_gate = b_gate;
  sa.q_all = q_all;
  sa.y_all = y_all;
  sa.tw_last = tw_last;
  sa.out = out;
  sa.B = batch;
  sa.S = seq;
  sa.D = (int)D;
  sa.H = H;
  sa.dqk = c.dim_qk;
  sa.dv = c.dim_v;
  sa.C = C;
  sa.Nq = H * c.dim_qk;
  sa.Nv = H * c.dim_v;
  using fwpkm::LaunchTiming;
  hipError_t e = timed(h, h->prof, 8, [&](const LaunchTiming* tm) { return fwpkm::launch_kf_project(sa, stream, tm); });
  if (e != hipSuccess) return fail(FWPKM_ERR_HIP, "projection kernel: %s", hipGetErrorString(e));
  for (int ci = 0; ci < nchunks; ++ci)
    if ((rc = chunk_call(ci, false)) != FWPKM_OK) return rc;
  e = timed(h, h->prof, 9, [&](const LaunchTiming* tm) { return fwpkm::launch_kf_gate(sa, stream, tm); });
  if (e != hipSuccess) return fail(FWPKM_ERR_HIP, "gate kernel: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return FWPKM_OK;
}

void fwpkm_destroy(fwpkm_handle* h) {
  if (!h) return;
  if (h->ws) {
    int prev = -1;
    if (hipGetDevice(&prev) == hipSuccess && prev != h->device) (void)hipSetDevice(h->device);
    (void)hipDeviceSynchronize();
    for (auto& m : h->marks) { (void)hipEventDestroy(m.beg); (void)hipEventDestroy(m.end); }
    for (auto e : h->spare) (void)hipEventDestroy(e);
    (void)hipFree(h->ws);
    if (prev >= 0 && prev != h->device) (void)hipSetDevice(prev);
  }
  delete h;
}

int32_t fwpkm_checked_build(void) { return FWPKM_DEVICE_CHECKS ? 1 : 0; }

const char* fwpkm_kernel_name(int32_t i) {
  return (i >= 0 && i < FWPKM_NUM_TIMED) ? kKernelNames[i] : "";
}

int fwpkm_profile_enable(fwpkm_handle* h, int32_t enable) {
  if (!h) return fail(FWPKM_ERR_INVALID_ARG, "handle is NULL");
  if (enable) {
    for (auto& m : h->marks) { h->spare.push_back(m.beg); h->spare.push_back(m.end); }
    h->marks.clear();
    for (int i = 0; i < FWPKM_NUM_TIMED; ++i) { h->ms[i] = 0.0; h->launches[i] = 0; }
  }
  h->prof = enable != 0;
  return FWPKM_OK;
}

int fwpkm_profile_read(fwpkm_handle* h, double* ms, int64_t* launches) {
  if (!h) return fail(FWPKM_ERR_INVALID_ARG, "handle is NULL");
  for (auto& m : h->marks) {
    hipError_t e = hipEventSynchronize(m.end);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, m.beg, m.end);
    if (e != hipSuccess) return fail(FWPKM_ERR_HIP, "timing events: %s", hipGetErrorString(e));
    h->ms[m.kernel] += t;
    h->launches[m.kernel] += 1;
    h->spare.push_back(m.beg);
    h->spare.push_back(m.end);
  }
  h->marks.clear();
  for (int i = 0; i < FWPKM_NUM_TIMED; ++i) {
    if (ms) ms[i] = h->ms[i];
    if (launches) launches[i] = h->launches[i];
  }
  return FWPKM_OK;
}

// out_rows_b: (token, head) rows between sequences in retrieved, out_slots
// and out_weights (0: tokens * H, the packed layout of a chunk call).
// dry_run: validate only, enqueue nothing.
// noalloc: use the fixed array `scratch` as the workspace (never the
// handle's, which is then neither allocated nor touched) and record no
// timing events.
#if FWPKM_DEVICE_CHECKS
// Checked builds: wait for the call's kernels and report the invariants they
// found broken (the word is cleared before the first kernel of every call).
static int read_device_checks(const unsigned int* word, hipStream_t stream) {
  static const char* const names[fwpkm::kNumDeviceChecks] = {
      "per-half sub-key index >= n", "fewer than k candidates", "selected slot outside [0, N)",
      "a slot selected twice", "selection weight not finite or outside [0, 1]",
      "grouped entry row or token out of range, or not its pair's row", "update batch over its LDS capacity",
      "grouped entries out of row order"};
  unsigned int bits = 0;
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemcpy(&bits, word, sizeof(bits), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(FWPKM_ERR_HIP, "reading the device-check word: %s", hipGetErrorString(e));
  if (bits == 0) {
    g_err[0] = '\0';
    return FWPKM_OK;
  }
  char msg[512];
  size_t at = 0;
  msg[0] = '\0';
  for (int i = 0; i < fwpkm::kNumDeviceChecks; ++i) {
    if (!(bits & (1u << i))) continue;
    const int w = snprintf(msg + at, sizeof(msg) - at, "%s%s", at ? "; " : "", names[i]);
    if (w < 0 || (size_t)w >= sizeof(msg) - at) break;
    at += (size_t)w;
  }
  return fail(FWPKM_ERR_DEVICE_CHECK, "device check failed (bits 0x%x): %s", bits, msg);
}
#endif

static int forward_impl(fwpkm_handle* h, const float* queries, const float* targets,
                        const float* token_weights, int32_t batch, int32_t tokens, float lr,
                        const fwpkm_state* past, const fwpkm_state* next,
                        float* retrieved, int32_t* out_slots, float* out_weights,
                        int64_t out_rows_b, hipStream_t stream, bool dry_run,
                        bool noalloc) {
  // ---------------------------------------------------------- validation
  if (!h) return fail(FWPKM_ERR_INVALID_ARG, "handle is NULL");
  const fwpkm_config& c = h->cfg;
  if (!queries || !targets || !retrieved) return fail(FWPKM_ERR_INVALID_ARG, "queries, targets and retrieved must be non-NULL");
  if (!past || !next) return fail(FWPKM_ERR_INVALID_ARG, "past_state and next_state must be non-NULL");
  if (!past->k1 || !past->k2 || !past->v || !next->k1 || !next->k2 || !next->v)
    return fail(FWPKM_ERR_INVALID_ARG, "state table pointers must be non-NULL");
  if (batch < 1 || batch > c.max_batch) return fail(FWPKM_ERR_INVALID_ARG, "batch %d outside [1, %d]", batch, c.max_batch);
  if (tokens < 1 || tokens > c.chunk_size) return fail(FWPKM_ERR_INVALID_ARG, "tokens %d outside [1, %d]", tokens, c.chunk_size);
  if (!std::isfinite(lr)) return fail(FWPKM_ERR_INVALID_ARG, "lr must be finite");

  const int n = c.sqrt_slots, half = c.dim_qk / 2, H = c.num_heads, k = c.topk;
  const int64_t N = (int64_t)n * n;
  const int64_t sk = (int64_t)H * n * half;        // elements of one sequence's K1 (or K2)
  const int64_t sv = (int64_t)H * N * c.dim_v;     // elements of one sequence's V
  auto stride_ok = [&](int64_t st, int64_t size, bool allow_zero) {
    return (st == 0 && allow_zero) || st >= size;
  };
  if (!stride_ok(past->batch_stride_k, sk, true) || !stride_ok(past->batch_stride_v, sv, true))
    return fail(FWPKM_ERR_INVALID_ARG, "past_state strides must be 0 or at least one sequence's tables");
  if (!stride_ok(next->batch_stride_k, sk, batch == 1) || !stride_ok(next->batch_stride_v, sv, batch == 1))
    return fail(FWPKM_ERR_INVALID_ARG, "next_state strides must cover one sequence's tables (0 only when batch == 1)");

  const Range pk1 = table_range(past->k1, past->batch_stride_k, sk, batch);
  const Range pk2 = table_range(past->k2, past->batch_stride_k, sk, batch);
  const Range pv = table_range(past->v, past->batch_stride_v, sv, batch);
  const Range nk1 = table_range(next->k1, next->batch_stride_k, sk, batch);
  const Range nk2 = table_range(next->k2, next->batch_stride_k, sk, batch);
  const Range nv = table_range(next->v, next->batch_stride_v, sv, batch);
  const bool inplace = past->k1 == next->k1 && past->k2 == next->k2 && past->v == next->v &&
                       past->batch_stride_k == next->batch_stride_k &&
                       past->batch_stride_v == next->batch_stride_v;
  if (overlap(nk1, nk2) || overlap(nk1, nv) || overlap(nk2, nv))
    return fail(FWPKM_ERR_ALIAS, "next_state tables overlap each other");
  if (!inplace) {
    const Range ps[3] = {pk1, pk2, pv};
    const Range ns[3] = {nk1, nk2, nv};
    for (const Range& a : ps)
      for (const Range& b : ns)
        if (overlap(a, b)) return fail(FWPKM_ERR_ALIAS, "next_state partially overlaps past_state");
  }
  const int64_t rows = (int64_t)batch * tokens * H;
  if (out_rows_b == 0) out_rows_b = (int64_t)tokens * H;
  // rows spanned by the outputs: the last sequence's rows end tokens * H past its start
  const int64_t orows = (int64_t)(batch - 1) * out_rows_b + (int64_t)tokens * H;
  const Range rq = {reinterpret_cast<uintptr_t>(queries), reinterpret_cast<uintptr_t>(queries + rows * c.dim_qk)};
  const Range ry = {reinterpret_cast<uintptr_t>(targets), reinterpret_cast<uintptr_t>(targets + rows * c.dim_v)};
  const Range rr = {reinterpret_cast<uintptr_t>(retrieved), reinterpret_cast<uintptr_t>(retrieved + orows * c.dim_v)};
  const Range rw = {reinterpret_cast<uintptr_t>(token_weights),
                    reinterpret_cast<uintptr_t>(token_weights + (token_weights ? rows : 0))};
  const Range outs[3] = {rr,
                         {reinterpret_cast<uintptr_t>(out_slots), reinterpret_cast<uintptr_t>(out_slots + (out_slots ? orows * k : 0))},
                         {reinterpret_cast<uintptr_t>(out_weights), reinterpret_cast<uintptr_t>(out_weights + (out_weights ? orows * k : 0))}};
  const Range ins[9] = {rq, ry, pk1, pk2, pv, nk1, nk2, nv, rw};
  for (int i = 0; i < 3; ++i) {
    if (outs[i].lo == outs[i].hi) continue;
    for (const Range& b : ins)
      if (b.lo != b.hi && overlap(outs[i], b)) return fail(FWPKM_ERR_ALIAS, "an output overlaps an input or the state");
    for (int j = i + 1; j < 3; ++j)
      if (outs[j].lo != outs[j].hi && overlap(outs[i], outs[j])) return fail(FWPKM_ERR_ALIAS, "outputs overlap each other");
  }
  for (const Range& b : {nk1, nk2, nv})
    if (overlap(b, rq) || overlap(b, ry) || (rw.lo != rw.hi && overlap(b, rw)))
      return fail(FWPKM_ERR_ALIAS, "next_state overlaps queries, targets or token weights");
  // ---------------------------------------------------------- workspace
  const int64_t U = (int64_t)batch * H;
  const WsLayout L = ws_layout(c, U, tokens);
  if (noalloc && L.total > (size_t)FWPKM_NOALLOC_SCRATCH_BYTES)
    return fail(FWPKM_ERR_UNSUPPORTED,
                "this call needs %zu bytes of workspace, more than the %u-byte fixed array of "
                "fwpkm_forward_chunk_noalloc (use fwpkm_forward_chunk)",
                L.total, (unsigned)FWPKM_NOALLOC_SCRATCH_BYTES);
  if (dry_run) return FWPKM_OK;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FWPKM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  char* ws = nullptr;
  if (noalloc) {
    const int rc = scratch_of_device(dev, &ws);
    if (rc != FWPKM_OK) return rc;
  } else {
    if (!h->ws) {
      e = hipMalloc(&h->ws, h->ws_bytes);
      if (e != hipSuccess) {
        h->ws = nullptr;
        (void)hipGetLastError();
        if (e == hipErrorOutOfMemory) return fail(FWPKM_ERR_OOM, "workspace of %zu bytes: %s", h->ws_bytes, hipGetErrorString(e));
        return fail(FWPKM_ERR_HIP, "hipMalloc: %s", hipGetErrorString(e));
      }
      h->device = dev;
    } else if (dev != h->device) {
      return fail(FWPKM_ERR_INVALID_ARG, "handle's workspace lives on device %d, current device is %d", h->device, dev);
    }
    ws = static_cast<char*>(h->ws);
  }
  // per-kernel events only on the handle's own path (creating events is an
  // allocation the fixed-workspace path must not make)
  const bool prof = h->prof && !noalloc;

  // ---------------------------------------------------------- enqueue
  if (!inplace) {
    const struct { float* d; const float* s; int64_t ds, ss, n; } cps[3] = {
        {next->k1, past->k1, next->batch_stride_k, past->batch_stride_k, sk},
        {next->k2, past->k2, next->batch_stride_k, past->batch_stride_k, sk},
        {next->v, past->v, next->batch_stride_v, past->batch_stride_v, sv}};
    e = timed(h, prof, 4, [&](const fwpkm::LaunchTiming* tm) {
      hipError_t r = tm ? hipEventRecord(tm->beg, stream) : hipSuccess;
      for (const auto& cp : cps) {
        for (int b = 0; b < batch && r == hipSuccess; ++b) {
          r = hipMemcpyAsync(cp.d + (int64_t)b * cp.ds, cp.s + (int64_t)b * cp.ss,
                             sizeof(float) * cp.n, hipMemcpyDeviceToDevice, stream);
        }
      }
      if (r == hipSuccess && tm) r = hipEventRecord(tm->end, stream);
      return r;
    });
    if (e != hipSuccess) return fail(FWPKM_ERR_HIP, "state copy: %s", hipGetErrorString(e));
  }

  fwpkm::ChunkArgs a{};
  a.n = n;
  a.half = half;
  a.dqk = c.dim_qk;
  a.dv = c.dim_v;
  a.k = k;
  a.T = tokens;
  a.H = H;
  a.U = (int)U;
  a.key_block = fwpkm::score_key_block((int)U, tokens, n);
  a.nblk = (n + a.key_block - 1) / a.key_block;
  a.P = tokens * k;
  a.mode = c.score_mode;
  a.eps = c.eps;
  a.lr = lr;
  a.q = queries;
  a.y = targets;
  a.tw = token_weights;
  a.k1 = next->k1;
  a.k2 = next->k2;
  a.v = next->v;
  a.stride_k = next->batch_stride_k;
  a.stride_v = next->batch_stride_v;
  a.retrieved = retrieved;
  a.out_rows_b = out_rows_b;
  a.out_slots = out_slots;
  a.out_weights = out_weights;
  a.half_o = reinterpret_cast<float*>(ws + L.half_o);
  a.half_i = reinterpret_cast<int*>(ws + L.half_i);
  a.qnorm = reinterpret_cast<float*>(ws + L.qnorm);
  a.sel_w = reinterpret_cast<float*>(ws + L.sel_w);
  a.g = reinterpret_cast<float*>(ws + L.g);
  a.keys = reinterpret_cast<int*>(ws + L.keys);
  a.coef = reinterpret_cast<float*>(ws + L.coef);
  a.ent_row = reinterpret_cast<int*>(ws + L.ent_row);
  a.ent_tw = reinterpret_cast<int2*>(ws + L.ent_tw);
  a.kinds = reinterpret_cast<int4*>(ws + L.kinds);
  a.regions = fwpkm::group_regions((int)U);
  a.region_bits = 0;
  while ((1 << a.region_bits) < a.regions) ++a.region_bits;
  a.pw = std::max(c.dim_v, half);
  a.npr = 0;
  for (int i = 0; i < k; ++i) a.npr += k / (i + 1);
  const bool write = lr != 0.0f;
  const bool addr = write && c.addr_weight != 0.0f;
  a.addr_weight = c.addr_weight;
  a.addr_s = addr ? reinterpret_cast<float*>(ws + L.addr_s) : nullptr;
  a.addr_np = (n + fwpkm::kAddrPad - 1) / fwpkm::kAddrPad * fwpkm::kAddrPad;
  a.addr_dk = reinterpret_cast<float*>(ws + L.addr_dk);
  a.addr_tok = reinterpret_cast<float*>(ws + L.addr_tok);
  a.addr_ell = reinterpret_cast<float*>(ws + L.addr_ell);
  a.check = reinterpret_cast<unsigned int*>(ws + L.check);
#if FWPKM_DEVICE_CHECKS
  // checked builds: every byte of the call's workspace starts as 0xFF (NaN as
  // a float, -1 as an index, so a kernel that reads workspace its call never
  // wrote gets values the device checks or the results expose), then the
  // check word is cleared
  if ((e = hipMemsetAsync(ws, 0xFF, L.total, stream)) != hipSuccess)
    return fail(FWPKM_ERR_HIP, "poisoning the workspace: %s", hipGetErrorString(e));
  if ((e = hipMemsetAsync(a.check, 0, sizeof(unsigned int), stream)) != hipSuccess)
    return fail(FWPKM_ERR_HIP, "clearing the device-check word: %s", hipGetErrorString(e));
#endif

  using fwpkm::LaunchTiming;
  if ((e = timed(h, prof, 0, [&](const LaunchTiming* tm) { return fwpkm::launch_ka(a, stream, tm); })) != hipSuccess)
    return fail(FWPKM_ERR_HIP, "score kernel: %s", hipGetErrorString(e));
  if ((e = timed(h, prof, 1, [&](const LaunchTiming* tm) { return fwpkm::launch_kb(a, write, stream, tm); })) != hipSuccess)
    return fail(FWPKM_ERR_HIP, "read kernel: %s", hipGetErrorString(e));
  if (write) {
    // the addressing gradient is taken at the starting keys, before the update
    if (addr) {
      if ((e = timed(h, prof, 5, [&](const LaunchTiming* tm) { return fwpkm::launch_ke_stats(a, stream, tm); })) != hipSuccess)
        return fail(FWPKM_ERR_HIP, "addressing statistics kernel: %s", hipGetErrorString(e));
      if ((e = timed(h, prof, 6, [&](const LaunchTiming* tm) { return fwpkm::launch_ke_grad(a, stream, tm); })) != hipSuccess)
        return fail(FWPKM_ERR_HIP, "addressing gradient kernel: %s", hipGetErrorString(e));
    }
    if (!fwpkm::kd_fuses_grouping(a) &&
        (e = timed(h, prof, 2, [&](const LaunchTiming* tm) { return fwpkm::launch_kc(a, stream, tm); })) != hipSuccess)
      return fail(FWPKM_ERR_HIP, "sort kernel: %s", hipGetErrorString(e));
    if ((e = timed(h, prof, 3, [&](const LaunchTiming* tm) { return fwpkm::launch_kd(a, stream, tm); })) != hipSuccess)
      return fail(FWPKM_ERR_HIP, "update kernel: %s", hipGetErrorString(e));
    if (addr) {
      if ((e = timed(h, prof, 7, [&](const LaunchTiming* tm) { return fwpkm::launch_ke_apply(a, stream, tm); })) != hipSuccess)
        return fail(FWPKM_ERR_HIP, "addressing step kernel: %s", hipGetErrorString(e));
    }
  }
#if FWPKM_DEVICE_CHECKS
  return read_device_checks(a.check, stream);
#else
  g_err[0] = '\0';
  return FWPKM_OK;
#endif
}

}  // extern "C"
