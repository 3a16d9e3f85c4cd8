// C ABI of libmsa (declared in include/msa.h): host-side argument checks,
// workspace layout, the walk over token windows, and the kernel chain of each
// entry point on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "msa.h"
#include "msa_internal.h"

namespace msa {
namespace {

constexpr size_t ALIGN = 256;
// The forward walks token windows whose query rows of one group (W R d bf16)
// stay within this many bytes: the items of a group re-read those rows once
// per selected block, and the last-level cache then serves most re-reads.
constexpr size_t FWD_WINDOW_Q_BYTES = (size_t)64 << 20;
constexpr size_t CAP_SELECT = (size_t)8 << 30;
// The Main Branch workspace a call asks for: one MI355X holds 288 GB, and fewer,
// longer windows (1M: 15 instead of 31 at half this size) cut launch tails
// and inverse-index rebuilds.
constexpr size_t CAP_MAIN = (size_t)80 << 30;

size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Layout {
  int W = 0;
  size_t total = 0;
  size_t pooled = 0;
  size_t counts = 0, base = 0, len = 0, items = 0, item_count = 0, list = 0, order = 0;
  int max_items = 0;
  size_t items2 = 0, item_count2 = 0, order2 = 0;  // merged call: backward items cut from the same inverse index
  int max_items2 = 0;
  size_t part_o = 0, part_lse = 0;
  size_t Dd = 0, dk_acc = 0, dv_acc = 0, dq_part = 0;
};

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = up(off + bytes);
    return o;
  }
};

void carve_inverse(Layout& L, Carver& c, const Geo& g, int W, int item_tokens) {
  const size_t BG = (size_t)g.B * g.G;
  const size_t nchunk = (W + INV_CHUNK - 1) / INV_CHUNK;
  L.max_items = inv_max_items(g, W, item_tokens);
  L.counts = c.take(BG * nchunk * g.N * 4);
  L.base = c.take(BG * g.N * 4);
  L.len = c.take(BG * g.N * 4);
  L.items = c.take(BG * (size_t)L.max_items * 16);
  L.item_count = c.take(BG * 4);
  L.list = c.take(BG * (size_t)W * g.K * 4);
  L.order = c.take(BG * (size_t)L.max_items * 4);
}

Layout layout(const Geo& g, msa_op op, int W) {
  Layout L;
  L.W = W;
  Carver c;
  const size_t BG = (size_t)g.B * g.G;
  const size_t pairs = BG * (size_t)W * g.K;
  if (op == MSA_OP_SELECT) {
    L.pooled = c.take(BG * (size_t)W * g.N * 4);
  } else if (op == MSA_OP_DECODE_SELECT) {
    L.pooled = c.take(BG * (size_t)g.N * 4);
  } else if (op == MSA_OP_DECODE_FWD) {
    L.part_o = c.take(BG * (size_t)g.K * g.R * g.D * 4);
    L.part_lse = c.take(BG * (size_t)g.K * g.R * 4);
  } else if (op == MSA_OP_FWD_BWD) {
    // One inverse index serves both halves; the forward partials are dead once
    // the window's combine has run, so the dQ partials reuse their memory.
    const size_t kv = (size_t)g.B * g.T * g.G * g.D;
    L.Dd = c.take((size_t)g.B * g.T * g.H * 4);
    L.dk_acc = c.take(kv * 4);
    L.dv_acc = c.take(kv * 4);
    carve_inverse(L, c, g, W, FWD_ITEM_TOKENS);
    L.max_items2 = inv_max_items(g, W, BWD_ITEM_TOKENS);
    L.items2 = c.take(BG * (size_t)L.max_items2 * 16);
    L.item_count2 = c.take(BG * 4);
    L.order2 = c.take(BG * (size_t)L.max_items2 * 4);
    L.part_lse = c.take((pairs + 1) * g.R * 4);
    L.part_o = c.take((pairs + 1) * g.R * g.D * 2);
    L.dq_part = L.part_o;
  } else if (op == MSA_OP_FWD) {
    carve_inverse(L, c, g, W, FWD_ITEM_TOKENS);
    L.part_o = c.take((pairs + 1) * g.R * g.D * 2);  // + a spare slot for rows past an item's list
    L.part_lse = c.take((pairs + 1) * g.R * 4);
  } else {
    const size_t kv = (size_t)g.B * g.T * g.G * g.D;
    L.Dd = c.take((size_t)g.B * g.T * g.H * 4);
    L.dk_acc = c.take(kv * 4);
    L.dv_acc = c.take(kv * 4);
    carve_inverse(L, c, g, W, BWD_ITEM_TOKENS);
    L.dq_part = c.take(pairs * g.R * g.D * 2);
  }
  L.total = c.off;
  return L;
}

// Window lengths are T itself or multiples of 256 tokens.
int min_window(const Geo& g) { return g.T < 256 ? g.T : 256; }

// Largest window whose layout fits in `bytes`; 0 if none does.
int fit_window(const Geo& g, msa_op op, size_t bytes) {
  if (layout(g, op, g.T).total <= bytes) return g.T;
  int lo = 0, hi = (g.T - 1) / 256;  // candidate windows 256 * m, m in [1, hi]
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (layout(g, op, 256 * mid).total <= bytes) lo = mid; else hi = mid - 1;
  }
  if (lo == 0) return layout(g, op, min_window(g)).total <= bytes ? min_window(g) : 0;
  return 256 * lo;
}

// Largest forward window (T, or a multiple of 256 tokens) whose query rows of
// one group fit FWD_WINDOW_Q_BYTES.
int fwd_window_cap(const Geo& g) {
  const size_t row = (size_t)g.R * g.D * 2;
  const size_t w = FWD_WINDOW_Q_BYTES / row;
  if (w >= (size_t)g.T) return g.T;
  return std::max<int>(256, (int)(w / 256 * 256));
}

bool is_pow2_le16(int r) { return r == 1 || r == 2 || r == 4 || r == 8 || r == 16; }

msa_status make_geo(const msa_dims* d, msa_op op, Geo* g) {
  if (!d) return MSA_ERR_NULL;
  if (d->B < 1 || d->T < 128 || d->T % 128 != 0 || d->T > (1 << 20) || d->G < 1 || d->topk < 1 ||
      d->topk > 1024 || !std::isfinite(d->scale))
    return MSA_ERR_SHAPE;
  if ((int64_t)d->T * d->topk >= ((int64_t)1 << 31) || (int64_t)d->B * d->T >= ((int64_t)1 << 30))
    return MSA_ERR_SHAPE;
  if ((int64_t)d->B * d->G > 65535) return MSA_ERR_SHAPE;  // (batch, group) is a grid dimension
  g->B = d->B; g->T = d->T; g->G = d->G; g->K = d->topk; g->N = d->T / 128;
  g->H = d->H; g->D = d->d; g->DP = d->dp;
  if (op == MSA_OP_SELECT) {
    if (d->dp != 32 && d->dp != 64 && d->dp != 128) return MSA_ERR_UNSUPPORTED;
    g->H = g->G; g->R = 1; g->D = 64;
  } else {
    if (d->H < 1 || d->H % d->G != 0) return MSA_ERR_SHAPE;
    g->R = d->H / d->G;
    if (!is_pow2_le16(g->R) || (d->d != 64 && d->d != 128)) return MSA_ERR_UNSUPPORTED;
  }
  g->scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt((float)g->D);
  return MSA_OK;
}

bool is_decode(msa_op op) { return op == MSA_OP_DECODE_SELECT || op == MSA_OP_DECODE_FWD; }

// Decode geometry: the training checks.
msa_status make_dec_geo(const msa_dims* d, msa_op op, Geo* g) {
  return make_geo(d, op == MSA_OP_DECODE_SELECT ? MSA_OP_SELECT : MSA_OP_FWD, g);
}

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The integer a caller passed for an enum argument.  C callers may pass any
// int; reading it through the object representation keeps values outside the
// enumerators defined (they select the "unknown" branches).
template <class E>
int enum_value(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "enums of the ABI are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

InvBufs inv_bufs(const Layout& L, char* ws) {
  InvBufs ib;
  ib.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  ib.base = reinterpret_cast<int32_t*>(ws + L.base);
  ib.len = reinterpret_cast<int32_t*>(ws + L.len);
  ib.items = reinterpret_cast<int4*>(ws + L.items);
  ib.item_count = reinterpret_cast<int32_t*>(ws + L.item_count);
  ib.list = reinterpret_cast<int32_t*>(ws + L.list);
  ib.order = reinterpret_cast<int32_t*>(ws + L.order);
  ib.max_items = L.max_items;
  return ib;
}

#define MSA_TRY(x)                                  \
  do {                                              \
    if ((x) != hipSuccess) return MSA_ERR_HIP;      \
  } while (0)

// ---- opt-in launch timing.  The state belongs to the calling host thread
// (created by its first msa_timing_enable, kept until the process ends), so
// calls from different threads never share it; with timing off a launch only
// reads this thread's null pointer.
constexpr int MAX_TIMED = 4096;
struct TimedLaunch {
  hipEvent_t a = nullptr, b = nullptr;
  int kernel = 0;
};
struct TimingState {
  bool on = false;
  int n = 0;
  TimedLaunch slot[MAX_TIMED];
};
thread_local TimingState* t_timing = nullptr;

int timing_begin(int kernel, hipStream_t st) {
  TimingState* ts = t_timing;
  if (!ts || !ts->on || ts->n >= MAX_TIMED) return -1;
  TimedLaunch& s = ts->slot[ts->n];
  if (!s.a && hipEventCreate(&s.a) != hipSuccess) return -1;
  if (!s.b && hipEventCreate(&s.b) != hipSuccess) return -1;
  if (hipEventRecord(s.a, st) != hipSuccess) return -1;
  s.kernel = kernel;
  return ts->n++;
}

void timing_end(int id, hipStream_t st) {
  if (id >= 0) (void)hipEventRecord(t_timing->slot[id].b, st);
}

// ---- allocation-free decode attention (msa_decode_fwd_static)
// Its per-slot partials live in this array instead of a caller workspace.
// In host code `scratch` names a host-side stand-in; the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with
// that device current and kept here.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)MSA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[MAX_DEVICES] = {};

// Device address of `scratch` on the device that `st` belongs to, which must
// be the current device.
msa_status scratch_for_stream(hipStream_t st, void** out) {
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MSA_ERR_HIP;
  if (hipStreamGetDevice(st, &sdev) != hipSuccess) return MSA_ERR_HIP;
  if (dev != sdev || dev < 0 || dev >= MAX_DEVICES) return MSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MSA_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MSA_OK;
}

// Launch `call` (a hipError_t expression), timed as `kernel` when timing is on.
#define MSA_LAUNCH(kernel, st, call)                 \
  do {                                               \
    const int tid_ = timing_begin((kernel), (st));   \
    const hipError_t e_ = (call);                    \
    timing_end(tid_, (st));                          \
    if (e_ != hipSuccess) return MSA_ERR_HIP;        \
  } while (0)

// Cache check, on when MSA_VALIDATE is set to a non-empty value other than "0".
bool validate_on() {
  const char* e = std::getenv("MSA_VALIDATE");
  return e && e[0] && std::strcmp(e, "0") != 0;
}

// Runs the device check of idx (its result in the first 16 bytes of ws) and
// waits for it: MSA_ERR_INDEX if a row fails.
msa_status check_cache(const Geo& g, const int32_t* idx, void* ws, hipStream_t st) {
  if (!validate_on()) return MSA_OK;
  int32_t* flag = static_cast<int32_t*>(ws);
  MSA_TRY(launch_fill_zero(reinterpret_cast<float*>(flag), 4, st));
  MSA_TRY(launch_check_idx(g, idx, flag, st));
  int32_t h = 0;
  MSA_TRY(hipMemcpyAsync(&h, flag, sizeof(h), hipMemcpyDeviceToHost, st));
  MSA_TRY(hipStreamSynchronize(st));
  return h ? MSA_ERR_INDEX : MSA_OK;
}

}  // namespace
}  // namespace msa

using namespace msa;

extern "C" {

size_t msa_workspace_bytes(const msa_dims* dims, msa_op op_in) {
  const int opv = enum_value(op_in);
  if (opv < MSA_OP_SELECT || opv > MSA_OP_FWD_BWD) return 0;
  const msa_op op = static_cast<msa_op>(opv);
  Geo g;
  if (is_decode(op)) return make_dec_geo(dims, op, &g) == MSA_OK ? layout(g, op, 0).total : 0;
  if (op != MSA_OP_SELECT && op != MSA_OP_FWD && op != MSA_OP_BWD && op != MSA_OP_FWD_BWD) return 0;
  if (make_geo(dims, op, &g) != MSA_OK) return 0;
  const int pref = (op == MSA_OP_FWD || op == MSA_OP_FWD_BWD) ? fwd_window_cap(g) : g.T;
  const size_t full = layout(g, op, pref).total;
  const size_t cap = op == MSA_OP_SELECT ? CAP_SELECT : CAP_MAIN;
  if (full <= cap) return full;
  const int W = fit_window(g, op, cap);
  return layout(g, op, W > 0 ? W : min_window(g)).total;
}

size_t msa_workspace_min_bytes(const msa_dims* dims, msa_op op_in) {
  const int opv = enum_value(op_in);
  if (opv < MSA_OP_SELECT || opv > MSA_OP_FWD_BWD) return 0;
  const msa_op op = static_cast<msa_op>(opv);
  Geo g;
  if (is_decode(op)) return make_dec_geo(dims, op, &g) == MSA_OK ? layout(g, op, 0).total : 0;
  if (op != MSA_OP_SELECT && op != MSA_OP_FWD && op != MSA_OP_BWD && op != MSA_OP_FWD_BWD) return 0;
  if (make_geo(dims, op, &g) != MSA_OK) return 0;
  return layout(g, op, min_window(g)).total;
}

msa_status msa_pattern_select(const msa_dims* dims, int32_t window, int32_t dilation, const int32_t* idx_in,
                              int32_t k_in, int32_t* idx_out, void* stream) {
  if (!dims) return MSA_ERR_NULL;
  const msa_dims& d = *dims;
  if (d.B < 1 || d.T < 128 || d.T % 128 != 0 || d.T > (1 << 20) || d.G < 1 || d.topk < 1 || d.topk > 1024)
    return MSA_ERR_SHAPE;
  if ((int64_t)d.T * d.topk >= ((int64_t)1 << 31) || (int64_t)d.B * d.T >= ((int64_t)1 << 30))
    return MSA_ERR_SHAPE;
  if (window < 0 || dilation < 0) return MSA_ERR_SHAPE;
  if (window == 0 && dilation == 0 && idx_in == nullptr) return MSA_ERR_SHAPE;
  if (idx_in != nullptr && (k_in < 1 || k_in > 1024)) return MSA_ERR_SHAPE;
  if (!idx_out) return MSA_ERR_NULL;
  if (!al16(idx_out) || (idx_in && !al16(idx_in))) return MSA_ERR_ALIGN;
  // the largest row the pattern can produce must fit the output width
  const int64_t N = d.T / 128, w = std::min<int64_t>(window, N);
  const int64_t far = dilation > 0 ? (std::max<int64_t>(0, N - window) + dilation - 1) / dilation : 0;
  const int64_t bound = std::min<int64_t>(N, w + far + (idx_in ? k_in : 0));
  if (d.topk < bound) return MSA_ERR_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  MSA_LAUNCH(MSA_K_PATTERN, st,
             launch_pattern(idx_in, idx_in ? k_in : 0, idx_out, d.topk, d.B, d.G, d.T, window, dilation, st));
  return MSA_OK;
}

msa_status msa_proxy_select(const msa_dims* dims, const msa_bf16* qp, const msa_bf16* kp, int32_t* idx, void* ws,
                            size_t ws_bytes, void* stream) {
  Geo g;
  const msa_status s = make_geo(dims, MSA_OP_SELECT, &g);
  if (s != MSA_OK) return s;
  if (!qp || !kp || !idx || !ws) return MSA_ERR_NULL;
  if (!al16(qp) || !al16(kp) || !al16(idx) || !al16(ws)) return MSA_ERR_ALIGN;
  const int W = fit_window(g, MSA_OP_SELECT, ws_bytes);
  if (W == 0) return MSA_ERR_WORKSPACE;
  const Layout L = layout(g, MSA_OP_SELECT, W);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float* pooled = reinterpret_cast<float*>(static_cast<char*>(ws) + L.pooled);
  for (int t0 = 0; t0 < g.T; t0 += W) {
    const Win w{t0, std::min(W, g.T - t0)};
    MSA_LAUNCH(MSA_K_PROXY_POOL, st, launch_proxy_pool(g, w, qp, kp, pooled, st));
    MSA_LAUNCH(MSA_K_TOPK, st, launch_topk(g, w, pooled, idx, st));
  }
  return MSA_OK;
}

msa_status msa_fwd(const msa_dims* dims, const msa_bf16* q, const msa_bf16* k, const msa_bf16* v, const int32_t* idx,
                   msa_bf16* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  Geo g;
  const msa_status s = make_geo(dims, MSA_OP_FWD, &g);
  if (s != MSA_OK) return s;
  if (!q || !k || !v || !idx || !o || !lse || !ws) return MSA_ERR_NULL;
  if (!al16(q) || !al16(k) || !al16(v) || !al16(idx) || !al16(o) || !al16(lse) || !al16(ws)) return MSA_ERR_ALIGN;
  int W = fit_window(g, MSA_OP_FWD, ws_bytes);
  if (W == 0) return MSA_ERR_WORKSPACE;
  W = std::min(W, fwd_window_cap(g));
  const Layout L = layout(g, MSA_OP_FWD, W);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (const msa_status c = check_cache(g, idx, ws, st); c != MSA_OK) return c;
  char* base = static_cast<char*>(ws);
  const InvBufs ib = inv_bufs(L, base);
  uint16_t* part_o = reinterpret_cast<uint16_t*>(base + L.part_o);
  float* part_lse = reinterpret_cast<float*>(base + L.part_lse);
  for (int t0 = 0; t0 < g.T; t0 += W) {
    const Win w{t0, std::min(W, g.T - t0)};
    MSA_LAUNCH(MSA_K_INVERSE, st, launch_inverse(g, w, idx, ib, FWD_ITEM_TOKENS, st));
    MSA_LAUNCH(MSA_K_FWD_PARTIALS, st, launch_fwd_partials(g, w, q, k, v, ib, part_o, part_lse, st));
    MSA_LAUNCH(MSA_K_FWD_COMBINE, st, launch_fwd_combine(g, w, idx, part_o, part_lse, o, lse, nullptr, nullptr, st));
  }
  return MSA_OK;
}

msa_status msa_bwd(const msa_dims* dims, const msa_bf16* q, const msa_bf16* k, const msa_bf16* v, const msa_bf16* o,
                   const msa_bf16* dout, const float* lse, const int32_t* idx, msa_bf16* dq, msa_bf16* dk,
                   msa_bf16* dv, void* ws, size_t ws_bytes, void* stream) {
  Geo g;
  const msa_status s = make_geo(dims, MSA_OP_BWD, &g);
  if (s != MSA_OK) return s;
  if (!q || !k || !v || !o || !dout || !lse || !idx || !dq || !dk || !dv || !ws) return MSA_ERR_NULL;
  if (!al16(q) || !al16(k) || !al16(v) || !al16(o) || !al16(dout) || !al16(lse) || !al16(idx) || !al16(dq) ||
      !al16(dk) || !al16(dv) || !al16(ws))
    return MSA_ERR_ALIGN;
  const int W = fit_window(g, MSA_OP_BWD, ws_bytes);
  if (W == 0) return MSA_ERR_WORKSPACE;
  const Layout L = layout(g, MSA_OP_BWD, W);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (const msa_status c = check_cache(g, idx, ws, st); c != MSA_OK) return c;
  char* base = static_cast<char*>(ws);
  const InvBufs ib = inv_bufs(L, base);
  float* Dd = reinterpret_cast<float*>(base + L.Dd);
  float* dk_acc = reinterpret_cast<float*>(base + L.dk_acc);
  float* dv_acc = reinterpret_cast<float*>(base + L.dv_acc);
  uint16_t* dq_part = reinterpret_cast<uint16_t*>(base + L.dq_part);
  const size_t kv = (size_t)g.B * g.T * g.G * g.D;
  MSA_LAUNCH(MSA_K_BWD_DOT, st, launch_bwd_dot(g, o, dout, Dd, st));
  MSA_LAUNCH(MSA_K_BWD_DOT, st, launch_fill_zero(dk_acc, kv, st));
  MSA_LAUNCH(MSA_K_BWD_DOT, st, launch_fill_zero(dv_acc, kv, st));
  for (int t0 = 0; t0 < g.T; t0 += W) {
    const Win w{t0, std::min(W, g.T - t0)};
    MSA_LAUNCH(MSA_K_INVERSE, st, launch_inverse(g, w, idx, ib, BWD_ITEM_TOKENS, st));
    MSA_LAUNCH(MSA_K_BWD_PARTIALS, st, launch_bwd_partials(g, w, q, k, v, dout, lse, Dd, ib, dq_part, dk_acc, dv_acc, st));
    MSA_LAUNCH(MSA_K_DQ_COMBINE, st, launch_dq_combine(g, w, idx, dq_part, dq, st));
  }
  MSA_LAUNCH(MSA_K_CONVERT, st, launch_cvt_bf16(dk_acc, dk, kv, st));
  MSA_LAUNCH(MSA_K_CONVERT, st, launch_cvt_bf16(dv_acc, dv, kv, st));
  return MSA_OK;
}

msa_status msa_fwd_bwd(const msa_dims* dims, const msa_bf16* q, const msa_bf16* k, const msa_bf16* v,
                       const msa_bf16* dout, const int32_t* idx, msa_bf16* o, float* lse, msa_bf16* dq, msa_bf16* dk,
                       msa_bf16* dv, void* ws, size_t ws_bytes, void* stream) {
  Geo g;
  const msa_status s = make_geo(dims, MSA_OP_FWD_BWD, &g);
  if (s != MSA_OK) return s;
  if (!q || !k || !v || !dout || !idx || !o || !lse || !dq || !dk || !dv || !ws) return MSA_ERR_NULL;
  if (!al16(q) || !al16(k) || !al16(v) || !al16(dout) || !al16(idx) || !al16(o) || !al16(lse) || !al16(dq) ||
      !al16(dk) || !al16(dv) || !al16(ws))
    return MSA_ERR_ALIGN;
  int W = fit_window(g, MSA_OP_FWD_BWD, ws_bytes);
  if (W == 0) return MSA_ERR_WORKSPACE;
  W = std::min(W, fwd_window_cap(g));
  const Layout L = layout(g, MSA_OP_FWD_BWD, W);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (const msa_status c = check_cache(g, idx, ws, st); c != MSA_OK) return c;
  char* base = static_cast<char*>(ws);
  const InvBufs ib = inv_bufs(L, base);
  InvBufs ib2 = ib;  // same list, backward-sized items
  ib2.items = reinterpret_cast<int4*>(base + L.items2);
  ib2.item_count = reinterpret_cast<int32_t*>(base + L.item_count2);
  ib2.order = reinterpret_cast<int32_t*>(base + L.order2);
  ib2.max_items = L.max_items2;
  float* Dd = reinterpret_cast<float*>(base + L.Dd);
  float* dk_acc = reinterpret_cast<float*>(base + L.dk_acc);
  float* dv_acc = reinterpret_cast<float*>(base + L.dv_acc);
  uint16_t* part_o = reinterpret_cast<uint16_t*>(base + L.part_o);
  float* part_lse = reinterpret_cast<float*>(base + L.part_lse);
  uint16_t* dq_part = reinterpret_cast<uint16_t*>(base + L.dq_part);
  const size_t kv = (size_t)g.B * g.T * g.G * g.D;
  MSA_LAUNCH(MSA_K_BWD_DOT, st, launch_fill_zero(dk_acc, kv, st));
  MSA_LAUNCH(MSA_K_BWD_DOT, st, launch_fill_zero(dv_acc, kv, st));
  for (int t0 = 0; t0 < g.T; t0 += W) {
    const Win w{t0, std::min(W, g.T - t0)};
    MSA_LAUNCH(MSA_K_INVERSE, st, launch_inverse(g, w, idx, ib, FWD_ITEM_TOKENS, st));
    MSA_LAUNCH(MSA_K_INVERSE, st, launch_inverse_items(g, ib2, BWD_ITEM_TOKENS, st));
    MSA_LAUNCH(MSA_K_FWD_PARTIALS, st, launch_fwd_partials(g, w, q, k, v, ib, part_o, part_lse, st));
    MSA_LAUNCH(MSA_K_FWD_COMBINE, st, launch_fwd_combine(g, w, idx, part_o, part_lse, o, lse, dout, Dd, st));
    MSA_LAUNCH(MSA_K_BWD_PARTIALS, st,
               launch_bwd_partials(g, w, q, k, v, dout, lse, Dd, ib2, dq_part, dk_acc, dv_acc, st));
    MSA_LAUNCH(MSA_K_DQ_COMBINE, st, launch_dq_combine(g, w, idx, dq_part, dq, st));
  }
  MSA_LAUNCH(MSA_K_CONVERT, st, launch_cvt_bf16(dk_acc, dk, kv, st));
  MSA_LAUNCH(MSA_K_CONVERT, st, launch_cvt_bf16(dv_acc, dv, kv, st));
  return MSA_OK;
}

msa_status msa_decode_select(const msa_dims* dims, const msa_bf16* qp, const msa_bf16* kp, const int32_t* len,
                             int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  Geo g;
  const msa_status s = make_dec_geo(dims, MSA_OP_DECODE_SELECT, &g);
  if (s != MSA_OK) return s;
  if (!qp || !kp || !len || !idx || !ws) return MSA_ERR_NULL;
  if (!al16(qp) || !al16(kp) || !al16(len) || !al16(idx) || !al16(ws)) return MSA_ERR_ALIGN;
  const Layout L = layout(g, MSA_OP_DECODE_SELECT, 0);
  if (ws_bytes < L.total) return MSA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float* pooled = reinterpret_cast<float*>(static_cast<char*>(ws) + L.pooled);
  MSA_LAUNCH(MSA_K_DEC_POOL, st, launch_dec_pool(g, qp, kp, len, pooled, st));
  MSA_LAUNCH(MSA_K_DEC_TOPK, st, launch_dec_topk(g, pooled, len, idx, st));
  return MSA_OK;
}

msa_status msa_decode_fwd(const msa_dims* dims, const msa_bf16* q, const msa_bf16* k, const msa_bf16* v,
                          const int32_t* len, const int32_t* idx, msa_bf16* o, float* lse, void* ws, size_t ws_bytes,
                          void* stream) {
  Geo g;
  const msa_status s = make_dec_geo(dims, MSA_OP_DECODE_FWD, &g);
  if (s != MSA_OK) return s;
  if (!q || !k || !v || !len || !idx || !o || !lse || !ws) return MSA_ERR_NULL;
  if (!al16(q) || !al16(k) || !al16(v) || !al16(len) || !al16(idx) || !al16(o) || !al16(lse) || !al16(ws))
    return MSA_ERR_ALIGN;
  const Layout L = layout(g, MSA_OP_DECODE_FWD, 0);
  if (ws_bytes < L.total) return MSA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  float* part_o = reinterpret_cast<float*>(base + L.part_o);
  float* part_lse = reinterpret_cast<float*>(base + L.part_lse);
  MSA_LAUNCH(MSA_K_DEC_ATTN, st, launch_dec_attn(g, q, k, v, len, idx, part_o, part_lse, st));
  MSA_LAUNCH(MSA_K_DEC_COMBINE, st, launch_dec_combine(g, part_o, part_lse, idx, len, o, lse, st));
  return MSA_OK;
}

msa_status msa_decode_fwd_static(const msa_dims* dims, const msa_bf16* q, const msa_bf16* k, const msa_bf16* v,
                                 const int32_t* len, const int32_t* idx, msa_bf16* o, float* lse, void* stream) {
  Geo g;
  const msa_status s = make_dec_geo(dims, MSA_OP_DECODE_FWD, &g);
  if (s != MSA_OK) return s;
  if (!q || !k || !v || !len || !idx || !o || !lse) return MSA_ERR_NULL;
  if (!al16(q) || !al16(k) || !al16(v) || !al16(len) || !al16(idx) || !al16(o) || !al16(lse)) return MSA_ERR_ALIGN;
  const Layout L = layout(g, MSA_OP_DECODE_FWD, 0);
  if (L.total > STATIC_SCRATCH_BYTES) return MSA_ERR_SCRATCH;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  void* base = nullptr;
  if (const msa_status e = scratch_for_stream(st, &base); e != MSA_OK) return e;
  char* b = static_cast<char*>(base);
  float* part_o = reinterpret_cast<float*>(b + L.part_o);
  float* part_lse = reinterpret_cast<float*>(b + L.part_lse);
  MSA_LAUNCH(MSA_K_DEC_ATTN, st, launch_dec_attn(g, q, k, v, len, idx, part_o, part_lse, st));
  MSA_LAUNCH(MSA_K_DEC_COMBINE, st, launch_dec_combine(g, part_o, part_lse, idx, len, o, lse, st));
  return MSA_OK;
}

const char* msa_status_str(msa_status s) {
  switch (enum_value(s)) {
    case MSA_OK: return "ok";
    case MSA_ERR_NULL: return "null pointer argument";
    case MSA_ERR_SHAPE: return "dimensions out of the supported range";
    case MSA_ERR_UNSUPPORTED: return "head dim, proxy dim or group ratio not supported";
    case MSA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MSA_ERR_WORKSPACE: return "workspace too small";
    case MSA_ERR_HIP: return "HIP runtime error";
    case MSA_ERR_INDEX: return "block-index cache fails the MSA_VALIDATE check";
    case MSA_ERR_SCRATCH: return "problem needs more than the library's static scratch (MSA_STATIC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

const char* msa_version(void) { return "msa-gfx950 0.1"; }

void msa_timing_enable(int on) {
  if (!t_timing) {
    if (!on) return;
    t_timing = new (std::nothrow) TimingState();
    if (!t_timing) return;
  }
  t_timing->on = on != 0;
  t_timing->n = 0;
}

msa_status msa_timing_read(double* ms, int32_t* launches, int32_t n) {
  for (int k = 0; k < n; ++k) {
    if (ms) ms[k] = 0.0;
    if (launches) launches[k] = 0;
  }
  const int n_rec = t_timing ? t_timing->n : 0;
  for (int i = 0; i < n_rec; ++i) {
    const TimedLaunch& s = t_timing->slot[i];
    float t = 0.f;
    if (hipEventSynchronize(s.b) != hipSuccess || hipEventElapsedTime(&t, s.a, s.b) != hipSuccess)
      return MSA_ERR_HIP;
    if (s.kernel < n) {
      if (ms) ms[s.kernel] += t;
      if (launches) launches[s.kernel] += 1;
    }
  }
  return MSA_OK;
}

}  // extern "C"
