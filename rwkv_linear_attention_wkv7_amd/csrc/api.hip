// C-ABI entry points (include/wkv7.h): argument validation, workspace carving
// and the launch sequences of the WKV7 and time-mix calls.  Validation runs
// before anything is enqueued, so every error path can be exercised without
// a GPU.

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/wkv7.h"
#include "common.hpp"
#include "gdn.hpp"
#include "moba.hpp"
#include "optim.hpp"
#include "stack_kernels.hpp"
#include "timemix_kernels.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(WKV7_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIPCHK(expr, what)                      \
  do {                                          \
    hipError_t e_ = (expr);                     \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_tok_ptr(const void* p, const char* name, int dtype, bool required) {
  if (!p) return required ? fail(WKV7_EINVAL, "%s is NULL", name) : WKV7_OK;
  if (!aligned(p, dtype == WKV7_BF16 ? 8 : 16))
    return fail(WKV7_EINVAL, "%s is not %d-byte aligned", name, dtype == WKV7_BF16 ? 8 : 16);
  return WKV7_OK;
}

int check_f32_ptr(const void* p, const char* name, bool required) {
  return check_tok_ptr(p, name, WKV7_F32, required);
}

int check_wkv_shape(int B, int T, int H, int N, int dtype) {
  if (N != WKV7_N) return fail(WKV7_EINVAL, "head size N=%d unsupported (must be 64)", N);
  if (B < 1 || T < 1 || H < 1) return fail(WKV7_EINVAL, "B, T, H must be >= 1 (got %d, %d, %d)", B, T, H);
  if (dtype != WKV7_F32 && dtype != WKV7_BF16) return fail(WKV7_EINVAL, "unknown dtype %d", dtype);
  if ((size_t)B * T * H * N > ((size_t)1 << 40)) return fail(WKV7_EINVAL, "problem too large");
  return WKV7_OK;
}

size_t tok_bytes(int B, int T, int H, int dtype) {
  return (size_t)B * T * H * WKV7_N * (dtype == WKV7_BF16 ? 2 : 4);
}
size_t state_bytes(int B, int H) { return (size_t)B * H * WKV7_N * WKV7_N * sizeof(float); }

// checkpoint states plus the forward's per-token sa (see wkv7_ckpt_sa)
size_t ckpt_floats(int B, int T, int H) { return wkv7_ckpt_total_floats(B, T, H); }

// bump allocator over a workspace (or a dry run for size queries)
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  float* take(size_t nfloats) {
    off = (off + 255) & ~(size_t)255;
    float* p = base ? (float*)(base + off) : nullptr;
    off += nfloats * sizeof(float);
    return p;
  }
};

#define CHK(x)                 \
  do {                         \
    int rc_ = (x);             \
    if (rc_ != WKV7_OK) return rc_; \
  } while (0)

// Byte ranges a call reads and writes.  check() fails with WKV7_EINVAL when a
// written range overlaps any other range (read or written); ranges that are
// only read may overlap.  NULL pointers and empty ranges are skipped.
// Permitted in-place updates (s0 == sT, the decode state) are entered once,
// as written.
struct Spans {
  struct S {
    uintptr_t lo, hi;
    bool w;
    const char* name;
  };
  std::vector<S> v;
  void rd(const void* p, size_t bytes, const char* n) {
    if (p && bytes) v.push_back({(uintptr_t)p, (uintptr_t)p + bytes, false, n});
  }
  void wr(const void* p, size_t bytes, const char* n) {
    if (p && bytes) v.push_back({(uintptr_t)p, (uintptr_t)p + bytes, true, n});
  }
  int check() {
    std::sort(v.begin(), v.end(), [](const S& a, const S& b) { return a.lo < b.lo; });
    // sweep in address order: the furthest end of every range so far and of
    // every written range so far
    uintptr_t end_any = 0, end_w = 0;
    const char *n_any = "", *n_w = "";
    for (const S& x : v) {
      if (x.lo < end_w) return fail(WKV7_EINVAL, "%s overlaps %s (written)", x.name, n_w);
      if (x.w && x.lo < end_any) return fail(WKV7_EINVAL, "%s (written) overlaps %s", x.name, n_any);
      if (x.hi > end_any) { end_any = x.hi; n_any = x.name; }
      if (x.w && x.hi > end_w) { end_w = x.hi; n_w = x.name; }
    }
    return WKV7_OK;
  }
};

// Optional caller-owned side stream: ev[0] fork, ev[1] and ev[2]
// intermediate fork points, ev[3] join.  nullptr when none (or when it is the
// caller's stream itself): everything then runs on the caller's stream.
int check_side(const wkv7_side* side, hipStream_t st, const wkv7_side*& use) {
  use = nullptr;
  if (!side) return WKV7_OK;
  if (!side->stream) return fail(WKV7_EINVAL, "side->stream is NULL");
  for (int i = 0; i < 4; i++)
    if (!side->ev[i]) return fail(WKV7_EINVAL, "side->ev[%d] is NULL", i);
  if (side->stream != st) use = side;
  return WKV7_OK;
}

}  // namespace

// ------------------------------------------------------------------ WKV7 --
extern "C" const char* wkv7_last_error(void) { return g_err; }

extern "C" int wkv7_side_create(wkv7_side* side) {
  g_err[0] = 0;
  if (!side) return fail(WKV7_EINVAL, "side is NULL");
  memset(side, 0, sizeof(*side));
  hipError_t e = hipStreamCreateWithFlags(&side->stream, hipStreamNonBlocking);
  for (int i = 0; i < 4 && e == hipSuccess; i++)
    e = hipEventCreateWithFlags(&side->ev[i], hipEventDisableTiming);
  if (e != hipSuccess) {
    (void)wkv7_side_destroy(side);
    return hip_fail(e, "wkv7_side_create");
  }
  return WKV7_OK;
}

extern "C" int wkv7_side_destroy(wkv7_side* side) {
  g_err[0] = 0;
  if (!side) return WKV7_OK;
  hipError_t e = hipSuccess, x;
  for (int i = 0; i < 4; i++)
    if (side->ev[i] && (x = hipEventDestroy(side->ev[i])) != hipSuccess && e == hipSuccess) e = x;
  if (side->stream && (x = hipStreamDestroy(side->stream)) != hipSuccess && e == hipSuccess) e = x;
  memset(side, 0, sizeof(*side));
  return e == hipSuccess ? WKV7_OK : hip_fail(e, "wkv7_side_destroy");
}

extern "C" int wkv7_checkpoint_interval(void) { return wkv7_ckpt_interval_const(); }

extern "C" size_t wkv7_checkpoint_floats(int B, int T, int H, int N) {
  if (N != WKV7_N || B < 1 || T < 1 || H < 1) return 0;
  return ckpt_floats(B, T, H);
}

extern "C" size_t wkv7_forward_workspace_bytes(int B, int T, int H, int N) {
  if (N != WKV7_N || B < 1 || T < 1 || H < 1) return 0;
  return wkv7_use_chunked(T) ? wkv7_chunk_ws_floats(B, T, H) * sizeof(float) : 0;
}

extern "C" int wkv7_forward(int B, int T, int H, int N, int dtype, const void* r, const void* w,
                            const void* k, const void* v, const void* a, const void* b,
                            const float* s0, void* y, float* sT, float* ckpt, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  CHK(check_wkv_shape(B, T, H, N, dtype));
  CHK(check_tok_ptr(r, "r", dtype, true));
  CHK(check_tok_ptr(w, "w", dtype, true));
  CHK(check_tok_ptr(k, "k", dtype, true));
  CHK(check_tok_ptr(v, "v", dtype, true));
  CHK(check_tok_ptr(a, "a", dtype, true));
  CHK(check_tok_ptr(b, "b", dtype, true));
  CHK(check_tok_ptr(y, "y", dtype, true));
  CHK(check_f32_ptr(s0, "s0", false));
  CHK(check_f32_ptr(sT, "sT", false));
  CHK(check_f32_ptr(ckpt, "ckpt", false));
  float* cws = nullptr;
  if (ws) {
    const size_t need = wkv7_forward_workspace_bytes(B, T, H, N);
    if (ws_bytes < need)
      return fail(WKV7_ENOSPC, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    CHK(check_f32_ptr(ws, "ws", true));
    if (need) cws = static_cast<float*>(ws);
  }
  {
    const size_t tb = tok_bytes(B, T, H, dtype), sb = state_bytes(B, H);
    Spans sp;
    sp.rd(r, tb, "r"); sp.rd(w, tb, "w"); sp.rd(k, tb, "k");
    sp.rd(v, tb, "v"); sp.rd(a, tb, "a"); sp.rd(b, tb, "b");
    if (s0 != sT) sp.rd(s0, sb, "s0");  // s0 == sT: the state is updated in place
    sp.wr(y, tb, "y");
    sp.wr(sT, sb, "sT");
    sp.wr(ckpt, ckpt_floats(B, T, H) * sizeof(float), "ckpt");
    if (cws) sp.wr(cws, wkv7_forward_workspace_bytes(B, T, H, N), "ws");
    CHK(sp.check());
  }
  HIPCHK(wkv7_launch_forward(dtype, B, T, H, r, w, k, v, a, b, s0, y, sT, ckpt, cws, stream),
         "wkv7_forward launch");
  return WKV7_OK;
}

namespace {
// fp32 floats of the region both backward paths share (only one of them
// produces results): the two-pass path's dsa and boundary state gradients,
// or the single-pass path's column partials.
size_t wkv7_bwd_region_floats(int B, int T, int H) {
  Carver one(nullptr), two(nullptr);
  one.take(wkv7_bwd_partial_floats(B, T, H));
  two.take(wkv7_bwd2_ws_floats(B, T, H));
  return (std::max(one.off, two.off) + sizeof(float) - 1) / sizeof(float);
}
}  // namespace

extern "C" size_t wkv7_backward_workspace_bytes(int B, int T, int H, int N, int have_ckpt) {
  if (N != WKV7_N || B < 1 || T < 1 || H < 1) return 0;
  Carver c(nullptr);
  c.take(wkv7_bwd_region_floats(B, T, H));
  c.take(1);  // path flag
  if (!have_ckpt) c.take(ckpt_floats(B, T, H));
  return c.off;
}

namespace {
int wkv7_backward_run(int B, int T, int H, int dtype, const void* r, const void* w, const void* k,
                      const void* v, const void* a, const void* b, const float* s0,
                      const float* ckpt, const void* dy, const float* dsT, void* dr, void* dw,
                      void* dk, void* dv, void* da, void* db, float* ds0, void* ws,
                      const wkv7_side* sd, hipStream_t stream);
}  // namespace

extern "C" int wkv7_backward(int B, int T, int H, int N, int dtype, const void* r, const void* w,
                             const void* k, const void* v, const void* a, const void* b,
                             const float* s0, const float* ckpt, const void* dy, const float* dsT,
                             void* dr, void* dw, void* dk, void* dv, void* da, void* db, float* ds0,
                             void* ws, size_t ws_bytes, const wkv7_side* side, hipStream_t stream) {
  g_err[0] = 0;
  CHK(check_wkv_shape(B, T, H, N, dtype));
  const char* names[] = {"r", "w", "k", "v", "a", "b", "dy", "dr", "dw", "dk", "dv", "da", "db"};
  const void* ptrs[] = {r, w, k, v, a, b, dy, dr, dw, dk, dv, da, db};
  for (int i = 0; i < 13; i++) CHK(check_tok_ptr(ptrs[i], names[i], dtype, true));
  CHK(check_f32_ptr(s0, "s0", false));
  CHK(check_f32_ptr(ckpt, "ckpt", false));
  CHK(check_f32_ptr(dsT, "dsT", false));
  CHK(check_f32_ptr(ds0, "ds0", false));
  const size_t need = wkv7_backward_workspace_bytes(B, T, H, N, ckpt != nullptr);
  if (!ws || ws_bytes < need)
    return fail(WKV7_ENOSPC, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  CHK(check_f32_ptr(ws, "ws", true));
  const wkv7_side* sd = nullptr;
  CHK(check_side(side, stream, sd));
  {
    const size_t tb = tok_bytes(B, T, H, dtype), sb = state_bytes(B, H);
    Spans sp;
    for (int i = 0; i < 7; i++) sp.rd(ptrs[i], tb, names[i]);
    for (int i = 7; i < 13; i++) sp.wr(ptrs[i], tb, names[i]);
    sp.rd(s0, sb, "s0");
    sp.rd(dsT, sb, "dsT");
    sp.rd(ckpt, ckpt_floats(B, T, H) * sizeof(float), "ckpt");
    sp.wr(ds0, sb, "ds0");
    sp.wr(ws, need, "ws");
    CHK(sp.check());
  }
  return wkv7_backward_run(B, T, H, dtype, r, w, k, v, a, b, s0, ckpt, dy, dsT, dr, dw, dk, dv, da,
                           db, ds0, ws, sd, stream);
}

namespace {
// The backward's launches, arguments already validated; ws holds
// wkv7_backward_workspace_bytes(.., ckpt != NULL).
int wkv7_backward_run(int B, int T, int H, int dtype, const void* r, const void* w, const void* k,
                      const void* v, const void* a, const void* b, const float* s0,
                      const float* ckpt, const void* dy, const float* dsT, void* dr, void* dw,
                      void* dk, void* dv, void* da, void* db, float* ds0, void* ws,
                      const wkv7_side* sd, hipStream_t stream) {
  Carver cv(ws);
  float* region = cv.take(wkv7_bwd_region_floats(B, T, H));
  int* gate = reinterpret_cast<int*>(cv.take(1));
  const float* ck = ckpt;
  if (!ck) {
    float* tmp = cv.take(ckpt_floats(B, T, H));
    HIPCHK(wkv7_launch_forward(dtype, B, T, H, r, w, k, v, a, b, s0, nullptr, nullptr, tmp, nullptr,
                               stream),
           "wkv7_backward checkpoint recompute");
    ck = tmp;
  }
  float* part = region;
  (void)sd;  // every launch of this call runs on `stream`
  // A call of a few chunks (at most 512 workgroups of the products kernel)
  // is launch-latency bound: the single-pass kernels alone, two launches,
  // take less time than the flag, scan and products (B=1 T=64 H=4: 31 against
  // 39 us).
  if ((long)B * H * ((T + wkv7_ckpt_interval_const() - 1) / wkv7_ckpt_interval_const()) <= 512) {
    HIPCHK(wkv7_launch_backward(dtype, B, T, H, r, w, k, v, a, b, dy, ck, dsT, dr, dw, dk, dv, da,
                                db, ds0, part, nullptr, stream),
           "wkv7_backward launch");
    return WKV7_OK;
  }
  // The two-pass backward (reverse state-gradient scan, then per-chunk
  // matrix-core products) serves decays in [1/8, 1]; its scan raises the
  // flag on any other decay, and then the single-pass kernels, launched after
  // it with the same flag, produce the results instead (the products return
  // at once).  Both use the one region.
  HIPCHK(stk_launch_fill_zero(reinterpret_cast<float*>(gate), 1, stream), "wkv7_backward flag");
  HIPCHK(wkv7_launch_backward2(dtype, B, T, H, r, w, k, v, a, b, dy, ck, dsT, dr, dw, dk, dv, da,
                               db, ds0, region, gate, stream),
         "wkv7_backward launch");
  HIPCHK(wkv7_launch_backward(dtype, B, T, H, r, w, k, v, a, b, dy, ck, dsT, dr, dw, dk, dv, da,
                              db, ds0, part, gate, stream),
         "wkv7_backward launch");
  return WKV7_OK;
}
}  // namespace

// ---------------------------------------------- backward without allocation --
// Fixed device scratch of wkv7_backward_noalloc, for callers that cannot
// allocate (graph capture, tight serving loops).  Each device holds its own
// copy until the process ends; host code never uses the array's name as an
// address, only the pointer hipGetSymbolAddress returns for the current
// device (looked up once per device and kept).  Every call on a device
// shares that device's copy: calls that overlap on one device race.
namespace {
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
constexpr int NOALLOC_MAX_DEVICES = 64;
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_ptr[NOALLOC_MAX_DEVICES];
std::mutex g_scratch_mu;

int scratch_of_current_device(void** out) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
    return fail(WKV7_EINVAL, "device %d beyond the %d the fixed scratch serves", dev,
                NOALLOC_MAX_DEVICES);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
      if (!p) return fail(WKV7_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return WKV7_OK;
}
}  // namespace

extern "C" int wkv7_backward_noalloc(int B, int T, int H, int N, int dtype, const void* r,
                                     const void* w, const void* k, const void* v, const void* a,
                                     const void* b, const float* s0, const float* ckpt,
                                     const void* dy, const float* dsT, void* dr, void* dw,
                                     void* dk, void* dv, void* da, void* db, float* ds0,
                                     const wkv7_side* side, hipStream_t stream) {
  g_err[0] = 0;
  CHK(check_wkv_shape(B, T, H, N, dtype));
  const char* names[] = {"r", "w", "k", "v", "a", "b", "dy", "dr", "dw", "dk", "dv", "da", "db"};
  const void* ptrs[] = {r, w, k, v, a, b, dy, dr, dw, dk, dv, da, db};
  for (int i = 0; i < 13; i++) CHK(check_tok_ptr(ptrs[i], names[i], dtype, true));
  CHK(check_f32_ptr(s0, "s0", false));
  CHK(check_f32_ptr(ckpt, "ckpt", false));
  CHK(check_f32_ptr(dsT, "dsT", false));
  CHK(check_f32_ptr(ds0, "ds0", false));
  const size_t need = wkv7_backward_workspace_bytes(B, T, H, N, ckpt != nullptr);
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(WKV7_ENOSPC, "this shape needs %zu bytes of scratch; the fixed scratch of "
                "wkv7_backward_noalloc holds %zu (use wkv7_backward with a workspace)",
                need, NOALLOC_SCRATCH_BYTES);
  const wkv7_side* sd = nullptr;
  CHK(check_side(side, stream, sd));
  {
    const size_t tb = tok_bytes(B, T, H, dtype), sb = state_bytes(B, H);
    Spans sp;
    for (int i = 0; i < 7; i++) sp.rd(ptrs[i], tb, names[i]);
    for (int i = 7; i < 13; i++) sp.wr(ptrs[i], tb, names[i]);
    sp.rd(s0, sb, "s0");
    sp.rd(dsT, sb, "dsT");
    sp.rd(ckpt, ckpt_floats(B, T, H) * sizeof(float), "ckpt");
    sp.wr(ds0, sb, "ds0");
    CHK(sp.check());
  }
  void* ws = nullptr;
  CHK(scratch_of_current_device(&ws));
  return wkv7_backward_run(B, T, H, dtype, r, w, k, v, a, b, s0, ckpt, dy, dsT, dr, dw, dk, dv, da,
                           db, ds0, ws, sd, stream);
}

extern "C" int wkv7_step(int B, int H, int N, int dtype, const void* r, const void* w,
                         const void* k, const void* v, const void* a, const void* b, float* state,
                         void* y, hipStream_t stream) {
  g_err[0] = 0;
  CHK(check_wkv_shape(B, 1, H, N, dtype));
  const char* names[] = {"r", "w", "k", "v", "a", "b", "y"};
  const void* ptrs[] = {r, w, k, v, a, b, y};
  for (int i = 0; i < 7; i++) CHK(check_tok_ptr(ptrs[i], names[i], dtype, true));
  CHK(check_f32_ptr(state, "state", true));
  {
    const size_t tb = tok_bytes(B, 1, H, dtype);
    Spans sp;
    for (int i = 0; i < 6; i++) sp.rd(ptrs[i], tb, names[i]);
    sp.wr(y, tb, "y");
    sp.wr(state, state_bytes(B, H), "state");  // read and written in place
    CHK(sp.check());
  }
  HIPCHK(wkv7_launch_step(dtype, B, H, r, w, k, v, a, b, state, y, stream), "wkv7_step launch");
  return WKV7_OK;
}

// -------------------------------------------------------------- time-mix --

namespace {

struct TmCache {
  float *xr, *xw, *xk, *xv, *xa, *xg;
  float *r, *k, *v, *tw, *ow, *la, *oa, *sg, *g, *lv, *ov;
  float *w, *a, *kk, *kmod, *vmod, *A, *Bv, *y, *tg;
  float *mean, *rstd, *alpha, *ckpt;
  float* wkv_ws;  // chunked-forward records (nullptr: token-sequential forward)
};

void carve_cache(Carver& c, const tm_shape* s, int B, int T, TmCache& m, bool with_ckpt = true) {
  const size_t BT = (size_t)B * T, tok = BT * s->C;
  float** toks[] = {&m.xr, &m.xw, &m.xk, &m.xv, &m.xa, &m.xg, &m.r, &m.k, &m.v, &m.ow, &m.oa,
                    &m.g, &m.w, &m.a, &m.kk, &m.kmod, &m.vmod, &m.A, &m.Bv, &m.y, &m.tg};
  for (float** p : toks) *p = c.take(tok);
  m.tw = c.take(BT * s->Dw);
  m.la = c.take(BT * s->Da);
  m.sg = c.take(BT * s->Dg);
  if (s->layer_id > 0) {
    m.lv = c.take(BT * s->Dv);
    m.ov = c.take(tok);
  } else {
    m.lv = m.ov = nullptr;
  }
  m.mean = c.take(BT * s->H);
  m.rstd = c.take(BT * s->H);
  m.alpha = c.take(BT * s->H);
  m.ckpt = with_ckpt ? c.take(ckpt_floats(B, T, s->H)) : nullptr;
  m.wkv_ws = nullptr;  // the time-mix runs the (faster) token-sequential recurrence
}

struct TmBwdBufs {
  float *dtg, *dg, *dy_wkv, *dr, *dkmod, *dvmod, *gr, *gw, *gk, *gv, *gA, *gB;
  float *dk, *dv, *dpre_a, *dpre_w, *dpre_v, *d_la, *d_lw, *d_lg, *d_lv;
  float *dxr, *dxw, *dxk, *dxv, *dxa, *dxg, *part_post, *part_pre, *part_shift, *splitk, *out_tmp;
  float* wkv_ws;  // the two-pass WKV7 backward's dsa and boundary state gradients
};

// split-K factor for a weight gradient [Mo][No] reduced over BT tokens
int splitk_for(int Mo, int No, int BT) {
  // workspace for either precision's choice
  return std::max(gemm_splitk_slices(GEMM_F32, Mo, No, BT), gemm_splitk_slices(GEMM_BF16, Mo, No, BT));
}

size_t splitk_scratch(const tm_shape* s, int BT) {
  const int C = s->C;
  size_t best = 0;
  const int dims[] = {C, s->Dw, s->Da, s->Dg, s->layer_id > 0 ? s->Dv : 0};
  for (int d : dims) {
    if (d <= 0) continue;
    const size_t x = (size_t)splitk_for(C, d, BT) * C * d;
    if (x > best) best = x;
    const size_t y = (size_t)splitk_for(d, C, BT) * C * d;
    if (y > best) best = y;
  }
  return best;
}

void carve_bwd(Carver& c, const tm_shape* s, int B, int T, TmBwdBufs& m) {
  const size_t BT = (size_t)B * T, tok = BT * s->C;
  float** toks[] = {&m.dtg, &m.dg, &m.dy_wkv, &m.dr, &m.dkmod, &m.dvmod, &m.gr, &m.gw, &m.gk,
                    &m.gv, &m.gA, &m.gB, &m.dk, &m.dv, &m.dpre_a, &m.dpre_w, &m.dxr, &m.dxw,
                    &m.dxk, &m.dxv, &m.dxa, &m.dxg};
  for (float** p : toks) *p = c.take(tok);
  m.dpre_v = s->layer_id > 0 ? c.take(tok) : nullptr;
  m.d_la = c.take(BT * s->Da);
  m.d_lw = c.take(BT * s->Dw);
  m.d_lg = c.take(BT * s->Dg);
  m.d_lv = s->layer_id > 0 ? c.take(BT * s->Dv) : nullptr;
  const int nblk = tm_num_token_blocks((int)BT);
  m.part_post = c.take((size_t)3 * nblk * s->C);
  m.part_pre = c.take((size_t)5 * nblk * s->C);
  m.part_shift = c.take((size_t)6 * nblk * s->C);
  m.splitk = c.take(splitk_scratch(s, (int)BT));
  m.wkv_ws = c.take(wkv7_bwd2_ws_floats(B, T, s->H));
  m.out_tmp = nullptr;
}

int check_tm_shape(const tm_shape* s, int B, int T) {
  if (!s) return fail(WKV7_EINVAL, "shape is NULL");
  if (s->N != WKV7_N) return fail(WKV7_EINVAL, "head size N=%d unsupported (must be 64)", s->N);
  if (s->H < 1 || s->C != s->H * s->N) return fail(WKV7_EINVAL, "C=%d must equal H*N=%d*%d", s->C, s->H, s->N);
  if (B < 1 || T < 1) return fail(WKV7_EINVAL, "B, T must be >= 1 (got %d, %d)", B, T);
  if (s->Dw < 4 || s->Da < 4 || s->Dg < 4 || s->Dw % 4 || s->Da % 4 || s->Dg % 4)
    return fail(WKV7_EINVAL, "LoRA ranks Dw, Da, Dg must be positive multiples of 4");
  if (s->layer_id < 0) return fail(WKV7_EINVAL, "layer_id must be >= 0");
  if (s->layer_id > 0 && (s->Dv < 4 || s->Dv % 4))
    return fail(WKV7_EINVAL, "LoRA rank Dv must be a positive multiple of 4 for layer_id > 0");
  if ((size_t)B * T * s->C > ((size_t)1 << 36)) return fail(WKV7_EINVAL, "problem too large");
  return WKV7_OK;
}

int check_weights(const tm_shape* s, const tm_weights* W) {
  if (!W) return fail(WKV7_EINVAL, "weights is NULL");
  const float* req[] = {W->mu_r, W->mu_w, W->mu_k, W->mu_v, W->mu_a, W->mu_g, W->Wr, W->Wk, W->Wv,
                        W->Wo, W->w0, W->W1, W->W2, W->a0, W->A1, W->A2, W->G1, W->G2, W->k_k,
                        W->k_a, W->r_k, W->ln_w, W->ln_b};
  const char* nm[] = {"mu_r", "mu_w", "mu_k", "mu_v", "mu_a", "mu_g", "Wr", "Wk", "Wv", "Wo",
                      "w0", "W1", "W2", "a0", "A1", "A2", "G1", "G2", "k_k", "k_a", "r_k",
                      "ln_w", "ln_b"};
  for (int i = 0; i < 23; i++) CHK(check_f32_ptr(req[i], nm[i], true));
  if (s->layer_id > 0) {
    CHK(check_f32_ptr(W->v0, "v0", true));
    CHK(check_f32_ptr(W->V1, "V1", true));
    CHK(check_f32_ptr(W->V2, "V2", true));
  }
  return WKV7_OK;
}

// Byte ranges of a time-mix block's weights (or gradients, same shapes).
template <typename WT>
void tm_weight_spans(Spans& sp, const tm_shape* s, const WT* W, bool written) {
  const size_t C = s->C, f = sizeof(float);
  auto add = [&](const void* p, size_t n, const char* nm) {
    if (written) sp.wr(p, n * f, nm); else sp.rd(p, n * f, nm);
  };
  const void* vec[] = {W->mu_r, W->mu_w, W->mu_k, W->mu_v, W->mu_a, W->mu_g, W->w0, W->a0,
                       W->k_k, W->k_a, W->r_k, W->ln_w, W->ln_b};
  const char* vn[] = {"mu_r", "mu_w", "mu_k", "mu_v", "mu_a", "mu_g", "w0", "a0", "k_k", "k_a",
                      "r_k", "ln_w", "ln_b"};
  for (int i = 0; i < 13; i++) add(vec[i], C, vn[i]);
  add(W->Wr, C * C, "Wr"); add(W->Wk, C * C, "Wk"); add(W->Wv, C * C, "Wv"); add(W->Wo, C * C, "Wo");
  add(W->W1, C * s->Dw, "W1"); add(W->W2, C * s->Dw, "W2");
  add(W->A1, C * s->Da, "A1"); add(W->A2, C * s->Da, "A2");
  add(W->G1, C * s->Dg, "G1"); add(W->G2, C * s->Dg, "G2");
  if (s->layer_id > 0) {
    add(W->v0, C, "v0"); add(W->V1, C * s->Dv, "V1"); add(W->V2, C * s->Dv, "V2");
  }
}

// decode: T == 1 with the WKV state updated in place (s0 == sT, no checkpoint),
// run by one fused kernel (pre-WKV, the step on the state in place, post-WKV).
// out = out_beta * out + tg Wo, or resid + tg Wo when resid is given
// (out_proj = false: tg is left in m.tg and the caller applies Wo).
int tm_forward_impl(const tm_shape* s, const tm_weights* W, int B, int T, const float* x,
                    const float* x_prev, float* v_first, const float* s0, float* sT, float* out,
                    float* x_last, const TmCache& m, hipStream_t st, bool decode = false,
                    float out_beta = 0.f, int prec = GEMM_F32, bool shifted = false,
                    bool out_proj = true, const float* resid = nullptr, __bf16* x16 = nullptr) {
  // x16: NULL or 3 BT C bf16 of scratch for the shift's bf16 copies of xr,
  // xk, xv, which the r/k/v products then take as their A operands
  const int BT = B * T, C = s->C;
  if (s->layer_id > 0 && (!m.lv || !m.ov))
    return fail(WKV7_EHIP, "internal: activation set without value-residual buffers for layer %d",
                s->layer_id);
  TmFwd p;
  memset(&p, 0, sizeof(p));
  p.BT = BT; p.T = T; p.C = C; p.layer_id = s->layer_id;
  p.x = x; p.x_prev = x_prev;
  p.mu_r = W->mu_r; p.mu_w = W->mu_w; p.mu_k = W->mu_k; p.mu_v = W->mu_v; p.mu_a = W->mu_a; p.mu_g = W->mu_g;
  p.xr = m.xr; p.xw = m.xw; p.xk = m.xk; p.xv = m.xv; p.xa = m.xa; p.xg = m.xg; p.x_last = x_last;
  const bool rkv16 = x16 && !shifted && prec == GEMM_BF16;  // the copies exist only if the shift runs here
  if (rkv16) {
    p.xr16 = x16;
    p.xk16 = x16 + (size_t)BT * C;
    p.xv16 = x16 + 2 * (size_t)BT * C;
    if (!decode) p.tg16 = x16;  // after the r/k/v products have read xr16
  }
  p.k = m.k; p.v = m.v; p.ow = m.ow; p.oa = m.oa; p.ov = m.ov;
  p.w0 = W->w0; p.a0 = W->a0; p.v0 = W->v0; p.k_k = W->k_k; p.k_a = W->k_a;
  p.v_first = v_first;
  p.w = m.w; p.a = m.a; p.kk = m.kk; p.kmod = m.kmod; p.vmod = m.vmod; p.A = m.A; p.Bv = m.Bv;
  p.y = m.y; p.r = m.r; p.g = m.g; p.r_k = W->r_k; p.ln_w = W->ln_w; p.ln_b = W->ln_b;
  p.tg = m.tg; p.mean = m.mean; p.rstd = m.rstd; p.alpha = m.alpha;

  // shifted: the caller already wrote xr..xg (and x_last) with its LayerNorm
  if (!shifted) HIPCHK(tm_launch_shift_fwd(p, st), "token shift");
  auto prob = [](int M, int N, int K, const float* A, int lda, const float* B, int ldb, float* C,
                 int ldc, int epi) {
    return GemmProblem{M, N, K, A, lda, B, ldb, C, ldc, 0.f, epi, nullptr, nullptr};
  };
  {  // r, k, v projections and the LoRA down-projections (tanh for w, sigmoid
     // for g).  Decode (latency bound, 2048-row products) runs them as one
     // launch; larger token batches as two, so the thin LoRA products keep
     // tiles of their own size.
    GemmBatch g;
    g.count = 3;
    g.p[0] = prob(BT, C, C, m.xr, C, W->Wr, C, m.r, C, EPI_NONE);
    g.p[1] = prob(BT, C, C, m.xk, C, W->Wk, C, m.k, C, EPI_NONE);
    g.p[2] = prob(BT, C, C, m.xv, C, W->Wv, C, m.v, C, EPI_NONE);
    if (rkv16) {
      g.p[0].A16 = p.xr16;
      g.p[1].A16 = p.xk16;
      g.p[2].A16 = p.xv16;
    }
    GemmBatch l;
    l.count = 3;
    l.p[0] = prob(BT, s->Dw, C, m.xw, C, W->W1, s->Dw, m.tw, s->Dw, EPI_TANH);
    l.p[1] = prob(BT, s->Da, C, m.xa, C, W->A1, s->Da, m.la, s->Da, EPI_NONE);
    l.p[2] = prob(BT, s->Dg, C, m.xg, C, W->G1, s->Dg, m.sg, s->Dg, EPI_SIGMOID);
    if (s->layer_id > 0) l.p[l.count++] = prob(BT, s->Dv, C, m.xv, C, W->V1, s->Dv, m.lv, s->Dv, EPI_NONE);
    if (decode) {
      for (int i = 0; i < l.count; i++) g.p[g.count++] = l.p[i];
      HIPCHK(gemm_batch(prec, false, false, g, st), "r/k/v + lora down");
    } else {
      HIPCHK(gemm_batch(prec, false, false, g, st), "r/k/v proj");
      HIPCHK(gemm_batch(prec, false, false, l, st), "lora down");
    }
  }
  {  // LoRA up-projections: one launch
    GemmBatch g;
    g.count = 3;
    g.p[0] = prob(BT, C, s->Dw, m.tw, s->Dw, W->W2, C, m.ow, C, EPI_NONE);
    g.p[1] = prob(BT, C, s->Da, m.la, s->Da, W->A2, C, m.oa, C, EPI_NONE);
    g.p[2] = prob(BT, C, s->Dg, m.sg, s->Dg, W->G2, C, m.g, C, EPI_NONE);
    if (s->layer_id > 0) g.p[g.count++] = prob(BT, C, s->Dv, m.lv, s->Dv, W->V2, C, m.ov, C, EPI_NONE);
    HIPCHK(gemm_batch(prec, false, false, g, st), "lora up");
  }
  if (decode) {
    HIPCHK(tm_launch_step_fused(p, sT, st), "pre-wkv + wkv7 step + post-wkv");
  } else {
    HIPCHK(tm_launch_pre_fwd(p, st), "pre-wkv");
    HIPCHK(wkv7_launch_forward(WKV7_F32, B, T, s->H, m.r, m.w, m.kmod, m.vmod, m.A, m.Bv, s0, m.y, sT,
                               m.ckpt, m.wkv_ws, st), "wkv7 forward");
    HIPCHK(tm_launch_post_fwd(p, st), "post-wkv");
  }
  if (out_proj && resid)  // out = resid + tg Wo
    HIPCHK(gemm_run_x(prec, false, false, BT, C, C, m.tg, C, W->Wo, C, out, C, 0.f, EPI_ADD, resid, 1, nullptr, st,
                      p.tg16, nullptr), "o proj");
  else if (out_proj)
    HIPCHK(gemm_run_x(prec, false, false, BT, C, C, m.tg, C, W->Wo, C, out, C, out_beta, 0, nullptr, 1, nullptr, st,
                      p.tg16, nullptr), "o proj");
  return WKV7_OK;
}

}  // namespace

namespace {
// Time-mix backward given the forward cache m and scratch bb.  dvf_accum:
// dv_first_out += (instead of =) for layer > 0 (a stack sums it over layers).
int tm_backward_impl(const tm_shape* s, const tm_weights* W, int B, int T, const float* x,
                     const float* x_prev, const float* v_first, const float* s0, const float* dout,
                     const float* dsT, const TmCache& m, const TmBwdBufs& bb, tm_grads* G, float* dx,
                     float* dx_prev, const float* dv_first_in, float* dv_first_out, bool dvf_accum,
                     float* ds0, hipStream_t st, int prec, const wkv7_side* sd,
                     __bf16* x16 = nullptr, const __bf16* dout16 = nullptr) {
  // x16: NULL or 3 BT C bf16 of scratch for the pre-WKV backward's bf16
  // copies of dr, dk, dv, which the r/k/v input-gradient products then take
  // as their A operands; dout16: NULL or dout already rounded to bf16
  const int BT = B * T, C = s->C, L = s->layer_id;

  // The weight gradients (X^T dY products, split along the tokens) feed
  // nothing else in the backward, so they run on the library side stream
  // while this stream carries on with the input-gradient chain.  Each waits
  // for the point of this stream where its operands are complete (fork:
  // start; mark[0]: after the pre-WKV backward; mark[1]: after the LoRA
  // input gradients), only they use the split-K scratch, and this stream
  // joins the side stream before returning, so the next call may reuse
  // every buffer.
  // sd: the caller's side stream (nullptr: none, everything on st)
  hipStream_t ss = sd ? sd->stream : st;
  auto fork_at = [&](int ev) -> hipError_t {
    if (!sd) return hipSuccess;
    hipError_t r = hipEventRecord(sd->ev[ev], st);
    return r != hipSuccess ? r : hipStreamWaitEvent(ss, sd->ev[ev], 0);
  };
  struct Join {  // joins the side stream on every return path
    const wkv7_side* sd;
    hipStream_t st;
    ~Join() {
      if (sd && hipEventRecord(sd->ev[3], sd->stream) == hipSuccess) (void)hipStreamWaitEvent(st, sd->ev[3], 0);
    }
  } join{sd, st};

  HIPCHK(fork_at(0), "backward fork");
  // output projection
  HIPCHK(gemm_run_x(prec, false, true, BT, C, C, dout, C, W->Wo, C, bb.dtg, C, 0.f, 0, nullptr, 1, nullptr, st,
                    prec == GEMM_BF16 ? dout16 : nullptr, nullptr), "dtg");
  HIPCHK(gemm_run(prec, true, false, C, C, BT, m.tg, C, dout, C, G->Wo, C, 0.f, 0, nullptr, splitk_for(C, C, BT), bb.splitk, ss), "dWo");
  TmBwd p;
  memset(&p, 0, sizeof(p));
  p.BT = BT; p.T = T; p.C = C; p.layer_id = L;
  p.dtg = bb.dtg; p.g = m.g; p.y = m.y; p.r = m.r; p.kmod = m.kmod; p.vmod = m.vmod;
  p.mean = m.mean; p.rstd = m.rstd; p.alpha = m.alpha; p.r_k = W->r_k; p.ln_w = W->ln_w; p.ln_b = W->ln_b;
  p.dg = bb.dg; p.dy_wkv = bb.dy_wkv; p.dr = bb.dr; p.dkmod = bb.dkmod; p.dvmod = bb.dvmod;
  p.part_post = bb.part_post;
  p.gr = bb.gr; p.gk = bb.gk; p.gv = bb.gv; p.gw = bb.gw; p.gA = bb.gA; p.gB = bb.gB;
  p.a = m.a; p.kk = m.kk; p.k = m.k; p.w = m.w; p.ow = m.ow; p.ov = m.ov; p.v = m.v;
  p.v_first = v_first; p.k_a = W->k_a; p.k_k = W->k_k; p.w0 = W->w0; p.v0 = W->v0;
  p.dvf_in = L == 0 ? dv_first_in : nullptr;
  p.dk = bb.dk; p.dv = bb.dv; p.dpre_a = bb.dpre_a; p.dpre_w = bb.dpre_w; p.dpre_v = bb.dpre_v;
  p.dvf_out = L > 0 ? dv_first_out : nullptr;
  p.dvf_accum = dvf_accum ? 1 : 0;
  p.part_pre = bb.part_pre;
  p.x = x; p.x_prev = x_prev;
  p.mu_r = W->mu_r; p.mu_w = W->mu_w; p.mu_k = W->mu_k; p.mu_v = W->mu_v; p.mu_a = W->mu_a; p.mu_g = W->mu_g;
  p.dxr = bb.dxr; p.dxw = bb.dxw; p.dxk = bb.dxk; p.dxv = bb.dxv; p.dxa = bb.dxa; p.dxg = bb.dxg;
  p.dx = dx; p.dx_prev = dx_prev; p.part_shift = bb.part_shift;
  if (x16 && prec == GEMM_BF16) {
    p.dr16 = x16;
    p.dk16 = x16 + (size_t)BT * C;
    p.dv16 = x16 + 2 * (size_t)BT * C;
  }

  HIPCHK(tm_launch_post_bwd(p, st), "post-wkv backward");
  // the time-mix decay exp(-0.606531 sigmoid(.)) lies in [0.545, 1]: the
  // two-pass backward applies to every call, no flag needed
  HIPCHK(wkv7_launch_backward2(WKV7_F32, B, T, s->H, m.r, m.w, m.kmod, m.vmod, m.A, m.Bv, bb.dy_wkv,
                               m.ckpt, dsT, bb.gr, bb.gw, bb.gk, bb.gv, bb.gA, bb.gB, ds0,
                               bb.wkv_ws, nullptr, st),
         "wkv7 backward");
  HIPCHK(tm_launch_pre_bwd(p, st), "pre-wkv backward");
  const int Dw = s->Dw, Da = s->Da, Dg = s->Dg, Dv = s->Dv;
  float* sk = bb.splitk;
  HIPCHK(fork_at(1), "backward fork");
  // r, k, v weight gradients (dr from the post-WKV backward, dk and dv from
  // the pre-WKV backward)
  HIPCHK(gemm_run(prec, true, false, C, C, BT, m.xr, C, bb.dr, C, G->Wr, C, 0.f, 0, nullptr, splitk_for(C, C, BT), sk, ss), "dWr");
  HIPCHK(gemm_run(prec, true, false, C, C, BT, m.xk, C, bb.dk, C, G->Wk, C, 0.f, 0, nullptr, splitk_for(C, C, BT), sk, ss), "dWk");
  HIPCHK(gemm_run(prec, true, false, C, C, BT, m.xv, C, bb.dv, C, G->Wv, C, 0.f, 0, nullptr, splitk_for(C, C, BT), sk, ss), "dWv");

  // a: a = sigmoid(a0 + (xa A1) A2)
  HIPCHK(gemm_run(prec, false, true, BT, Da, C, bb.dpre_a, C, W->A2, C, bb.d_la, Da, 0.f, 0, nullptr, 1, nullptr, st), "d_la");
  HIPCHK(gemm_run(prec, true, false, Da, C, BT, m.la, Da, bb.dpre_a, C, G->A2, C, 0.f, 0, nullptr, splitk_for(Da, C, BT), sk, ss), "dA2");
  HIPCHK(gemm_run(prec, false, true, BT, C, Da, bb.d_la, Da, W->A1, Da, bb.dxa, C, 0.f, 0, nullptr, 1, nullptr, st), "dxa");
  // w: w = exp(-c sigmoid(w0 + tanh(xw W1) W2))
  HIPCHK(gemm_run(prec, false, true, BT, Dw, C, bb.dpre_w, C, W->W2, C, bb.d_lw, Dw, 0.f, 3, m.tw, 1, nullptr, st), "d_lw");
  HIPCHK(gemm_run(prec, true, false, Dw, C, BT, m.tw, Dw, bb.dpre_w, C, G->W2, C, 0.f, 0, nullptr, splitk_for(Dw, C, BT), sk, ss), "dW2");
  HIPCHK(gemm_run(prec, false, true, BT, C, Dw, bb.d_lw, Dw, W->W1, Dw, bb.dxw, C, 0.f, 0, nullptr, 1, nullptr, st), "dxw");
  // g: g = sigmoid(xg G1) G2
  HIPCHK(gemm_run(prec, false, true, BT, Dg, C, bb.dg, C, W->G2, C, bb.d_lg, Dg, 0.f, 4, m.sg, 1, nullptr, st), "d_lg");
  HIPCHK(gemm_run(prec, true, false, Dg, C, BT, m.sg, Dg, bb.dg, C, G->G2, C, 0.f, 0, nullptr, splitk_for(Dg, C, BT), sk, ss), "dG2");
  HIPCHK(gemm_run(prec, false, true, BT, C, Dg, bb.d_lg, Dg, W->G1, Dg, bb.dxg, C, 0.f, 0, nullptr, 1, nullptr, st), "dxg");
  // value residual LoRA (layer > 0)
  if (L > 0) {
    HIPCHK(gemm_run(prec, false, true, BT, Dv, C, bb.dpre_v, C, W->V2, C, bb.d_lv, Dv, 0.f, 0, nullptr, 1, nullptr, st), "d_lv");
    HIPCHK(gemm_run(prec, true, false, Dv, C, BT, m.lv, Dv, bb.dpre_v, C, G->V2, C, 0.f, 0, nullptr, splitk_for(Dv, C, BT), sk, ss), "dV2");
    HIPCHK(gemm_run(prec, false, true, BT, C, Dv, bb.d_lv, Dv, W->V1, Dv, bb.dxv, C, 0.f, 0, nullptr, 1, nullptr, st), "dxv lora");
  }
  HIPCHK(fork_at(2), "backward fork");
  HIPCHK(gemm_run(prec, true, false, C, Da, BT, m.xa, C, bb.d_la, Da, G->A1, Da, 0.f, 0, nullptr, splitk_for(C, Da, BT), sk, ss), "dA1");
  HIPCHK(gemm_run(prec, true, false, C, Dw, BT, m.xw, C, bb.d_lw, Dw, G->W1, Dw, 0.f, 0, nullptr, splitk_for(C, Dw, BT), sk, ss), "dW1");
  HIPCHK(gemm_run(prec, true, false, C, Dg, BT, m.xg, C, bb.d_lg, Dg, G->G1, Dg, 0.f, 0, nullptr, splitk_for(C, Dg, BT), sk, ss), "dG1");
  if (L > 0)
    HIPCHK(gemm_run(prec, true, false, C, Dv, BT, m.xv, C, bb.d_lv, Dv, G->V1, Dv, 0.f, 0, nullptr, splitk_for(C, Dv, BT), sk, ss), "dV1");
  // r, k, v projections
  HIPCHK(gemm_run_x(prec, false, true, BT, C, C, bb.dr, C, W->Wr, C, bb.dxr, C, 0.f, 0, nullptr, 1, nullptr, st,
                    p.dr16, nullptr), "dxr");
  HIPCHK(gemm_run_x(prec, false, true, BT, C, C, bb.dk, C, W->Wk, C, bb.dxk, C, 0.f, 0, nullptr, 1, nullptr, st,
                    p.dk16, nullptr), "dxk");
  HIPCHK(gemm_run_x(prec, false, true, BT, C, C, bb.dv, C, W->Wv, C, bb.dxv, C, L > 0 ? 1.f : 0.f, 0, nullptr, 1,
                    nullptr, st, p.dv16, nullptr), "dxv");

  HIPCHK(tm_launch_shift_bwd(p, st), "token shift backward");
  const int nblk = tm_num_token_blocks(BT);
  VecOut o1 = {{G->r_k, G->ln_w, G->ln_b, nullptr, nullptr, nullptr, nullptr, nullptr}};
  HIPCHK(tm_launch_reduce(bb.part_post, 3, nblk, C, o1, st), "reduce post");
  VecOut o2 = {{G->k_a, G->k_k, G->a0, G->w0, L > 0 ? G->v0 : nullptr, nullptr, nullptr, nullptr}};
  HIPCHK(tm_launch_reduce(bb.part_pre, 5, nblk, C, o2, st), "reduce pre");
  VecOut o3 = {{G->mu_r, G->mu_w, G->mu_k, G->mu_v, G->mu_a, G->mu_g, nullptr, nullptr}};
  HIPCHK(tm_launch_reduce(bb.part_shift, 6, nblk, C, o3, st), "reduce shift");
  return WKV7_OK;
}
}  // namespace

extern "C" size_t timemix_cache_bytes(const tm_shape* s, int B, int T) {
  if (check_tm_shape(s, B, T) != WKV7_OK) return 0;
  Carver c(nullptr);
  TmCache m;
  carve_cache(c, s, B, T, m);
  return c.off + 256;
}

extern "C" size_t timemix_forward_workspace_bytes(const tm_shape* s, int B, int T) {
  return timemix_cache_bytes(s, B, T);
}

extern "C" size_t timemix_backward_workspace_bytes(const tm_shape* s, int B, int T) {
  if (check_tm_shape(s, B, T) != WKV7_OK) return 0;
  Carver c(nullptr);
  TmCache m;
  carve_cache(c, s, B, T, m);
  c.take((size_t)B * T * s->C);  // forward output when the cache is recomputed
  TmBwdBufs bb;
  carve_bwd(c, s, B, T, bb);
  return c.off + 256;
}

extern "C" int timemix_forward(const tm_shape* s, const tm_weights* W, int B, int T, const float* x,
                               const float* x_prev, float* v_first, const float* s0, float* sT,
                               float* out, float* x_last, void* cache, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  g_err[0] = 0;
  CHK(check_tm_shape(s, B, T));
  CHK(check_weights(s, W));
  CHK(check_f32_ptr(x, "x", true));
  CHK(check_f32_ptr(x_prev, "x_prev", false));
  CHK(check_f32_ptr(v_first, "v_first", true));
  CHK(check_f32_ptr(s0, "s0", false));
  CHK(check_f32_ptr(sT, "sT", false));
  CHK(check_f32_ptr(out, "out", true));
  CHK(check_f32_ptr(x_last, "x_last", false));
  void* base = cache;
  if (!base) {
    const size_t need = timemix_forward_workspace_bytes(s, B, T);
    if (!ws || ws_bytes < need)
      return fail(WKV7_ENOSPC, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    base = ws;
  }
  CHK(check_f32_ptr(base, cache ? "cache" : "ws", true));
  {
    const size_t tb = (size_t)B * T * s->C * sizeof(float), rb = (size_t)B * s->C * sizeof(float);
    const size_t sb = state_bytes(B, s->H);
    Spans sp;
    tm_weight_spans(sp, s, W, false);
    sp.rd(x, tb, "x");
    // x_last may replace x_prev in place for one token (the same thread reads, then writes)
    if (!(T == 1 && x_last == x_prev)) sp.rd(x_prev, rb, "x_prev");
    if (s->layer_id == 0) sp.wr(v_first, tb, "v_first"); else sp.rd(v_first, tb, "v_first");
    if (s0 != sT) sp.rd(s0, sb, "s0");
    sp.wr(sT, sb, "sT");
    sp.wr(out, tb, "out");
    sp.wr(x_last, rb, "x_last");
    sp.wr(base, timemix_cache_bytes(s, B, T), cache ? "cache" : "ws");
    CHK(sp.check());
  }
  Carver c(base);
  TmCache m;
  carve_cache(c, s, B, T, m);
  return tm_forward_impl(s, W, B, T, x, x_prev, v_first, s0, sT, out, x_last, m, stream);
}

extern "C" int timemix_backward(const tm_shape* s, const tm_weights* W, int B, int T,
                                const float* x, const float* x_prev, const float* v_first,
                                const float* s0, const float* dout, const float* dsT,
                                const void* cache, tm_grads* G, float* dx, float* dx_prev,
                                const float* dv_first_in, float* dv_first_out, float* ds0,
                                void* ws, size_t ws_bytes, const wkv7_side* side,
                                hipStream_t stream) {
  g_err[0] = 0;
  CHK(check_tm_shape(s, B, T));
  CHK(check_weights(s, W));
  if (!G) return fail(WKV7_EINVAL, "grads is NULL");
  float* greq[] = {G->mu_r, G->mu_w, G->mu_k, G->mu_v, G->mu_a, G->mu_g, G->Wr, G->Wk, G->Wv,
                   G->Wo, G->w0, G->W1, G->W2, G->a0, G->A1, G->A2, G->G1, G->G2, G->k_k,
                   G->k_a, G->r_k, G->ln_w, G->ln_b};
  for (float* p : greq) CHK(check_f32_ptr(p, "a gradient field", true));
  if (s->layer_id > 0) {
    CHK(check_f32_ptr(G->v0, "G.v0", true));
    CHK(check_f32_ptr(G->V1, "G.V1", true));
    CHK(check_f32_ptr(G->V2, "G.V2", true));
  }
  CHK(check_f32_ptr(x, "x", true));
  CHK(check_f32_ptr(x_prev, "x_prev", false));
  CHK(check_f32_ptr(v_first, "v_first", s->layer_id > 0));
  CHK(check_f32_ptr(s0, "s0", false));
  CHK(check_f32_ptr(dout, "dout", true));
  CHK(check_f32_ptr(dsT, "dsT", false));
  CHK(check_f32_ptr(dx, "dx", true));
  CHK(check_f32_ptr(dx_prev, "dx_prev", false));
  CHK(check_f32_ptr(dv_first_in, "dv_first_in", false));
  CHK(check_f32_ptr(dv_first_out, "dv_first_out", false));
  CHK(check_f32_ptr(ds0, "ds0", false));
  CHK(check_f32_ptr(cache, "cache", false));
  const size_t need = timemix_backward_workspace_bytes(s, B, T);
  if (!ws || ws_bytes < need)
    return fail(WKV7_ENOSPC, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  CHK(check_f32_ptr(ws, "ws", true));
  const wkv7_side* sd = nullptr;
  CHK(check_side(side, stream, sd));
  {
    const size_t tb = (size_t)B * T * s->C * sizeof(float), rb = (size_t)B * s->C * sizeof(float);
    const size_t sb = state_bytes(B, s->H);
    Spans sp;
    tm_weight_spans(sp, s, W, false);
    tm_weight_spans(sp, s, G, true);
    sp.rd(x, tb, "x");
    sp.rd(x_prev, rb, "x_prev");
    if (s->layer_id > 0) sp.rd(v_first, tb, "v_first");
    sp.rd(s0, sb, "s0");
    sp.rd(dout, tb, "dout");
    sp.rd(dsT, sb, "dsT");
    sp.rd(cache, cache ? timemix_cache_bytes(s, B, T) : 0, "cache");
    if (s->layer_id == 0) sp.rd(dv_first_in, tb, "dv_first_in");
    sp.wr(dx, tb, "dx");
    sp.wr(dx_prev, rb, "dx_prev");
    if (s->layer_id > 0) sp.wr(dv_first_out, tb, "dv_first_out");
    sp.wr(ds0, sb, "ds0");
    sp.wr(ws, need, "ws");
    CHK(sp.check());
  }

  const int BT = B * T, C = s->C, L = s->layer_id;
  Carver cw(ws);
  TmCache m;
  carve_cache(cw, s, B, T, m);  // used when the cache must be recomputed
  float* out_tmp = cw.take((size_t)BT * C);
  TmBwdBufs bb;
  carve_bwd(cw, s, B, T, bb);
  if (cache) {
    Carver cc((void*)cache);
    carve_cache(cc, s, B, T, m);
  } else {
    // layer 0 republishes v_first; send it to a scratch buffer so the caller's
    // (const) v_first is never written
    float* vf = L == 0 ? bb.dxg : (float*)v_first;
    CHK(tm_forward_impl(s, W, B, T, x, x_prev, vf, s0, nullptr, out_tmp, nullptr, m, stream));
  }
  return tm_backward_impl(s, W, B, T, x, x_prev, v_first, s0, dout, dsT, m, bb, G, dx, dx_prev,
                          dv_first_in, dv_first_out, false, ds0, stream, GEMM_F32, sd);
}

// ----------------------------------------------------------------- GEMM --
namespace {
int gemm_abi(int prec, int transA, int transB, int M, int N, int K, const float* A, int lda,
             const float* B, int ldb, float* C, int ldc, float beta, void* ws, size_t ws_bytes,
             hipStream_t stream) {
  g_err[0] = 0;
  if (M < 1 || N < 1 || K < 1) return fail(WKV7_EINVAL, "M, N, K must be >= 1");
  CHK(check_f32_ptr(A, "A", true));
  CHK(check_f32_ptr(B, "B", true));
  CHK(check_f32_ptr(C, "C", true));
  const int a_inner = transA ? M : K, b_inner = transB ? K : N;
  if (a_inner % 4 || b_inner % 4 || lda % 4 || ldb % 4)
    return fail(WKV7_EINVAL, "contiguous GEMM dimensions and leading dims must be multiples of 4");
  if (lda < a_inner || ldb < b_inner || ldc < N) return fail(WKV7_EINVAL, "leading dimension too small");
  {
    const size_t f = sizeof(float);
    const size_t a_rows = transA ? K : M, b_rows = transB ? N : K;
    Spans sp;
    sp.rd(A, ((a_rows - 1) * lda + a_inner) * f, "A");
    sp.rd(B, ((b_rows - 1) * ldb + b_inner) * f, "B");
    sp.wr(C, ((size_t)(M - 1) * ldc + N) * f, "C");
    if (ws) sp.wr(ws, ws_bytes, "ws");
    CHK(sp.check());
  }
  if (ws && ((uintptr_t)ws & 255)) return fail(WKV7_EINVAL, "ws must be 256-byte aligned");
  // operands packed to bf16 only when the workspace holds the whole copy
  const size_t need = (prec == GEMM_BF16 && !transA) ? gemm_pack_need(M, N, K) : 0;
  if (ws && ws_bytes < need)
    return fail(WKV7_ENOSPC, "workspace %zu bytes, this GEMM needs %zu", ws_bytes, need);
  GemmPackScope pack_scope(need && ws ? ws : nullptr, ws_bytes);
  HIPCHK(gemm_run(prec, transA != 0, transB != 0, M, N, K, A, lda, B, ldb, C, ldc, beta, 0, nullptr,
                  1, nullptr, stream),
         "gemm launch");
  return WKV7_OK;
}
}  // namespace

extern "C" int wkv7_gemm_f32(int transA, int transB, int M, int N, int K, const float* A, int lda,
                             const float* B, int ldb, float* C, int ldc, float beta,
                             hipStream_t stream) {
  return gemm_abi(GEMM_F32, transA, transB, M, N, K, A, lda, B, ldb, C, ldc, beta, nullptr, 0,
                  stream);
}

extern "C" size_t wkv7_gemm_bf16_workspace_bytes(int transA, int transB, int M, int N, int K) {
  (void)transB;
  if (M < 1 || N < 1 || K < 1 || transA) return 0;
  return gemm_pack_need(M, N, K);
}

extern "C" int wkv7_gemm_bf16(int transA, int transB, int M, int N, int K, const float* A,
                              int lda, const float* B, int ldb, float* C, int ldc, float beta,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  return gemm_abi(GEMM_BF16, transA, transB, M, N, K, A, lda, B, ldb, C, ldc, beta, ws, ws_bytes,
                  stream);
}

// --------------------------------------------------------- decode stack --
namespace {

struct DecodeBufs {
  float *x, *h, *vf, *sh, *ka;
  float* part;  // split-K partials of the channel-mix value product
  TmCache tm;
};
// Slices of the channel-mix value product (K = F) in decode: every layer but
// the last leaves them for the next layer's LN1 to add to the residual.
// The output projection (K = C) leaves its slices for LN2 the same way.
constexpr int DECODE_CM_SPLIT = 4;
constexpr int DECODE_O_SPLIT = 2;

int check_cfg(const rwkv7_config* c, int B) {
  if (!c) return fail(WKV7_EINVAL, "config is NULL");
  if (c->N != WKV7_N) return fail(WKV7_EINVAL, "head size N=%d unsupported (must be 64)", c->N);
  if (c->gemm_dtype != WKV7_F32 && c->gemm_dtype != WKV7_BF16)
    return fail(WKV7_EINVAL, "gemm_dtype must be WKV7_F32 or WKV7_BF16");
  if (c->train_recompute != 0 && c->train_recompute != 1)
    return fail(WKV7_EINVAL, "train_recompute must be 0 or 1");
  if (c->H < 1 || c->C != c->H * c->N) return fail(WKV7_EINVAL, "C=%d must equal H*N", c->C);
  if (c->C > stk_max_layernorm_width()) return fail(WKV7_EINVAL, "C=%d above the supported %d", c->C, stk_max_layernorm_width());
  if (c->n_layer < 1 || B < 1) return fail(WKV7_EINVAL, "n_layer and B must be >= 1");
  if (c->F < 4 || c->F % 4 || c->V < 4 || c->V % 4) return fail(WKV7_EINVAL, "F and V must be positive multiples of 4");
  if (c->n_attn < 0) return fail(WKV7_EINVAL, "n_attn must be >= 0");
  if (c->n_attn > 0 && (c->moba_chunk < 1 || c->moba_topk < 1 || c->moba_topk > 64))
    return fail(WKV7_EINVAL, "attention blocks need moba_chunk >= 1 and moba_topk in [1, 64]");
  tm_shape s = {c->C, c->H, c->N, c->Dw, c->Da, c->Dv, c->Dg, c->n_layer > 1 ? 1 : 0};
  return check_tm_shape(&s, B, 1);
}

void carve_decode(Carver& c, const rwkv7_config* cfg, int B, DecodeBufs& d) {
  const size_t BC = (size_t)B * cfg->C;
  d.x = c.take(BC);
  d.h = c.take(BC);
  d.vf = c.take(BC);
  d.sh = c.take(BC);
  d.ka = c.take((size_t)B * cfg->F);
  d.part = c.take((size_t)std::max(DECODE_CM_SPLIT, DECODE_O_SPLIT) * BC);
  tm_shape s = {cfg->C, cfg->H, cfg->N, cfg->Dw, cfg->Da, cfg->Dv, cfg->Dg, 1};
  carve_cache(c, &s, B, 1, d.tm, false);
}

// Streams split into groups advanced concurrently (B >= 512: one group per
// 512 streams, at most DECODE_MAX_GROUPS): every kernel of the step is
// either HBM bound over the whole batch (wkv7_step) or a small latency-bound
// GEMM / row kernel, so the groups' chains overlap on the GPU.  Group 0 runs
// on the caller's stream, the others on library streams forked from it and
// joined back with events (all recorded into a HIP graph when the caller
// captures).  Every group but the last has a multiple of 4 streams so each
// group pointer keeps its alignment.  Measured on MI355X, 12 layers C = 256,
// 2048 streams: 1.82 ms per step in one group, 1.64 ms in two, 2.01 ms in
// four (smaller groups make every GEMM and row kernel less efficient).
constexpr int DECODE_SPLIT_MIN = 512;
constexpr int DECODE_MAX_GROUPS = 2;  // the caller's stream and the side stream

int decode_groups(int B, int nb[DECODE_MAX_GROUPS]) {
  const int g = B < DECODE_SPLIT_MIN ? 1 : std::min(DECODE_MAX_GROUPS, B / DECODE_SPLIT_MIN + (B % DECODE_SPLIT_MIN ? 1 : 0));
  if (g == 1) {
    nb[0] = B;
    return 1;
  }
  const int per = (B / g) / 4 * 4;
  for (int i = 0; i < g - 1; i++) nb[i] = per;
  nb[g - 1] = B - per * (g - 1);
  return g;
}

void carve_decode_all(Carver& c, const rwkv7_config* cfg, int B, DecodeBufs d[DECODE_MAX_GROUPS]) {
  int nb[DECODE_MAX_GROUPS];
  const int g = decode_groups(B, nb);
  for (int i = 0; i < g; i++) carve_decode(c, cfg, nb[i], d[i]);
}

// One group of nb streams starting at stream b0 of B: the per-layer state
// rows, tokens and logits are the group's contiguous sub-blocks.
int decode_run(const rwkv7_config* cfg, const rwkv7_model* M, int B, int b0, int nb,
               const int* tokens, float* att_x_prev, float* att_state, float* ffn_x_prev,
               float* logits, DecodeBufs& d, int prec, hipStream_t st) {
  const int C = cfg->C, F = cfg->F, V = cfg->V, L = cfg->n_layer, H = cfg->H;
  const size_t BC = (size_t)B * C, NN = (size_t)WKV7_N * WKV7_N;
  tokens += b0;
  logits += (size_t)b0 * V;
  HIPCHK(stk_launch_emb_gather(nb, C, V, tokens, M->emb, d.x, st), "embedding");
  if (cfg->use_ln0) HIPCHK(stk_launch_layernorm(nb, C, d.x, M->ln0_w, M->ln0_b, d.x, nullptr, nullptr, st), "ln0");
  int pend = 0;  // split-K partials of the previous layer's channel-mix value product
  for (int l = 0; l < L; l++) {
    const rwkv7_block& bl = M->blocks[l];
    tm_shape s = {C, H, cfg->N, cfg->Dw, cfg->Da, cfg->Dv, cfg->Dg, l};
    float* axp = att_x_prev + (size_t)l * BC + (size_t)b0 * C;
    float* ast = att_state + ((size_t)l * B + b0) * H * NN;
    float* fxp = ffn_x_prev + (size_t)l * BC + (size_t)b0 * C;
    {  // (residual add,) LN1 fused with the six time-mix lerps; att_x_prev <- this token's LN1 output
      LnMix lm{nb, C, 6, d.x, bl.ln1_w, bl.ln1_b, axp, axp,
               {bl.tm.mu_r, bl.tm.mu_w, bl.tm.mu_k, bl.tm.mu_v, bl.tm.mu_a, bl.tm.mu_g},
               {d.tm.xr, d.tm.xw, d.tm.xk, d.tm.xv, d.tm.xa, d.tm.xg},
               d.part, pend, d.x};
      HIPCHK(stk_launch_ln_mix(lm, st), "ln1 + shift");
      pend = 0;
    }
    CHK(tm_forward_impl(&s, &bl.tm, nb, 1, nullptr, nullptr, d.vf, ast, ast, d.x, nullptr, d.tm, st,
                        true, 1.f, prec, true, false));
    // output projection as split-K partials, added to the residual by LN2
    HIPCHK(gemm_run_partials(prec, nb, C, C, d.tm.tg, C, bl.tm.Wo, C, DECODE_O_SPLIT, d.part, &pend, st),
           "o proj");
    {  // residual add, LN2 fused with the channel-mix lerp; ffn_x_prev <- this token's LN2 output
      LnMix lm{nb, C, 1, d.x, bl.ln2_w, bl.ln2_b, fxp, fxp, {bl.cm_mu_k}, {d.sh}, d.part, pend, d.x};
      HIPCHK(stk_launch_ln_mix(lm, st), "ln2 + shift");
      pend = 0;
    }
    HIPCHK(gemm_run(prec, false, false, nb, F, C, d.sh, C, bl.cm_Wk, F, d.ka, F, 0.f, 5, nullptr, 1, nullptr, st), "cm key");
    if (l + 1 < L)  // the next layer's LN1 adds the slices to the residual
      HIPCHK(gemm_run_partials(prec, nb, C, F, d.ka, F, bl.cm_Wv, C, DECODE_CM_SPLIT, d.part, &pend, st),
             "cm value");
    else
      HIPCHK(gemm_run(prec, false, false, nb, C, F, d.ka, F, bl.cm_Wv, C, d.x, C, 1.f, 0, nullptr, 1, nullptr, st), "cm value");
  }
  HIPCHK(stk_launch_layernorm(nb, C, d.x, M->ln_out_w, M->ln_out_b, d.h, nullptr, nullptr, st), "ln_out");
  HIPCHK(gemm_run(prec, false, false, nb, V, C, d.h, C, M->head, V, logits, V, 0.f, 0, nullptr, 1, nullptr, st), "head");
  return WKV7_OK;
}

}  // namespace

namespace {
// Byte ranges of a model's weights (or of its gradients, same shapes).
template <typename MT>
void model_spans(Spans& sp, const rwkv7_config* cfg, const MT* M, bool written) {
  const size_t f = sizeof(float), C = cfg->C, F = cfg->F, V = cfg->V;
  auto add = [&](const void* p, size_t n, const char* nm) {
    if (written) sp.wr(p, n * f, nm); else sp.rd(p, n * f, nm);
  };
  add(M->emb, V * C, "emb");
  add(M->head, C * V, "head");
  add(M->ln_out_w, C, "ln_out_w");
  add(M->ln_out_b, C, "ln_out_b");
  if (cfg->use_ln0) {
    add(M->ln0_w, C, "ln0_w");
    add(M->ln0_b, C, "ln0_b");
  }
  for (int l = 0; l < cfg->n_layer; l++) {
    const auto& bl = M->blocks[l];
    add(bl.ln1_w, C, "ln1_w"); add(bl.ln1_b, C, "ln1_b");
    add(bl.ln2_w, C, "ln2_w"); add(bl.ln2_b, C, "ln2_b");
    add(bl.cm_mu_k, C, "cm_mu_k"); add(bl.cm_Wk, C * F, "cm_Wk"); add(bl.cm_Wv, F * C, "cm_Wv");
    tm_shape s = {cfg->C, cfg->H, cfg->N, cfg->Dw, cfg->Da, cfg->Dv, cfg->Dg, l};
    tm_weight_spans(sp, &s, &bl.tm, written);
  }
  for (int a = 0; a < cfg->n_attn; a++) {
    const auto& ab = M->attn[a];
    add(ab.ln1_w, C, "attn ln1_w"); add(ab.ln1_b, C, "attn ln1_b");
    add(ab.ln2_w, C, "attn ln2_w"); add(ab.ln2_b, C, "attn ln2_b");
    add(ab.Wq, C * C, "Wq"); add(ab.Wk, C * C, "attn Wk"); add(ab.Wv, C * C, "attn Wv");
    add(ab.Wo, C * C, "attn Wo");
    add(ab.cm_mu_k, C, "attn cm_mu_k"); add(ab.cm_Wk, C * F, "attn cm_Wk"); add(ab.cm_Wv, F * C, "attn cm_Wv");
  }
}
}  // namespace

extern "C" size_t rwkv7_decode_workspace_bytes(const rwkv7_config* cfg, int B) {
  if (check_cfg(cfg, B) != WKV7_OK || cfg->n_attn != 0) return 0;
  Carver c(nullptr);
  DecodeBufs d[DECODE_MAX_GROUPS];
  carve_decode_all(c, cfg, B, d);
  return c.off + 256;
}

extern "C" int rwkv7_decode_step(const rwkv7_config* cfg, const rwkv7_model* M, int B,
                                 const int* tokens, float* att_x_prev, float* att_state,
                                 float* ffn_x_prev, float* logits, void* ws, size_t ws_bytes,
                                 const wkv7_side* side, hipStream_t st) {
  g_err[0] = 0;
  CHK(check_cfg(cfg, B));
  if (cfg->n_attn != 0) return fail(WKV7_EINVAL, "attention blocks are supported by rwkv7_train_step only");
  const int prec = cfg->gemm_dtype == WKV7_BF16 ? GEMM_BF16 : GEMM_F32;
  if (!M || !M->blocks) return fail(WKV7_EINVAL, "model or model->blocks is NULL");
  CHK(check_f32_ptr(M->emb, "emb", true));
  CHK(check_f32_ptr(M->head, "head", true));
  CHK(check_f32_ptr(M->ln_out_w, "ln_out_w", true));
  CHK(check_f32_ptr(M->ln_out_b, "ln_out_b", true));
  CHK(check_f32_ptr(M->ln0_w, "ln0_w", cfg->use_ln0 != 0));
  CHK(check_f32_ptr(M->ln0_b, "ln0_b", cfg->use_ln0 != 0));
  CHK(check_tok_ptr(tokens, "tokens", WKV7_F32, true));
  CHK(check_f32_ptr(att_x_prev, "att_x_prev", true));
  CHK(check_f32_ptr(att_state, "att_state", true));
  CHK(check_f32_ptr(ffn_x_prev, "ffn_x_prev", true));
  CHK(check_f32_ptr(logits, "logits", true));
  for (int l = 0; l < cfg->n_layer; l++) {
    const rwkv7_block& bl = M->blocks[l];
    tm_shape s = {cfg->C, cfg->H, cfg->N, cfg->Dw, cfg->Da, cfg->Dv, cfg->Dg, l};
    CHK(check_weights(&s, &bl.tm));
    const float* req[] = {bl.ln1_w, bl.ln1_b, bl.ln2_w, bl.ln2_b, bl.cm_mu_k, bl.cm_Wk, bl.cm_Wv};
    for (const float* p : req) CHK(check_f32_ptr(p, "a block weight", true));
  }
  const size_t need = rwkv7_decode_workspace_bytes(cfg, B);
  if (!ws || ws_bytes < need)
    return fail(WKV7_ENOSPC, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  CHK(check_f32_ptr(ws, "ws", true));
  const wkv7_side* sd = nullptr;
  CHK(check_side(side, st, sd));
  {
    const size_t f = sizeof(float), L = cfg->n_layer, BC = (size_t)B * cfg->C;
    Spans sp;
    model_spans(sp, cfg, M, false);
    sp.rd(tokens, (size_t)B * sizeof(int), "tokens");
    sp.wr(att_x_prev, L * BC * f, "att_x_prev");  // the state tensors are updated in place
    sp.wr(att_state, L * state_bytes(B, cfg->H), "att_state");
    sp.wr(ffn_x_prev, L * BC * f, "ffn_x_prev");
    sp.wr(logits, (size_t)B * cfg->V * f, "logits");
    sp.wr(ws, need, "ws");
    CHK(sp.check());
  }
  Carver cw(ws);
  DecodeBufs d[DECODE_MAX_GROUPS];
  carve_decode_all(cw, cfg, B, d);
  int nb[DECODE_MAX_GROUPS], b0[DECODE_MAX_GROUPS];
  const int ng = decode_groups(B, nb);
  for (int g = 0, o = 0; g < ng; o += nb[g], g++) b0[g] = o;
  if (ng == 1)
    return decode_run(cfg, M, B, 0, B, tokens, att_x_prev, att_state, ffn_x_prev, logits, d[0],
                      prec, st);
  if (!sd) {  // no side stream: the groups one after the other
    for (int g = 0; g < ng; g++)
      CHK(decode_run(cfg, M, B, b0[g], nb[g], tokens, att_x_prev, att_state, ffn_x_prev, logits,
                     d[g], prec, st));
    return WKV7_OK;
  }
  // group 1 on the side stream, forked from and joined back to `st`
  HIPCHK(hipEventRecord(sd->ev[0], st), "decode fork");
  HIPCHK(hipStreamWaitEvent(sd->stream, sd->ev[0], 0), "decode fork");
  int rc = decode_run(cfg, M, B, b0[1], nb[1], tokens, att_x_prev, att_state, ffn_x_prev, logits,
                      d[1], prec, sd->stream);
  // the join is enqueued whatever happened, so the caller's stream (or
  // capture) never leaves the side stream dangling
  hipError_t ej = hipEventRecord(sd->ev[3], sd->stream);
  if (rc == WKV7_OK)
    rc = decode_run(cfg, M, B, 0, nb[0], tokens, att_x_prev, att_state, ffn_x_prev, logits, d[0],
                    prec, st);
  const hipError_t e = hipStreamWaitEvent(st, sd->ev[3], 0);
  if (ej == hipSuccess) ej = e;
  HIPCHK(ej, "decode join");
  return rc;
}

// ---------------------------------------------------------- training step --
namespace {

// Activations of one block kept from the forward for its backward.
struct BlockActs {
  float *h, *x1, *h2, *sh, *ka;  // LN1 out, x + TM, LN2 out, cm shift, relu(sh Wk)^2
  TmCache tm;
};

struct TrainBufs {
  float *block_in, *x_emb, *vf, *dvf, *h, *dsh, *dh, *dx, *dx1;
  float *dfk, *logits, *loss_row, *part_ln, *part_cm, *splitk;
  int *count, *off, *perm, *n_valid;
  std::vector<BlockActs> act;  // every block's (train_recompute == 0), or one reused
  TmBwdBufs tb;
  float* pack = nullptr;  // bf16 operand copies of the GEMMs (gemm_dtype == WKV7_BF16)
  size_t pack_bytes = 0;
  // bf16 copy [BT][F] of the channel-mix hidden activation (forward) or its
  // gradient (backward), written by the producing product and read as the
  // next product's A, and before that in each block the time-mix shift's
  // copies of xr, xk, xv [3][BT][C] (gemm_dtype == WKV7_BF16; one buffer,
  // reused on the caller's stream)
  __bf16* act16 = nullptr;
  __bf16* sh16 = nullptr;  // the channel-mix shift's bf16 copy, past act16's [BT][max(F, 3C)]
  // bf16 copy [BT][C] of the upstream gradient a LayerNorm backward leaves in
  // dx (every producer of t.dx writes it; read by the channel-mix dfk product)
  // or dx1 (read by the time-mix output product's input gradient)
  __bf16* dx16 = nullptr;
  // bf16 copy [BT][V] of dlogits written by the cross-entropy kernel, the A of
  // the head's input-gradient product (gemm_dtype == WKV7_BF16)
  __bf16* logits16 = nullptr;
  // attention blocks (n_attn > 0): activations of each (or one reused set)
  // and the backward's buffers
  struct AttnActs {
    float *h, *q, *k, *v, *y, *x1, *h2, *sh, *ka, *lse;
    uint64_t* sel;
  };
  std::vector<AttnActs> aact;
  float *dyc = nullptr, *dq = nullptr, *dk = nullptr, *dv = nullptr, *mws = nullptr;
  size_t mws_bytes = 0;
};

// Largest arena of bf16 operand copies any one GEMM launch of the training
// step asks for (the X W and dY W^T products; the X^T dY ones read fp32).
size_t train_pack_bytes(const rwkv7_config* cfg, size_t BT) {
  const int C = cfg->C, F = cfg->F, V = cfg->V, M = (int)BT;
  const int D[4] = {cfg->Dw, cfg->Da, cfg->Dg, cfg->Dv};
  size_t best = 3 * gemm_pack_need(M, C, C);  // r, k, v in one launch
  size_t down = 0, up = 0;
  for (int d : D) {
    down += gemm_pack_need(M, d, C);
    up += gemm_pack_need(M, C, d);
  }
  best = std::max({best, down, up, gemm_pack_need(M, F, C), gemm_pack_need(M, C, F),
                   gemm_pack_need(M, V, C), gemm_pack_need(M, C, V), gemm_pack_need_b(M, C, V)});
  return best;
}

tm_shape block_shape(const rwkv7_config* c, int l) {
  return tm_shape{c->C, c->H, c->N, c->Dw, c->Da, c->Dv, c->Dg, l};
}

void carve_train(Carver& c, const rwkv7_config* cfg, int B, int T, TrainBufs& t) {
  const size_t BT = (size_t)B * T, tok = BT * cfg->C, L = cfg->n_layer;
  t.block_in = c.take((L + cfg->n_attn + 1) * tok);
  t.x_emb = cfg->use_ln0 ? c.take(tok) : nullptr;
  float** toks[] = {&t.vf, &t.dvf, &t.h, &t.dsh, &t.dh, &t.dx, &t.dx1};
  for (float** p : toks) *p = c.take(tok);
  t.dfk = c.take(BT * cfg->F);
  t.logits = c.take(BT * cfg->V);
  t.loss_row = c.take(BT);
  t.part_ln = c.take((size_t)2 * stk_num_ln_blocks((int)BT) * cfg->C);
  t.part_cm = c.take((size_t)stk_num_shift_blocks((int)BT, cfg->C) * cfg->C);
  const int C = cfg->C, F = cfg->F, V = cfg->V;
  size_t sk = 0;
  const int pairs[][2] = {{F, C}, {C, F}, {C, V}};
  for (auto& pr : pairs) sk = std::max(sk, (size_t)splitk_for(pr[0], pr[1], (int)BT) * pr[0] * pr[1]);
  t.splitk = c.take(sk);
  t.count = (int*)c.take((size_t)V);
  t.off = (int*)c.take((size_t)V);
  t.perm = (int*)c.take(BT);
  t.n_valid = (int*)c.take(1);
  if (cfg->gemm_dtype == WKV7_BF16) {
    t.pack_bytes = train_pack_bytes(cfg, BT);
    t.pack = c.take(t.pack_bytes / sizeof(float));
    t.act16 = reinterpret_cast<__bf16*>(c.take(BT * (std::max(cfg->F, 3 * cfg->C) + cfg->C) / 2));
    t.sh16 = t.act16 + BT * std::max(cfg->F, 3 * cfg->C);
    t.dx16 = reinterpret_cast<__bf16*>(c.take(BT * cfg->C / 2));
    t.logits16 = reinterpret_cast<__bf16*>(c.take((BT * cfg->V + 1) / 2));
  }
  const bool keep = cfg->train_recompute == 0;
  t.act.resize(keep ? L : 1);
  for (size_t i = 0; i < t.act.size(); i++) {
    BlockActs& a = t.act[i];
    float** bt[] = {&a.h, &a.x1, &a.h2, &a.sh};
    for (float** p : bt) *p = c.take(tok);
    a.ka = c.take(BT * cfg->F);
    // a reused set is sized for a block with the value-residual LoRA (layer > 0)
    tm_shape s = block_shape(cfg, keep ? (int)i : 1);
    carve_cache(c, &s, B, T, a.tm);
  }
  tm_shape s = block_shape(cfg, 1);
  carve_bwd(c, &s, B, T, t.tb);
  if (cfg->n_attn > 0) {
    const size_t rows = BT / T * cfg->H * T;  // B H T
    t.aact.resize(keep ? cfg->n_attn : 1);
    for (auto& a : t.aact) {
      float** bt[] = {&a.h, &a.q, &a.k, &a.v, &a.y, &a.x1, &a.h2, &a.sh};
      for (float** p : bt) *p = c.take(tok);
      a.ka = c.take(BT * cfg->F);
      a.lse = c.take(rows);
      a.sel = (uint64_t*)c.take(2 * rows);
    }
    float** bb[] = {&t.dyc, &t.dq, &t.dk, &t.dv};
    for (float** p : bb) *p = c.take(tok);
    t.mws_bytes = moba_ws_bytes(B, T, cfg->H, cfg->moba_chunk, cfg->moba_topk);
    t.mws = c.take(t.mws_bytes / sizeof(float) + 1);
  }
}

}  // namespace

extern "C" size_t rwkv7_train_workspace_bytes(const rwkv7_config* cfg, int B, int T) {
  if (check_cfg(cfg, B) != WKV7_OK || T < 1) return 0;
  Carver c(nullptr);
  TrainBufs t;
  carve_train(c, cfg, B, T, t);
  return c.off + 256;
}

namespace {
// Arguments shared by rwkv7_train_step and rwkv7_online_segment; `extra`
// adds the caller's other tensors to the overlap check.
int check_train(const rwkv7_config* cfg, const rwkv7_model* M, rwkv7_model_grads* G, int B, int T,
                const int* tokens, const int* targets, float* loss, void* ws, size_t ws_bytes,
                size_t need, const wkv7_side* side, hipStream_t st, const wkv7_side*& sd,
                Spans& sp) {
  CHK(check_cfg(cfg, B));
  if (T < 1) return fail(WKV7_EINVAL, "T must be >= 1");
  if (!M || !M->blocks || !G || !G->blocks) return fail(WKV7_EINVAL, "model/grads or their blocks are NULL");
  CHK(check_f32_ptr(M->emb, "emb", true));
  CHK(check_f32_ptr(M->head, "head", true));
  CHK(check_f32_ptr(M->ln_out_w, "ln_out_w", true));
  CHK(check_f32_ptr(M->ln_out_b, "ln_out_b", true));
  CHK(check_f32_ptr(M->ln0_w, "ln0_w", cfg->use_ln0 != 0));
  CHK(check_f32_ptr(M->ln0_b, "ln0_b", cfg->use_ln0 != 0));
  float* greq[] = {G->emb, G->head, G->ln_out_w, G->ln_out_b};
  for (float* p : greq) CHK(check_f32_ptr(p, "a model gradient", true));
  if (cfg->use_ln0) {
    CHK(check_f32_ptr(G->ln0_w, "grad ln0_w", true));
    CHK(check_f32_ptr(G->ln0_b, "grad ln0_b", true));
  }
  CHK(check_tok_ptr(tokens, "tokens", WKV7_F32, true));
  CHK(check_tok_ptr(targets, "targets", WKV7_F32, true));
  CHK(check_f32_ptr(loss, "loss", true));
  const int V = cfg->V, L = cfg->n_layer;
  if ((size_t)B * T * V > ((size_t)1 << 34)) return fail(WKV7_EINVAL, "B*T*V too large");
  for (int l = 0; l < L; l++) {
    tm_shape s = block_shape(cfg, l);
    CHK(check_weights(&s, &M->blocks[l].tm));
    const rwkv7_block& bl = M->blocks[l];
    const float* req[] = {bl.ln1_w, bl.ln1_b, bl.ln2_w, bl.ln2_b, bl.cm_mu_k, bl.cm_Wk, bl.cm_Wv};
    for (const float* p : req) CHK(check_f32_ptr(p, "a block weight", true));
    const rwkv7_block_grads& gb = G->blocks[l];
    float* gq[] = {gb.ln1_w, gb.ln1_b, gb.ln2_w, gb.ln2_b, gb.cm_mu_k, gb.cm_Wk, gb.cm_Wv,
                   gb.tm.mu_r, gb.tm.mu_w, gb.tm.mu_k, gb.tm.mu_v, gb.tm.mu_a, gb.tm.mu_g,
                   gb.tm.Wr, gb.tm.Wk, gb.tm.Wv, gb.tm.Wo, gb.tm.w0, gb.tm.W1, gb.tm.W2, gb.tm.a0,
                   gb.tm.A1, gb.tm.A2, gb.tm.G1, gb.tm.G2, gb.tm.k_k, gb.tm.k_a, gb.tm.r_k,
                   gb.tm.ln_w, gb.tm.ln_b};
    for (float* p : gq) CHK(check_f32_ptr(p, "a block gradient", true));
    if (l > 0) {
      CHK(check_f32_ptr(gb.tm.v0, "grad v0", true));
      CHK(check_f32_ptr(gb.tm.V1, "grad V1", true));
      CHK(check_f32_ptr(gb.tm.V2, "grad V2", true));
    }
  }
  if (cfg->n_attn > 0) {
    if (!M->attn || !G->attn) return fail(WKV7_EINVAL, "model/grads attn arrays are NULL with n_attn > 0");
    if (moba_num_chunks(T, cfg->moba_chunk) > 64)
      return fail(WKV7_EINVAL, "T=%d in chunks of %d gives more than 64 chunks", T, cfg->moba_chunk);
    for (int a = 0; a < cfg->n_attn; a++) {
      const rwkv7_attn_block& ab = M->attn[a];
      const float* req[] = {ab.ln1_w, ab.ln1_b, ab.ln2_w, ab.ln2_b, ab.Wq, ab.Wk, ab.Wv, ab.Wo,
                            ab.cm_mu_k, ab.cm_Wk, ab.cm_Wv};
      for (const float* p : req) CHK(check_f32_ptr(p, "an attention-block weight", true));
      const rwkv7_attn_grads& ga = G->attn[a];
      float* gq[] = {ga.ln1_w, ga.ln1_b, ga.ln2_w, ga.ln2_b, ga.Wq, ga.Wk, ga.Wv, ga.Wo,
                     ga.cm_mu_k, ga.cm_Wk, ga.cm_Wv};
      for (float* p : gq) CHK(check_f32_ptr(p, "an attention-block gradient", true));
    }
  }
  if (!ws || ws_bytes < need)
    return fail(WKV7_ENOSPC, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  CHK(check_f32_ptr(ws, "ws", true));
  CHK(check_side(side, st, sd));
  model_spans(sp, cfg, G, true);
  sp.rd(tokens, (size_t)B * T * sizeof(int), "tokens");
  sp.rd(targets, (size_t)B * T * sizeof(int), "targets");
  sp.wr(loss, sizeof(float), "loss");
  sp.wr(ws, need, "ws");
  return WKV7_OK;
}

// The training step's launches; arguments validated.  st0: NULL (zero
// initial state) or the streaming state the batch starts from (per layer
// att_x_prev [B][C], att_state [B][H][N][N], ffn_x_prev [B][C]); the
// gradients stop at it.
struct StartState {
  const float *att_x_prev, *att_state, *ffn_x_prev;
};

// Stack order of a hybrid model (the fullmodel page's fm_build): after every
// n_layer / n_attn RWKV-7 blocks one attention block, then the remaining
// RWKV-7 blocks.  Entries: (0, RWKV-7 block index) or (1, attention block index).
std::vector<std::pair<int, int>> block_order(int n_rwkv, int n_attn) {
  std::vector<std::pair<int, int>> o;
  if (n_attn == 0) {
    for (int i = 0; i < n_rwkv; i++) o.push_back({0, i});
    return o;
  }
  const int interval = n_rwkv / n_attn;
  for (int a = 0; a < n_attn; a++) {
    for (int j = a * interval; j < (a + 1) * interval; j++) o.push_back({0, j});
    o.push_back({1, a});
  }
  for (int j = n_attn * interval; j < n_rwkv; j++) o.push_back({0, j});
  return o;
}
int train_run(const rwkv7_config* cfg, const rwkv7_model* M, rwkv7_model_grads* G, int B, int T,
              const int* tokens, const int* targets, float* loss, const StartState* st0, TrainBufs& t,
              const wkv7_side* sd, hipStream_t st) {
  const int prec = cfg->gemm_dtype == WKV7_BF16 ? GEMM_BF16 : GEMM_F32;
  GemmPackScope pack_scope(t.pack, t.pack_bytes);  // bf16 operand copies (null for fp32)
  const int C = cfg->C, F = cfg->F, V = cfg->V, L = cfg->n_layer;
  const size_t NN = (size_t)WKV7_N * WKV7_N;
  auto xp_tm = [&](int l) -> const float* { return st0 ? st0->att_x_prev + (size_t)l * B * C : nullptr; };
  auto s0_tm = [&](int l) -> const float* { return st0 ? st0->att_state + (size_t)l * B * cfg->H * NN : nullptr; };
  auto xp_cm = [&](int l) -> const float* { return st0 ? st0->ffn_x_prev + (size_t)l * B * C : nullptr; };

  const int BT = B * T;
  const size_t tokC = (size_t)BT * C;
  auto bin = [&](int l) { return t.block_in + (size_t)l * tokC; };
  auto reduce_ln = [&](float* gw, float* gb) -> hipError_t {
    VecOut o = {{gw, gb, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr}};
    return tm_launch_reduce(t.part_ln, 2, stk_num_ln_blocks(BT), C, o, st);
  };

  const bool keep = cfg->train_recompute == 0;
  // RWKV-7 block l's forward from xin (its output is x1 + ka Wv), activations into a
  auto block_fwd = [&](int l, const float* xin, BlockActs& a) -> int {
    const rwkv7_block& bl = M->blocks[l];
    tm_shape s = block_shape(cfg, l);
    HIPCHK(stk_launch_layernorm(BT, C, xin, bl.ln1_w, bl.ln1_b, a.h, nullptr, nullptr, st), "ln1");
    // x1 = xin + the time mix (the residual added in the output projection)
    CHK(tm_forward_impl(&s, &bl.tm, B, T, a.h, xp_tm(l), t.vf, s0_tm(l), nullptr, a.x1, nullptr, a.tm,
                        st, false, 0.f, prec, false, true, xin, t.act16));
    HIPCHK(stk_launch_layernorm(BT, C, a.x1, bl.ln2_w, bl.ln2_b, a.h2, nullptr, nullptr, st), "ln2");
    HIPCHK(stk_launch_cm_shift(BT, T, C, a.h2, xp_cm(l), bl.cm_mu_k, a.sh, nullptr, st, t.sh16), "cm shift");
    HIPCHK(gemm_run_x(prec, false, false, BT, F, C, a.sh, C, bl.cm_Wk, F, a.ka, F, 0.f, EPI_SQRELU, nullptr, 1,
                      nullptr, st, t.sh16, t.act16), "cm key");
    return WKV7_OK;
  };
  // attention block i's forward from xin (its output is x1 + ka Wv)
  const int H = cfg->H;
  auto attn_fwd = [&](int i, const float* xin, TrainBufs::AttnActs& a) -> int {
    const rwkv7_attn_block& ab = M->attn[i];
    HIPCHK(stk_launch_layernorm(BT, C, xin, ab.ln1_w, ab.ln1_b, a.h, nullptr, nullptr, st), "attn ln1");
    {
      GemmBatch g;
      g.count = 3;
      const float* W[3] = {ab.Wq, ab.Wk, ab.Wv};
      float* out[3] = {a.q, a.k, a.v};
      for (int j = 0; j < 3; j++) g.p[j] = GemmProblem{BT, C, C, a.h, C, W[j], C, out[j], C, 0.f, EPI_NONE, nullptr, nullptr};
      HIPCHK(gemm_batch(prec, false, false, g, st), "q/k/v proj");
    }
    HIPCHK(moba_launch_forward(B, T, H, cfg->moba_chunk, cfg->moba_topk, a.q, a.k, a.v, a.y, a.lse, a.sel,
                               t.mws, st), "moba forward");
    HIPCHK(gemm_run(prec, false, false, BT, C, C, a.y, C, ab.Wo, C, a.x1, C, 0.f, EPI_ADD, xin, 1, nullptr, st), "o proj");
    HIPCHK(stk_launch_layernorm(BT, C, a.x1, ab.ln2_w, ab.ln2_b, a.h2, nullptr, nullptr, st), "attn ln2");
    HIPCHK(stk_launch_cm_shift(BT, T, C, a.h2, nullptr, ab.cm_mu_k, a.sh, nullptr, st, t.sh16), "attn cm shift");
    HIPCHK(gemm_run_x(prec, false, false, BT, F, C, a.sh, C, ab.cm_Wk, F, a.ka, F, 0.f, EPI_SQRELU, nullptr, 1,
                      nullptr, st, t.sh16, t.act16), "attn cm key");
    return WKV7_OK;
  };
  const auto order = block_order(L, cfg->n_attn);
  const int NB = (int)order.size();

  // ---------------- forward (every block's activations, or only its input, kept)
  HIPCHK(stk_launch_emb_gather(BT, C, V, tokens, M->emb, cfg->use_ln0 ? t.x_emb : bin(0), st), "embedding");
  if (cfg->use_ln0)
    HIPCHK(stk_launch_layernorm(BT, C, t.x_emb, M->ln0_w, M->ln0_b, bin(0), nullptr, nullptr, st), "ln0");
  for (int pos = 0; pos < NB; pos++) {
    const int i = order[pos].second;
    const float *x1, *ka, *Wv;
    if (order[pos].first == 0) {
      BlockActs& a = t.act[keep ? i : 0];
      CHK(block_fwd(i, bin(pos), a));
      x1 = a.x1, ka = a.ka, Wv = M->blocks[i].cm_Wv;
    } else {
      TrainBufs::AttnActs& a = t.aact[keep ? i : 0];
      CHK(attn_fwd(i, bin(pos), a));
      x1 = a.x1, ka = a.ka, Wv = M->attn[i].cm_Wv;
    }
    float* xo = bin(pos + 1);  // x1 + the channel mix
    HIPCHK(gemm_run_x(prec, false, false, BT, C, F, ka, F, Wv, C, xo, C, 0.f, EPI_ADD, x1, 1, nullptr, st,
                      t.act16, nullptr), "cm value");
  }
  HIPCHK(stk_launch_layernorm(BT, C, bin(NB), M->ln_out_w, M->ln_out_b, t.h, nullptr, nullptr, st), "ln_out");
  HIPCHK(gemm_run(prec, false, false, BT, V, C, t.h, C, M->head, V, t.logits, V, 0.f, EPI_NONE, nullptr, 1, nullptr, st), "head");
  HIPCHK(stk_launch_ce(BT, V, t.logits, targets, t.loss_row, loss, t.n_valid, st, t.logits16), "cross-entropy");

  // ---------------- backward
  // Weight gradients run on the side stream (see tm_backward_impl): here the
  // head's and each channel-mix's, which only use t.splitk among the scratch
  // buffers; every block's time-mix backward joins the side stream before
  // returning, before any buffer they read is written again.
  hipStream_t ss = sd ? sd->stream : st;
  auto fork_here = [&]() -> hipError_t {
    if (!sd) return hipSuccess;
    hipError_t r = hipEventRecord(sd->ev[0], st);
    return r != hipSuccess ? r : hipStreamWaitEvent(ss, sd->ev[0], 0);
  };
  struct Join {
    const wkv7_side* sd;
    hipStream_t st;
    ~Join() {
      if (sd && hipEventRecord(sd->ev[3], sd->stream) == hipSuccess) (void)hipStreamWaitEvent(st, sd->ev[3], 0);
    }
  } join{sd, st};
  HIPCHK(fork_here(), "backward fork");
  HIPCHK(gemm_run_x(prec, false, true, BT, C, V, t.logits, V, M->head, V, t.dh, C, 0.f, EPI_NONE, nullptr, 1,
                    nullptr, st, t.logits16, nullptr), "dh");
  HIPCHK(gemm_run(prec, true, false, C, V, BT, t.h, C, t.logits, V, G->head, V, 0.f, EPI_NONE, nullptr,
                      splitk_for(C, V, BT), t.splitk, ss), "dhead");
  HIPCHK(stk_launch_layernorm_bwd(BT, C, bin(NB), M->ln_out_w, t.dh, nullptr, t.dx, t.part_ln, st, t.dx16), "ln_out bwd");
  HIPCHK(reduce_ln(G->ln_out_w, G->ln_out_b), "ln_out grads");
  HIPCHK(stk_launch_fill_zero(t.dvf, tokC, st), "zero dv_first");
  auto join_side = [&]() -> hipError_t {
    if (!sd) return hipSuccess;
    hipError_t r = hipEventRecord(sd->ev[2], ss);
    return r != hipSuccess ? r : hipStreamWaitEvent(st, sd->ev[2], 0);
  };
  // attention block i's backward (upstream t.dx; result into t.dx)
  auto attn_bwd = [&](int i, int pos) -> int {
    const rwkv7_attn_block& ab = M->attn[i];
    rwkv7_attn_grads& ga = G->attn[i];
    TrainBufs::AttnActs& a = t.aact[keep ? i : 0];
    if (!keep) CHK(attn_fwd(i, bin(pos), a));  // recompute this block's forward from its input
    // channel-mix backward (as in the RWKV-7 blocks)
    HIPCHK(gemm_run_x(prec, false, true, BT, F, C, t.dx, C, ab.cm_Wv, C, t.dfk, F, 0.f, EPI_SQRELU_BWD, a.ka, 1,
                      nullptr, st, t.dx16, t.act16), "attn dfk");
    HIPCHK(fork_here(), "backward fork");
    HIPCHK(gemm_run(prec, true, false, F, C, BT, a.ka, F, t.dx, C, ga.cm_Wv, C, 0.f, EPI_NONE, nullptr,
                    splitk_for(F, C, BT), t.splitk, ss), "attn dWv");
    HIPCHK(gemm_run(prec, true, false, C, F, BT, a.sh, C, t.dfk, F, ga.cm_Wk, F, 0.f, EPI_NONE, nullptr,
                    splitk_for(C, F, BT), t.splitk, ss), "attn dWk");
    HIPCHK(gemm_run_x(prec, false, true, BT, C, F, t.dfk, F, ab.cm_Wk, F, t.dsh, C, 0.f, EPI_NONE, nullptr, 1,
                      nullptr, st, t.act16, nullptr), "attn dsh");
    HIPCHK(stk_launch_cm_shift_bwd(BT, T, C, a.h2, nullptr, ab.cm_mu_k, t.dsh, t.dh, nullptr, t.part_cm, st), "attn cm shift bwd");
    {
      VecOut o = {{ga.cm_mu_k, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr}};
      HIPCHK(tm_launch_reduce(t.part_cm, 1, stk_num_shift_blocks(BT, C), C, o, st), "attn cm mu grad");
    }
    HIPCHK(stk_launch_layernorm_bwd(BT, C, a.x1, ab.ln2_w, t.dh, t.dx, t.dx1, t.part_ln, st), "attn ln2 bwd");
    HIPCHK(reduce_ln(ga.ln2_w, ga.ln2_b), "attn ln2 grads");
    // output projection: dy_core = dx1 Wo^T, dWo = y^T dx1
    HIPCHK(gemm_run(prec, false, true, BT, C, C, t.dx1, C, ab.Wo, C, t.dyc, C, 0.f, EPI_NONE, nullptr, 1, nullptr, st), "attn dy");
    HIPCHK(fork_here(), "backward fork");  // t.dx1 complete
    HIPCHK(gemm_run(prec, true, false, C, C, BT, a.y, C, t.dx1, C, ga.Wo, C, 0.f, EPI_NONE, nullptr,
                    splitk_for(C, C, BT), t.splitk, ss), "attn dWo");
    HIPCHK(moba_launch_backward(B, T, H, cfg->moba_chunk, cfg->moba_topk, a.q, a.k, a.v, a.y, a.lse, a.sel,
                                t.dyc, t.dq, t.dk, t.dv, t.mws, st), "moba backward");
    HIPCHK(fork_here(), "backward fork");  // dq, dk, dv complete
    const float* dqkv[3] = {t.dq, t.dk, t.dv};
    const float* Wqkv[3] = {ab.Wq, ab.Wk, ab.Wv};
    float* gqkv[3] = {ga.Wq, ga.Wk, ga.Wv};
    for (int j = 0; j < 3; j++) {
      HIPCHK(gemm_run(prec, true, false, C, C, BT, a.h, C, dqkv[j], C, gqkv[j], C, 0.f, EPI_NONE, nullptr,
                      splitk_for(C, C, BT), t.splitk, ss), "attn dWq/dWk/dWv");
      HIPCHK(gemm_run(prec, false, true, BT, C, C, dqkv[j], C, Wqkv[j], C, t.dh, C, j ? 1.f : 0.f, EPI_NONE,
                      nullptr, 1, nullptr, st), "attn dh1");
    }
    // the side stream's weight gradients read t.dx, t.dx1 and this block's
    // activations: joined before t.dx is written again
    HIPCHK(join_side(), "backward join");
    HIPCHK(stk_launch_layernorm_bwd(BT, C, bin(pos), ab.ln1_w, t.dh, t.dx1, t.dx, t.part_ln, st, t.dx16), "attn ln1 bwd");
    HIPCHK(reduce_ln(ga.ln1_w, ga.ln1_b), "attn ln1 grads");
    return WKV7_OK;
  };
  for (int pos = NB - 1; pos >= 0; pos--) {
    if (order[pos].first == 1) {
      CHK(attn_bwd(order[pos].second, pos));
      continue;
    }
    const int l = order[pos].second;
    const rwkv7_block& bl = M->blocks[l];
    rwkv7_block_grads& gb = G->blocks[l];
    tm_shape s = block_shape(cfg, l);
    BlockActs& a = t.act[keep ? l : 0];
    if (!keep) CHK(block_fwd(l, bin(pos), a));  // recompute this block's forward from its input
    // channel-mix backward
    HIPCHK(gemm_run_x(prec, false, true, BT, F, C, t.dx, C, bl.cm_Wv, C, t.dfk, F, 0.f, EPI_SQRELU_BWD, a.ka, 1,
                      nullptr, st, t.dx16, t.act16), "dfk");
    HIPCHK(fork_here(), "backward fork");  // t.dx and t.dfk complete
    HIPCHK(gemm_run(prec, true, false, F, C, BT, a.ka, F, t.dx, C, gb.cm_Wv, C, 0.f, EPI_NONE, nullptr,
                        splitk_for(F, C, BT), t.splitk, ss), "dWv");
    HIPCHK(gemm_run(prec, true, false, C, F, BT, a.sh, C, t.dfk, F, gb.cm_Wk, F, 0.f, EPI_NONE, nullptr,
                        splitk_for(C, F, BT), t.splitk, ss), "dWk");
    HIPCHK(gemm_run_x(prec, false, true, BT, C, F, t.dfk, F, bl.cm_Wk, F, t.dsh, C, 0.f, EPI_NONE, nullptr, 1,
                      nullptr, st, t.act16, nullptr), "dsh");
    HIPCHK(stk_launch_cm_shift_bwd(BT, T, C, a.h2, xp_cm(l), bl.cm_mu_k, t.dsh, t.dh, nullptr, t.part_cm, st), "cm shift bwd");
    {
      VecOut o = {{gb.cm_mu_k, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr}};
      HIPCHK(tm_launch_reduce(t.part_cm, 1, stk_num_shift_blocks(BT, C), C, o, st), "cm mu grad");
    }
    HIPCHK(stk_launch_layernorm_bwd(BT, C, a.x1, bl.ln2_w, t.dh, t.dx, t.dx1, t.part_ln, st, t.dx16), "ln2 bwd");
    HIPCHK(reduce_ln(gb.ln2_w, gb.ln2_b), "ln2 grads");
    // time-mix backward (input h, upstream dx1); v_first gradient summed over layers > 0
    CHK(tm_backward_impl(&s, &bl.tm, B, T, a.h, xp_tm(l), t.vf, s0_tm(l), t.dx1, nullptr, a.tm, t.tb,
                         &gb.tm, t.dh, nullptr, l == 0 ? t.dvf : nullptr, l > 0 ? t.dvf : nullptr, true,
                         nullptr, st, prec, sd, t.act16, t.dx16));
    HIPCHK(stk_launch_layernorm_bwd(BT, C, bin(pos), bl.ln1_w, t.dh, t.dx1, t.dx, t.part_ln, st, t.dx16), "ln1 bwd");
    HIPCHK(reduce_ln(gb.ln1_w, gb.ln1_b), "ln1 grads");
  }
  const float* demb_src = t.dx;
  if (cfg->use_ln0) {
    HIPCHK(stk_launch_layernorm_bwd(BT, C, t.x_emb, M->ln0_w, t.dx, nullptr, t.dx1, t.part_ln, st), "ln0 bwd");
    HIPCHK(reduce_ln(G->ln0_w, G->ln0_b), "ln0 grads");
    demb_src = t.dx1;
  }
  HIPCHK(stk_launch_emb_bwd(BT, V, C, tokens, demb_src, t.count, t.off, t.perm, G->emb, st), "embedding bwd");
  return WKV7_OK;
}
}  // namespace

extern "C" int rwkv7_train_step(const rwkv7_config* cfg, const rwkv7_model* M,
                                rwkv7_model_grads* G, int B, int T, const int* tokens,
                                const int* targets, float* loss, void* ws, size_t ws_bytes,
                                const wkv7_side* side, hipStream_t st) {
  g_err[0] = 0;
  const wkv7_side* sd = nullptr;
  Spans sp;
  const size_t need = rwkv7_train_workspace_bytes(cfg, B, T);
  CHK(check_train(cfg, M, G, B, T, tokens, targets, loss, ws, ws_bytes, need, side, st, sd, sp));
  model_spans(sp, cfg, M, false);
  CHK(sp.check());
  Carver cw(ws);
  TrainBufs t;
  carve_train(cw, cfg, B, T, t);
  return train_run(cfg, M, G, B, T, tokens, targets, loss, nullptr, t, sd, st);
}


// ------------------------------------------------------ online TBPTT segment --
namespace {

// Every parameter tensor of the model with its gradient, Adam moments (or
// NULL) and element count, in one fixed order.
template <typename Fn>
void for_each_param(const rwkv7_config* cfg, const rwkv7_model* M, const rwkv7_model_grads* G,
                    const rwkv7_model_grads* Mm, const rwkv7_model_grads* Vv, Fn fn) {
  const size_t C = cfg->C, F = cfg->F, V = cfg->V;
  auto P = [](const float* p) { return const_cast<float*>(p); };
  auto one = [&](const float* p, float* g, float* m, float* v, size_t n) { fn(P(p), g, m, v, n); };
  one(M->emb, G->emb, Mm ? Mm->emb : nullptr, Vv ? Vv->emb : nullptr, V * C);
  one(M->head, G->head, Mm ? Mm->head : nullptr, Vv ? Vv->head : nullptr, C * V);
  one(M->ln_out_w, G->ln_out_w, Mm ? Mm->ln_out_w : nullptr, Vv ? Vv->ln_out_w : nullptr, C);
  one(M->ln_out_b, G->ln_out_b, Mm ? Mm->ln_out_b : nullptr, Vv ? Vv->ln_out_b : nullptr, C);
  if (cfg->use_ln0) {
    one(M->ln0_w, G->ln0_w, Mm ? Mm->ln0_w : nullptr, Vv ? Vv->ln0_w : nullptr, C);
    one(M->ln0_b, G->ln0_b, Mm ? Mm->ln0_b : nullptr, Vv ? Vv->ln0_b : nullptr, C);
  }
  typedef const float* const tm_weights::*WF;
  typedef float* tm_grads::*GF;
  struct TmField {
    WF w;
    GF g;
    int rows, cols;  // in units: 0 -> C, -1 Dw, -2 Da, -3 Dv, -4 Dg, 1 -> 1
    bool v_lora;
  };
  static const TmField tmf[] = {
      {&tm_weights::mu_r, &tm_grads::mu_r, 1, 0, false}, {&tm_weights::mu_w, &tm_grads::mu_w, 1, 0, false},
      {&tm_weights::mu_k, &tm_grads::mu_k, 1, 0, false}, {&tm_weights::mu_v, &tm_grads::mu_v, 1, 0, false},
      {&tm_weights::mu_a, &tm_grads::mu_a, 1, 0, false}, {&tm_weights::mu_g, &tm_grads::mu_g, 1, 0, false},
      {&tm_weights::Wr, &tm_grads::Wr, 0, 0, false},     {&tm_weights::Wk, &tm_grads::Wk, 0, 0, false},
      {&tm_weights::Wv, &tm_grads::Wv, 0, 0, false},     {&tm_weights::Wo, &tm_grads::Wo, 0, 0, false},
      {&tm_weights::w0, &tm_grads::w0, 1, 0, false},     {&tm_weights::W1, &tm_grads::W1, 0, -1, false},
      {&tm_weights::W2, &tm_grads::W2, -1, 0, false},    {&tm_weights::a0, &tm_grads::a0, 1, 0, false},
      {&tm_weights::A1, &tm_grads::A1, 0, -2, false},    {&tm_weights::A2, &tm_grads::A2, -2, 0, false},
      {&tm_weights::v0, &tm_grads::v0, 1, 0, true},      {&tm_weights::V1, &tm_grads::V1, 0, -3, true},
      {&tm_weights::V2, &tm_grads::V2, -3, 0, true},     {&tm_weights::G1, &tm_grads::G1, 0, -4, false},
      {&tm_weights::G2, &tm_grads::G2, -4, 0, false},    {&tm_weights::k_k, &tm_grads::k_k, 1, 0, false},
      {&tm_weights::k_a, &tm_grads::k_a, 1, 0, false},   {&tm_weights::r_k, &tm_grads::r_k, 1, 0, false},
      {&tm_weights::ln_w, &tm_grads::ln_w, 1, 0, false}, {&tm_weights::ln_b, &tm_grads::ln_b, 1, 0, false}};
  auto dim = [&](int u) -> size_t {
    return u == 0 ? C : u == 1 ? 1 : u == -1 ? cfg->Dw : u == -2 ? cfg->Da : u == -3 ? cfg->Dv : cfg->Dg;
  };
  for (int l = 0; l < cfg->n_layer; l++) {
    const rwkv7_block& b = M->blocks[l];
    const rwkv7_block_grads& g = G->blocks[l];
    const rwkv7_block_grads* bm = Mm ? &Mm->blocks[l] : nullptr;
    const rwkv7_block_grads* bv = Vv ? &Vv->blocks[l] : nullptr;
    one(b.ln1_w, g.ln1_w, bm ? bm->ln1_w : nullptr, bv ? bv->ln1_w : nullptr, C);
    one(b.ln1_b, g.ln1_b, bm ? bm->ln1_b : nullptr, bv ? bv->ln1_b : nullptr, C);
    one(b.ln2_w, g.ln2_w, bm ? bm->ln2_w : nullptr, bv ? bv->ln2_w : nullptr, C);
    one(b.ln2_b, g.ln2_b, bm ? bm->ln2_b : nullptr, bv ? bv->ln2_b : nullptr, C);
    one(b.cm_mu_k, g.cm_mu_k, bm ? bm->cm_mu_k : nullptr, bv ? bv->cm_mu_k : nullptr, C);
    one(b.cm_Wk, g.cm_Wk, bm ? bm->cm_Wk : nullptr, bv ? bv->cm_Wk : nullptr, C * F);
    one(b.cm_Wv, g.cm_Wv, bm ? bm->cm_Wv : nullptr, bv ? bv->cm_Wv : nullptr, F * C);
    for (const TmField& tf : tmf) {
      if (tf.v_lora && l == 0) continue;
      one(b.tm.*(tf.w), g.tm.*(tf.g), bm ? bm->tm.*(tf.g) : nullptr, bv ? bv->tm.*(tf.g) : nullptr,
          dim(tf.rows) * dim(tf.cols));
    }
  }
}

// The segment replayed with the updated weights from the start state: the
// forward of every block, writing each layer's new streaming state (the WKV
// state in place; the two token-shift states through xl, then copied).
int replay_run(const rwkv7_config* cfg, const rwkv7_model* M, int B, int T, const int* tokens,
               float* axp, float* ast, float* fxp, TrainBufs& t, float* xl, hipStream_t st) {
  const int prec = cfg->gemm_dtype == WKV7_BF16 ? GEMM_BF16 : GEMM_F32;
  GemmPackScope pack_scope(t.pack, t.pack_bytes);
  const int C = cfg->C, F = cfg->F, V = cfg->V, L = cfg->n_layer, BT = B * T;
  const size_t tokC = (size_t)BT * C, BC = (size_t)B * C, NN = (size_t)WKV7_N * WKV7_N;
  auto bin = [&](int l) { return t.block_in + (size_t)l * tokC; };
  HIPCHK(stk_launch_emb_gather(BT, C, V, tokens, M->emb, cfg->use_ln0 ? t.x_emb : bin(0), st), "embedding");
  if (cfg->use_ln0)
    HIPCHK(stk_launch_layernorm(BT, C, t.x_emb, M->ln0_w, M->ln0_b, bin(0), nullptr, nullptr, st), "ln0");
  const bool keep = cfg->train_recompute == 0;
  for (int l = 0; l < L; l++) {
    // the layer's own activation set (kept mode: sized for its layer id) or
    // the one reused set (sized for a block with the value-residual LoRA)
    BlockActs& a = t.act[keep ? l : 0];
    const rwkv7_block& bl = M->blocks[l];
    tm_shape s = block_shape(cfg, l);
    float* st_l = ast + (size_t)l * B * cfg->H * NN;
    HIPCHK(stk_launch_layernorm(BT, C, bin(l), bl.ln1_w, bl.ln1_b, a.h, nullptr, nullptr, st), "ln1");
    CHK(tm_forward_impl(&s, &bl.tm, B, T, a.h, axp + (size_t)l * BC, t.vf, st_l, st_l, a.x1,
                        xl + (size_t)l * BC, a.tm, st, false, 0.f, prec, false, true, bin(l)));
    HIPCHK(stk_launch_layernorm(BT, C, a.x1, bl.ln2_w, bl.ln2_b, a.h2, nullptr, nullptr, st), "ln2");
    HIPCHK(stk_launch_cm_shift(BT, T, C, a.h2, fxp + (size_t)l * BC, bl.cm_mu_k, a.sh,
                               xl + (size_t)(L + l) * BC, st), "cm shift");
    HIPCHK(gemm_run(prec, false, false, BT, F, C, a.sh, C, bl.cm_Wk, F, a.ka, F, 0.f, EPI_SQRELU, nullptr, 1, nullptr, st), "cm key");
    HIPCHK(gemm_run(prec, false, false, BT, C, F, a.ka, F, bl.cm_Wv, C, bin(l + 1), C, 0.f, EPI_ADD, a.x1, 1, nullptr, st), "cm value");
  }
  HIPCHK(hipMemcpyAsync(axp, xl, (size_t)L * BC * sizeof(float), hipMemcpyDeviceToDevice, st), "state copy");
  HIPCHK(hipMemcpyAsync(fxp, xl + (size_t)L * BC, (size_t)L * BC * sizeof(float), hipMemcpyDeviceToDevice, st), "state copy");
  return WKV7_OK;
}

}  // namespace

extern "C" size_t rwkv7_online_workspace_bytes(const rwkv7_config* cfg, int B, int S) {
  if (check_cfg(cfg, B) != WKV7_OK || S < 1 || cfg->n_attn != 0) return 0;
  Carver c(nullptr);
  TrainBufs t;
  carve_train(c, cfg, B, S, t);
  c.take((size_t)2 * cfg->n_layer * B * cfg->C);  // the replay's new token-shift states
  return c.off + 256;
}

extern "C" int rwkv7_online_segment(const rwkv7_config* cfg, const rwkv7_model* M,
                                    rwkv7_model_grads* G, rwkv7_model_grads* adam_m,
                                    rwkv7_model_grads* adam_v, const rwkv7_optim* opt, int B, int S,
                                    const int* tokens, const int* targets, float* att_x_prev,
                                    float* att_state, float* ffn_x_prev, float* loss, void* ws,
                                    size_t ws_bytes, const wkv7_side* side, hipStream_t st) {
  g_err[0] = 0;
  if (cfg && cfg->n_attn != 0) return fail(WKV7_EINVAL, "attention blocks are supported by rwkv7_train_step only");
  if (!opt) return fail(WKV7_EINVAL, "optimiser settings are NULL");
  if (opt->optimizer != 0 && opt->optimizer != 1) return fail(WKV7_EINVAL, "optimizer must be 0 (SGD) or 1 (Adam)");
  if (!(opt->lr >= 0.f) || !(opt->clip >= 0.f) || opt->lr > 1e30f || opt->clip > 1e30f)
    return fail(WKV7_EINVAL, "lr and clip must be finite and >= 0");
  const bool adam = opt->optimizer == 1;
  if (adam && opt->step < 1) return fail(WKV7_EINVAL, "Adam step must be >= 1 (got %d)", opt->step);
  if (adam && (!adam_m || !adam_v || !adam_m->blocks || !adam_v->blocks))
    return fail(WKV7_EINVAL, "Adam needs both moment mirrors");
  CHK(check_f32_ptr(att_x_prev, "att_x_prev", true));
  CHK(check_f32_ptr(att_state, "att_state", true));
  CHK(check_f32_ptr(ffn_x_prev, "ffn_x_prev", true));
  const wkv7_side* sd = nullptr;
  Spans sp;
  const size_t need = rwkv7_online_workspace_bytes(cfg, B, S);
  CHK(check_train(cfg, M, G, B, S, tokens, targets, loss, ws, ws_bytes, need, side, st, sd, sp));
  int bad = 0;
  if (adam)
    for_each_param(cfg, M, G, adam_m, adam_v, [&](float*, float*, float* m, float* v, size_t) {
      if (bad == 0 && (check_f32_ptr(m, "an Adam moment", true) || check_f32_ptr(v, "an Adam moment", true))) bad = 1;
    });
  if (bad) return WKV7_EINVAL;
  model_spans(sp, cfg, M, true);  // the weights are updated in place
  if (adam) {
    model_spans(sp, cfg, adam_m, true);
    model_spans(sp, cfg, adam_v, true);
  }
  const size_t f = sizeof(float), L = cfg->n_layer, BC = (size_t)B * cfg->C;
  sp.wr(att_x_prev, L * BC * f, "att_x_prev");  // start state in, live state out
  sp.wr(att_state, L * state_bytes(B, cfg->H), "att_state");
  sp.wr(ffn_x_prev, L * BC * f, "ffn_x_prev");
  CHK(sp.check());

  Carver cw(ws);
  TrainBufs t;
  carve_train(cw, cfg, B, S, t);
  float* xl = cw.take(2 * L * BC);
  // 1. gradients of the segment from the start state (truncated there)
  const StartState s0{att_x_prev, att_state, ffn_x_prev};
  CHK(train_run(cfg, M, G, B, S, tokens, targets, loss, &s0, t, sd, st));
  // 2. the update, up to OPT_MAX tensors per launch
  OptBatch ob;
  memset(&ob, 0, sizeof(ob));
  hipError_t e = hipSuccess;
  auto flush = [&]() {
    if (ob.n && e == hipSuccess) e = opt_launch(ob, adam ? 1 : 0, opt->lr, opt->clip, opt->step, st);
    ob.n = 0;
  };
  for_each_param(cfg, M, G, adam_m, adam_v, [&](float* p, float* g, float* m, float* v, size_t n) {
    ob.p[ob.n] = p; ob.g[ob.n] = g; ob.m[ob.n] = m; ob.v[ob.n] = v; ob.count[ob.n] = n;
    if (++ob.n == OPT_MAX) flush();
  });
  flush();
  HIPCHK(e, "parameter update");
  // 3. the live state: the segment replayed with the updated weights
  return replay_run(cfg, M, B, S, tokens, att_x_prev, att_state, ffn_x_prev, t, xl, st);
}

// ------------------------------------------------------------ GatedDeltaNet --
namespace {

int check_gdn(const gdn_shape* s, const gdn_weights* W, int B, int T) {
  if (!s || !W) return fail(WKV7_EINVAL, "shape or weights is NULL");
  if ((s->dk != 64 && s->dk != 128) || (s->dv != 64 && s->dv != 128))
    return fail(WKV7_EINVAL, "dk and dv must be 64 or 128 (got %d, %d)", s->dk, s->dv);
  if (s->nk < 1 || s->nv < 1 || s->nv % s->nk || s->nv / s->nk > 16)
    return fail(WKV7_EINVAL, "nv must be a multiple of nk with at most 16 value heads per key head");
  if (s->kk < 1 || s->kk > 8) return fail(WKV7_EINVAL, "kk must be in 1..8 (got %d)", s->kk);
  if (!(s->rms_eps >= 0.f)) return fail(WKV7_EINVAL, "rms_eps must be >= 0");
  if (B < 1 || T < 1) return fail(WKV7_EINVAL, "B, T must be >= 1 (got %d, %d)", B, T);
  const size_t cdim = 2 * (size_t)s->nk * s->dk + (size_t)s->nv * s->dv;
  if ((size_t)B * T * cdim > ((size_t)1 << 36)) return fail(WKV7_EINVAL, "problem too large");
  CHK(check_f32_ptr(W->conv, "conv", true));
  CHK(check_f32_ptr(W->A_log, "A_log", true));
  CHK(check_f32_ptr(W->dt_bias, "dt_bias", true));
  CHK(check_f32_ptr(W->norm, "norm", true));
  return WKV7_OK;
}

size_t gdn_cdim(const gdn_shape* s) { return 2 * (size_t)s->nk * s->dk + (size_t)s->nv * s->dv; }

void carve_gdn_cache(Carver& c, const gdn_shape* s, int B, int T, GdnArgs& p) {
  const size_t BT = (size_t)B * T, cd = gdn_cdim(s);
  p.pre = c.take(BT * cd);
  p.cq = c.take(BT * cd);
  p.qh = c.take(BT * s->nk * s->dk);
  p.kh = c.take(BT * s->nk * s->dk);
  p.g = c.take(BT * s->nv);
  p.beta = c.take(BT * s->nv);
  p.o = c.take(BT * s->nv * s->dv);
  p.ckpt = c.take(gdn_ckpt_floats(B, T, s->nv, s->dk, s->dv));
  p.kv = c.take(BT * s->nv * s->dv);
}

void carve_gdn_bwd(Carver& c, const gdn_shape* s, int B, int T, GdnArgs& p) {
  const size_t BT = (size_t)B * T;
  p.dobuf = c.take(BT * s->nv * s->dv);
  p.dcq = c.take(BT * gdn_cdim(s));
  p.part = c.take(gdn_partial_floats(B, T, s->nv, s->dk, s->dv));
  p.gend = p.du = p.anc = nullptr;
  if (gdn_two_pass(s->dk, s->dv)) {
    const size_t nblk = (T + 15) / 16;
    p.gend = c.take(gdn_ckpt_floats(B, T, s->nv, s->dk, s->dv));
    p.du = c.take(BT * s->nv * s->dv);
    p.anc = c.take((size_t)B * s->nv * nblk * s->dv);
  }
}

void gdn_fill(GdnArgs& p, const gdn_shape* s, const gdn_weights* W, int B, int T,
              const float* raw, const float* z, const float* a, const float* b) {
  p.B = B; p.T = T; p.nk = s->nk; p.nv = s->nv; p.dk = s->dk; p.dv = s->dv; p.kk = s->kk;
  p.rms_eps = s->rms_eps;
  p.raw = raw; p.z = z; p.a = a; p.b = b;
  p.conv = W->conv; p.A_log = W->A_log; p.dt_bias = W->dt_bias; p.norm = W->norm;
}

void gdn_input_spans(Spans& sp, const gdn_shape* s, int B, int T, const float* raw,
                     const float* z, const float* a, const float* b, const gdn_weights* W) {
  const size_t BT = (size_t)B * T, f = sizeof(float);
  sp.rd(raw, BT * gdn_cdim(s) * f, "raw");
  sp.rd(z, BT * s->nv * s->dv * f, "z");
  sp.rd(a, BT * s->nv * f, "a");
  sp.rd(b, BT * s->nv * f, "b");
  sp.rd(W->conv, gdn_cdim(s) * s->kk * f, "conv");
  sp.rd(W->A_log, s->nv * f, "A_log");
  sp.rd(W->dt_bias, s->nv * f, "dt_bias");
  sp.rd(W->norm, s->dv * f, "norm");
}

}  // namespace

extern "C" size_t gdn_cache_bytes(const gdn_shape* s, int B, int T) {
  if (!s || B < 1 || T < 1) return 0;
  Carver c(nullptr);
  GdnArgs p;
  carve_gdn_cache(c, s, B, T, p);
  return c.off + 256;
}

extern "C" size_t gdn_backward_workspace_bytes(const gdn_shape* s, int B, int T, int have_cache) {
  if (!s || B < 1 || T < 1) return 0;
  Carver c(nullptr);
  GdnArgs p;
  if (!have_cache) carve_gdn_cache(c, s, B, T, p);
  carve_gdn_bwd(c, s, B, T, p);
  return c.off + 256;
}

extern "C" int gdn_forward(const gdn_shape* s, const gdn_weights* W, int B, int T, const float* raw,
                           const float* z, const float* a, const float* b, float* out, void* cache,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  CHK(check_gdn(s, W, B, T));
  const float* ins[] = {raw, z, a, b, out};
  const char* nm[] = {"raw", "z", "a", "b", "out"};
  for (int i = 0; i < 5; i++) CHK(check_f32_ptr(ins[i], nm[i], true));
  const size_t need = gdn_cache_bytes(s, B, T);
  void* base = cache;
  if (!base) {
    if (!ws || ws_bytes < need)
      return fail(WKV7_ENOSPC, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    base = ws;
  }
  CHK(check_f32_ptr(base, cache ? "cache" : "ws", true));
  {
    Spans sp;
    gdn_input_spans(sp, s, B, T, raw, z, a, b, W);
    sp.wr(out, (size_t)B * T * s->nv * s->dv * sizeof(float), "out");
    sp.wr(base, need, cache ? "cache" : "ws");
    CHK(sp.check());
  }
  GdnArgs p;
  memset(&p, 0, sizeof(p));
  gdn_fill(p, s, W, B, T, raw, z, a, b);
  Carver c(base);
  carve_gdn_cache(c, s, B, T, p);
  p.out = out;
  HIPCHK(gdn_launch_forward(p, stream), "gdn_forward launch");
  return WKV7_OK;
}

extern "C" int gdn_backward(const gdn_shape* s, const gdn_weights* W, int B, int T, const float* raw,
                            const float* z, const float* a, const float* b, const float* dout,
                            const void* cache, float* draw, float* dz, float* da, float* db,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  CHK(check_gdn(s, W, B, T));
  const float* ins[] = {raw, z, a, b, dout, draw, dz, da, db};
  const char* nm[] = {"raw", "z", "a", "b", "dout", "draw", "dz", "da", "db"};
  for (int i = 0; i < 9; i++) CHK(check_f32_ptr(ins[i], nm[i], true));
  CHK(check_f32_ptr(cache, "cache", false));
  const size_t need = gdn_backward_workspace_bytes(s, B, T, cache != nullptr);
  if (!ws || ws_bytes < need)
    return fail(WKV7_ENOSPC, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  CHK(check_f32_ptr(ws, "ws", true));
  {
    const size_t BT = (size_t)B * T, f = sizeof(float);
    Spans sp;
    gdn_input_spans(sp, s, B, T, raw, z, a, b, W);
    sp.rd(dout, BT * s->nv * s->dv * f, "dout");
    sp.rd(cache, cache ? gdn_cache_bytes(s, B, T) : 0, "cache");
    sp.wr(draw, BT * gdn_cdim(s) * f, "draw");
    sp.wr(dz, BT * s->nv * s->dv * f, "dz");
    sp.wr(da, BT * s->nv * f, "da");
    sp.wr(db, BT * s->nv * f, "db");
    sp.wr(ws, need, "ws");
    CHK(sp.check());
  }
  GdnArgs p;
  memset(&p, 0, sizeof(p));
  gdn_fill(p, s, W, B, T, raw, z, a, b);
  Carver cw(ws);
  if (!cache) carve_gdn_cache(cw, s, B, T, p);
  carve_gdn_bwd(cw, s, B, T, p);
  if (!cache) {
    // recompute the cache; the forward's output itself is not needed, so it
    // goes to dobuf, which the backward's first kernel overwrites
    p.out = p.dobuf;
    HIPCHK(gdn_launch_forward(p, stream), "gdn_backward forward recompute");
  } else {
    Carver cc((void*)cache);
    carve_gdn_cache(cc, s, B, T, p);
  }
  p.dout = dout;
  p.dz = dz; p.draw = draw; p.da = da; p.db = db;
  HIPCHK(gdn_launch_backward(p, stream), "gdn_backward launch");
  return WKV7_OK;
}

// ------------------------------------------------------- MoBA attention --
namespace {
int check_moba(int B, int T, int H, int N, int chunk, int topk) {
  if (N != WKV7_N) return fail(WKV7_EINVAL, "head size N=%d unsupported (must be 64)", N);
  if (B < 1 || T < 1 || H < 1) return fail(WKV7_EINVAL, "B, T, H must be >= 1 (got %d, %d, %d)", B, T, H);
  if (chunk < 1) return fail(WKV7_EINVAL, "chunk must be >= 1 (got %d)", chunk);
  if (moba_num_chunks(T, chunk) > 64)
    return fail(WKV7_EINVAL, "T=%d in chunks of %d gives %d chunks (at most 64)", T, chunk,
                moba_num_chunks(T, chunk));
  if (topk < 1 || topk > 64) return fail(WKV7_EINVAL, "topk must be in [1, 64] (got %d)", topk);
  if ((size_t)B * T * H * N > ((size_t)1 << 36)) return fail(WKV7_EINVAL, "problem too large");
  return WKV7_OK;
}
int check_sel_ptr(const void* p, const char* name) {
  if (!p) return fail(WKV7_EINVAL, "%s is NULL", name);
  if ((uintptr_t)p & 7) return fail(WKV7_EINVAL, "%s must be 8-byte aligned", name);
  return WKV7_OK;
}
}  // namespace

extern "C" size_t moba_workspace_bytes(int B, int T, int H, int N, int chunk, int topk) {
  if (check_moba(B, T, H, N, chunk, topk) != WKV7_OK) return 0;
  return moba_ws_bytes(B, T, H, chunk, topk);
}

extern "C" int moba_forward(int B, int T, int H, int N, int chunk, int topk, const float* q,
                            const float* k, const float* v, float* y, float* lse, uint64_t* sel,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  CHK(check_moba(B, T, H, N, chunk, topk));
  const float* ptr[] = {q, k, v, y, lse, (const float*)ws};
  const char* nm[] = {"q", "k", "v", "y", "lse", "ws"};
  for (int i = 0; i < 6; i++) CHK(check_f32_ptr(ptr[i], nm[i], true));
  CHK(check_sel_ptr(sel, "sel"));
  const size_t need = moba_workspace_bytes(B, T, H, N, chunk, topk);
  if (ws_bytes < need) return fail(WKV7_ENOSPC, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  {
    const size_t tok = (size_t)B * T * H * N * sizeof(float), row = (size_t)B * H * T;
    Spans sp;
    sp.rd(q, tok, "q");
    sp.rd(k, tok, "k");
    sp.rd(v, tok, "v");
    sp.wr(y, tok, "y");
    sp.wr(lse, row * sizeof(float), "lse");
    sp.wr(sel, row * sizeof(uint64_t), "sel");
    sp.wr(ws, need, "ws");
    CHK(sp.check());
  }
  HIPCHK(moba_launch_forward(B, T, H, chunk, topk, q, k, v, y, lse, sel, ws, stream),
         "moba_forward launch");
  return WKV7_OK;
}

extern "C" int moba_backward(int B, int T, int H, int N, int chunk, int topk, const float* q,
                             const float* k, const float* v, const float* y, const float* lse,
                             const uint64_t* sel, const float* dy, float* dq, float* dk, float* dv,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  CHK(check_moba(B, T, H, N, chunk, topk));
  const float* ptr[] = {q, k, v, y, lse, dy, dq, dk, dv, (const float*)ws};
  const char* nm[] = {"q", "k", "v", "y", "lse", "dy", "dq", "dk", "dv", "ws"};
  for (int i = 0; i < 10; i++) CHK(check_f32_ptr(ptr[i], nm[i], true));
  CHK(check_sel_ptr(sel, "sel"));
  const size_t need = moba_workspace_bytes(B, T, H, N, chunk, topk);
  if (ws_bytes < need) return fail(WKV7_ENOSPC, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  {
    const size_t tok = (size_t)B * T * H * N * sizeof(float), row = (size_t)B * H * T;
    Spans sp;
    sp.rd(q, tok, "q");
    sp.rd(k, tok, "k");
    sp.rd(v, tok, "v");
    sp.rd(y, tok, "y");
    sp.rd(dy, tok, "dy");
    sp.rd(lse, row * sizeof(float), "lse");
    sp.rd(sel, row * sizeof(uint64_t), "sel");
    sp.wr(dq, tok, "dq");
    sp.wr(dk, tok, "dk");
    sp.wr(dv, tok, "dv");
    sp.wr(ws, need, "ws");
    CHK(sp.check());
  }
  HIPCHK(moba_launch_backward(B, T, H, chunk, topk, q, k, v, y, lse, sel, dy, dq, dk, dv, ws, stream),
         "moba_backward launch");
  return WKV7_OK;
}
