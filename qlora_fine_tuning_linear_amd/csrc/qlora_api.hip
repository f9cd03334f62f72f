// C ABI entry points (include/qlora.h): validate, then enqueue the kernels of
// one pass on the caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "qlora.h"
#include "qlora_launch.h"
#include "qlora_plan.h"
#include "qlora_validate.h"

// Scratch of qlora_linear_fwd_static: one array per GPU, in this file's
// device code object, held until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: never pass it to a kernel.
constexpr size_t kStaticScratchBytes = QLORA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

// Per-device answer to "is this a gfx950": 0 unknown, 1 yes, 2 no.
std::atomic<int> g_dev_ok[64];
// qlora_debug_force_arch: when set, the architecture name every device is
// taken to have (0: the device's own, the normal case).
std::atomic<int> g_arch_forced{0};
char g_arch_name[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QLORA_ERR_HIP;
  if (dev < 0 || dev >= 64) return QLORA_ERR_UNSUPPORTED_DEVICE;
  if (g_arch_forced.load(std::memory_order_acquire))
    return strncmp(g_arch_name, "gfx950", 6) == 0 ? QLORA_OK : QLORA_ERR_UNSUPPORTED_DEVICE;
  int s = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QLORA_ERR_HIP;
    s = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_ok[dev].store(s, std::memory_order_relaxed);
  }
  return s == 1 ? QLORA_OK : QLORA_ERR_UNSUPPORTED_DEVICE;
}

// Scratch of qlora_linear_fwd_static (the array itself is defined at file
// scope above this namespace).  Its device address is looked up once per
// device, with that device current, and only that address is ever handed to
// kernels or host-side HIP calls.
std::atomic<void*> g_scratch[64];
std::mutex g_scratch_mu;

int static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QLORA_ERR_HIP;
  if (dev < 0 || dev >= 64) return QLORA_ERR_UNSUPPORTED_DEVICE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return QLORA_ERR_HIP;
      p = addr;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return QLORA_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP; }

// Launch tracing (qlora_trace_install): caller-owned event arrays.
struct Trace {
  void** begin = nullptr;
  void** end = nullptr;
  int32_t* kinds = nullptr;
  int32_t capacity = 0;
  int32_t* count = nullptr;
} g_trace;

// One GEMM launch, bracketed by trace events when tracing is installed.
// bf16: the bf16-staged kernel (the weight already expanded into a.wb).
hipError_t traced_gemm(int mode, bool bf16, const GemmArgs& a, const qplan::GemmPlan& pl, hipStream_t st) {
  int32_t idx = -1;
  if (g_trace.capacity > 0 && g_trace.count) {
    idx = (*g_trace.count)++;
    if (idx < g_trace.capacity) {
      hipError_t e = hipEventRecord(static_cast<hipEvent_t>(g_trace.begin[idx]), st);
      if (e != hipSuccess) return e;
      g_trace.kinds[idx] = mode + (bf16 ? 8 : 0);
    } else {
      idx = -1;
    }
  }
  hipError_t e = bf16 ? launch_bgemm(mode, a, st) : launch_qgemm(mode, a, pl, st);
  if (e == hipSuccess && idx >= 0) e = hipEventRecord(static_cast<hipEvent_t>(g_trace.end[idx]), st);
  return e;
}

// Trace slot around one launch (-1: not traced).
int32_t trace_begin(int32_t kind, hipStream_t st, hipError_t* err) {
  *err = hipSuccess;
  if (g_trace.capacity <= 0 || !g_trace.count) return -1;
  const int32_t idx = (*g_trace.count)++;
  if (idx >= g_trace.capacity) return -1;
  *err = hipEventRecord(static_cast<hipEvent_t>(g_trace.begin[idx]), st);
  g_trace.kinds[idx] = kind;
  return idx;
}
hipError_t trace_end(int32_t idx, hipError_t e, hipStream_t st) {
  if (e == hipSuccess && idx >= 0) e = hipEventRecord(static_cast<hipEvent_t>(g_trace.end[idx]), st);
  return e;
}

// Skinny-M forward GEMM (the streaming form when the activations were re-laid
// out), traced as kind mode + 16.
hipError_t traced_skinny_fwd(const SkinnyArgs& a, const qplan::SkinnyPlan& pl, hipStream_t st) {
  hipError_t e;
  const int32_t idx = trace_begin(MODE_FWD + 16, st, &e);
  if (e != hipSuccess) return e;
  return trace_end(idx, a.Xt ? launch_skinny_fwd2(a, pl, st) : launch_skinny_fwd(a, pl, st), st);
}

// Skinny-M transposed product, traced as kind MODE_BWD + 16.
hipError_t traced_skinny_bwd(const SkinnyBwdArgs& a, int splits, hipStream_t st) {
  hipError_t e;
  const int32_t idx = trace_begin(MODE_BWD + 16, st, &e);
  if (e != hipSuccess) return e;
  return trace_end(idx, launch_skinny_bwd(a, splits, st), st);
}

hipError_t traced_gemm_q(int mode, const GemmArgs& a, const qplan::GemmPlan& pl, hipStream_t st) {
  return traced_gemm(mode, false, a, pl, st);
}
hipError_t traced_gemm_b(int mode, const GemmArgs& a, hipStream_t st) {
  return traced_gemm(mode, true, a, qplan::GemmPlan{}, st);
}

Nf4Dev to_dev(const qlora_nf4& w) {
  Nf4Dev d;
  d.codes = w.codes;
  d.absmax = w.absmax;
  d.absmax_q = w.absmax_q;
  d.absmax_scale = w.absmax_scale;
  d.N = w.N;
  d.K = w.K;
  d.dq = w.dq_group;
  return d;
}

float lora_s(const qlora_linear& L) { return L.alpha / (float)L.r; }

// LoRA term with the B [N, r] matrix (forward side).
LoraSide side_B(const qlora_linear& L, const float* V) {
  return LoraSide{V, static_cast<const uint16_t*>(L.B), (int64_t)L.r, 1, L.r, lora_s(L)};
}
// LoRA term with the A [r, K] matrix (backward side), read from its
// transposed copy AT [K, r] (rows contiguous in j, as the GEMM wants).
LoraSide side_AT(const qlora_linear& L, const float* V, const uint16_t* AT) {
  return LoraSide{V, AT, (int64_t)L.r, 1, L.r, lora_s(L)};
}

GemmArgs gemm_args() {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  return a;
}

#define QTRY(expr)                  \
  do {                              \
    const int _st = (expr);         \
    if (_st != QLORA_OK) return _st; \
  } while (0)
#define QHIP(expr) QTRY(hip_status(expr))

const uint16_t* u16(const void* p) { return static_cast<const uint16_t*>(p); }
uint16_t* u16m(void* p) { return static_cast<uint16_t*>(p); }
char* bytes(void* p) { return static_cast<char*>(p); }

}  // namespace

extern "C" {

int qlora_trace_install(void** begin_events, void** end_events, int32_t* kinds, int32_t capacity, int32_t* count) {
  if (capacity <= 0 || !begin_events || !end_events || !kinds || !count) {
    g_trace = Trace{};
    return QLORA_OK;
  }
  g_trace.begin = begin_events;
  g_trace.end = end_events;
  g_trace.kinds = kinds;
  g_trace.capacity = capacity;
  g_trace.count = count;
  return QLORA_OK;
}

int qlora_debug_force_arch(const char* gcn_arch_name) {
  if (!gcn_arch_name) {
    g_arch_forced.store(0, std::memory_order_release);
    return QLORA_OK;
  }
  if (strlen(gcn_arch_name) >= sizeof(g_arch_name)) return QLORA_ERR_INVALID_ARG;
  g_arch_forced.store(0, std::memory_order_release);
  strncpy(g_arch_name, gcn_arch_name, sizeof(g_arch_name) - 1);
  g_arch_name[sizeof(g_arch_name) - 1] = 0;
  g_arch_forced.store(1, std::memory_order_release);
  return QLORA_OK;
}

int nf4_quantize(const float* W, int64_t N, int64_t K, const float* codebook16, int32_t blocksize, int32_t dq_group,
                 uint8_t* codes, float* absmax, uint8_t* absmax_q, float* absmax_scale, void* stream) {
  QTRY(qv_quantize(W, N, K, codebook16, blocksize, dq_group, codes, absmax, absmax_q, absmax_scale));
  if (N == 0 || K == 0) return QLORA_OK;
  QTRY(check_device());
  return hip_status(launch_nf4_quantize(W, N * K / 64, codebook16, dq_group, codes, absmax, absmax_q, absmax_scale,
                                        static_cast<hipStream_t>(stream)));
}

int nf4_dequantize(const qlora_nf4* w, int32_t out_dtype, void* out, void* stream) {
  QTRY(qv_dequantize(w, out_dtype, out));
  QTRY(check_device());
  return hip_status(launch_nf4_dequantize(to_dev(*w), w->codebook, out_dtype == QLORA_DTYPE_F32 ? 1 : 0, out,
                                          static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ groups
// The packed groups as one layer: W0 and the stacked A as given, B the
// block-diagonal of bf16(s_g B_g) held in the workspace, s = 1.
static int linear_bwd_impl(const qlora_linear* L, const void* dY, const void* X, const float* XA_saved, int64_t M,
                           void* dX, void* dA, void* dB, const GroupDesc* grp, bool* grp_done, void* ws,
                           size_t ws_bytes, void* stream);

static qlora_linear grouped_layer(const qlora_grouped* Q, GroupDesc* d) {
  memset(d, 0, sizeof(*d));
  d->G = Q->G;
  for (int g = 0; g < Q->G; ++g) {
    d->B[g] = static_cast<const uint16_t*>(Q->B[g]);
    d->noff[g + 1] = d->noff[g] + Q->N[g];
    d->roff[g + 1] = d->roff[g] + Q->r[g];
    d->s[g] = Q->alpha[g] / (float)Q->r[g];
  }
  qlora_linear L;
  memset(&L, 0, sizeof(L));
  L.W0 = Q->W0;
  L.A = Q->A;
  L.B = nullptr;  // set to the block-diagonal copy
  L.r = d->roff[Q->G];
  L.alpha = (float)L.r;  // s = alpha / r = 1
  return L;
}

static size_t grouped_bcat_bytes(const qlora_grouped* Q, int r) {
  return qplan::align256((size_t)Q->W0.N * (size_t)r * 2);
}

size_t qlora_grouped_workspace_bytes(const qlora_grouped* Q, int64_t M) {
  if (qv_grouped(Q)) return 0;
  GroupDesc d;
  qlora_linear L = grouped_layer(Q, &d);
  L.B = L.A;  // any non-null pointer: only the shapes matter for sizing
  return 2 * grouped_bcat_bytes(Q, L.r) + qlora_linear_workspace_bytes(&L, M);
}

int qlora_grouped_fwd(const qlora_grouped* Q, const void* X, int64_t M, void* Y, float* XA_saved, void* ws,
                      size_t ws_bytes, void* stream) {
  QTRY(qv_grouped(Q));
  GroupDesc d;
  qlora_linear L = grouped_layer(Q, &d);
  const size_t bc = grouped_bcat_bytes(Q, L.r);
  if (M > 0 && ws_bytes < 2 * bc) return QLORA_ERR_WORKSPACE_TOO_SMALL;
  L.B = M > 0 ? ws : Q->A;  // where the block-diagonal B goes; validated with the rest first
  QTRY(qv_linear_fwd(&L, X, M, Y, XA_saved, M > 0 ? bytes(ws) + 2 * bc : ws, M > 0 ? ws_bytes - 2 * bc : 0));
  if (M == 0) return QLORA_OK;
  QTRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint16_t* bcat = reinterpret_cast<uint16_t*>(bytes(ws));
  QHIP(launch_grouped_bcat(d, (int)Q->W0.N, L.r, bcat, st));
  L.B = bcat;
  return qlora_linear_fwd(&L, X, M, Y, XA_saved, bytes(ws) + 2 * bc, ws_bytes - 2 * bc, stream);
}

int qlora_grouped_bwd(const qlora_grouped* Q, const void* dY, const void* X, const float* XA_saved, int64_t M,
                      void* dX, void* dA, void* const* dB, void* ws, size_t ws_bytes, void* stream) {
  QTRY(qv_grouped(Q));
  QTRY(qv_grouped_dB(Q, dB));
  GroupDesc d;
  qlora_linear L = grouped_layer(Q, &d);
  for (int g = 0; g < Q->G; ++g) d.dB[g] = static_cast<uint16_t*>(dB[g]);
  const size_t bc = grouped_bcat_bytes(Q, L.r);
  if (ws_bytes < 2 * bc) return QLORA_ERR_WORKSPACE_TOO_SMALL;
  L.B = ws;  // where the block-diagonal B goes; validated with the rest first
  QTRY(qv_linear_bwd(&L, dY, X, XA_saved, M, dX, dA, bytes(ws) + bc, bytes(ws) + 2 * bc, ws_bytes - 2 * bc));
  QTRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint16_t* bcat = reinterpret_cast<uint16_t*>(bytes(ws));
  uint16_t* dbcat = reinterpret_cast<uint16_t*>(bytes(ws) + bc);
  QHIP(launch_grouped_bcat(d, (int)Q->W0.N, L.r, bcat, st));
  L.B = bcat;
  bool done = false;
  QTRY(linear_bwd_impl(&L, dY, X, XA_saved, M, dX, dA, dbcat, &d, &done, bytes(ws) + 2 * bc, ws_bytes - 2 * bc,
                       stream));
  if (done) return QLORA_OK;
  return hip_status(launch_grouped_db(d, (int)Q->W0.N, L.r, dbcat, st));
}

int rmsnorm_fwd(const void* X, const void* w, int64_t M, int64_t D, float eps, void* Y, float* rstd,
                void* stream) {
  QTRY(qv_rmsnorm_fwd(X, w, M, D, eps, Y, rstd));
  if (M == 0) return QLORA_OK;
  QTRY(check_device());
  return hip_status(launch_rmsnorm_fwd(u16(X), u16(w), M, D, eps, u16m(Y), rstd, static_cast<hipStream_t>(stream)));
}

size_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t D) { return qv_rmsnorm_ws(M, D); }

int rmsnorm_bwd(const void* dY, const void* X, const void* w, const float* rstd, int64_t M, int64_t D, void* dX,
                float* dw, void* ws, size_t ws_bytes, void* stream) {
  QTRY(qv_rmsnorm_bwd(dY, X, w, rstd, M, D, dX, dw, ws, ws_bytes));
  if (M == 0 && !dw) return QLORA_OK;
  QTRY(check_device());
  return hip_status(launch_rmsnorm_bwd(u16(dY), u16(X), u16(w), rstd, M, D, u16m(dX), dw,
                                       reinterpret_cast<float*>(ws), static_cast<hipStream_t>(stream)));
}

size_t qlora_linear_ce_workspace_bytes(int64_t T, int64_t D, int64_t V, int64_t chunk, int32_t want_dx) {
  return qv_linear_ce_ws(T, D, V, chunk, want_dx);
}

int qlora_linear_ce(const void* X, int64_t T, int64_t D, const void* W, int64_t V, const int32_t* targets,
                    int32_t ignore_index, int64_t chunk, float* loss, float* token_loss, void* dX, void* ws,
                    size_t ws_bytes, void* stream) {
  QTRY(qv_linear_ce(X, T, D, W, V, targets, chunk, loss, token_loss, dX, ws, ws_bytes));
  QTRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (T == 0) return hip_status(launch_ce_loss(nullptr, 0, nullptr, loss, st));
  const bool want_dx = dX != nullptr;
  const qplan::CeWs w = qplan::ce_ws(T, D, V, chunk, want_dx);
  char* b = bytes(ws);
  int32_t* nvalid = reinterpret_cast<int32_t*>(b);
  float* tl = token_loss ? token_loss : reinterpret_cast<float*>(b + w.nvalid);
  float* z = reinterpret_cast<float*>(b + w.nvalid + w.tloss);
  float* part = reinterpret_cast<float*>(b + w.nvalid + w.tloss + w.logits);
  QHIP(launch_ce_count(targets, T, V, ignore_index, nvalid, st));
  for (int64_t c0 = 0; c0 < T; c0 += w.C) {
    const int64_t C = (T - c0) < w.C ? (T - c0) : w.C;
    // logits of the chunk: z = X_c W^T, fp32 [C, V]
    GemmArgs a = gemm_args();
    a.act0 = u16(X) + c0 * D;
    a.M = C;
    a.Nout = V;
    a.Kred0 = D;
    a.wb = u16(W);
    a.ldw = D;
    a.wrows = V;
    a.partial = z;
    a.out_f32 = 1;
    QHIP(traced_gemm_b(MODE_FWD, a, st));
    // loss terms; with dX wanted, each row of z becomes the bf16 row
    // (softmax - onehot) / n (row stride 2V bf16 elements)
    QHIP(launch_ce_rows(z, C, V, targets + c0, ignore_index, nvalid, want_dx ? 1 : 0, tl + c0, st));
    if (!want_dx) continue;
    // dX_c = g W, the vocabulary reduction split into fp32 partials; the head
    // [V, D] is read K-major (rows of the reduction) as it is stored
    GemmArgs g = gemm_args();
    g.act0 = reinterpret_cast<const uint16_t*>(z);
    g.lda = 2 * V;
    g.M = C;
    g.Nout = D;
    g.Kred0 = V;
    g.wb = u16(W);
    g.ldw = D;
    g.wrows = D;
    g.w_kmajor = 1;
    g.out0 = u16m(dX) + c0 * D;
    if (w.splits > 1) {
      g.partial = part;
      g.ktiles_per_split = w.kps;
    }
    QHIP(traced_gemm_b(MODE_FWD, g, st));
    if (w.splits > 1) QHIP(launch_splitk_finish(part, w.splits, C, D, u16m(dX) + c0 * D, st));
  }
  return hip_status(launch_ce_loss(tl, T, nvalid, loss, st));
}

int qlora_merge(const qlora_linear* L, int32_t out_dtype, void* out, void* stream) {
  QTRY(qv_merge(L, out_dtype, out));
  QTRY(check_device());
  return hip_status(launch_merge(to_dev(L->W0), L->W0.codebook, u16(L->A), u16(L->B), L->r, lora_s(*L),
                                 out_dtype == QLORA_DTYPE_F16 ? 1 : 0, u16m(out), static_cast<hipStream_t>(stream)));
}

int qlora_linear_fwd(const qlora_linear* L, const void* X, int64_t M, void* Y, float* XA_saved, void* ws,
                     size_t ws_bytes, void* stream) {
  QTRY(qv_linear_fwd(L, X, M, Y, XA_saved, ws, ws_bytes));
  if (M == 0) return QLORA_OK;
  QTRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t N = L->W0.N, K = L->W0.K;
  const qplan::LinearWs w = qplan::linear_ws(M, N, K, L->r);
  float* part = reinterpret_cast<float*>(bytes(ws));
  float* down_part = reinterpret_cast<float*>(bytes(ws) + w.fwd_part);

  if (qplan::use_skinny_fwd(M, L->r)) {
    // XA partials; the skinny GEMM sums them, writes XA and adds s XA B^T
    const int ds = qplan::plan_down_splits(M, K, L->r);
    const int dsu = qplan::down_splits_used(K, ds);
    const bool stream2 = qplan::use_skinny_fwd2(M, N, K, L->r);
    const qplan::SkinnyPlan sp = stream2 ? qplan::plan_skinny_fwd2(N, K) : qplan::plan_skinny_fwd(N, K);
    // the streaming form's activation re-layout comes from the same pass
    // over X when the rank allows (<= 16), else from its own launch
    uint16_t* xt = stream2 ? reinterpret_cast<uint16_t*>(bytes(ws) + w.fwd_part + w.fwd_down) : nullptr;
    const bool xt_fused = stream2 && L->r <= 16;
    QHIP(launch_lora_down(u16(X), M, K, u16(L->A), L->r, nullptr, 0, XA_saved, nullptr, ds, down_part, st, false,
                          false, xt_fused ? xt : nullptr, xt_fused ? qplan::skinny_mp(M) : 0));
    SkinnyArgs a;
    memset(&a, 0, sizeof(a));
    a.X = u16(X);
    a.M = M;
    a.N = N;
    a.K = K;
    a.w = to_dev(L->W0);
    a.codebook = L->W0.codebook;
    a.vpart = dsu > 1 ? down_part : XA_saved;
    a.vsplits = dsu;
    a.vout = dsu > 1 ? XA_saved : nullptr;
    a.Wl = static_cast<const uint16_t*>(L->B);
    a.wl_sc = L->r;
    a.wl_sj = 1;
    a.r = L->r;
    a.s = lora_s(*L);
    a.out = u16m(Y);
    a.part = sp.splits > 1 ? part : nullptr;
    a.kps = sp.kps;
    if (stream2) {
      a.Mp = qplan::skinny_mp(M);
      a.Xt = xt;
      if (!xt_fused) QHIP(launch_xtile(u16(X), M, K, a.Mp, xt, st));
    }
    QHIP(traced_skinny_fwd(a, sp, st));
    if (sp.splits > 1) QHIP(launch_splitk_finish(part, sp.splits, M, N, u16m(Y), st));
    return QLORA_OK;
  }
  // XA = X A^T (kept for the backward)
  QHIP(launch_lora_down(u16(X), M, K, u16(L->A), L->r, nullptr, 0, XA_saved, nullptr,
                        qplan::plan_down_splits(M, K, L->r), down_part, st));
  // Y = X W0^T + s XA B^T
  const qplan::GemmPlan pl = qplan::plan_gemm(M, N, K, true);
  GemmArgs a = gemm_args();
  a.act0 = u16(X);
  a.M = M;
  a.Nout = N;
  a.Kred0 = K;
  a.w0 = to_dev(L->W0);
  a.codebook = L->W0.codebook;
  a.l0 = side_B(*L, XA_saved);
  a.out0 = u16m(Y);
  a.partial = part;
  if (qplan::use_bgemm(M)) {
    uint16_t* wbuf = reinterpret_cast<uint16_t*>(bytes(ws) + w.fwd_part + w.fwd_down);
    QHIP(launch_dequant_rows(a.w0, nullptr, a.codebook, nullptr, N, wbuf, st));
    a.wb = wbuf;
    a.ldw = K;
    a.wrows = N;
    return hip_status(traced_gemm_b(MODE_FWD, a, st));
  }
  QHIP(traced_gemm_q(MODE_FWD, a, pl, st));
  if (pl.splits > 1) QHIP(launch_splitk_finish(part, pl.splits, M, N, u16m(Y), st));
  return QLORA_OK;
}

int qlora_linear_fwd_static(const qlora_linear* L, const void* X, int64_t M, void* Y, float* XA_saved, void* stream) {
  QTRY(qv_linear_fwd_static(L, X, M, Y, XA_saved, kStaticScratchBytes));
  if (M == 0) return QLORA_OK;
  QTRY(check_device());
  void* ws = nullptr;
  QTRY(static_scratch(&ws));
  return qlora_linear_fwd(L, X, M, Y, XA_saved, ws, kStaticScratchBytes, stream);
}

int qlora_linear_bwd(const qlora_linear* L, const void* dY, const void* X, const float* XA_saved, int64_t M, void* dX,
                     void* dA, void* dB, void* ws, size_t ws_bytes, void* stream) {
  return linear_bwd_impl(L, dY, X, XA_saved, M, dX, dA, dB, nullptr, nullptr, ws, ws_bytes, stream);
}

// grp: the layer is packed LoRA groups (B block-diagonal); when the dB
// reduction can run per group (grouped_grad_ok), each group's dB is written
// straight from dY and its own ranks of XA, dB is left alone and *grp_done
// set; otherwise dB receives the [N, r] block-diagonal gradient.
static int linear_bwd_impl(const qlora_linear* L, const void* dY, const void* X, const float* XA_saved, int64_t M,
                           void* dX, void* dA, void* dB, const GroupDesc* grp, bool* grp_done, void* ws,
                           size_t ws_bytes, void* stream) {
  QTRY(qv_linear_bwd(L, dY, X, XA_saved, M, dX, dA, dB, ws, ws_bytes));
  QTRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t N = L->W0.N, K = L->W0.K;
  const int r = L->r;
  const float s = lora_s(*L);
  if (M == 0) {
    QHIP(launch_lora_grad(0, nullptr, nullptr, 0, N, nullptr, r, s, 1, nullptr, 0, u16m(dB), st));
    QHIP(launch_lora_grad(0, nullptr, nullptr, 0, K, nullptr, r, s, 1, nullptr, 1, u16m(dA), st));
    return QLORA_OK;
  }
  const qplan::LinearWs w = qplan::linear_ws(M, N, K, r);
  char* base = bytes(ws);
  float* T = reinterpret_cast<float*>(base);
  uint16_t* BT = reinterpret_cast<uint16_t*>(base + w.bwd_T);
  uint16_t* AT = reinterpret_cast<uint16_t*>(base + w.bwd_T + qplan::align256((size_t)N * r * 2));
  char* after_bt = base + w.bwd_T + w.bwd_BT;
  float* part = reinterpret_cast<float*>(after_bt);
  float* down_part = reinterpret_cast<float*>(after_bt + w.bwd_part);
  float* grad_part = reinterpret_cast<float*>(after_bt + w.bwd_part + w.bwd_down);

  const qplan::GemmPlan pl = qplan::plan_gemm(M, K, N, true, true);
  const bool sk_bwd = skinny_bwd_supported(M, N, K);
  if (!qplan::use_bgemm(M) && pl.cfg == qplan::CFG_SKINNY_TR && skinny_finish_supported(M, r) &&
      (sk_bwd || pl.splits > 1)) {
    // Skinny M: T partials, the split transposed product without its LoRA
    // term (the skinny kernel when the shape allows, else the dequant-staged
    // GEMM), then one finish launch for dX (+ s T A), dA and dB.
    // T = dY B: B read as stored when the rank allows (<= 16), else B^T first
    const int ds = qplan::plan_down_splits(M, N, r);
    const int dsu = qplan::down_splits_used(N, ds);
    if (r <= 16) {
      QHIP(launch_lora_down(u16(dY), M, N, u16(L->B), r, nullptr, 0, T, nullptr, ds, down_part, st, false, true));
    } else {
      QHIP(launch_transpose_rn(u16(L->B), N, r, BT, st));
      QHIP(launch_lora_down(u16(dY), M, N, BT, r, nullptr, 0, T, nullptr, ds, down_part, st, false));
    }
    if (sk_bwd) {
      SkinnyBwdArgs b;
      memset(&b, 0, sizeof(b));
      b.dY = u16(dY);
      b.M = M;
      b.N = N;
      b.K = K;
      b.w = to_dev(L->W0);
      b.codebook = L->W0.codebook;
      b.part = part;
      b.kps = pl.ktiles_per_split;
      QHIP(traced_skinny_bwd(b, pl.splits, st));
    } else {
      GemmArgs a = gemm_args();
      a.act0 = u16(dY);
      a.M = M;
      a.Nout = K;
      a.Kred0 = N;
      a.w0 = to_dev(L->W0);
      a.codebook = L->W0.codebook;
      a.partial = part;
      QHIP(traced_gemm_q(MODE_BWD, a, pl, st));
    }
    SkinnyFinishArgs f;
    memset(&f, 0, sizeof(f));
    f.M = M;
    f.N = N;
    f.K = K;
    f.r = r;
    f.s = s;
    f.part = part;
    f.splits = pl.splits;
    f.tpart = dsu > 1 ? down_part : T;
    f.tsplits = dsu;
    f.XA = XA_saved;
    f.X = u16(X);
    f.dY = u16(dY);
    f.A = u16(L->A);
    f.dX = u16m(dX);
    f.dA = u16m(dA);
    f.dB = u16m(dB);
    return hip_status(launch_skinny_bwd_finish(f, st));
  }
  // T = dY B  (B^T first, so that the product reads rows)
  {
    TransposeBatch tb;
    tb.add(u16(L->B), N, r, BT);  // B [N, r] -> B^T [r, N]
    tb.add(u16(L->A), r, K, AT);  // A [r, K] -> A^T [K, r]
    QHIP(launch_transpose_multi(tb.J, st));
  }
  const bool pair = r <= 16;
  if (pair) {
    // T = dY B and dB = s dY^T XA from one pass over dY
    PairArgs pa{};
    plan_lora_pair(pa, M, N, r);
    pa.njobs = 1;
    pa.job[0] = PairJob{u16(dY), BT, XA_saved, r, s, grad_part, grad_part + (size_t)pa.nb * M * r, T, u16m(dB)};
    QHIP(launch_lora_pair(pa, st));
  } else {
    QHIP(launch_lora_down(u16(dY), M, N, BT, r, nullptr, 0, T, nullptr, qplan::plan_down_splits(M, N, r), down_part,
                          st));
  }
  // dX = dY W0 + s T A
  GemmArgs a = gemm_args();
  a.act0 = u16(dY);
  a.M = M;
  a.Nout = K;
  a.Kred0 = N;
  a.w0 = to_dev(L->W0);
  a.codebook = L->W0.codebook;
  a.l0 = side_AT(*L, T, AT);
  a.out0 = u16m(dX);
  a.partial = part;
  if (qplan::use_bgemm(M)) {
    // W0^T expanded to bf16 [K, N]: the reduction over N becomes row-contiguous
    uint16_t* wbuf = reinterpret_cast<uint16_t*>(after_bt + w.bwd_part + w.bwd_down + w.bwd_grad);
    QHIP(launch_dequant_trans(a.w0, a.codebook, wbuf, N, 0, st));
    a.wb = wbuf;
    a.ldw = N;
    a.wrows = K;
    QHIP(traced_gemm_b(MODE_BWD, a, st));
  } else {
    QHIP(traced_gemm_q(MODE_BWD, a, pl, st));
    if (pl.splits > 1) QHIP(launch_splitk_finish(part, pl.splits, M, K, u16m(dX), st));
  }
  // dB = s dY^T XA  ([N, r], unless done above);  dA = s T^T X  ([r, K])
  const int64_t grp_cap = (int64_t)(w.bwd_grad / ((size_t)N * 64));  // [S][N][16] fp32 partials that fit
  if (!pair && grp && grp_cap >= 1 && grouped_grad_ok(*grp, N)) {
    int ms = qplan::plan_grad_msplits(M, N, 16);
    if (ms > grp_cap) ms = (int)grp_cap;
    QHIP(launch_grouped_grad(*grp, u16(dY), M, N, XA_saved, r, ms, grad_part, st));
    *grp_done = true;
  } else if (!pair) {
    QHIP(launch_lora_grad(0, u16(dY), nullptr, M, N, XA_saved, r, s, qplan::plan_grad_msplits(M, N, r), grad_part,
                          0, u16m(dB), st));
  }
  QHIP(launch_lora_grad(0, u16(X), nullptr, M, K, T, r, s, qplan::plan_grad_msplits(M, K, r), grad_part, 1, u16m(dA),
                        st));
  return QLORA_OK;
}

// The RMSNorm in front of the block folded into its first GEMM: the norm
// weight multiplies the expanded gate/up weights' columns, the inverse RMS of
// each token row scales that GEMM's product (its LoRA term included, which
// therefore uses the unscaled X (A w)^T).
struct RmsFold {
  const uint16_t* w;   // norm weight [D]
  const float* rstd;   // [M]
  const float* xa_g;   // X (A_g w)^T, fp32 [M, r_g]
  const float* xa_u;   // X (A_u w)^T
};

// The MLP forward on validated arguments (X the block's input; with rf, the
// pre-norm input and XA_g / XA_u already written by the caller).
static int mlp_fwd_impl(const qlora_mlp* P, const void* X, int64_t M, void* Y, const qlora_mlp_saved* S, void* ws,
                        hipStream_t st, const RmsFold* rf) {
  const int64_t I = P->gate.W0.N, D = P->gate.W0.K;
  const qplan::MlpWs w = qplan::mlp_ws(M, D, I, P->gate.r, P->up.r, P->down.r);
  uint16_t* H = reinterpret_cast<uint16_t*>(bytes(ws));
  float* down_part = reinterpret_cast<float*>(bytes(ws) + w.fwd_H);
  float* had_part = w.fwd_had ? reinterpret_cast<float*>(bytes(ws) + w.fwd_H + w.fwd_down) : nullptr;
  uint16_t* ext_act =
      w.fwd_ext ? reinterpret_cast<uint16_t*>(bytes(ws) + w.fwd_H + w.fwd_down + w.fwd_had) : nullptr;
  uint16_t* wbuf = w.fwd_wbuf
                       ? reinterpret_cast<uint16_t*>(bytes(ws) + w.fwd_H + w.fwd_down + w.fwd_had + w.fwd_ext)
                       : nullptr;

  // XA_g | XA_u in one pass over X (the down-projection kernels take a
  // combined rank of at most 128; above that, one pass per layer)
  if (rf) {
    // done by the caller
  } else if (P->gate.r + P->up.r <= 128) {
    QHIP(launch_lora_down(u16(X), M, D, u16(P->gate.A), P->gate.r, u16(P->up.A), P->up.r, S->XA_g, S->XA_u,
                          qplan::plan_down_splits(M, D, P->gate.r + P->up.r), down_part, st));
  } else {
    QHIP(launch_lora_down(u16(X), M, D, u16(P->gate.A), P->gate.r, nullptr, 0, S->XA_g, nullptr,
                          qplan::plan_down_splits(M, D, P->gate.r), down_part, st));
    QHIP(launch_lora_down(u16(X), M, D, u16(P->up.A), P->up.r, nullptr, 0, S->XA_u, nullptr,
                          qplan::plan_down_splits(M, D, P->up.r), down_part, st));
  }
  // G, U = gate/up(X) and H = silu(G) * U in one dual GEMM
  {
    GemmArgs a = gemm_args();
    a.act0 = u16(X);
    a.M = M;
    a.Nout = I;
    a.Kred0 = D;
    a.w0 = to_dev(P->gate.W0);
    a.w1 = to_dev(P->up.W0);
    a.codebook = P->gate.W0.codebook;
    a.codebook1 = P->up.W0.codebook;
    a.l0 = side_B(P->gate, rf ? rf->xa_g : S->XA_g);
    a.l1 = side_B(P->up, rf ? rf->xa_u : S->XA_u);
    if (rf) a.row_scale = rf->rstd;
    a.out0 = u16m(S->G);
    a.out1 = u16m(S->U);
    a.out2 = H;
    if (wbuf) {
      // the LoRA terms as extra reduction columns: [s_g XA_g | s_u XA_u]
      // against [B_g | 0] (gate rows) and [0 | B_u] (up rows)
      const int rg = P->gate.r, ru = P->up.r;
      const int64_t ext = qplan::lora_ext_cols(rg, ru);
      QHIP(launch_dequant_rows(a.w0, &a.w1, a.codebook, a.codebook1, qplan::pair_rows(I), wbuf, st,
                               rf ? rf->w : nullptr, D + ext));
      QHIP(launch_lora_ext_cols(u16(P->gate.B), rg, u16(P->up.B), ru, I, qplan::pair_rows(I), D, D + ext, ext, wbuf,
                                st));
      QHIP(launch_lora_ext_act(a.l0.V, rg, a.l0.s, a.l1.V, ru, a.l1.s, M, ext, ext_act, st));
      a.act1 = ext_act;
      a.lda1 = ext;
      a.Kred1 = ext;
      a.wb = wbuf;
      a.ldw = D + ext;
      a.wrows = qplan::pair_rows(I);
      if (had_part) {  // HA_d from the GEMM's own H, as column-tile partials
        a.had_A = u16(P->down.A);
        a.had_r = P->down.r;
        a.had_part = had_part;
      }
      QHIP(traced_gemm_b(MODE_FWD_SWIGLU, a, st));
    } else {
      QHIP(traced_gemm_q(MODE_FWD_SWIGLU, a, qplan::plan_gemm(M, I, D, false), st));
    }
  }
  // HA_d = H A_d^T
  if (had_part)
    QHIP(launch_had_finish(had_part, (int)qplan::cdiv(I, 128), M, P->down.r, S->HA_d, st));
  else
    QHIP(launch_lora_down(H, M, I, u16(P->down.A), P->down.r, nullptr, 0, S->HA_d, nullptr,
                          qplan::plan_down_splits(M, I, P->down.r), down_part, st));
  // Y = H W_d^T + s_d HA_d B_d^T
  {
    GemmArgs a = gemm_args();
    a.act0 = H;
    a.M = M;
    a.Nout = D;
    a.Kred0 = I;
    a.w0 = to_dev(P->down.W0);
    a.codebook = P->down.W0.codebook;
    a.l0 = side_B(P->down, S->HA_d);
    a.out0 = u16m(Y);
    if (wbuf) {
      QHIP(launch_dequant_rows(a.w0, nullptr, a.codebook, nullptr, D, wbuf, st));
      a.wb = wbuf;
      a.ldw = I;
      a.wrows = D;
      QHIP(traced_gemm_b(MODE_FWD, a, st));
    } else {
      QHIP(traced_gemm_q(MODE_FWD, a, qplan::plan_gemm(M, D, I, false), st));
    }
  }
  return QLORA_OK;
}

int qlora_mlp_fwd(const qlora_mlp* P, const void* X, int64_t M, void* Y, const qlora_mlp_saved* S, void* ws,
                  size_t ws_bytes, void* stream) {
  QTRY(qv_mlp_fwd(P, X, M, Y, S, ws, ws_bytes));
  if (M == 0) return QLORA_OK;
  QTRY(check_device());
  return mlp_fwd_impl(P, X, M, Y, S, ws, static_cast<hipStream_t>(stream), nullptr);
}

int qlora_mlp_fwd_rmsnorm(const qlora_mlp* P, const void* X, const void* norm_w, float eps, int64_t M, void* Y,
                          const qlora_mlp_saved* S, float* rstd, void* Xn, void* ws, size_t ws_bytes, void* stream) {
  QTRY(qv_mlp_fwd_rmsnorm(P, X, norm_w, eps, M, Y, S, rstd, Xn, ws, ws_bytes));
  if (M == 0) return QLORA_OK;
  QTRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t I = P->gate.W0.N, D = P->gate.W0.K;
  const int rg = P->gate.r, ru = P->up.r;
  const qplan::MlpRmsWs w = qplan::mlp_rms_ws(M, D, I, rg, ru, P->down.r);
  char* extra = bytes(ws) + w.base;
  if (!qplan::use_bgemm(M)) {
    // below the bf16-GEMM threshold the GEMM expands NF4 in its own tiles:
    // the norm runs as its own pass into Xn (or the workspace)
    uint16_t* xn = Xn ? u16m(Xn) : reinterpret_cast<uint16_t*>(extra + w.at_g + w.at_u + w.xa);
    QHIP(launch_rmsnorm_fwd(u16(X), u16(norm_w), M, D, eps, xn, rstd, st));
    return mlp_fwd_impl(P, xn, M, Y, S, ws, st, nullptr);
  }
  uint16_t* ag = reinterpret_cast<uint16_t*>(extra);
  uint16_t* au = reinterpret_cast<uint16_t*>(extra + w.at_g);
  float* xag = reinterpret_cast<float*>(extra + w.at_g + w.at_u);
  float* xau = xag + (size_t)M * rg;
  float* down_part = reinterpret_cast<float*>(bytes(ws) + qplan::mlp_ws(M, D, I, rg, ru, P->down.r).fwd_H);
  // rstd (and Xn when the caller keeps it for the backward)
  QHIP(launch_rmsnorm_fwd(u16(X), u16(norm_w), M, D, eps, Xn ? u16m(Xn) : nullptr, rstd, st));
  // X (A w)^T, then XA = rstd * X (A w)^T for the backward
  QHIP(launch_scale_cols(u16(P->gate.A), rg, D, u16(norm_w), ag, st));
  QHIP(launch_scale_cols(u16(P->up.A), ru, D, u16(norm_w), au, st));
  if (rg + ru <= 128) {
    QHIP(launch_lora_down(u16(X), M, D, ag, rg, au, ru, xag, xau, qplan::plan_down_splits(M, D, rg + ru), down_part,
                          st));
  } else {
    QHIP(launch_lora_down(u16(X), M, D, ag, rg, nullptr, 0, xag, nullptr, qplan::plan_down_splits(M, D, rg), down_part,
                          st));
    QHIP(launch_lora_down(u16(X), M, D, au, ru, nullptr, 0, xau, nullptr, qplan::plan_down_splits(M, D, ru), down_part,
                          st));
  }
  QHIP(launch_scale_rows(xag, M, rg, rstd, S->XA_g, st));
  QHIP(launch_scale_rows(xau, M, ru, rstd, S->XA_u, st));
  const RmsFold rf{u16(norm_w), rstd, xag, xau};
  return mlp_fwd_impl(P, X, M, Y, S, ws, st, &rf);
}

int qlora_mlp_bwd(const qlora_mlp* P, const void* dY, const void* X, const qlora_mlp_saved* S, int64_t M, void* dX,
                  const qlora_mlp_grads* G, void* ws, size_t ws_bytes, void* stream) {
  QTRY(qv_mlp_bwd(P, dY, X, S, M, dX, G, ws, ws_bytes));
  QTRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t I = P->gate.W0.N, D = P->gate.W0.K;
  const int rg = P->gate.r, ru = P->up.r, rd = P->down.r;
  const float sg = lora_s(P->gate), su = lora_s(P->up), sd = lora_s(P->down);
  if (M == 0) {
    QHIP(launch_lora_grad(0, nullptr, nullptr, 0, D, nullptr, rd, sd, 1, nullptr, 0, u16m(G->dB_d), st));
    QHIP(launch_lora_grad(0, nullptr, nullptr, 0, I, nullptr, rd, sd, 1, nullptr, 1, u16m(G->dA_d), st));
    QHIP(launch_lora_grad(0, nullptr, nullptr, 0, I, nullptr, rg, sg, 1, nullptr, 0, u16m(G->dB_g), st));
    QHIP(launch_lora_grad(0, nullptr, nullptr, 0, D, nullptr, rg, sg, 1, nullptr, 1, u16m(G->dA_g), st));
    QHIP(launch_lora_grad(0, nullptr, nullptr, 0, I, nullptr, ru, su, 1, nullptr, 0, u16m(G->dB_u), st));
    QHIP(launch_lora_grad(0, nullptr, nullptr, 0, D, nullptr, ru, su, 1, nullptr, 1, u16m(G->dA_u), st));
    return QLORA_OK;
  }
  const qplan::MlpWs w = qplan::mlp_ws(M, D, I, rg, ru, rd);
  char* b = bytes(ws);
  float* Td = reinterpret_cast<float*>(b);
  b += w.bwd_Td;
  uint16_t* dG = reinterpret_cast<uint16_t*>(b);
  b += w.bwd_dG;
  uint16_t* dU = reinterpret_cast<uint16_t*>(b);
  b += w.bwd_dU;
  float* Tg = reinterpret_cast<float*>(b);
  b += w.bwd_Tg;
  float* Tu = reinterpret_cast<float*>(b);
  b += w.bwd_Tu;
  uint16_t* BdT = reinterpret_cast<uint16_t*>(b);
  uint16_t* BgT = reinterpret_cast<uint16_t*>(b + qplan::align256((size_t)rd * D * 2));
  uint16_t* BuT = reinterpret_cast<uint16_t*>(b + qplan::align256((size_t)rd * D * 2) +
                                              qplan::align256((size_t)rg * I * 2));
  char* at0 = b + qplan::align256((size_t)rd * D * 2) + qplan::align256((size_t)rg * I * 2) +
              qplan::align256((size_t)ru * I * 2);
  uint16_t* AdT = reinterpret_cast<uint16_t*>(at0);                                        // [I, rd]
  uint16_t* AgT = reinterpret_cast<uint16_t*>(at0 + qplan::align256((size_t)I * rd * 2));  // [D, rg]
  uint16_t* AuT = reinterpret_cast<uint16_t*>(at0 + qplan::align256((size_t)I * rd * 2) +
                                              qplan::align256((size_t)D * rg * 2));       // [D, ru]
  b += w.bwd_BT;
  float* down_part = reinterpret_cast<float*>(b);
  b += w.bwd_down;
  float* grad_part = reinterpret_cast<float*>(b);
  b += w.bwd_grad;
  float* pair_part = reinterpret_cast<float*>(b);
  b += w.bwd_pair;
  uint16_t* tdt = reinterpret_cast<uint16_t*>(b);
  b += w.bwd_tdt;
  uint16_t* wbuf = w.bwd_wbuf ? reinterpret_cast<uint16_t*>(b) : nullptr;
  const bool pair = qplan::use_lora_pair(rg, ru, rd);
  // T_d^T in bf16 for the dH epilogue's dA_d (bf16-GEMM path): from the
  // single-pass T + dB finish when it runs, else its own pass
  const bool tt_in_pair = pair && wbuf && qplan::fuse_dad(rd);
  const int64_t tt_ld = 8 * qplan::cdiv(M, 8);

  // Td = dY B_d
  {
    TransposeBatch tb;
    tb.add(u16(P->down.B), D, rd, BdT);
    tb.add(u16(P->gate.B), I, rg, BgT);
    tb.add(u16(P->up.B), I, ru, BuT);
    tb.add(u16(P->down.A), rd, I, AdT);
    tb.add(u16(P->gate.A), rg, D, AgT);
    tb.add(u16(P->up.A), ru, D, AuT);
    QHIP(launch_transpose_multi(tb.J, st));
  }
  if (pair) {
    // Td = dY B_d and dB_d = s_d dY^T HA_d from one pass over dY
    PairArgs pa{};
    plan_lora_pair(pa, M, D, rd);
    pa.njobs = 1;
    pa.job[0] = PairJob{u16(dY), BdT, S->HA_d, rd, sd, pair_part, pair_part + (size_t)pa.nb * M * rd, Td,
                        u16m(G->dB_d)};
    if (tt_in_pair) {  // its finish also writes T_d^T in bf16 for the dH epilogue
      pa.job[0].Tt = tdt;
      pa.job[0].tt_ld = tt_ld;
    }
    QHIP(launch_lora_pair(pa, st));
  } else {
    QHIP(launch_lora_down(u16(dY), M, D, BdT, rd, nullptr, 0, Td, nullptr, qplan::plan_down_splits(M, D, rd),
                          down_part, st));
  }
  // dH = dY W_d + s_d Td A_d, with the SwiGLU backward in the epilogue -> dG, dU
  {
    GemmArgs a = gemm_args();
    a.act0 = u16(dY);
    a.M = M;
    a.Nout = I;
    a.Kred0 = D;
    a.w0 = to_dev(P->down.W0);
    a.codebook = P->down.W0.codebook;
    a.l0 = side_AT(P->down, Td, AdT);
    a.in0 = u16(S->G);
    a.in1 = u16(S->U);
    a.out0 = dG;
    a.out1 = dU;
    if (wbuf) {
      // W_d^T as bf16 [I, D]
      QHIP(launch_dequant_trans(a.w0, a.codebook, wbuf, D, 0, st));
      a.wb = wbuf;
      a.ldw = D;
      a.wrows = I;
      // dA_d = s_d Td^T H from the epilogue's own G, U (per-token-tile
      // partials), with Td^T in bf16 so that a lane's operand is one load
      if (qplan::fuse_dad(rd)) {
        if (!tt_in_pair) QHIP(launch_t_bf16_trans(Td, M, rd, tt_ld, tdt, st));
        a.dad_part = grad_part;
        a.dad_tt = tdt;
        a.dad_tt_ld = tt_ld;
      }
      QHIP(traced_gemm_b(MODE_BWD_SWIGLU, a, st));
      if (qplan::fuse_dad(rd))
        QHIP(launch_grad_finish(grad_part, (int)qplan::cdiv(M, 256), I, rd, sd, 1, u16m(G->dA_d), st));
    } else {
      QHIP(traced_gemm_q(MODE_BWD_SWIGLU, a, qplan::plan_gemm(M, I, D, false), st));
    }
  }
  // down-layer LoRA gradients: dB_d = s_d dY^T HA_d, dA_d = s_d Td^T H (H
  // recomputed from G, U when the dH GEMM did not)
  if (!pair)
    QHIP(launch_lora_grad(0, u16(dY), nullptr, M, D, S->HA_d, rd, sd, qplan::plan_grad_msplits(M, D, rd), grad_part,
                          0, u16m(G->dB_d), st));
  if (!(wbuf && qplan::fuse_dad(rd)))
    QHIP(launch_lora_grad(1, u16(S->G), u16(S->U), M, I, Td, rd, sd, qplan::plan_grad_msplits(M, I, rd), grad_part,
                          1, u16m(G->dA_d), st));
  if (pair) {
    // Tg = dG B_g, dB_g = s_g dG^T XA_g, Tu = dU B_u, dB_u = s_u dU^T XA_u:
    // one pass over dG and one over dU, in one launch
    PairArgs pa{};
    plan_lora_pair(pa, M, I, rg > ru ? rg : ru, 2);
    pa.njobs = 2;
    float* pg = pair_part;
    float* pu = pg + qplan::pair_part_floats(M, I, rg);
    pa.job[0] = PairJob{dG, BgT, S->XA_g, rg, sg, pg, pg + (size_t)pa.nb * M * rg, Tg, u16m(G->dB_g)};
    pa.job[1] = PairJob{dU, BuT, S->XA_u, ru, su, pu, pu + (size_t)pa.nb * M * ru, Tu, u16m(G->dB_u)};
    QHIP(launch_lora_pair(pa, st));
  } else {
    // Tg = dG B_g, Tu = dU B_u
    QHIP(launch_lora_down(dG, M, I, BgT, rg, nullptr, 0, Tg, nullptr, qplan::plan_down_splits(M, I, rg), down_part,
                          st));
    QHIP(launch_lora_down(dU, M, I, BuT, ru, nullptr, 0, Tu, nullptr, qplan::plan_down_splits(M, I, ru), down_part,
                          st));
  }
  // dX = dG W_g + dU W_u + s_g Tg A_g + s_u Tu A_u  (one GEMM, reduction over 2I)
  {
    GemmArgs a = gemm_args();
    a.act0 = dG;
    a.act1 = dU;
    a.M = M;
    a.Nout = D;
    a.Kred0 = I;
    a.Kred1 = I;
    a.w0 = to_dev(P->gate.W0);
    a.w1 = to_dev(P->up.W0);
    a.codebook = P->gate.W0.codebook;
    a.codebook1 = P->up.W0.codebook;
    a.l0 = side_AT(P->gate, Tg, AgT);
    a.l1 = side_AT(P->up, Tu, AuT);
    a.out0 = u16m(dX);
    if (wbuf) {
      // [W_g^T | W_u^T] as bf16 [D, 2I]
      QHIP(launch_dequant_trans(a.w0, a.codebook, wbuf, 2 * I, 0, st));
      QHIP(launch_dequant_trans(a.w1, a.codebook1, wbuf, 2 * I, I, st));
      a.wb = wbuf;
      a.ldw = 2 * I;
      a.wrows = D;
      QHIP(traced_gemm_b(MODE_BWD_DUAL, a, st));
    } else {
      QHIP(traced_gemm_q(MODE_BWD_DUAL, a, qplan::plan_gemm(M, D, 2 * I, false), st));
    }
  }
  // gate / up LoRA gradients (dB_g, dB_u already done by the single pass)
  if (pair) {
    // dA_g = s_g Tg^T X and dA_u = s_u Tu^T X from one pass over X
    QHIP(launch_lora_grad2(u16(X), M, D, Tg, rg, sg, u16m(G->dA_g), Tu, ru, su, u16m(G->dA_u), grad_part, st));
    return QLORA_OK;
  }
  QHIP(launch_lora_grad(0, dG, nullptr, M, I, S->XA_g, rg, sg, qplan::plan_grad_msplits(M, I, rg), grad_part, 0,
                        u16m(G->dB_g), st));
  QHIP(launch_lora_grad(0, u16(X), nullptr, M, D, Tg, rg, sg, qplan::plan_grad_msplits(M, D, rg), grad_part, 1,
                        u16m(G->dA_g), st));
  QHIP(launch_lora_grad(0, dU, nullptr, M, I, S->XA_u, ru, su, qplan::plan_grad_msplits(M, I, ru), grad_part, 0,
                        u16m(G->dB_u), st));
  QHIP(launch_lora_grad(0, u16(X), nullptr, M, D, Tu, ru, su, qplan::plan_grad_msplits(M, D, ru), grad_part, 1,
                        u16m(G->dA_u), st));
  return QLORA_OK;
}

}  // extern "C"
