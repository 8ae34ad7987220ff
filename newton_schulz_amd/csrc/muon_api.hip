// libmuon C ABI: context, argument validation and the Newton-Schulz driver.
//
// The driver enqueues, per batched call: the deterministic norm reduction,
// then `steps` times Gram -> symmetric square -> update, all on the caller's
// stream, with no host synchronisation and no device allocation (blog "Muon
// Optimizer + FSDP", section "Memory control", item 2: one preallocated
// workspace, only views per micro-bucket).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "muon.h"
#include "muon_internal.h"
#include "ns_layout.h"

namespace {

constexpr int kTabSlots = 4;
constexpr int64_t kTabCap = 65536;  // pointers per table (per in/out) per slot

struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

}  // namespace

struct muon_ctx {
  int device = 0;
  int cus = 256;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  uint64_t* host_tab = nullptr;  // pinned staging, kTabSlots * 2 * kTabCap
  uint64_t* dev_tab = nullptr;   // device tables, same layout
  hipEvent_t tab_ev[kTabSlots] = {};
  bool tab_used[kTabSlots] = {};
  int tab_next = 0;
  // timing
  bool timing = false;
  uint32_t tmask = (1u << MUON_K_COUNT) - 1;  // classes that record events
  std::vector<hipEvent_t> tev;
  std::vector<int> tcls;
  size_t tused = 0;  // events recorded (pairs * 2)
  std::string err;
};

namespace {

muon_status_t fail(muon_ctx* c, muon_status_t s, const char* what) {
  if (c) c->err = what;
  return s;
}

muon_status_t hip_fail(muon_ctx* c, hipError_t e, const char* where) {
  if (c) {
    c->err = std::string(where) + ": " + hipGetErrorString(e);
  }
  return MUON_EHIP;
}

// Record the start event of a timed launch; returns the pair index or -1.
long tstart(muon_ctx* c, hipStream_t s, int cls) {
  if (!c->timing || !((c->tmask >> cls) & 1u) || c->tused + 2 > c->tev.size()) return -1;
  // launches recorded into a graph are not timed (the events would be
  // re-recorded by every replay)
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return -1;
  const long k = static_cast<long>(c->tused);
  if (hipEventRecord(c->tev[k], s) != hipSuccess) return -1;
  c->tcls[k / 2] = cls;
  return k;
}
void tstop(muon_ctx* c, hipStream_t s, long k) {
  if (k < 0) return;
  if (hipEventRecord(c->tev[k + 1], s) == hipSuccess) c->tused = static_cast<size_t>(k) + 2;
}

bool is_dtype(int32_t d) { return d == MUON_F32 || d == MUON_BF16; }
size_t esize(int32_t d) { return d == MUON_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return na && nb && x < y + nb && y < x + na;
}

// Does some out[j] (bytes long) overlap an in[k] other than in[j] == out[j]
// exactly?  Inputs sorted by address; each output checks the inputs starting
// less than `bytes` away.
bool cross_overlap(const void* const* in, const void* const* out, int64_t count, int64_t bytes) {
  std::vector<std::pair<uintptr_t, int64_t>> v(static_cast<size_t>(count));
  for (int64_t i = 0; i < count; ++i) v[i] = {reinterpret_cast<uintptr_t>(in[i]), i};
  std::sort(v.begin(), v.end());
  const uintptr_t b = static_cast<uintptr_t>(bytes);
  for (int64_t j = 0; j < count; ++j) {
    const uintptr_t o = reinterpret_cast<uintptr_t>(out[j]);
    const uintptr_t lo = o >= b ? o - b + 1 : 0;
    auto it = std::lower_bound(v.begin(), v.end(), std::make_pair(lo, int64_t{-1}));
    for (; it != v.end() && it->first < o + b; ++it)
      if (it->second != j || it->first != o) return true;
  }
  return false;
}

}  // namespace

extern "C" {

const char* muon_status_string(muon_status_t s) {
  switch (s) {
    case MUON_OK: return "ok";
    case MUON_EINVAL: return "invalid argument";
    case MUON_ESHAPE: return "invalid shape";
    case MUON_EDTYPE: return "unsupported dtype";
    case MUON_EWORKSPACE: return "workspace too small";
    case MUON_EHIP: return "HIP runtime error";
    case MUON_ENOMEM: return "out of host memory";
  }
  return "unknown status";
}

const char* muon_last_error(const muon_ctx_t* ctx) { return ctx ? ctx->err.c_str() : ""; }

void muon_ns_params_default(muon_ns_params_t* p) {
  if (!p) return;
  p->steps = 5;
  p->a = 3.4445f;
  p->b = -4.7750f;
  p->c = 2.0315f;
  p->eps = 1e-7f;
  p->compute = MUON_BF16;
  p->method = MUON_NS_QUINTIC;
  p->fuse = MUON_FUSE_AUTO;
  p->coeffs = nullptr;
  p->sq_partials = nullptr;
  p->sq_base = nullptr;
  p->sq_count = 0;
}

size_t muon_ctx_workspace_bytes(const muon_ctx_t* ctx) { return ctx ? ctx->ws_bytes : 0; }

muon_status_t muon_create(int device, size_t workspace_bytes, muon_ctx_t** out) {
  if (out == nullptr) return MUON_EINVAL;
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return MUON_EHIP;
  DeviceGuard g(device);
  if (!g.ok) return MUON_EHIP;
  muon_ctx* c = new (std::nothrow) muon_ctx;
  if (c == nullptr) return MUON_ENOMEM;
  c->device = device;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess &&
      cus > 0)
    c->cus = cus;
  const size_t tab_bytes = sizeof(uint64_t) * kTabSlots * 2 * kTabCap;
  bool ok = hipMalloc(reinterpret_cast<void**>(&c->ws), std::max<size_t>(workspace_bytes, 256)) ==
            hipSuccess;
  ok = ok && hipMalloc(reinterpret_cast<void**>(&c->dev_tab), tab_bytes) == hipSuccess;
  ok = ok && hipHostMalloc(reinterpret_cast<void**>(&c->host_tab), tab_bytes, 0) == hipSuccess;
  for (int i = 0; ok && i < kTabSlots; ++i)
    ok = hipEventCreateWithFlags(&c->tab_ev[i], hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    muon_destroy(c);
    return MUON_EHIP;
  }
  c->ws_bytes = workspace_bytes;
  *out = c;
  return MUON_OK;
}

muon_status_t muon_destroy(muon_ctx_t* c) {
  if (c == nullptr) return MUON_OK;
  DeviceGuard g(c->device);
  (void)hipDeviceSynchronize();
  for (auto& e : c->tev) (void)hipEventDestroy(e);
  for (int i = 0; i < kTabSlots; ++i)
    if (c->tab_ev[i]) (void)hipEventDestroy(c->tab_ev[i]);
  if (c->host_tab) (void)hipHostFree(c->host_tab);
  if (c->dev_tab) (void)hipFree(c->dev_tab);
  if (c->ws) (void)hipFree(c->ws);
  delete c;
  return MUON_OK;
}

muon_status_t muon_timing_enable(muon_ctx_t* c, int32_t enable, int32_t capacity) {
  if (c == nullptr || capacity < 0) return MUON_EINVAL;
  DeviceGuard g(c->device);
  c->timing = false;
  if (!enable) return MUON_OK;
  const size_t want = static_cast<size_t>(capacity > 0 ? capacity : 8192) * 2;
  try {
    while (c->tev.size() < want) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return hip_fail(c, hipGetLastError(), "hipEventCreate");
      c->tev.push_back(e);
    }
    c->tcls.assign(c->tev.size() / 2, 0);
  } catch (...) {
    return MUON_ENOMEM;
  }
  c->tused = 0;
  c->timing = true;
  return MUON_OK;
}

muon_status_t muon_timing_select(muon_ctx_t* c, uint32_t class_mask) {
  if (c == nullptr || (class_mask >> MUON_K_COUNT) != 0) return MUON_EINVAL;
  c->tmask = class_mask;
  return MUON_OK;
}

muon_status_t muon_timing_reset(muon_ctx_t* c) {
  if (c == nullptr) return MUON_EINVAL;
  c->tused = 0;
  return MUON_OK;
}

muon_status_t muon_timing_read(muon_ctx_t* c, int32_t cls, double* total_ms, int64_t* launches) {
  if (c == nullptr || total_ms == nullptr || launches == nullptr) return MUON_EINVAL;
  if (cls < 0 || cls >= MUON_K_COUNT) return MUON_EINVAL;
  DeviceGuard g(c->device);
  double tot = 0.0;
  int64_t n = 0;
  for (size_t k = 0; k + 1 < c->tused; k += 2) {
    if (c->tcls[k / 2] != cls) continue;
    hipError_t e = hipEventSynchronize(c->tev[k + 1]);
    if (e != hipSuccess) return hip_fail(c, e, "hipEventSynchronize");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, c->tev[k], c->tev[k + 1]);
    if (e != hipSuccess) return hip_fail(c, e, "hipEventElapsedTime");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return MUON_OK;
}

static muon_status_t momentum_impl(muon_ctx_t* c, void* stream, const void* grad, int32_t grad_dtype,
                            float* momentum, void* update_out, int32_t update_dtype,
                            int64_t numel, float beta, int32_t nesterov, double* sq) {
  if (c == nullptr) return MUON_EINVAL;
  if (numel < 0) return fail(c, MUON_EINVAL, "numel < 0");
  if (!is_dtype(grad_dtype) || !is_dtype(update_dtype)) return fail(c, MUON_EDTYPE, "dtype");
  if (numel == 0) return MUON_OK;
  if (!grad || !momentum || !update_out) return fail(c, MUON_EINVAL, "null pointer");
  if (!(beta >= 0.0f && beta <= 1.0f)) return fail(c, MUON_EINVAL, "beta outside [0, 1]");
  const size_t nb = static_cast<size_t>(numel);
  if (ranges_overlap(update_out, nb * esize(update_dtype), grad, nb * esize(grad_dtype)) ||
      ranges_overlap(update_out, nb * esize(update_dtype), momentum, nb * 4) ||
      ranges_overlap(grad, nb * esize(grad_dtype), momentum, nb * 4))
    return fail(c, MUON_EINVAL, "aliasing buffers");
  if ((reinterpret_cast<uintptr_t>(grad) % esize(grad_dtype)) ||
      (reinterpret_cast<uintptr_t>(momentum) % 4) ||
      (reinterpret_cast<uintptr_t>(update_out) % esize(update_dtype)))
    return fail(c, MUON_EINVAL, "misaligned pointer");
  if (sq != nullptr) {
    const size_t qb = static_cast<size_t>((numel + MUON_SQ_BLOCK - 1) / MUON_SQ_BLOCK) * 8;
    if (reinterpret_cast<uintptr_t>(sq) % 8) return fail(c, MUON_EINVAL, "misaligned sq_partials");
    if (ranges_overlap(sq, qb, grad, nb * esize(grad_dtype)) || ranges_overlap(sq, qb, momentum, nb * 4) ||
        ranges_overlap(sq, qb, update_out, nb * esize(update_dtype)))
      return fail(c, MUON_EINVAL, "sq_partials overlaps a buffer");
  }
  DeviceGuard g(c->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float c1 = 1.0f - beta;
  const long tk = tstart(c, s, MUON_K_MOMENTUM);
  const hipError_t e = launch_momentum(s, c->cus, grad, grad_dtype, momentum, update_out,
                                       update_dtype, numel, beta, c1, nesterov ? 1 : 0, sq);
  tstop(c, s, tk);
  if (e != hipSuccess) return hip_fail(c, e, "momentum launch");
  return MUON_OK;
}

muon_status_t muon_momentum_update(muon_ctx_t* c, void* stream, const void* grad,
                                   int32_t grad_dtype, float* momentum, void* update_out,
                                   int32_t update_dtype, int64_t numel, float beta,
                                   int32_t nesterov) {
  return momentum_impl(c, stream, grad, grad_dtype, momentum, update_out, update_dtype, numel,
                       beta, nesterov, nullptr);
}

muon_status_t muon_momentum_update_sq(muon_ctx_t* c, void* stream, const void* grad,
                                      int32_t grad_dtype, float* momentum, void* update_out,
                                      int32_t update_dtype, int64_t numel, float beta,
                                      int32_t nesterov, double* sq_partials) {
  if (c == nullptr) return MUON_EINVAL;
  if (sq_partials == nullptr) return fail(c, MUON_EINVAL, "sq_partials NULL");
  return momentum_impl(c, stream, grad, grad_dtype, momentum, update_out, update_dtype, numel,
                       beta, nesterov, sq_partials);
}

muon_status_t muon_apply(muon_ctx_t* c, void* stream, float* master, const void* update,
                         int32_t update_dtype, void* weight_bf16, int64_t numel, float lr,
                         float scale, float weight_decay) {
  if (c == nullptr) return MUON_EINVAL;
  if (numel < 0) return fail(c, MUON_EINVAL, "numel < 0");
  if (!is_dtype(update_dtype)) return fail(c, MUON_EDTYPE, "dtype");
  if (numel == 0) return MUON_OK;
  if (!master || !update) return fail(c, MUON_EINVAL, "null pointer");
  const size_t nb = static_cast<size_t>(numel);
  if (ranges_overlap(master, nb * 4, update, nb * esize(update_dtype)) ||
      (weight_bf16 && (ranges_overlap(weight_bf16, nb * 2, master, nb * 4) ||
                       ranges_overlap(weight_bf16, nb * 2, update, nb * esize(update_dtype)))))
    return fail(c, MUON_EINVAL, "aliasing buffers");
  if ((reinterpret_cast<uintptr_t>(master) % 4) ||
      (reinterpret_cast<uintptr_t>(update) % esize(update_dtype)) ||
      (weight_bf16 && (reinterpret_cast<uintptr_t>(weight_bf16) % 2)))
    return fail(c, MUON_EINVAL, "misaligned pointer");
  DeviceGuard g(c->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float eta = lr * scale;
  const float decay = 1.0f - lr * weight_decay;
  const long tk = tstart(c, s, MUON_K_APPLY);
  const hipError_t e = launch_apply(s, c->cus, master, update, update_dtype, weight_bf16, numel,
                                    eta, decay, weight_decay != 0.0f ? 1 : 0);
  tstop(c, s, tk);
  if (e != hipSuccess) return hip_fail(c, e, "apply launch");
  return MUON_OK;
}

}  // extern "C"

namespace {

// Describe `count` matrices (each `per` units of unit_bytes) as a unit-level
// MatRef: uniform stride when possible, else a device table staged through
// the pinned ring.  `tab` receives the host-side slot to fill.
struct UnitsRef {
  MatRef ref{nullptr, 0, nullptr};
  bool needs_table = false;
};

UnitsRef describe(const void* const* p, int64_t count, int64_t per, int64_t unit_bytes) {
  UnitsRef r;
  const char* b0 = static_cast<const char*>(p[0]);
  if (count == 1) {
    r.ref = MatRef{b0, unit_bytes, nullptr};
    return r;
  }
  const int64_t d = static_cast<const char*>(p[1]) - b0;
  bool uniform = (per == 1) || (d == per * unit_bytes);
  for (int64_t i = 2; uniform && i < count; ++i)
    uniform = (static_cast<const char*>(p[i]) - b0) == i * d;
  if (uniform) {
    r.ref = MatRef{b0, per == 1 ? d : unit_bytes, nullptr};
  } else {
    r.needs_table = true;
  }
  return r;
}

void fill_table(uint64_t* dst, const void* const* p, int64_t count, int64_t per,
                int64_t unit_bytes) {
  for (int64_t i = 0; i < count; ++i)
    for (int64_t k = 0; k < per; ++k)
      dst[i * per + k] = reinterpret_cast<uint64_t>(static_cast<const char*>(p[i]) + k * unit_bytes);
}

}  // namespace

namespace {

muon_status_t efail(const NsEnv& env, muon_status_t st, const char* what) {
  if (env.ctx) env.ctx->err = what;
  if (env.err) *env.err = what;
  return st;
}
muon_status_t ehip(const NsEnv& env, hipError_t e, const char* where) {
  if (env.ctx) return hip_fail(env.ctx, e, where);
  if (env.err) *env.err = where;
  return MUON_EHIP;
}
long etstart(const NsEnv& env, hipStream_t s, int cls) { return env.ctx ? tstart(env.ctx, s, cls) : -1; }
void etstop(const NsEnv& env, hipStream_t s, long k) {
  if (env.ctx) tstop(env.ctx, s, k);
}

}  // namespace

// The Newton-Schulz driver behind both batched entry points.  env.ctx is the
// context (workspace slab, pointer-table ring, timing events, error text), or
// null for the allocation-free entry point, which brings its own workspace,
// takes uniformly placed matrices only (no pointer tables) and records its
// error text as a static string.
muon_status_t ns_batched(const NsEnv& env, void* stream, const void* const* mats, int64_t count,
                         muon_shape_t shape, int32_t io_dtype, const muon_ns_params_t* prm,
                         void* const* out, int* nonfinite_flag) {
  muon_ctx* c = env.ctx;

  if (count < 0) return efail(env, MUON_EINVAL, "count < 0");
  if (prm == nullptr) return efail(env, MUON_EINVAL, "params NULL");
  if (!is_dtype(io_dtype) || !is_dtype(prm->compute)) return efail(env, MUON_EDTYPE, "dtype");
  if (io_dtype != prm->compute)
    return efail(env, MUON_EDTYPE, "io dtype must equal the compute dtype");
  if (prm->steps < 0 || !(prm->eps >= 0.0f)) return efail(env, MUON_EINVAL, "steps/eps");
  if (prm->method != MUON_NS_QUINTIC && prm->method != MUON_NS_GRAM)
    return efail(env, MUON_EINVAL, "method");
  if (prm->fuse != MUON_FUSE_AUTO && prm->fuse != MUON_FUSE_OFF && prm->fuse != MUON_FUSE_ON)
    return efail(env, MUON_EINVAL, "fuse");
  if (prm->coeffs != nullptr)
    for (int64_t k = 0; k < 3 * static_cast<int64_t>(prm->steps); ++k)
      if (!std::isfinite(prm->coeffs[k])) return efail(env, MUON_EINVAL, "coefficients not finite");
  NsLayout L;
  if (!ns_layout(shape, count, prm->compute, &L)) return efail(env, MUON_ESHAPE, "shape");
  if (count == 0) return MUON_OK;
  if (mats == nullptr) return efail(env, MUON_EINVAL, "mats NULL");
  const size_t es = esize(io_dtype);
  for (int64_t i = 0; i < count; ++i) {
    if (mats[i] == nullptr || (out && out[i] == nullptr)) return efail(env, MUON_EINVAL, "null matrix");
    if ((reinterpret_cast<uintptr_t>(mats[i]) % es) || (out && reinterpret_cast<uintptr_t>(out[i]) % es))
      return efail(env, MUON_EINVAL, "misaligned matrix");
  }
  const int64_t per = L.units / count;
  const int64_t unit_elems = L.ur * L.uc;
  const int64_t unit_bytes = unit_elems * static_cast<int64_t>(es);
  // norms from the momentum pass: every unit on whole blocks inside the partials
  const int64_t block_bytes = int64_t{MUON_SQ_BLOCK} * static_cast<int64_t>(es);
  if (prm->sq_partials != nullptr) {
    if (prm->sq_base == nullptr || prm->sq_count < 0 ||
        reinterpret_cast<uintptr_t>(prm->sq_partials) % 8 || unit_elems % MUON_SQ_BLOCK)
      return efail(env, MUON_EINVAL, "sq_partials: units must span whole blocks");
    const uintptr_t base = reinterpret_cast<uintptr_t>(prm->sq_base);
    const int64_t nblk = per * (unit_elems / MUON_SQ_BLOCK);
    for (int64_t i = 0; i < count; ++i) {
      const uintptr_t a = reinterpret_cast<uintptr_t>(mats[i]);
      if (a < base || (a - base) % static_cast<uintptr_t>(block_bytes) ||
          static_cast<int64_t>((a - base) / static_cast<uintptr_t>(block_bytes)) > prm->sq_count - nblk)
        return efail(env, MUON_EINVAL, "sq_partials do not cover a matrix on block boundaries");
    }
  }
  if (L.total > env.ws_bytes) return efail(env, MUON_EWORKSPACE, "workspace too small for this call");
  const void* const* outp = out ? reinterpret_cast<const void* const*>(out) : mats;

  UnitsRef in = describe(mats, count, per, unit_bytes);
  UnitsRef ot = describe(outp, count, per, unit_bytes);
  if ((in.needs_table || ot.needs_table) && c == nullptr)
    return efail(env, MUON_EINVAL, "matrices not evenly spaced: pointer tables need a context");
  if ((in.needs_table || ot.needs_table) && L.units > kTabCap)
    return efail(env, MUON_EINVAL, "too many irregularly placed units in one call (max 65536)");

  // vector paths need 16-byte aligned units
  bool al = (unit_bytes % 16) == 0;
  for (int64_t i = 0; al && i < count; ++i) al = aligned16(mats[i]) && aligned16(outp[i]);
  const bool mfma = prm->compute == MUON_BF16 && al && (L.ur % 8 == 0) && (L.uc % 8 == 0) &&
                    unit_bytes < (int64_t(1) << 31);

  DeviceGuard g(env.device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;

  if (in.needs_table || ot.needs_table) {
    // the tables are uploaded from a host ring that later calls reuse: a
    // replayed graph would copy whatever the ring holds then
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs) != hipSuccess ||
        cs != hipStreamCaptureStatusNone)
      return efail(env, MUON_EINVAL, "matrices not evenly spaced: their pointer tables cannot be recorded into a graph");
    const int slot = c->tab_next;
    c->tab_next = (c->tab_next + 1) % kTabSlots;
    if (c->tab_used[slot]) {
      e = hipEventSynchronize(c->tab_ev[slot]);
      if (e != hipSuccess) return ehip(env, e, "table slot wait");
    }
    uint64_t* hin = c->host_tab + static_cast<size_t>(slot) * 2 * kTabCap;
    uint64_t* hout = hin + kTabCap;
    uint64_t* din = c->dev_tab + static_cast<size_t>(slot) * 2 * kTabCap;
    uint64_t* dout = din + kTabCap;
    if (in.needs_table) {
      fill_table(hin, mats, count, per, unit_bytes);
      e = hipMemcpyAsync(din, hin, sizeof(uint64_t) * L.units, hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return ehip(env, e, "table upload");
      in.ref = MatRef{nullptr, 0, din};
    }
    if (ot.needs_table) {
      fill_table(hout, outp, count, per, unit_bytes);
      e = hipMemcpyAsync(dout, hout, sizeof(uint64_t) * L.units, hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return ehip(env, e, "table upload");
      ot.ref = MatRef{nullptr, 0, dout};
    }
    e = hipEventRecord(c->tab_ev[slot], s);
    if (e != hipSuccess) return ehip(env, e, "table event");
    c->tab_used[slot] = true;
  }

  // BF16 units whose smaller side is under kNsTinySide run the iteration in
  // fp32: their bf16 A and B' alone take some Gaussian draws past the bf16
  // error bar.  The inputs are widened into the slab, the fp32 call runs in
  // place there (norms recomputed from the same values), and its result is
  // rounded to bf16 into the outputs.
  if (prm->compute == MUON_BF16 && L.m < kNsTinySide) {
    char* stage = env.ws + L.stage;
    const MatRef SR{stage, unit_elems * 4, nullptr};
    e = launch_convert(s, in.ref, 1, SR, 0, unit_elems, L.units, nullptr);
    if (e != hipSuccess) return ehip(env, e, "widen launch");
    std::vector<const void*> sp(static_cast<size_t>(L.units));
    for (int64_t i = 0; i < L.units; ++i) sp[static_cast<size_t>(i)] = stage + i * unit_elems * 4;
    muon_ns_params_t p32 = *prm;
    p32.compute = MUON_F32;
    p32.sq_partials = nullptr;
    p32.sq_base = nullptr;
    p32.sq_count = 0;
    NsEnv sub = env;
    sub.ws = env.ws + L.sub;
    sub.ws_bytes = env.ws_bytes - L.sub;
    sub.outputs_in_place = true;
    const muon_shape_t us{L.ur, L.uc, 0};
    const muon_status_t st =
        ns_batched(sub, stream, sp.data(), L.units, us, MUON_F32, &p32, nullptr, nonfinite_flag);
    if (st != MUON_OK) return st;
    e = launch_convert(s, SR, 0, ot.ref, 1, unit_elems, L.units, nullptr);
    return e == hipSuccess ? MUON_OK : ehip(env, e, "narrow launch");
  }

  char* ws = env.ws;
  const int64_t xbytes = L.m * L.n * static_cast<int64_t>(es);
  const int64_t abytes = L.m * L.m * static_cast<int64_t>(es);
  const MatRef XA{ws + L.xa, xbytes, nullptr}, XB{ws + L.xb, xbytes, nullptr};
  const MatRef AR{ws + L.a, abytes, nullptr}, BR{ws + L.b, abytes, nullptr};
  float* scale = reinterpret_cast<float*>(ws + L.scale);
  int* zflag = reinterpret_cast<int*>(ws + L.zflag);
  double* partial = reinterpret_cast<double*>(ws + L.partial);
  // BF16 compute carries the iterate past bf16: residual plane and B's diagonal
  char* lo_plane = prm->compute == MUON_BF16 ? ws + L.lo : nullptr;
  float* dvec = prm->compute == MUON_BF16 ? reinterpret_cast<float*>(ws + L.dvec) : nullptr;
  const int io_bf16 = io_dtype == MUON_BF16;
  const bool tall = L.ur > L.uc;
  const int64_t m = L.m, n = L.n;

  auto setup = [&](NsGemmArgs& a, int epi, int T) {
    a.tiles_m = static_cast<int>((a.M + T - 1) / T);
    a.tiles_n = static_cast<int>((a.N + T - 1) / T);
    a.tiles_per_unit = (epi == EPI_UPDATE) ? a.tiles_m * a.tiles_n : a.tiles_m * (a.tiles_m + 1) / 2;
    a.units = L.units;
    a.cus = env.cus;
    a.zflag = zflag;
  };
  // (a, b, c) of iteration k: the per-iteration table's row k, else the fixed
  // coefficients
  auto coef = [&](int k, float* ca, float* cb, float* cc) {
    const float* r = prm->coeffs ? prm->coeffs + 3 * static_cast<int64_t>(k) : nullptr;
    *ca = r ? r[0] : prm->a;
    *cb = r ? r[1] : prm->b;
    *cc = r ? r[2] : prm->c;
  };

  // Deterministic norm, then per iteration Gram -> symmetric square ->
  // update.  Iterates stay in the input's orientation; K-major operands are
  // read in place (transposed reads), never copied.
  NsNormArgs na;
  na.in = in.ref;
  na.unit_elems = unit_elems;
  na.units = L.units;
  na.parts = L.parts;
  na.partial = partial;
  na.scale = scale;
  na.zflag = zflag;
  na.nonfinite = nonfinite_flag;
  na.eps = prm->eps;
  na.sq = prm->sq_partials;
  na.sq_base = static_cast<const char*>(prm->sq_base);
  na.block_bytes = block_bytes;
  na.blocks_per_unit = unit_elems / MUON_SQ_BLOCK;
  long tk = etstart(env, s, MUON_K_NORM);
  e = launch_norm(s, na, io_bf16, al && (unit_elems % 8 == 0));
  etstop(env, s, tk);
  if (e != hipSuccess) return ehip(env, e, "norm launch");
  if (prm->steps == 0) {
    e = launch_scale_copy(s, in.ref, ot.ref, unit_elems, L.units, scale, io_bf16);
    return e == hipSuccess ? MUON_OK : ehip(env, e, "copy launch");
  }
  auto gemm = [&](int cls, NsGemmArgs& a, int epi, bool tm, bool tn) -> hipError_t {
    // 256 x 256 tiles once the smaller output side reaches 256, 128 x 128
    // where that leaves most CUs idle (the same bits either way)
    const int T = mfma ? ns_mfma_tile(a.M, a.N, epi != EPI_UPDATE, L.units, env.cus) : 64;
    setup(a, epi, T);
    const long k = etstart(env, s, cls);
    const hipError_t r = mfma ? launch_ns_gemm_mfma(s, a, epi, tm, tn, T)
                              : launch_ns_gemm_simple(s, a, epi, tm, tn, io_bf16);
    etstop(env, s, k);
    return r;
  };
  // Does the output touch the input?  `alias`: the spans of the inputs and
  // the outputs overlap at all (conservative).
  bool alias = false;
  {
    const int64_t call_bytes = unit_bytes * per;
    const char *ilo = nullptr, *ihi = nullptr, *olo = nullptr, *ohi = nullptr;
    for (int64_t i = 0; i < count; ++i) {
      const char* pi = static_cast<const char*>(mats[i]);
      const char* po = static_cast<const char*>(outp[i]);
      alias = alias || pi == po;
      ilo = (i == 0 || pi < ilo) ? pi : ilo;
      ihi = (i == 0 || pi + call_bytes > ihi) ? pi + call_bytes : ihi;
      olo = (i == 0 || po < olo) ? po : olo;
      ohi = (i == 0 || po + call_bytes > ohi) ? po + call_bytes : ohi;
    }
    alias = alias || ranges_overlap(ilo, ihi - ilo, olo, ohi - olo);
  }
  // The Gram form squares the singular values into A_0; in bf16 that loses
  // the small ones once m nears n (relative error ~1e-1 on square Gaussian
  // inputs against ~1e-2 for the quintic), so bf16 runs it only on units with
  // 2 m <= n, where its error stays at the quintic's level.
  const bool gram_form =
      prm->method == MUON_NS_GRAM && (prm->compute == MUON_F32 || 2 * m <= n);
  // Small wide units: every iteration in one launch.  A workgroup writes only
  // its own unit, so an output may be its own input but may not touch any
  // other matrix's input.
  const bool small_ok = mfma && !tall && m <= 128 && prm->fuse != MUON_FUSE_OFF &&
                        (prm->coeffs == nullptr || prm->steps <= MUON_NS_FUSED_MAX_ROWS) &&
                        (!alias || (c == nullptr ? env.outputs_in_place
                                                 : !cross_overlap(mats, outp, count, unit_bytes * per)));
  // AUTO: a unit for every CU, or units narrow enough that one workgroup per
  // unit finishes before the separate launches would with most CUs idle
  // (MI355X, 8 waves per workgroup: ~0.05 + 0.0155 ms per 128-column block
  // and round of units, against >= 0.28 ms for the fifteen launches; at
  // 128 x 4096 with a few units the separate launches win)
  constexpr int64_t kFuseAnyCols = 3072;
  if (small_ok && (prm->fuse == MUON_FUSE_ON || L.units >= env.cus || n <= kFuseAnyCols)) {
    NsSmallArgs fa{};
    fa.src = in.ref;
    fa.dst = ot.ref;
    fa.xa = XA;
    fa.xb = XB;
    fa.m = static_cast<int>(m);
    fa.n = static_cast<int>(n);
    fa.steps = prm->steps;
    fa.gram = gram_form ? 1 : 0;
    fa.units = L.units;
    fa.scale = scale;
    fa.zflag = zflag;
    // a fixed triple is one row that every iteration reuses
    fa.dvec = dvec;
    fa.lo = lo_plane;
    fa.ncoef = prm->coeffs ? prm->steps : 1;
    for (int k = 0; k < fa.ncoef; ++k) coef(k, &fa.coef[k][0], &fa.coef[k][1], &fa.coef[k][2]);
    const long k = etstart(env, s, MUON_K_FUSED);
    e = launch_ns_small(s, fa);
    etstop(env, s, k);
    return e == hipSuccess ? MUON_OK : ehip(env, e, "fused launch");
  }

  if (gram_form) {
    // m x m matrices live in A, B and (at m x m stride) the two iterate
    // regions; the input is read by the first and the last product only.
    const MatRef R2{ws + L.xa, abytes, nullptr}, R3{ws + L.xb, abytes, nullptr};
    auto sym_prod = [&](int cls, const MatRef& p, const MatRef& q, const MatRef& d) {
      // d = p q for symmetric commuting p, q: the Gram product p q^T, upper tiles
      NsGemmArgs pa{};
      pa.pm = p; pa.pn = q; pa.dst = d; pa.epi = d;
      pa.ldm = pa.ldn = pa.ldd = pa.lde = m;
      pa.M = pa.N = pa.K = static_cast<int>(m);
      return gemm(cls, pa, EPI_GRAM, false, false);
    };
    NsGemmArgs ga{};
    ga.pm = in.ref; ga.pn = in.ref; ga.dst = AR; ga.epi = AR;
    ga.ldm = ga.ldn = tall ? m : n;
    ga.ldd = ga.lde = m;
    ga.M = ga.N = static_cast<int>(m);
    ga.K = static_cast<int>(n);
    ga.scale = scale;
    ga.scale_pow = 2;
    e = gemm(MUON_K_GRAM, ga, EPI_GRAM, tall, tall);
    if (e != hipSuccess) return ehip(env, e, "gram launch");
    MatRef Q = R2, other = R3;
    for (int k = 0; k < prm->steps; ++k) {
      // P_k = a I + b A_k + c A_k^2; P_0 is Q_1 itself
      const MatRef P = (k == 0) ? R2 : BR;
      NsGemmArgs sa{};
      sa.pm = AR; sa.pn = AR; sa.dst = P; sa.epi = AR;
      sa.ldm = sa.ldn = sa.ldd = sa.lde = m;
      sa.M = sa.N = sa.K = static_cast<int>(m);
      coef(k, &sa.ca, &sa.cb, &sa.cc);
      e = gemm(MUON_K_SYMSQ, sa, EPI_SYMSQ, false, false);
      if (e != hipSuccess) return ehip(env, e, "symsq launch");
      if (k > 0) {
        e = sym_prod(MUON_K_PROD, P, Q, other);  // Q_{k+1} = P_k Q_k
        if (e != hipSuccess) return ehip(env, e, "product launch");
        std::swap(Q, other);
      }
      if (k + 1 < prm->steps) {
        // A_{k+1} = (P_k A_k) P_k, through the free region
        e = sym_prod(MUON_K_PROD, P, AR, other);
        if (e == hipSuccess) e = sym_prod(MUON_K_PROD, other, P, AR);
        if (e != hipSuccess) return ehip(env, e, "product launch");
      }
    }
    // X = s Q X_0 (tall: Y Q).  Written straight to the output unless the
    // output overlaps the input, then through the free iterate region.
    const MatRef freeX = (Q.base == R2.base) ? XB : XA;
    NsGemmArgs ua{};
    ua.dst = alias ? freeX : ot.ref;
    ua.scale = scale;
    ua.scale_pow = 1;
    ua.zero_write = 1;
    if (!tall) {
      ua.pm = Q; ua.ldm = m;
      ua.pn = in.ref; ua.ldn = n;
      ua.ldd = ua.lde = n;
      ua.M = static_cast<int>(m);
      ua.N = static_cast<int>(n);
    } else {
      ua.pm = in.ref; ua.ldm = m;
      ua.pn = Q; ua.ldn = m;
      ua.ldd = ua.lde = m;
      ua.M = static_cast<int>(n);
      ua.N = static_cast<int>(m);
    }
    ua.K = static_cast<int>(m);
    e = gemm(MUON_K_UPDATE, ua, EPI_UPDATE, false, !tall);
    if (e != hipSuccess) return ehip(env, e, "update launch");
    if (alias) {
      e = launch_scale_copy(s, freeX, ot.ref, unit_elems, L.units, nullptr, io_bf16);
      if (e != hipSuccess) return ehip(env, e, "copy launch");
    }
    return MUON_OK;
  }

  // The products skip zero units (their result is exactly zero, written by
  // the last update).  The updates but the last run over a list of the
  // nonzero units, so that the others take no tile slot at all and a call
  // with many zero units (experts without tokens) does not leave workgroups
  // idle behind the busiest one (update -15% at 25% zero units, 768 x 2048);
  // the Gram and symmetric-square launches, with 6 tiles per such unit and
  // whole rounds either way, measured faster without it.  The list goes
  // where the norm's partial sums were (at least 8 bytes per unit, free once
  // the norms are taken).  The last update writes every unit.
  const int* ulist = nullptr;
  const int* ucount = nullptr;
  if (mfma && prm->steps > 1) {
    int* lst = reinterpret_cast<int*>(partial);
    e = launch_compact_units(s, zflag, L.units, lst, lst + L.units);
    if (e != hipSuccess) return ehip(env, e, "unit list launch");
    ulist = lst;
    ucount = lst + L.units;
  }

  for (int k = 0; k < prm->steps; ++k) {
    const bool last = (k == prm->steps - 1);
    const MatRef src = (k == 0) ? in.ref : (((k - 1) % 2 == 0) ? XA : XB);
    // one-step calls go through XA so the input is never overwritten while read
    const MatRef dstX = (last && prm->steps > 1) ? ot.ref : ((k % 2 == 0) ? XA : XB);

    NsGemmArgs ga{};
    ga.pm = src; ga.pn = src; ga.dst = AR; ga.epi = AR;
    ga.ldm = ga.ldn = tall ? m : n;
    ga.ldd = ga.lde = m;
    ga.M = ga.N = static_cast<int>(m);
    ga.K = static_cast<int>(n);
    ga.scale = scale;
    ga.scale_pow = (k == 0) ? 2 : 0;
    e = gemm(MUON_K_GRAM, ga, EPI_GRAM, tall, tall);
    if (e != hipSuccess) return ehip(env, e, "gram launch");

    NsGemmArgs sa{};
    sa.pm = AR; sa.pn = AR; sa.dst = BR; sa.epi = AR;
    sa.ldm = sa.ldn = sa.ldd = sa.lde = m;
    sa.M = sa.N = sa.K = static_cast<int>(m);
    sa.dvec = dvec;
    coef(k, &sa.ca, &sa.cb, &sa.cc);
    e = gemm(MUON_K_SYMSQ, sa, EPI_SYMSQ, false, false);
    if (e != hipSuccess) return ehip(env, e, "symsq launch");

    NsGemmArgs ua{};
    ua.dst = dstX;
    ua.scale = scale;
    ua.scale_pow = (k == 0) ? 1 : 0;
    ua.zero_write = last ? 1 : 0;
    // B's diagonal completed in fp32 and the residual carried from update to
    // update (read and rewritten tile by tile, in place) out of every update
    // but the last two: rounding left in the second-to-last update is lifted
    // by one more iteration only (a bf16 emulation of rank-deficient inputs
    // moves by at most 1e-3 relative).  The generic kernel reads the iterate
    // at the output position through epi.
    ua.dvec = dvec;
    ua.epi = src;
    ua.lde = tall ? m : n;
    ua.lo_in = (lo_plane != nullptr && ns_lo_read(k, prm->steps)) ? lo_plane : nullptr;
    ua.lo_out = (lo_plane != nullptr && ns_lo_written(k, prm->steps)) ? lo_plane : nullptr;
    if (!tall) {
      // X' = B' X : rows from B', columns from X (K-major)
      ua.pm = BR; ua.ldm = m;
      ua.pn = src; ua.ldn = n;
      ua.ldd = ua.lde = n;
      ua.M = static_cast<int>(m);
      ua.N = static_cast<int>(n);
    } else {
      // Y' = Y B' : rows from Y, columns from B' (symmetric)
      ua.pm = src; ua.ldm = m;
      ua.pn = BR; ua.ldn = m;
      ua.ldd = ua.lde = m;
      ua.M = static_cast<int>(n);
      ua.N = static_cast<int>(m);
    }
    ua.K = static_cast<int>(m);
    if (!last) {
      ua.ulist = ulist;
      ua.ucount = ucount;
    }
    e = gemm(MUON_K_UPDATE, ua, EPI_UPDATE, false, !tall);
    if (e != hipSuccess) return ehip(env, e, "update launch");
  }
  if (prm->steps == 1) {
    e = launch_scale_copy(s, XA, ot.ref, unit_elems, L.units, nullptr, io_bf16);
    if (e != hipSuccess) return ehip(env, e, "copy launch");
  }
  return MUON_OK;
}

extern "C" muon_status_t muon_newton_schulz_batched(muon_ctx_t* c, void* stream,
                                                    const void* const* mats, int64_t count,
                                                    muon_shape_t shape, int32_t io_dtype,
                                                    const muon_ns_params_t* prm,
                                                    void* const* out, int* nonfinite_flag) {
  if (c == nullptr) return MUON_EINVAL;
  NsEnv env;
  env.ctx = c;
  env.ws = c->ws;
  env.ws_bytes = c->ws_bytes;
  env.cus = c->cus;
  env.device = c->device;
  return ns_batched(env, stream, mats, count, shape, io_dtype, prm, out, nonfinite_flag);
}
