// The allocation-free Newton-Schulz entry point: the same kernels as
// muon_newton_schulz_batched, with the workspace in a static device array
// instead of a context's slab, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).
//
// The array, `scratch`, is part of the library's code object: the runtime
// allocates it on every GPU the library runs on when it loads the code object
// there, and it stays until the process ends.  On the host its name is only a
// stand-in, not a device address: the address comes from hipGetSymbolAddress,
// once per device with that device current, and is cached per device.  Every
// call on one GPU shares that GPU's copy (calls that overlap on one GPU race);
// the array keeps the last call's contents, and nothing in it has to start at
// zero (the norm pass writes every unit's scale and zero flag, the residual
// plane and B's diagonal are written before they are read).
#include <hip/hip_runtime.h>

#include <mutex>

#include "muon.h"
#include "muon_internal.h"
#include "ns_layout.h"

namespace {

constexpr size_t kScratchBytes = MUON_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex g_mu;
char* g_scratch[kMaxDevices] = {};  // device address of `scratch` per device
int g_cus[kMaxDevices] = {};
thread_local const char* g_err = "";

// The device address of this device's copy of `scratch` and its compute
// units, looked up on the first call on the device.
muon_status_t scratch_on(int device, char** p, int* cus) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[device] == nullptr) {
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (hipSetDevice(device) != hipSuccess) {
      (void)hipGetLastError();
      g_err = "hipSetDevice failed";
      return MUON_EHIP;
    }
    void* q = nullptr;
    hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    int n = 0;
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device);
    if (prev >= 0) (void)hipSetDevice(prev);
    if (e != hipSuccess || q == nullptr) {
      (void)hipGetLastError();
      g_err = "hipGetSymbolAddress of the static scratch failed";
      return MUON_EHIP;
    }
    g_scratch[device] = static_cast<char*>(q);
    g_cus[device] = n > 0 ? n : 256;
  }
  *p = g_scratch[device];
  *cus = g_cus[device];
  return MUON_OK;
}

muon_status_t reject(muon_status_t st, const char* what) {
  g_err = what;
  return st;
}

}  // namespace

extern "C" muon_status_t muon_newton_schulz_batched_noalloc(int device, void* stream,
                                                            const void* const* mats, int64_t count,
                                                            muon_shape_t shape, int32_t io_dtype,
                                                            const muon_ns_params_t* params,
                                                            void* const* out, int* nonfinite_flag) {
  g_err = "";
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev || device >= kMaxDevices)
    return reject(MUON_EINVAL, "no such device");
  if (params == nullptr || count < 0) return reject(MUON_EINVAL, "params NULL or count < 0");
  if (io_dtype != MUON_F32 && io_dtype != MUON_BF16) return reject(MUON_EDTYPE, "dtype");
  NsLayout L;
  if (!ns_layout(shape, count, params->compute, &L)) return reject(MUON_ESHAPE, "shape");
  if (count == 0) return MUON_OK;
  if (mats == nullptr) return reject(MUON_EINVAL, "mats NULL");
  if (L.total > kScratchBytes)
    return reject(MUON_EWORKSPACE, "the call needs more than the static scratch holds");
  // Placement: evenly spaced inputs; outputs either the inputs themselves
  // (in place) or evenly spaced and disjoint from every input.
  const int64_t bytes = shape.rows * shape.cols * (io_dtype == MUON_BF16 ? 2 : 4);
  auto addr = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
  auto even = [&](const void* const* p) {
    for (int64_t i = 0; i < count; ++i)
      if (p[i] == nullptr) return false;
    if (count < 2) return true;
    const intptr_t d = static_cast<intptr_t>(addr(p[1]) - addr(p[0]));
    if (d < bytes && -d < bytes) return false;  // neighbours overlap
    for (int64_t i = 2; i < count; ++i)
      if (static_cast<intptr_t>(addr(p[i]) - addr(p[0])) != d * i) return false;
    return true;
  };
  if (!even(mats)) return reject(MUON_EINVAL, "inputs must be evenly spaced and not overlap");
  bool in_place = out == nullptr;
  if (!in_place) {
    in_place = true;
    for (int64_t i = 0; i < count; ++i) in_place = in_place && out[i] == mats[i];
    if (!in_place) {
      if (!even(out)) return reject(MUON_EINVAL, "outputs must be evenly spaced and not overlap");
      auto span = [&](const void* const* p, uintptr_t* lo, uintptr_t* hi) {
        *lo = addr(p[0]);
        *hi = addr(p[0]) + bytes;
        for (int64_t i = 1; i < count; ++i) {
          *lo = addr(p[i]) < *lo ? addr(p[i]) : *lo;
          *hi = addr(p[i]) + bytes > *hi ? addr(p[i]) + bytes : *hi;
        }
      };
      uintptr_t ilo, ihi, olo, ohi;
      span(mats, &ilo, &ihi);
      span(reinterpret_cast<const void* const*>(out), &olo, &ohi);
      if (ilo < ohi && olo < ihi)
        return reject(MUON_EINVAL, "outputs must be the inputs themselves or disjoint from them");
    }
  }
  char* ws = nullptr;
  int cus = 256;
  const muon_status_t st = scratch_on(device, &ws, &cus);
  if (st != MUON_OK) return st;
  NsEnv env;
  env.ctx = nullptr;
  env.ws = ws;
  env.ws_bytes = kScratchBytes;
  env.cus = cus;
  env.device = device;
  env.outputs_in_place = in_place;
  env.err = &g_err;
  return ns_batched(env, stream, mats, count, shape, io_dtype, params, in_place ? nullptr : out,
                    nonfinite_flag);
}

extern "C" const char* muon_noalloc_last_error(void) { return g_err; }
