// fa_bwd_noalloc: the backward pass with its workspace in a fixed, file-scope
// device array instead of a caller buffer, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// The array is `scratch`, kScratchBytes long, one copy per GPU the library runs
// on, held until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is a stand-in, not a device address): the device address
// of each GPU's copy is looked up once per device with hipGetSymbolAddress, with
// that device current, and kept.  The backward's kernels take that address as
// their workspace, exactly as they take the caller's buffer in fa_bwd.
//
// The workspace holds per-row terms that the first phase writes in full before
// the other phases read them, so nothing needs clearing between calls.  Calls
// that overlap on one GPU (two streams, two host threads) share the array and
// race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"
#include "fa_launch.h"

namespace {

constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, or nullptr if the
// runtime cannot provide it.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(g_lock);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                              const float* lse, void* dQ, void* dK, void* dV, int B, int H, int Tq, int Tk, int d,
                              float scale, int causal, int dtype, int o_dtype, int grad_dtype, void* stream) {
  // every argument check of fa_bwd, without a workspace and before any HIP call
  const int st = fa::check_bwd_args(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, d, scale, dtype, o_dtype,
                                    grad_dtype);
  if (st != FA_OK) return st;
  if (fa_bwd_workspace_bytes(B, H, Tq, Tk, d, dtype, grad_dtype) > kScratchBytes) return FA_ERR_SCRATCH;
  void* ws = scratch_address();
  if (!ws) return FA_ERR_LAUNCH;
  return fa_bwd(Q, K, V, O, dO, lse, dQ, dK, dV, B, H, Tq, Tk, d, scale, causal, dtype, o_dtype, grad_dtype, ws,
                kScratchBytes, stream);
}
