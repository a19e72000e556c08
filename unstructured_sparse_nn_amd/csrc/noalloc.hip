// noalloc.hip -- snack_prune_regrow_static: the restructure step with its
// workspace in a file-scope device array instead of a caller's buffer, for
// callers that cannot allocate (code under graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// `scratch` below is one device array per GPU the library runs on; its
// device address comes from hipGetSymbolAddress once per device, with that
// device current, and only that address is passed to kernels and copies
// (the array's name is a host-side stand-in in host code).  Every call on a
// GPU shares that GPU's array, so calls that overlap on one GPU race; the
// restructure writes every word of the workspace it reads (nothing relies on
// a cleared array), and its result words come back by a copy into the
// caller's stack.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/snack.h"
#include "internal.h"

// The workspace of every call on a GPU (one copy per device).
static __device__ __align__(256) unsigned char scratch[SNACK_STATIC_WS_MAX];

namespace {

constexpr int MAX_DEVICES = 64;

std::mutex g_init_mutex;
std::atomic<void*> g_scratch[MAX_DEVICES];

// Device address of this device's scratch array (resolved once per device);
// NULL if the lookup fails.
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_init_mutex);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_scratch[dev].store(addr, std::memory_order_release);
  return addr;
}

}  // namespace

extern "C" {

snack_status snack_prune_regrow_static(int32_t* row, int32_t* col, void* vals, snack_dtype dtype,
                                       int32_t M, int32_t K, int64_t nnz, int64_t n_drop,
                                       uint64_t seed, uint64_t step, int64_t* dropped_lin,
                                       int64_t* grown_lin, void* stream) {
  size_t need = 0;
  const snack_status st = snack_prune_regrow_workspace(M, K, nnz, n_drop, &need);
  if (st != SNACK_OK) return st;
  if (need > (size_t)SNACK_STATIC_WS_MAX) return SNACK_E_WORKSPACE;
  if (n_drop == 0) return snack_prune_regrow(row, col, vals, dtype, M, K, nnz, 0, seed, step,
                                             dropped_lin, grown_lin, nullptr, 0, stream);
  void* ws = scratch_of_current_device();
  if (!ws) return SNACK_E_HIP;
  return snack_prune_regrow(row, col, vals, dtype, M, K, nnz, n_drop, seed, step, dropped_lin,
                            grown_lin, ws, (size_t)SNACK_STATIC_WS_MAX, stream);
}

}  // extern "C"
