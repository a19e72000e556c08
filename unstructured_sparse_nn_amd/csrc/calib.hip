// calib.hip -- calibration kernels for the benchmark's floors: an empty
// kernel (launch and drain), a streaming read and a streaming write of a
// buffer (HBM bandwidth), and a chain of dependent loads (memory latency).
// They measure the machine, not the layer, and take no part in it.
#include <hip/hip_runtime.h>

#include "../../include/snack.h"
#include "common.h"
#include "internal.h"

namespace {

__global__ void k_calib_empty() {}

// Every 16-byte word of the buffer is read once (grid-stride, eight
// non-temporal loads in flight per thread); a word is stored only if the
// running xor hits an improbable value, so no load can be dropped and nothing
// is written in practice.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_calib_read(const uint4* __restrict__ p, int64_t n,
                                                    uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  const u32x4* __restrict__ q = reinterpret_cast<const u32x4*>(p);
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = __builtin_nontemporal_load(&q[i + u * stride]);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
  }
  for (; i < n; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ __launch_bounds__(256) void k_calib_write(uint4* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) p[i] = z;
}

// Slot i (128 bytes, one line) holds the index of the next slot of a
// full-period linear congruential cycle over the n slots (n a power of two,
// multiplier 1 mod 4, odd increment): consecutive hops land far apart.
__global__ __launch_bounds__(256) void k_calib_chain(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n)
    p[i * 32] = (uint32_t)(((uint64_t)i * 0x9E3779B1ull + 0x7F4A7C15ull) & (uint64_t)(n - 1));
}

// One thread follows `hops` links from slot 0, each load depending on the
// previous one; the last index is stored in slot 0's second word.
// (Indices are masked to the slot count, so a buffer the chain kernel did not
// write still reads in bounds.)
__global__ void k_calib_chase(const uint32_t* __restrict__ p, int64_t hops, uint32_t mask,
                              uint32_t* __restrict__ out) {
  uint32_t j = 0;
  for (int64_t h = 0; h < hops; ++h) j = __builtin_nontemporal_load(&p[(int64_t)j * 32]) & mask;
  out[1] = j;
}

}  // namespace

extern "C" {

snack_status snack_calibrate(int32_t kind, void* buf, size_t bytes, int64_t n, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (kind) {
    case SNACK_CALIB_EMPTY:
      if (n < 1 || n > (1 << 20)) return SNACK_E_SHAPE;
      hipLaunchKernelGGL(k_calib_empty, dim3((unsigned)n), dim3(64), 0, s);
      break;
    case SNACK_CALIB_READ:
    case SNACK_CALIB_WRITE: {
      if (!buf) return SNACK_E_NULL;
      if (bytes < 16 || bytes % 16 || n < 1 || n > (1 << 20)) return SNACK_E_SHAPE;
      const int64_t words = (int64_t)(bytes / 16);
      if (kind == SNACK_CALIB_READ)
        hipLaunchKernelGGL(k_calib_read, dim3((unsigned)n), dim3(256), 0, s, (const uint4*)buf,
                           words - 1, (uint32_t*)((uint4*)buf + words - 1));
      else
        hipLaunchKernelGGL(k_calib_write, dim3((unsigned)n), dim3(256), 0, s, (uint4*)buf,
                           words);
      break;
    }
    case SNACK_CALIB_CHAIN:
    case SNACK_CALIB_CHASE: {
      if (!buf) return SNACK_E_NULL;
      int64_t slots = 1;
      while (slots * 2 * 128 <= (int64_t)bytes && slots < ((int64_t)1 << 31)) slots *= 2;
      if (slots < 2) return SNACK_E_SHAPE;
      if (kind == SNACK_CALIB_CHAIN) {
        hipLaunchKernelGGL(k_calib_chain, dim3((unsigned)snk::cdiv(slots, 256)), dim3(256), 0, s,
                           (uint32_t*)buf, slots);
      } else {
        if (n < 1) return SNACK_E_SHAPE;
        hipLaunchKernelGGL(k_calib_chase, dim3(1), dim3(1), 0, s, (const uint32_t*)buf, n,
                           (uint32_t)(slots - 1), (uint32_t*)buf);
      }
      break;
    }
    default: return SNACK_E_SHAPE;
  }
  return hipGetLastError() == hipSuccess ? SNACK_OK : SNACK_E_HIP;
}

}  // extern "C"
