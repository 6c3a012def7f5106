// Sustained HBM read rate on this device: the plain streaming read that the
// decode kernels' bandwidth is compared with (a measurement helper, not part
// of the matrix-product path).
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace lowbit {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per thread per step

// Every 16-byte piece is read once with a nontemporal load in a grid-stride
// loop; each workgroup XOR-folds what it read into *out (so no load can be
// dropped).
__global__ __launch_bounds__(kProbeThreads) void hbm_read(const v4u* __restrict__ p, int64_t n16,
                                                         uint32_t* out) {
  uint32_t acc = 0;
  const int64_t step = (int64_t)gridDim.x * kProbeThreads * kProbeUnroll;
  for (int64_t i = (int64_t)blockIdx.x * kProbeThreads * kProbeUnroll + threadIdx.x; i < n16;
       i += step) {
    v4u v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; u++) {
      const int64_t j = i + (int64_t)u * kProbeThreads;
      v[u] = j < n16 ? __builtin_nontemporal_load(p + j) : v4u{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(out, acc);
}

}  // namespace

hipError_t launch_hbm_read(const void* src, int64_t bytes, uint32_t* out, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t n16 = bytes / 16;
  const int64_t per_block = (int64_t)kProbeThreads * kProbeUnroll;
  const int64_t want = (n16 + per_block - 1) / per_block;
  // one workgroup per CU with 8 loads in flight per thread (32 KiB per CU)
  // reads fastest: measured 7.36 TB/s, against 7.23 at two workgroups with
  // 4 loads and 6.1 at eight with 4 (more concurrent streams read HBM less
  // efficiently)
  const int64_t grid = want < (int64_t)cus ? want : (int64_t)cus;
  hipLaunchKernelGGL(hbm_read, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(kProbeThreads), 0, s,
                     (const v4u*)src, n16, out);
  return hipGetLastError();
}

}  // namespace lowbit
