// Reference kernel for the HBM roofline of the memory-bound kernels: a plain
// streaming read.  It is not part of the NVFP4 path; the benchmark times it
// beside the path's kernels so that their GB/s can be set against what this
// device sustains on reads alone (the published 8 TB/s is a peak, not a
// sustainable rate).
//
// Every lane reads 16-byte chunks with eight loads in flight, grid-stride,
// and folds them into one word, which is stored only if it equals a value the
// caller chooses to make the store practically impossible; the loads are
// therefore live and the kernel writes nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ p, uint64_t n16,
                                                   uint32_t* __restrict__ sink, uint32_t magic) {
  uint32_t acc = 0;
  const uint64_t stride = (uint64_t)gridDim.x * 256u;
  uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  for (; i + 7u * stride < n16; i += 8u * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + (uint64_t)u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == magic) sink[0] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16, 16-byte aligned) from device memory `p`
// with `grid` workgroups of 256 threads on `stream`.  sink: one device word.
// Returns 0 when the launch was accepted, 1 on bad arguments, 2 when the
// runtime reported a launch error.
extern "C" int nvfp4_probe_read(const void* p, uint64_t bytes, uint32_t* sink, uint32_t magic, int grid,
                                void* stream) {
  if (!p || !sink || bytes % 16 || ((uintptr_t)p % 16) || grid < 1) return 1;
  read_kernel<<<grid, 256, 0, (hipStream_t)stream>>>((const uint4*)p, bytes / 16, sink, magic);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
