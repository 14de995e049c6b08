// Streaming-read probe: the practical HBM read bandwidth of this device, the
// floor a bandwidth-bound kernel of the step is compared with. Not part of
// the step; the benchmark calls it.
//
// A grid of workgroups of 256 threads strides over the buffer with 16-byte
// loads (each wave reads 1 KiB contiguous per load) and writes its fp32 sum to
// one sink word, so nothing is optimized away.

#include "dsa_kernels.h"

namespace dsa {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const float4* __restrict__ src,
                                                                   long long n16,
                                                                   float* __restrict__ sink) {
  float acc = 0.0f;
  const long long stride = (long long)gridDim.x * kProbeThreads;
  for (long long i = (long long)blockIdx.x * kProbeThreads + threadIdx.x; i < n16; i += stride) {
    const float4 v = src[i];
    acc += (v.x + v.y) + (v.z + v.w);
  }
  __shared__ float part[kProbeThreads / 64];
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
    for (int w = 0; w < kProbeThreads / 64; ++w) t += part[w];
    sink[blockIdx.x] = t;
  }
}

hipError_t launch_read_probe(const void* src, long long bytes, float* sink, int blocks,
                             hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(kProbeThreads), 0, stream,
                     static_cast<const float4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace dsa
