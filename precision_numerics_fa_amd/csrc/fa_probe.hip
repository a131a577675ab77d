// Measured ceilings for the roofline figures: a kernel that does nothing but
// bf16 MFMAs (v_mfma_f32_32x32x16_bf16, the instruction of every product in
// the attention kernels), so that achieved TFLOP/s can be quoted against the
// dense rate this chip sustains under load as well as against its data-sheet
// peak.  Each wave keeps eight independent accumulator chains in flight, two
// waves per SIMD; operands stay in registers, so neither memory nor LDS takes
// part.  The result is written out so that the chains are not removed.
// A second probe reads a buffer through HBM (16-byte loads, four in flight
// per lane) for the read-bandwidth ceiling of the memory-bound kernels, whose
// traffic is almost all reads.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kProbeChains = 8;

__global__ __launch_bounds__(256, 2) void mfma_probe_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)((float)((lane + j) & 7) * (1.0f / 1024.0f));
    b[j] = (__bf16)((float)((lane * 3 + j) & 7) * (1.0f / 1024.0f));
  }
  f32x16 c[kProbeChains];
#pragma unroll
  for (int t = 0; t < kProbeChains; ++t) c[t] = zero16();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int t = 0; t < kProbeChains; ++t) c[t] = mfma<__bf16>(a, b, c[t]);
  }
  float s = 0.0f;
#pragma unroll
  for (int t = 0; t < kProbeChains; ++t) s += c[t][t];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Reads src[0 .. n16) (16-byte units): each workgroup streams one
// contiguous slice, 16 KB per step (four 16-byte loads in flight per lane),
// and each lane folds its words into one value (written to sink[thread]) so
// that the loads are kept.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, uint32_t* __restrict__ sink,
                                                         long long n16) {
  const long long chunk = (n16 + gridDim.x - 1) / gridDim.x;
  const long long begin = (long long)blockIdx.x * chunk;
  const long long end = min(n16, begin + chunk);
  long long i = begin + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 768 < end; i += 1024) {
    const uint4 a = src[i], b = src[i + 256], c = src[i + 512], d = src[i + 768];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < end; i += 256) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* src, uint32_t* sink, long long n16, hipStream_t s) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kHbmProbeBlocks), dim3(256), 0, s, (const uint4*)src, sink, n16);
  return hipGetLastError();
}

long long mfma_probe_flop(int blocks, int iters) {
  return (long long)blocks * 4 * iters * kProbeChains * (2LL * 32 * 32 * 16);
}

hipError_t launch_mfma_probe(float* out, int blocks, int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, s, out, iters);
  return hipGetLastError();
}

}  // namespace fa
