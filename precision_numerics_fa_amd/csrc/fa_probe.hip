// Measured ceilings for the roofline figures: a kernel that does nothing but
// bf16 MFMAs (v_mfma_f32_32x32x16_bf16, the instruction of every product in
// the attention kernels), so that achieved TFLOP/s can be quoted against the
// dense rate this chip sustains under load as well as against its data-sheet
// peak.  Each wave keeps eight independent accumulator chains in flight, two
// waves per SIMD; operands stay in registers, so neither memory nor LDS takes
// part.  The result is written out so that the chains are not removed.
// A second probe reads a buffer through HBM (16-byte loads, four in flight
// per lane) for the read-bandwidth ceiling of the memory-bound kernels, whose
// traffic is almost all reads.  A third measures what the instructions of
// the softmax cost on a SIMD beside MFMA work, and what LDS operand reads
// add (issue_probe_kernel).
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

// Instruction-issue probe: 512-thread workgroups with 96 KB of LDS, so one
// per CU and waves w and w + 4 on the same SIMD; waves numbered `active` and
// up skip the loop (active 4: one wave per SIMD, 8: two).  Per iteration an
// active wave issues, on registers only:
//   kind 0: 8 MFMAs on four accumulators
//   kind 1..5: 64 instructions of one type on eight independent chains:
//     v_fma_f32, v_max3_f32, v_med3_f32, v_exp_f32, v_cvt_pk_bf16_f32
//   kind 6: 8 MFMAs, each followed by 8 v_fma_f32
//   kind 7: waves 0-3 16 MFMAs, waves 4-7 128 v_fma_f32
//   kind 12: 8 MFMAs, each followed by 8 v_exp_f32
//   kind 13: 8 MFMAs, each followed by 8 instructions of the softmax's mix
//     (2 v_exp_f32, 2 v_fma_f32, 2 v_add_f32, 1 v_max3_f32, 1 v_med3_f32)
//   kind 14: 8 MFMAs, each followed by 8 v_max3_f32
//   kind 15: 8 MFMAs, each followed by 8 v_cvt_pk_bf16_f32
//   kind 16: 8 MFMAs, each followed by 8 two-operand v_max_f32
// One float per thread goes to out so that nothing is removed.
template <int KIND>
__global__ __launch_bounds__(512, 1) void issue_probe_kernel(float* __restrict__ out, int iters, int active) {
  __shared__ __attribute__((aligned(16))) float pad[24576];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the first 64 KB hold small bf16 values: the LDS kinds read 16-byte chunks
  // of it (chunk index below 4096)
  for (int i = tid; i < 16384; i += 512) {
    typedef __bf16 two_bf16 __attribute__((ext_vector_type(2)));
    two_bf16 v;
    v[0] = (__bf16)((float)(i & 63) * (1.0f / 256.0f));
    v[1] = (__bf16)((float)(i & 31) * (-1.0f / 256.0f));
    pad[i] = __builtin_bit_cast(float, v);
  }
  __syncthreads();
  const bf16x8* chunks = reinterpret_cast<const bf16x8*>(pad);
  uint32_t xr = 0;
  const float s0 = 1.0f + (float)(tid & 1) * 1e-7f;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(s0 * (float)(i + 1) * (1.0f / 64.0f));
    b[i] = (__bf16)((s0 - (float)i) * (1.0f / 64.0f));
  }
  f32x16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = zero16();
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = s0 * 0.01f * (float)(i + 1) + (float)tid * 1e-6f;
  const float m = 0.999f * s0, c = 1e-3f;
  // (the work of a wave is decided outside its loop, so the loop has no branch)
  auto valu_step = [&](int i) {
    if (KIND == 1 || KIND == 6 || KIND == 7) x[i] = __builtin_fmaf(x[i], m, c);
    if (KIND == 2 || KIND == 14) x[i] = __builtin_fmaxf(x[i], __builtin_fmaxf(x[(i + 1) & 7], c));
    if (KIND == 16) x[i] = __builtin_fmaxf(x[i], x[(i + 1) & 7]);
    if (KIND == 3) x[i] = __builtin_amdgcn_fmed3f(x[i], x[(i + 1) & 7], c);
    if (KIND == 4 || KIND == 12) x[i] = -exp2_fast(x[i]);
    if (KIND == 13) {
      if (i < 2) x[i] = -exp2_fast(x[i]);
      else if (i < 4) x[i] = __builtin_fmaf(x[i], m, c);
      else if (i < 6) x[i] = x[i] + x[(i + 1) & 7];
      else if (i == 6) x[i] = __builtin_fmaxf(x[i], __builtin_fmaxf(x[(i + 1) & 7], c));
      else x[i] = __builtin_amdgcn_fmed3f(x[i], x[(i + 1) & 7], c);
    }
    if (KIND == 5 || KIND == 15) {  // one v_cvt_pk_bf16_f32, its packed bits fed back as a float
      typedef __bf16 two_bf16 __attribute__((ext_vector_type(2)));
      two_bf16 r;
      r[0] = (__bf16)x[i];
      r[1] = (__bf16)x[(i + 2) & 7];
      x[i] = __builtin_bit_cast(float, r);
    }
  };
  if (wave < active) {
    if (KIND == 0) {
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r & 3] = mfma<__bf16>(a, b, acc[r & 3]);
    } else if (KIND == 6 || KIND >= 12) {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          acc[r & 3] = mfma<__bf16>(a, b, acc[r & 3]);
#pragma unroll
          for (int i = 0; i < 8; ++i) valu_step(i);
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
      }
    } else if (KIND == 8) {
      // LDS reads only: 8 ds_read_b128 (1 KB per wave each), folded by XOR
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const uint4 u = __builtin_bit_cast(uint4, chunks[(tid + r * 512 + it * 67) & 4095]);
          xr ^= u.x ^ u.y ^ u.z ^ u.w;
        }
    } else if (KIND == 9) {
      // 8 MFMAs, each with its A operand read from LDS (1 KB per wave)
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int r = 0; r < 8; ++r)
          acc[r & 3] = mfma<__bf16>(chunks[(tid + r * 512 + it * 67) & 4095], b, acc[r & 3]);
    } else if (KIND == 10) {
      // transposing LDS reads only: 16 ds_read_b64_tr_b16 (512 B per wave each)
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const s16x4 u = lds_load_tr4(reinterpret_cast<const bf16_t*>(
              reinterpret_cast<const char*>(pad) + ((tid * 8 + r * 4096 + it * 536) & 65535)));
          xr ^= (uint32_t)(uint16_t)u[0] ^ ((uint32_t)(uint16_t)u[1] << 16) ^ (uint32_t)(uint16_t)u[2] ^
                ((uint32_t)(uint16_t)u[3] << 16);
        }
    } else if (KIND == 11) {
      // 8 MFMAs, each with its A operand from two transposing LDS reads (1 KB)
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const char* base = reinterpret_cast<const char*>(pad);
          const s16x4 lo = lds_load_tr4(reinterpret_cast<const bf16_t*>(base + ((tid * 8 + r * 8192 + it * 536) & 65535)));
          const s16x4 hi = lds_load_tr4(
              reinterpret_cast<const bf16_t*>(base + ((tid * 8 + r * 8192 + 4096 + it * 536) & 65535)));
          acc[r & 3] = mfma<__bf16>(join8(lo, hi), b, acc[r & 3]);
        }
    } else if (KIND == 7) {
      if (wave < 4) {
        for (int it = 0; it < iters; ++it)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r & 3] = mfma<__bf16>(a, b, acc[r & 3]);
      } else {
        for (int it = 0; it < iters; ++it)
#pragma unroll
          for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int i = 0; i < 8; ++i) valu_step(i);
      }
    } else {
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int i = 0; i < 8; ++i) valu_step(i);
    }
  }
  float sum = pad[(tid + 1) & 511];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += acc[t][i];
#pragma unroll
  for (int i = 0; i < 8; ++i) sum += x[i];
  sum += (float)(xr & 255u);
  out[(size_t)blockIdx.x * 512 + tid] = sum;
}

}  // namespace

hipError_t launch_read_probe(const void* src, uint32_t* sink, long long n16, hipStream_t s) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kHbmProbeBlocks), dim3(256), 0, s, (const uint4*)src, sink, n16);
  return hipGetLastError();
}

long long mfma_probe_flop(int blocks, int iters) {
  return (long long)blocks * 4 * iters * kProbeChains * (2LL * 32 * 32 * 16);
}

hipError_t launch_issue_probe(int kind, int active, float* out, int blocks, int iters, hipStream_t s) {
  const dim3 g((unsigned)blocks), t(512);
  switch (kind) {
    case 0: hipLaunchKernelGGL(issue_probe_kernel<0>, g, t, 0, s, out, iters, active); break;
    case 1: hipLaunchKernelGGL(issue_probe_kernel<1>, g, t, 0, s, out, iters, active); break;
    case 2: hipLaunchKernelGGL(issue_probe_kernel<2>, g, t, 0, s, out, iters, active); break;
    case 3: hipLaunchKernelGGL(issue_probe_kernel<3>, g, t, 0, s, out, iters, active); break;
    case 4: hipLaunchKernelGGL(issue_probe_kernel<4>, g, t, 0, s, out, iters, active); break;
    case 5: hipLaunchKernelGGL(issue_probe_kernel<5>, g, t, 0, s, out, iters, active); break;
    case 6: hipLaunchKernelGGL(issue_probe_kernel<6>, g, t, 0, s, out, iters, active); break;
    case 7: hipLaunchKernelGGL(issue_probe_kernel<7>, g, t, 0, s, out, iters, active); break;
    case 8: hipLaunchKernelGGL(issue_probe_kernel<8>, g, t, 0, s, out, iters, active); break;
    case 9: hipLaunchKernelGGL(issue_probe_kernel<9>, g, t, 0, s, out, iters, active); break;
    case 10: hipLaunchKernelGGL(issue_probe_kernel<10>, g, t, 0, s, out, iters, active); break;
    case 11: hipLaunchKernelGGL(issue_probe_kernel<11>, g, t, 0, s, out, iters, active); break;
    case 12: hipLaunchKernelGGL(issue_probe_kernel<12>, g, t, 0, s, out, iters, active); break;
    case 13: hipLaunchKernelGGL(issue_probe_kernel<13>, g, t, 0, s, out, iters, active); break;
    case 14: hipLaunchKernelGGL(issue_probe_kernel<14>, g, t, 0, s, out, iters, active); break;
    case 15: hipLaunchKernelGGL(issue_probe_kernel<15>, g, t, 0, s, out, iters, active); break;
    default: hipLaunchKernelGGL(issue_probe_kernel<16>, g, t, 0, s, out, iters, active); break;
  }
  return hipGetLastError();
}

hipError_t launch_mfma_probe(float* out, int blocks, int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, s, out, iters);
  return hipGetLastError();
}

}  // namespace fa
