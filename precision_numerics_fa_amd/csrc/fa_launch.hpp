// Host-side launchers of the HIP kernels.  Arguments are assumed validated
// by the C ABI layer (fa_api.hip); each launcher only sizes the grid and
// enqueues on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Element type of the 16-bit tensors (the values of fa_dtype in fa.h).
constexpr int kBF16 = 0;
constexpr int kF16 = 1;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  uint8_t* row_shifted;  // may be null (then no per-row report is written)
  int B, H, N, d;
  bool causal;
  bool stabilize;
  float scale;
  int dtype;  // kBF16 or kF16
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* dvec;
  void* dq;
  void* dk;
  void* dv;
  int B, H, N, d;
  bool causal;
  float scale;
  int dtype;  // kBF16 or kF16
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

// The split-key forward (bf16): partial results of `splits` key ranges in
// caller-supplied fp32 buffers, then a merge kernel writes O and LSE.
struct SplitArgs {
  float* obar;  // (splits, B*H, N, d)
  float* lrow;  // (splits, B*H, N)
  float* mrow;  // (splits, B*H, N)
  int splits;
};
constexpr int kMaxSplits = 64;
hipError_t launch_fwd_split(const FwdArgs& a, const SplitArgs& sa, hipStream_t stream);
hipError_t launch_bwd_dot(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
// dK, dV and dQ in one launch (the two kernels above, fused horizontally)
hipError_t launch_bwd_grads(const BwdArgs& a, hipStream_t stream);

// scale * log2(e), rounded once to fp32 (the factor that folds the softmax
// scale into the base-2 exponent).
float scale_log2e(float scale);

// The unfused baseline attention (fa_base.hip): the FP32 score matrix S and
// the BF16 probability matrix P are (B, H, N, ld) with ld = base_ld(N).
struct BaseArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* s;
  void* p;
  int B, H, N, d, ld;
  bool causal;
  float scale;
};

// Longest row the baseline's softmax keeps in registers (keys per row).
constexpr int kBaseMaxN = 16384;

int base_ld(int N);
hipError_t launch_base_scores(const BaseArgs& a, hipStream_t stream);
hipError_t launch_base_softmax(const BaseArgs& a, hipStream_t stream);
hipError_t launch_base_pv(const BaseArgs& a, hipStream_t stream);

// The bf16 MFMA throughput probe (fa_probe.hip): FLOP done by one launch of
// `blocks` workgroups of `iters` iterations, and the launch.
long long mfma_probe_flop(int blocks, int iters);
hipError_t launch_mfma_probe(float* out, int blocks, int iters, hipStream_t stream);
hipError_t launch_issue_probe(int kind, int active, float* out, int blocks, int iters, hipStream_t stream);
// The HBM read-bandwidth probe: reads n16 16-byte units of src; one folded
// value per thread goes to sink (kHbmProbeBlocks * 256 of them).
constexpr int kHbmProbeBlocks = 4096;
hipError_t launch_read_probe(const void* src, uint32_t* sink, long long n16, hipStream_t stream);

constexpr int kFwdBlockQ = 128;
// Keys per block of the forward (both head sizes): one K and one V tile of
// 128 keys; the running maximum and repeated-maximum bookkeeping advance a
// block at a time.
constexpr int fwd_block_k(int d) { return d == 64 || d == 128 ? 128 : 0; }

}  // namespace fa
