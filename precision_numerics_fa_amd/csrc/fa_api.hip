// C ABI of the attention library (declared in include/fa.h): argument
// validation, device check, and dispatch to the kernel launchers.  Nothing
// here allocates or keeps per-call state; the only cached state is a per-device
// "is this a gfx950" flag, written with relaxed atomics (idempotent).
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "fa.h"
#include "fa_device.hpp"
#include "fa_launch.hpp"

// Scratch of fa_bwd_noalloc: the D vector, one fixed array per device.  The
// name is only a host-side handle; the device address is looked up once per
// device (with that device current) and cached, and only that address is
// ever handed to a kernel.
static __device__ __align__(256) float scratch[FA_BWD_NOALLOC_MAX_ROWS];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int known = g_device_ok[dev].load(std::memory_order_relaxed);
    if (known != 0) return known > 0 ? FA_OK : FA_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_device_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
  return ok ? FA_OK : FA_ERR_DEVICE;
}

bool aligned(const void* p, size_t a) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const long double elems = (long double)B * H * N * d;
  if (elems >= (long double)(1ULL << 40)) return FA_ERR_INVALID_ARG;
  // grid sizes (B*H*ceil(N/64)) must fit a 32-bit launch dimension
  if ((long double)B * H * ((N + 63) / 64) >= 2147483647.0L) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int check_scale(float scale) { return (std::isfinite(scale) && scale > 0.0f) ? FA_OK : FA_ERR_INVALID_ARG; }

int launched(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

int check_dtype(int dtype) { return (dtype == FA_BF16 || dtype == FA_F16) ? FA_OK : FA_ERR_UNSUPPORTED; }

int fwd_impl(int dtype, const void* Q, const void* K, const void* V, void* O, float* LSE, unsigned char* flags,
             int B, int H, int N, int d, int causal, float scale, int stabilize, void* stream) {
  int st = check_dtype(dtype);
  if (st != FA_OK) return st;
  if ((st = check_shape(B, H, N, d)) != FA_OK) return st;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(LSE, 4))
    return FA_ERR_INVALID_ARG;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if ((st = check_device()) != FA_OK) return st;
  fa::FwdArgs a{Q, K, V, O, LSE, flags, B, H, N, d, causal != 0, stabilize != 0, scale,
                dtype == FA_F16 ? fa::kF16 : fa::kBF16};
  (void)hipGetLastError();  // clear a stale error so a failure below is ours
  return launched(fa::launch_fwd(a, static_cast<hipStream_t>(stream)));
}

int bwd_args(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
             const float* Dvec, int B, int H, int N, int d, float scale) {
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(dO, 16) || !aligned(LSE, 4) ||
      !aligned(Dvec, 4))
    return FA_ERR_INVALID_ARG;
  return check_scale(scale);
}

int bwd_impl(int dtype, const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* LSE, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes, int B, int H,
             int N, int d, int causal, float scale, int stabilize, void* stream) {
  (void)stabilize;  // the backward recomputes P from LSE; the shift has no influence on it
  int st = check_dtype(dtype);
  if (st != FA_OK) return st;
  if ((st = check_shape(B, H, N, d)) != FA_OK) return st;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(dO, 16) ||
      !aligned(LSE, 4) || !aligned(dQ, 16) || !aligned(dK, 16) || !aligned(dV, 16))
    return FA_ERR_INVALID_ARG;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (workspace == nullptr || !aligned(workspace, 4) ||
      workspace_bytes < fa_bwd_workspace_bytes(B, H, N, d, causal))
    return FA_ERR_WORKSPACE;
  if ((st = check_device()) != FA_OK) return st;
  float* Dvec = static_cast<float*>(workspace);
  fa::BwdArgs a{Q, K, V, O, dO, LSE, Dvec, dQ, dK, dV, B, H, N, d, causal != 0, scale,
                dtype == FA_F16 ? fa::kF16 : fa::kBF16};
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if ((st = launched(fa::launch_bwd_dot(a, s))) != FA_OK) return st;
  return launched(fa::launch_bwd_grads(a, s));
}

std::atomic<float*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_DEVICE;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* a = nullptr;
      if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || a == nullptr) return FA_ERR_DEVICE;
      p = static_cast<float*>(a);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FA_OK;
}

// The baseline's extra limits: rows of at most kBaseMaxN keys (its softmax
// holds a row in registers) and one softmax workgroup per row.
int check_base_shape(int B, int H, int N, int d) {
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (N > fa::kBaseMaxN) return FA_ERR_UNSUPPORTED;
  if ((long double)B * H * N >= 2147483647.0L) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

size_t base_matrix_elems(int B, int H, int N) { return (size_t)B * H * N * (size_t)fa::base_ld(N); }

size_t base_p_offset(int B, int H, int N) {
  return (base_matrix_elems(B, H, N) * sizeof(float) + 255) & ~(size_t)255;
}

fa::BaseArgs base_args(const void* Q, const void* K, const void* V, void* O, float* LSE, float* S, void* P, int B,
                       int H, int N, int d, int causal, float scale) {
  return fa::BaseArgs{Q, K, V, O, LSE, S, P, B, H, N, d, fa::base_ld(N), causal != 0, scale};
}

// Workspace of fa_fwd_split: O_bar (splits, B*H, N, d) fp32, then l and M
// (splits, B*H, N) fp32 each, every part at a 256-byte boundary.
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t split_obar_bytes(int splits, int B, int H, int N, int d) {
  return round256((size_t)splits * B * H * N * d * sizeof(float));
}
size_t split_vec_bytes(int splits, int B, int H, int N) { return round256((size_t)splits * B * H * N * sizeof(float)); }

int check_splits(int splits, int B, int H, int N) {
  if (splits < 1 || splits > fa::kMaxSplits) return FA_ERR_INVALID_ARG;
  const long long n_qblk = (N + fa::kFwdBlockQ - 1) / fa::kFwdBlockQ;
  if ((long double)B * H * n_qblk * splits >= 2147483647.0L) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N, int d,
           int causal, float scale, int stabilize, void* stream) {
  return fwd_impl(FA_BF16, Q, K, V, O, LSE, nullptr, B, H, N, d, causal, scale, stabilize, stream);
}

int fa_fwd_diag(const void* Q, const void* K, const void* V, void* O, float* LSE, unsigned char* row_shifted,
                int B, int H, int N, int d, int causal, float scale, int stabilize, void* stream) {
  if (row_shifted == nullptr) return FA_ERR_INVALID_ARG;
  return fwd_impl(FA_BF16, Q, K, V, O, LSE, row_shifted, B, H, N, d, causal, scale, stabilize, stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int causal) {
  (void)causal;
  if (check_shape(B, H, N, d) != FA_OK) return 0;
  const size_t bytes = (size_t)B * H * N * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

int fa_bwd_dot(const void* O, const void* dO, float* Dvec, int B, int H, int N, int d, void* stream) {
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned(O, 16) || !aligned(dO, 16) || !aligned(Dvec, 4)) return FA_ERR_INVALID_ARG;
  if ((st = check_device()) != FA_OK) return st;
  fa::BwdArgs a{};
  a.o = O;
  a.dout = dO;
  a.dvec = Dvec;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  (void)hipGetLastError();
  return launched(fa::launch_bwd_dot(a, static_cast<hipStream_t>(stream)));
}

int fa_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                const float* Dvec, void* dK, void* dV, int B, int H, int N, int d, int causal, float scale,
                void* stream) {
  int st = bwd_args(Q, K, V, dO, LSE, Dvec, B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (!aligned(dK, 16) || !aligned(dV, 16)) return FA_ERR_INVALID_ARG;
  if ((st = check_device()) != FA_OK) return st;
  fa::BwdArgs a{Q, K, V, nullptr, dO, LSE, const_cast<float*>(Dvec), nullptr, dK, dV, B, H, N, d, causal != 0, scale};
  (void)hipGetLastError();
  return launched(fa::launch_bwd_dkdv(a, static_cast<hipStream_t>(stream)));
}

int fa_bwd_dq(const void* Q, const void* K, const void* V, const void* dO, const float* LSE, const float* Dvec,
              void* dQ, int B, int H, int N, int d, int causal, float scale, void* stream) {
  int st = bwd_args(Q, K, V, dO, LSE, Dvec, B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (!aligned(dQ, 16)) return FA_ERR_INVALID_ARG;
  if ((st = check_device()) != FA_OK) return st;
  fa::BwdArgs a{Q, K, V, nullptr, dO, LSE, const_cast<float*>(Dvec), dQ, nullptr, nullptr, B, H, N, d, causal != 0, scale};
  (void)hipGetLastError();
  return launched(fa::launch_bwd_dq(a, static_cast<hipStream_t>(stream)));
}

int fa_bwd_grads(const void* Q, const void* K, const void* V, const void* dO, const float* LSE, const float* Dvec,
                 void* dQ, void* dK, void* dV, int B, int H, int N, int d, int causal, float scale, void* stream) {
  int st = bwd_args(Q, K, V, dO, LSE, Dvec, B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (!aligned(dQ, 16) || !aligned(dK, 16) || !aligned(dV, 16)) return FA_ERR_INVALID_ARG;
  if ((st = check_device()) != FA_OK) return st;
  fa::BwdArgs a{Q, K, V, nullptr, dO, LSE, const_cast<float*>(Dvec), dQ, dK, dV, B, H, N, d, causal != 0, scale};
  (void)hipGetLastError();
  return launched(fa::launch_bwd_grads(a, static_cast<hipStream_t>(stream)));
}

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE, void* dQ,
           void* dK, void* dV, void* workspace, size_t workspace_bytes, int B, int H, int N, int d, int causal,
           float scale, int stabilize, void* stream) {
  return bwd_impl(FA_BF16, Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes, B, H, N, d, causal, scale,
                  stabilize, stream);
}

int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                   void* dQ, void* dK, void* dV, int B, int H, int N, int d, int causal, float scale, int stabilize,
                   void* stream) {
  (void)stabilize;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if ((long double)B * H * N > (long double)FA_BWD_NOALLOC_MAX_ROWS) return FA_ERR_TOO_LARGE;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(dO, 16) ||
      !aligned(LSE, 4) || !aligned(dQ, 16) || !aligned(dK, 16) || !aligned(dV, 16))
    return FA_ERR_INVALID_ARG;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if ((st = check_device()) != FA_OK) return st;
  float* Dvec = nullptr;
  if ((st = scratch_address(&Dvec)) != FA_OK) return st;
  // D is written in full by the row-dot launch before the gradient launch
  // reads it, so nothing in the scratch needs clearing between calls
  fa::BwdArgs a{Q, K, V, O, dO, LSE, Dvec, dQ, dK, dV, B, H, N, d, causal != 0, scale, fa::kBF16};
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if ((st = launched(fa::launch_bwd_dot(a, s))) != FA_OK) return st;
  return launched(fa::launch_bwd_grads(a, s));
}

int fa_fwd_ex(int dtype, const void* Q, const void* K, const void* V, void* O, float* LSE,
              unsigned char* row_shifted, int B, int H, int N, int d, int causal, float scale, int stabilize,
              void* stream) {
  return fwd_impl(dtype, Q, K, V, O, LSE, row_shifted, B, H, N, d, causal, scale, stabilize, stream);
}

int fa_bwd_ex(int dtype, const void* Q, const void* K, const void* V, const void* O, const void* dO,
              const float* LSE, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes, int B, int H,
              int N, int d, int causal, float scale, int stabilize, void* stream) {
  return bwd_impl(dtype, Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes, B, H, N, d, causal, scale,
                  stabilize, stream);
}

size_t fa_fwd_split_workspace_bytes(int B, int H, int N, int d, int splits) {
  if (check_shape(B, H, N, d) != FA_OK || check_splits(splits, B, H, N) != FA_OK) return 0;
  return split_obar_bytes(splits, B, H, N, d) + 2 * split_vec_bytes(splits, B, H, N);
}

int fa_fwd_split(const void* Q, const void* K, const void* V, void* O, float* LSE, int splits, void* workspace,
                 size_t workspace_bytes, int B, int H, int N, int d, int causal, float scale, int stabilize,
                 void* stream) {
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if ((st = check_splits(splits, B, H, N)) != FA_OK) return st;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(LSE, 4))
    return FA_ERR_INVALID_ARG;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (workspace == nullptr || !aligned(workspace, 256) ||
      workspace_bytes < fa_fwd_split_workspace_bytes(B, H, N, d, splits))
    return FA_ERR_WORKSPACE;
  if ((st = check_device()) != FA_OK) return st;
  char* w = static_cast<char*>(workspace);
  const size_t ob = split_obar_bytes(splits, B, H, N, d), vb = split_vec_bytes(splits, B, H, N);
  fa::SplitArgs sa{reinterpret_cast<float*>(w), reinterpret_cast<float*>(w + ob),
                   reinterpret_cast<float*>(w + ob + vb), splits};
  fa::FwdArgs a{Q, K, V, O, LSE, nullptr, B, H, N, d, causal != 0, stabilize != 0, scale, fa::kBF16};
  (void)hipGetLastError();
  return launched(fa::launch_fwd_split(a, sa, static_cast<hipStream_t>(stream)));
}

int fa_base_ld(int N) { return N < 1 ? 0 : fa::base_ld(N); }

size_t fa_base_workspace_bytes(int B, int H, int N, int d, int causal) {
  (void)causal;
  if (check_base_shape(B, H, N, d) != FA_OK) return 0;
  const size_t bytes = base_p_offset(B, H, N) + base_matrix_elems(B, H, N) * 2;
  return (bytes + 255) & ~(size_t)255;
}

int fa_base_scores(const void* Q, const void* K, float* S, int B, int H, int N, int d, int causal, float scale,
                   void* stream) {
  int st = check_base_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(S, 16)) return FA_ERR_INVALID_ARG;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if ((st = check_device()) != FA_OK) return st;
  const fa::BaseArgs a = base_args(Q, K, nullptr, nullptr, nullptr, S, nullptr, B, H, N, d, causal, scale);
  (void)hipGetLastError();
  return launched(fa::launch_base_scores(a, static_cast<hipStream_t>(stream)));
}

int fa_base_softmax(const float* S, void* P, float* LSE, int B, int H, int N, int causal, void* stream) {
  int st = check_base_shape(B, H, N, 64);
  if (st != FA_OK) return st;
  if (!aligned(S, 16) || !aligned(P, 16) || !aligned(LSE, 4)) return FA_ERR_INVALID_ARG;
  if ((st = check_device()) != FA_OK) return st;
  const fa::BaseArgs a =
      base_args(nullptr, nullptr, nullptr, nullptr, LSE, const_cast<float*>(S), P, B, H, N, 64, causal, 1.0f);
  (void)hipGetLastError();
  return launched(fa::launch_base_softmax(a, static_cast<hipStream_t>(stream)));
}

int fa_base_pv(const void* P, const void* V, void* O, int B, int H, int N, int d, int causal, void* stream) {
  int st = check_base_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned(P, 16) || !aligned(V, 16) || !aligned(O, 16)) return FA_ERR_INVALID_ARG;
  if ((st = check_device()) != FA_OK) return st;
  const fa::BaseArgs a =
      base_args(nullptr, nullptr, V, O, nullptr, nullptr, const_cast<void*>(P), B, H, N, d, causal, 1.0f);
  (void)hipGetLastError();
  return launched(fa::launch_base_pv(a, static_cast<hipStream_t>(stream)));
}

int fa_base_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, void* workspace,
                size_t workspace_bytes, int B, int H, int N, int d, int causal, float scale, void* stream) {
  int st = check_base_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(LSE, 4))
    return FA_ERR_INVALID_ARG;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (workspace == nullptr || !aligned(workspace, 256) ||
      workspace_bytes < fa_base_workspace_bytes(B, H, N, d, causal))
    return FA_ERR_WORKSPACE;
  if ((st = check_device()) != FA_OK) return st;
  float* S = static_cast<float*>(workspace);
  void* P = static_cast<char*>(workspace) + base_p_offset(B, H, N);
  const fa::BaseArgs a = base_args(Q, K, V, O, LSE, S, P, B, H, N, d, causal, scale);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if ((st = launched(fa::launch_base_scores(a, s))) != FA_OK) return st;
  if ((st = launched(fa::launch_base_softmax(a, s))) != FA_OK) return st;
  return launched(fa::launch_base_pv(a, s));
}

long long fa_mfma_probe(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || !aligned(out, 4) || blocks < 1 || iters < 1 || blocks > (1 << 24)) return FA_ERR_INVALID_ARG;
  const int st = check_device();
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  const int ls = launched(fa::launch_mfma_probe(out, blocks, iters, static_cast<hipStream_t>(stream)));
  return ls != FA_OK ? ls : fa::mfma_probe_flop(blocks, iters);
}

int fa_issue_probe(int kind, int waves_per_simd, float* out, int blocks, int iters, void* stream) {
  if (kind < 0 || kind > 16 || (waves_per_simd != 1 && waves_per_simd != 2) || (kind == 7 && waves_per_simd != 2) ||
      out == nullptr || !aligned(out, 4) || blocks < 1 || blocks > (1 << 20) || iters < 1)
    return FA_ERR_INVALID_ARG;
  const int st = check_device();
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  return launched(fa::launch_issue_probe(kind, 4 * waves_per_simd, out, blocks, iters, static_cast<hipStream_t>(stream)));
}

int fa_hbm_probe(const void* src, size_t bytes, unsigned int* sink, void* stream) {
  if (!aligned(src, 16) || !aligned(sink, 4) || bytes == 0 || bytes % 16 != 0) return FA_ERR_INVALID_ARG;
  const int st = check_device();
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  return launched(fa::launch_read_probe(src, sink, (long long)(bytes / 16), static_cast<hipStream_t>(stream)));
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size, or bad scale)";
    case FA_ERR_UNSUPPORTED: return "unsupported shape (d must be 64 or 128; the baseline takes N <= 16384)";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than fa_bwd_workspace_bytes()";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_DEVICE: return "current device is not a gfx950 GPU, or a device query failed";
    case FA_ERR_TOO_LARGE: return "B*H*N exceeds the allocation-free backward's scratch (FA_BWD_NOALLOC_MAX_ROWS)";
    default: return "unknown status";
  }
}

void fa_stabilize_params(float* delta_min, float* delta_max, float* fold) {
  if (delta_min) *delta_min = fa::kDeltaMin;
  if (delta_max) *delta_max = fa::kDeltaMax;
  if (fold) *fold = fa::kFold;
}

int fa_stabilize_params_ex(int dtype, float* delta_min, float* delta_max, float* fold) {
  if (check_dtype(dtype) != FA_OK) return FA_ERR_UNSUPPORTED;
  const bool h = dtype == FA_F16;
  if (delta_min) *delta_min = fa::kDeltaMin;
  if (delta_max) *delta_max = h ? fa::kF16DeltaMax : fa::kDeltaMax;
  if (fold) *fold = h ? fa::kF16Fold : fa::kFold;
  return FA_OK;
}

void fa_fwd_tile(int d, int* block_q, int* block_k) {
  const bool ok = d == 64 || d == 128;
  if (block_q) *block_q = ok ? fa::kFwdBlockQ : 0;
  if (block_k) *block_k = ok ? fa::fwd_block_k(d) : 0;
}

int fa_version(void) { return 300; }

}  // extern "C"
