// Unfused baseline attention with FP32 accumulation, for gfx950 (MI355X).
//
// Page 3 ("What did Meta's study find") measures FlashAttention's numeric
// deviation against a baseline attention that accumulates in FP32, in an
// isolated BF16 forward pass.  This file is that baseline, so that the two
// can be compared on the same inputs and the same device.  The steps are the
// plain definition, one kernel each, with the score and probability matrices
// materialised in HBM:
//
//   base_scores_kernel   S = fl32(fl32(Q K^T) * scale), FP32, (B,H,N,ld)
//   base_softmax_kernel  r = row max, e = 2^((S - r) log2 e), l = sum e (FP32),
//                        P = bf16(e * (1/l)), LSE = r + ln l
//   base_pv_kernel       O = bf16(P V), FP32 accumulation
//
// The only difference in rounding from the FlashAttention kernels is where
// the probabilities meet BF16: here they are normalised first (one maximum
// over the whole row, no rescaling), there the unnormalised block values
// are cast and the output is divided by the FP32 row sum at the end.
//
// Layout: S and P rows have a stride of ld = N rounded up to 64, so that
// every 64-key block of a row is 16-byte aligned.  For causal attention only
// the key blocks up to the diagonal are computed and read.  The softmax
// writes P for every key the PV kernel reads (zeros past the row's last
// visible key), so the PV kernel needs no mask.
//
// All three are bound by HBM traffic (the N x N matrices), not by the MFMAs;
// the contractions still run on v_mfma_f32_32x32x16_bf16 with the operand
// layouts of the FlashAttention forward.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBaseBQ = 128;  // query rows per workgroup (4 waves x 32)
constexpr int kBaseBK = 64;   // keys per block

// Workgroup -> (head, query block).  The hardware hands workgroup i to XCD
// i % 8; with `remap` each XCD gets a contiguous group of G heads, walked
// head-major with the heaviest causal block first, so that a head's K (or V)
// stays in that XCD's L2 while the N x N matrix streams past it.  Returns
// false for the padding workgroups of the last group.
__device__ __forceinline__ bool base_block(int n_qblk, int total, int remap, int BH, int G, int& bh, int& qb) {
  int bid = blockIdx.x;
  if (remap) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int per_group = G * n_qblk;
  const int g = bid / per_group;
  const int r = bid - g * per_group;
  bh = g * G + r / n_qblk;
  qb = n_qblk - 1 - r % n_qblk;
  return bh < BH;
}

struct BaseGrid {
  int n_qblk, total, remap, BH, G;
};

BaseGrid base_grid(const BaseArgs& a) {
  BaseGrid g;
  g.n_qblk = (a.N + kBaseBQ - 1) / kBaseBQ;
  g.BH = a.B * a.H;
  g.G = (g.BH + 7) / 8;
  g.total = (g.BH + g.G - 1) / g.G * g.G * g.n_qblk;
  g.remap = g.total % 8 == 0 ? 1 : 0;
  return g;
}

// ---------------------------------------------------------------- S = scale * Q K^T
// S = Q K^T on MFMA with the wave's Q rows as A operands (registers) and K
// rows from a swizzled LDS tile as B operands: lane l holds key l % 32 of a
// 32-key subtile and query rows 8 (i/4) + 4 (l/32) + i%4, so each store
// instruction writes two 128-byte row segments.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void base_scores_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                                                          float* __restrict__ S, int N, int ld, BaseGrid grid,
                                                          float scale) {
  constexpr int TILE = kBaseBK * D;
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * TILE];
  int bh, qb;
  if (!base_block(grid.n_qblk, grid.total, grid.remap, grid.BH, grid.G, bh, qb)) return;
  const int q0 = qb * kBaseBQ;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const bf16_t* Kh = K + hoff;
  float* Sh = S + (size_t)bh * (size_t)N * ld;

  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + l32;
  const bool wave_live = qw0 < N;
  const int last_row = min(q0 + kBaseBQ, N) - 1;
  const int n_kblk = CAUSAL ? (last_row / kBaseBK + 1) : (N + kBaseBK - 1) / kBaseBK;
  const int n_wave = !wave_live ? 0 : (CAUSAL ? min(n_kblk, min(qw0 + 31, N - 1) / kBaseBK + 1) : n_kblk);

  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (myq < N) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(Q + hoff + (size_t)myq * D + kk * 16 + hi * 8);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[kk][j] = (__bf16)0.0f;
    }
  }
  const uint32_t kx0 = 2u * (uint32_t)tile_off<D>(l32, hi * 8);
  int ldoff[kBaseBK * D / 8 / 256];
  tile_offsets<D, kBaseBK, 256>(ldoff, wave, lane);

  load_tile_async<D, kBaseBK, 256>(ldoff, Kh, 0, N, smem, wave, lane);
  wait_vmem();
  wait_vmem_tracked();
  zero_tail<D, kBaseBK, 256>(0, N, smem, wave, lane);
  __syncthreads();

  for (int j = 0; j < n_kblk; ++j) {
    bf16_t* const next = smem + ((j + 1) & 1) * TILE;
    if (j + 1 < n_kblk) load_tile_async<D, kBaseBK, 256>(ldoff, Kh, (j + 1) * kBaseBK, N, next, wave, lane);
    if (j < n_wave) {
      const bf16_t* Ks = smem + (j & 1) * TILE;
      const uint32_t kx = (uint32_t)opaque((int)kx0);
#pragma unroll
      for (int t = 0; t < kBaseBK / 32; ++t) {
        f32x16 s = zero16();
        const char* base = reinterpret_cast<const char*>(Ks + t * 32 * D);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          s = mfma<__bf16>(qf[kk], lds_load8(reinterpret_cast<const bf16_t*>(base + (kx ^ (uint32_t)(kk << 5)))),
                           s);
        const int key = j * kBaseBK + t * 32 + l32;
        if (key < N) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int q = qw0 + 8 * (i >> 2) + 4 * hi + (i & 3);
            if (q < N) Sh[(size_t)q * ld + key] = s[i] * scale;
          }
        }
      }
    }
    wait_vmem();
    if (j + 1 < n_kblk) zero_tail<D, kBaseBK, 256>((j + 1) * kBaseBK, N, next, wave, lane);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- row softmax
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = __builtin_fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Row softmax.  A team of WPR waves owns a row: one wave per row (four rows
// per workgroup) when rows are at most kBaseWaveRow keys, else the whole
// workgroup.  The row's visible scores are read once into registers, 4 per
// chunk; chunks past the row's end are skipped by team-uniform branches.  The
// maximum and the sum are reduced within each wave and, for a workgroup team,
// over its four waves in a fixed order, so the result does not depend on
// timing.
constexpr int kBaseWaveRow = 4096;

template <bool CAUSAL, int WPR>
__global__ __launch_bounds__(256) void base_softmax_kernel(const float* __restrict__ S, bf16_t* __restrict__ P,
                                                           float* __restrict__ LSE, int N, int ld, long long rows) {
  constexpr int TEAM = 64 * WPR;                     // threads per row
  constexpr int CH = (WPR == 1 ? kBaseWaveRow : kBaseMaxN) / (4 * TEAM);  // float4 chunks per thread
  __shared__ float red[2][4];
  const int tid = threadIdx.x, wave = tid >> 6;
  const long long row = WPR == 1 ? (long long)blockIdx.x * 4 + wave : (long long)blockIdx.x;  // (b*H + h)*N + i
  if (WPR == 1 && row >= rows) return;              // a whole wave; this variant has no barrier
  const int t = WPR == 1 ? (tid & 63) : tid;
  const int i = (int)(row % N);
  const int L = CAUSAL ? i + 1 : N;                                            // visible keys
  const int W = CAUSAL ? min(ld, kBaseBK * (i / kBaseBK + 1)) : ld;           // keys the PV kernel reads
  const float* Srow = S + row * ld;
  bf16_t* Prow = P + row * ld;

  float4 x[CH];
  float mx = kNegInf;
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    x[u] = make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
    if (4 * TEAM * u < L) {
      const int j = 4 * (t + TEAM * u);
      if (j < L) {
        x[u] = *reinterpret_cast<const float4*>(Srow + j);
        if (j + 1 >= L) x[u].y = kNegInf;
        if (j + 2 >= L) x[u].z = kNegInf;
        if (j + 3 >= L) x[u].w = kNegInf;
      }
      mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fmaxf(x[u].x, x[u].y), __builtin_fmaxf(x[u].z, x[u].w)));
    }
  }
  mx = wave_max(mx);
  float r = mx;
  if (WPR == 4) {
    if ((tid & 63) == 0) red[0][wave] = mx;
    __syncthreads();
    r = __builtin_fmaxf(__builtin_fmaxf(red[0][0], red[0][1]), __builtin_fmaxf(red[0][2], red[0][3]));
  }

  float sum = 0.0f;
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    if (4 * TEAM * u < L) {
      x[u].x = exp2_fast((x[u].x - r) * kLog2e);  // masked: exp2(-inf) = 0
      x[u].y = exp2_fast((x[u].y - r) * kLog2e);
      x[u].z = exp2_fast((x[u].z - r) * kLog2e);
      x[u].w = exp2_fast((x[u].w - r) * kLog2e);
      sum += x[u].x;
      sum += x[u].y;
      sum += x[u].z;
      sum += x[u].w;
    } else {
      x[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  }
  sum = wave_sum(sum);
  float l = sum;
  if (WPR == 4) {
    if ((tid & 63) == 0) red[1][wave] = sum;
    __syncthreads();
    l = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
  }
  const float inv = 1.0f / l;

#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const int j = 4 * (t + TEAM * u);
    if (4 * TEAM * u < W && j < W) {
      uint2 w;
      w.x = pack2<__bf16>(x[u].x * inv, x[u].y * inv);
      w.y = pack2<__bf16>(x[u].z * inv, x[u].w * inv);
      *reinterpret_cast<uint2*>(Prow + j) = w;
    }
  }
  if (t == 0) LSE[row] = r + __builtin_log2f(l) * kLn2;
}

// ---------------------------------------------------------------- O = P V
// O^T = V^T P^T as in the FlashAttention forward: V^T through the
// transposing LDS read of a swizzled V tile (A operand), the workgroup's 128
// rows of P for the block copied straight from HBM into a swizzled LDS tile
// (whole 128-byte row segments) and read back as the B operand, O^T
// accumulated in FP32 registers.  V and P tiles are double-buffered.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void base_pv_kernel(const bf16_t* __restrict__ P, const bf16_t* __restrict__ V,
                                                      bf16_t* __restrict__ O, int N, int ld, BaseGrid grid) {
  constexpr int TILE = kBaseBK * D;         // one V tile (elements)
  constexpr int PTILE = kBaseBQ * kBaseBK;  // one P tile: 128 rows x 64 keys
  constexpr int PPER = PTILE / 8 / 256;     // 16-byte copies per lane per P tile
  constexpr int NK = kBaseBK / 16;
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * TILE + 2 * PTILE];
  bf16_t* const vbuf = smem;
  bf16_t* const pbuf = smem + 2 * TILE;
  int bh, qb;
  if (!base_block(grid.n_qblk, grid.total, grid.remap, grid.BH, grid.G, bh, qb)) return;
  const int q0 = qb * kBaseBQ;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const bf16_t* Vh = V + hoff;
  const bf16_t* Pq = P + ((size_t)bh * (size_t)N + (size_t)q0) * ld;  // row q0 of this head

  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + l32;
  const bool wave_live = qw0 < N;
  const int last_row = min(q0 + kBaseBQ, N) - 1;
  const int n_kblk = CAUSAL ? (last_row / kBaseBK + 1) : (N + kBaseBK - 1) / kBaseBK;
  const int n_wave = !wave_live ? 0 : (CAUSAL ? min(n_kblk, min(qw0 + 31, N - 1) / kBaseBK + 1) : n_kblk);

  // V^T operand of key step ks: slot e of the lane holds key 16 ks + 8 hi + e
  // (the order of the lane's P operand), read as two transposing reads of
  // rows 8 hi + 0..3 and 8 hi + 4..7.
  const int j16 = lane & 15, dsub = (lane >> 4) & 1;
  const uint32_t vx0 = 2u * (uint32_t)tile_off<D>(8 * hi + (j16 >> 2), 16 * dsub + 4 * (j16 & 3));
  const uint32_t vx1 = 2u * (uint32_t)tile_off<D>(8 * hi + 4 + (j16 >> 2), 16 * dsub + 4 * (j16 & 3));
  // P operand of key step ks: row 32 wave + l32, keys 16 ks + 8 hi + 0..7
  // (chunk 2 ks + hi) at offset ^ (ks << 5)
  const uint32_t px0 = 2u * (uint32_t)tile_off<kBaseBK>(wave * 32 + l32, hi * 8);
  int ldoff[kBaseBK * D / 8 / 256];
  tile_offsets<D, kBaseBK, 256>(ldoff, wave, lane);
  // P tile copies: copy r of this lane fills physical chunk c = 256 r +
  // 64 wave + lane, which holds logical chunk (c % 8) ^ swz(row) of row c / 8;
  // rows past N read row N - 1 (in bounds; those rows' outputs are not kept)
  uint32_t poff[PPER];
#pragma unroll
  for (int r = 0; r < PPER; ++r) {
    const int c = r * 256 + wave * 64 + lane;
    const int row = c >> 3;
    const int lc = (c & 7) ^ swz<kBaseBK>(row);
    const int src = min(q0 + row, N - 1) - q0;
    poff[r] = (uint32_t)(((size_t)src * ld + lc * 8) * 2);
  }
  auto copy_p = [&](int j, bf16_t* dst) {
#pragma unroll
    for (int r = 0; r < PPER; ++r) dma16(Pq + j * kBaseBK, poff[r], lds_addr(dst + (r * 256 + wave * 64) * 8));
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) o[t] = zero16();

  load_tile_async<D, kBaseBK, 256>(ldoff, Vh, 0, N, vbuf, wave, lane);
  copy_p(0, pbuf);
  wait_vmem();
  wait_vmem_tracked();
  zero_tail<D, kBaseBK, 256>(0, N, vbuf, wave, lane);
  __syncthreads();

  for (int j = 0; j < n_kblk; ++j) {
    // block j + 1's tiles go into the buffers block j - 1 used (released by
    // the barrier that ended it)
    bf16_t* const vnext = vbuf + ((j + 1) & 1) * TILE;
    if (j + 1 < n_kblk) {
      load_tile_async<D, kBaseBK, 256>(ldoff, Vh, (j + 1) * kBaseBK, N, vnext, wave, lane);
      copy_p(j + 1, pbuf + ((j + 1) & 1) * PTILE);
    }
    if (j < n_wave) {
      const bf16_t* Vs = vbuf + (j & 1) * TILE;
      const char* Ps = reinterpret_cast<const char*>(pbuf + (j & 1) * PTILE);
      const uint32_t va = (uint32_t)opaque((int)vx0), vb = (uint32_t)opaque((int)vx1);
      const uint32_t pa = (uint32_t)opaque((int)px0);
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const bf16x8 pb = lds_load8(reinterpret_cast<const bf16_t*>(Ps + (pa ^ (uint32_t)(ks << 5))));
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const char* base = reinterpret_cast<const char*>(Vs + ks * 16 * D);
          const bf16x8 a = join8(lds_load_tr4(reinterpret_cast<const bf16_t*>(base + (va ^ (uint32_t)(dt << 6)))),
                                 lds_load_tr4(reinterpret_cast<const bf16_t*>(base + (vb ^ (uint32_t)(dt << 6)))));
          o[dt] = mfma<__bf16>(a, pb, o[dt]);
        }
      }
    }
    wait_vmem();
    if (j + 1 < n_kblk) zero_tail<D, kBaseBK, 256>((j + 1) * kBaseBK, N, vnext, wave, lane);
    __syncthreads();
  }

  if (wave_live && myq < N) {
    bf16_t* Orow = O + hoff + (size_t)myq * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack2<__bf16>(o[t][4 * g + 0], o[t][4 * g + 1]);
        w.y = pack2<__bf16>(o[t][4 * g + 2], o[t][4 * g + 3]);
        *reinterpret_cast<uint2*>(Orow + t * 32 + g * 8 + 4 * hi) = w;
      }
  }
}

template <int D>
hipError_t scores_d(const BaseArgs& a, hipStream_t s) {
  const BaseGrid g = base_grid(a);
  if (a.causal)
    hipLaunchKernelGGL((base_scores_kernel<D, true>), dim3((unsigned)g.total), dim3(256), 0, s, (const bf16_t*)a.q,
                       (const bf16_t*)a.k, a.s, a.N, a.ld, g, a.scale);
  else
    hipLaunchKernelGGL((base_scores_kernel<D, false>), dim3((unsigned)g.total), dim3(256), 0, s, (const bf16_t*)a.q,
                       (const bf16_t*)a.k, a.s, a.N, a.ld, g, a.scale);
  return hipGetLastError();
}

template <int D>
hipError_t pv_d(const BaseArgs& a, hipStream_t s) {
  const BaseGrid g = base_grid(a);
  if (a.causal)
    hipLaunchKernelGGL((base_pv_kernel<D, true>), dim3((unsigned)g.total), dim3(256), 0, s, (const bf16_t*)a.p,
                       (const bf16_t*)a.v, (bf16_t*)a.o, a.N, a.ld, g);
  else
    hipLaunchKernelGGL((base_pv_kernel<D, false>), dim3((unsigned)g.total), dim3(256), 0, s, (const bf16_t*)a.p,
                       (const bf16_t*)a.v, (bf16_t*)a.o, a.N, a.ld, g);
  return hipGetLastError();
}

}  // namespace

int base_ld(int N) { return (N + kBaseBK - 1) / kBaseBK * kBaseBK; }

hipError_t launch_base_scores(const BaseArgs& a, hipStream_t s) {
  return a.d == 64 ? scores_d<64>(a, s) : scores_d<128>(a, s);
}

hipError_t launch_base_softmax(const BaseArgs& a, hipStream_t s) {
  const long long rows = (long long)a.B * a.H * a.N;
  if (a.ld <= kBaseWaveRow) {
    const unsigned grid = (unsigned)((rows + 3) / 4);
    if (a.causal)
      hipLaunchKernelGGL((base_softmax_kernel<true, 1>), dim3(grid), dim3(256), 0, s, a.s, (bf16_t*)a.p, a.lse, a.N,
                         a.ld, rows);
    else
      hipLaunchKernelGGL((base_softmax_kernel<false, 1>), dim3(grid), dim3(256), 0, s, a.s, (bf16_t*)a.p, a.lse,
                         a.N, a.ld, rows);
  } else {
    const unsigned grid = (unsigned)rows;
    if (a.causal)
      hipLaunchKernelGGL((base_softmax_kernel<true, 4>), dim3(grid), dim3(256), 0, s, a.s, (bf16_t*)a.p, a.lse, a.N,
                         a.ld, rows);
    else
      hipLaunchKernelGGL((base_softmax_kernel<false, 4>), dim3(grid), dim3(256), 0, s, a.s, (bf16_t*)a.p, a.lse,
                         a.N, a.ld, rows);
  }
  return hipGetLastError();
}

hipError_t launch_base_pv(const BaseArgs& a, hipStream_t s) { return a.d == 64 ? pv_d<64>(a, s) : pv_d<128>(a, s); }

}  // namespace fa
