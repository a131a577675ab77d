// Tiled BF16 attention forward for gfx950 (MI355X).
//
// The method (page 3, "Flash Attention: from academic breakthrough to
// industry standard"; page 2, "Mechanism 2: where the bias comes from"):
// keys are consumed block by block; every query row keeps a running maximum
// m, a running sum l and an unnormalised output O_bar in FP32; the block's
// unnormalised probabilities P = exp(S - m) are cast to BF16 for the product
// with V; the row is normalised by l at the end, and LSE = m + ln l is kept
// for the backward.  With `stabilize`, a row whose running maximum has been
// attained at least twice gets its shift moved so that the exponent at the
// maximum is strictly below 1 (the rule is in fa_device.hpp).
//
// Mapping onto CDNA4.  A workgroup of 4 waves owns 128 query rows, 32 per
// wave; keys arrive in blocks of 64, staged through LDS in two buffers (the
// next block's global loads are in flight while the current one computes).
// Scores are formed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16: K
// rows come from LDS as the A operand, the wave's Q rows stay in registers as
// the B operand, and each lane ends up owning one query row (lanes l and l+32
// split its keys).  So the row maximum, the tie detection and the row sum are
// in-lane work plus one exchange with lane l^32, and the BF16 probabilities
// are already laid out as the B operand of O^T = V^T P^T: no LDS round trip
// for P.  V^T is read from the row-major V tile with the gfx950 transposing
// LDS read.  O^T and l stay in registers until the epilogue.
//
// Exponentials use exp2 with scale*log2(e) folded into one FMA:
// P = 2^(t*c - M), t the raw FP32 dot product, c = scale*log2 e, M the shift
// in base-2 units.  Ties are detected on the raw FP32 scores (equal raw
// scores are equal scaled scores).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

template <int D>
struct FwdTile {
  static constexpr int BQ = kFwdBlockQ;  // query rows per workgroup (4 waves x 32)
  static constexpr int BK = kFwdBlockK;  // keys per block
  static constexpr int KS = D + 8;       // LDS row stride of the K tile (elements)
  static constexpr int VS = D + 16;      // LDS row stride of the V tile (transposing reads)
  static constexpr int K_ELEMS = BK * KS;
  static constexpr int V_ELEMS = BK * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int CHUNKS = BK * D / 8 / 256;  // 16-byte chunks per thread per tensor
  static_assert(CHUNKS >= 1 && BK * D / 8 % 256 == 0, "tile/thread mismatch");
};

template <int D, bool CAUSAL, bool STAB, bool DIAG>
__global__ __launch_bounds__(256, 2) void fwd_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    bf16_t* __restrict__ O, float* __restrict__ LSE, uint8_t* __restrict__ row_shifted,
    int N, int n_qblk, int total_blocks, int xcd_remap, float c2) {
  using T = FwdTile<D>;
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * T::STAGE];

  // Workgroup -> (head, query block).  The hardware hands workgroup i to XCD
  // i % 8; the remap gives each XCD a contiguous range of heads so that a
  // head's K/V stay in that XCD's L2.  Within a head the heaviest (last,
  // for causal) query block goes first.
  int bid = blockIdx.x;
  if (xcd_remap) bid = (bid & 7) * (total_blocks >> 3) + (bid >> 3);
  const int bh = bid / n_qblk;
  const int qb = n_qblk - 1 - (bid - bh * n_qblk);
  const int q0 = qb * T::BQ;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const bf16_t* Qh = Q + hoff;
  const bf16_t* Kh = K + hoff;
  const bf16_t* Vh = V + hoff;

  const int qw0 = q0 + wave * 32;  // first query row of this wave
  const int myq = qw0 + l32;       // this lane's query row
  const bool wave_live = qw0 < N;
  const int wave_last_q = min(qw0 + 31, N - 1);

  // Q rows of this wave as B operands: element j of step kk is d = 16 kk + 8 hi + j.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (myq < N) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)myq * D + kk * 16 + hi * 8);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[kk][j] = (__bf16)0.0f;
    }
  }

  const int last_row = min(q0 + T::BQ, N) - 1;
  const int n_kblk = CAUSAL ? (last_row / T::BK + 1) : (N + T::BK - 1) / T::BK;

  // Global -> register -> LDS staging of one K block and one V block.
  uint4 kr[T::CHUNKS], vr[T::CHUNKS];
  auto gload = [&](int j) {
    const int kb0 = j * T::BK;
#pragma unroll
    for (int r = 0; r < T::CHUNKS; ++r) {
      const int c = tid + 256 * r;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int key = kb0 + row;
      if (key < N) {
        kr[r] = *reinterpret_cast<const uint4*>(Kh + (size_t)key * D + col);
        vr[r] = *reinterpret_cast<const uint4*>(Vh + (size_t)key * D + col);
      } else {
        kr[r] = make_uint4(0, 0, 0, 0);  // zero keys/values past N: masked scores
        vr[r] = make_uint4(0, 0, 0, 0);  // get probability 0, and 0 * 0 stays 0
      }
    }
  };
  auto lstore = [&](int st) {
    bf16_t* Ks = smem + st * T::STAGE;
    bf16_t* Vs = Ks + T::K_ELEMS;
#pragma unroll
    for (int r = 0; r < T::CHUNKS; ++r) {
      const int c = tid + 256 * r;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(Ks + row * T::KS + col) = kr[r];
      *reinterpret_cast<uint4*>(Vs + row * T::VS + col) = vr[r];
    }
  };

  // Running row state (both lanes of a row hold the same m, M, tie flag;
  // each keeps the partial sum of its own half of the keys).
  float m = kNegInf;   // running max of raw scores
  float M = kNegInf;   // current shift, base-2 units
  float l = 0.0f;      // partial row sum of this lane's probabilities
  bool tied = false;   // running max attained at least twice
  bool ever = false;   // the shift was applied at some block
  f32x16 o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) o[t] = zero16();

  const int g16 = lane >> 4, j16 = lane & 15;
  const int dsub = g16 & 1;  // lanes 16..31 and 48..63 read d + 16 in the V^T operand

  gload(0);
  lstore(0);
  for (int j = 0; j < n_kblk; ++j) {
    if (j + 1 < n_kblk) gload(j + 1);
    __syncthreads();
    const bf16_t* Ks = smem + (j & 1) * T::STAGE;
    const bf16_t* Vs = Ks + T::K_ELEMS;
    const int kb0 = j * T::BK;

    if (wave_live && (!CAUSAL || kb0 <= wave_last_q)) {
      // ---- S^T = K Q^T: two 32-key subtiles, raw FP32 dot products
      f32x16 s[T::BK / 32];
#pragma unroll
      for (int t = 0; t < T::BK / 32; ++t) s[t] = zero16();
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
        for (int t = 0; t < T::BK / 32; ++t) {
          const bf16x8 a = lds_load8(Ks + (t * 32 + l32) * T::KS + kk * 16 + hi * 8);
          s[t] = mfma32x32x16(a, qf[kk], s[t]);
        }
      }
      // ---- mask keys past N and, on the diagonal, keys after the query
      const bool edge = (kb0 + T::BK > N) || (CAUSAL && kb0 + T::BK - 1 > qw0);
      if (edge) {
#pragma unroll
        for (int t = 0; t < T::BK / 32; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb0 + t * 32 + (i >> 2) * 8 + hi * 4 + (i & 3);
            if (key >= N || (CAUSAL && key > myq)) s[t][i] = kNegInf;
          }
      }
      // ---- block row maximum (and, stabilised, the second largest value)
      float mx = kNegInf, m2 = kNegInf;
#pragma unroll
      for (int t = 0; t < T::BK / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (STAB) m2 = __builtin_amdgcn_fmed3f(mx, m2, s[t][i]);
          mx = __builtin_fmaxf(mx, s[t][i]);
        }
      const float omx = __shfl_xor(mx, 32);
      const float bm = __builtin_fmaxf(mx, omx);
      if (STAB) {
        const float om2 = __shfl_xor(m2, 32);
        const float b2 = __builtin_fmaxf(__builtin_fminf(mx, omx), __builtin_fmaxf(m2, om2));
        const bool btie = (b2 == bm) && (bm > kNegInf);
        // Running count >= 2: a new maximum restarts the count with this
        // block's; an equal maximum adds to it; a smaller one leaves it.
        tied = (bm > m) ? btie : ((bm == m && bm > kNegInf) ? true : tied);
      }
      const float m_new = __builtin_fmaxf(m, bm);
      const float R = m_new * c2;
      float Mn = R;
      if (STAB && tied) {
        Mn = shifted_offset(R);
        if (DIAG) ever = true;
      }
      const float alpha = exp2_fast(M - Mn);  // 0 on the first block (M = -inf)
      M = Mn;
      m = m_new;

      // ---- P = 2^(t c - M); partial row sum
      float lsum = 0.0f;
#pragma unroll
      for (int t = 0; t < T::BK / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2_fast(__builtin_fmaf(s[t][i], c2, -M));
          s[t][i] = p;
          lsum += p;
        }
      l = alpha * l + lsum;

      // ---- O^T = alpha O^T + V^T bf16(P)^T
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
      bf16x8 pb[T::BK / 16];
#pragma unroll
      for (int ks = 0; ks < T::BK / 16; ++ks) pb[ks] = pack8(s[ks >> 1], (ks & 1) * 8);
#pragma unroll
      for (int ks = 0; ks < T::BK / 16; ++ks) {
        const int row_lo = ks * 16 + 4 * hi + (j16 >> 2);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int col = dt * 32 + 16 * dsub + 4 * (j16 & 3);
          const s16x4 lo = lds_load_tr4(Vs + row_lo * T::VS + col);
          const s16x4 up = lds_load_tr4(Vs + (row_lo + 8) * T::VS + col);
          o[dt] = mfma32x32x16(join8(lo, up), pb[ks], o[dt]);
        }
      }
    }
    if (j + 1 < n_kblk) lstore((j + 1) & 1);
  }

  // ---- epilogue: O = O_bar / l (as O_bar * (1/l)), LSE = (M + log2 l) ln 2
  const float lt = l + __shfl_xor(l, 32);
  if (wave_live && myq < N) {
    const float rinv = 1.0f / lt;
    bf16_t* Orow = O + hoff + (size_t)myq * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack2(o[t][4 * g + 0] * rinv, o[t][4 * g + 1] * rinv);
        w.y = pack2(o[t][4 * g + 2] * rinv, o[t][4 * g + 3] * rinv);
        *reinterpret_cast<uint2*>(Orow + t * 32 + g * 8 + 4 * hi) = w;
      }
    if (hi == 0) {
      LSE[(size_t)bh * N + myq] = (M + __builtin_log2f(lt)) * kLn2;
      if (DIAG) row_shifted[(size_t)bh * N + myq] = ever ? 1 : 0;
    }
  }
}

template <int D, bool CAUSAL, bool STAB, bool DIAG>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int n_qblk = (a.N + kFwdBlockQ - 1) / kFwdBlockQ;
  const long long total = (long long)a.B * a.H * n_qblk;
  const int remap = (total % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, STAB, DIAG>), dim3((unsigned)total), dim3(256), 0, stream,
                     (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (bf16_t*)a.o, a.lse,
                     a.row_shifted, a.N, n_qblk, (int)total, remap, scale_log2e(a.scale));
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t s) {
  const bool diag = a.row_shifted != nullptr;
  if (a.stabilize)
    return diag ? launch_fwd_t<D, CAUSAL, true, true>(a, s) : launch_fwd_t<D, CAUSAL, true, false>(a, s);
  return diag ? launch_fwd_t<D, CAUSAL, false, true>(a, s) : launch_fwd_t<D, CAUSAL, false, false>(a, s);
}

}  // namespace

float scale_log2e(float scale) { return (float)((double)scale * 1.4426950408889634); }

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch_fwd_d<64, true>(a, s) : launch_fwd_d<64, false>(a, s);
  return a.causal ? launch_fwd_d<128, true>(a, s) : launch_fwd_d<128, false>(a, s);
}

}  // namespace fa
