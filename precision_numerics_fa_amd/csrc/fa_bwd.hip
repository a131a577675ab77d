// Tiled BF16 attention backward for gfx950 (MI355X), recomputing the
// probabilities from the forward's LSE (so the stabilised shift, which only
// changes the forward's intermediate scaling, plays no part here).
//
// Gradients of L = sum(O * dO) for softmax attention:
//   D_i   = sum_t dO_it O_it               (bwd_dot, from the bf16 forward O)
//   P_ij  = exp(S_ij - LSE_i)               (FP32, recomputed)
//   dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - D_i)              (FP32, cast to bf16 for the products)
//   dV_j  = sum_i bf16(P_ij) dO_i
//   dK_j  = scale * sum_i bf16(dS_ij) q_i
//   dQ_i  = scale * sum_j bf16(dS_ij) k_j
// Page 1 (section 4.3) notes that gradients of Q and K inherit the forward's
// errors through these quantities; the recipe itself is the standard one.
//
// Two kinds of compute workgroup, no atomics, deterministic:
//   dK/dV: a workgroup owns 128 keys (32 per wave; K rows in an LDS tile,
//     V rows in registers as B operands) and walks 32-query blocks of Q and
//     dO.  It works in the S layout (rows = queries, lane = key), so P and dS
//     are already B operands of dV^T = dO^T P and dK^T = Q^T dS, whose A
//     operands dO^T and Q^T come from the LDS tiles through the transposing
//     LDS read.
//   dQ: a workgroup owns 128 queries (Q and dO rows in registers) and
//     walks 64-key blocks of K and V in LDS.  It works in the S^T layout
//     (lane = query), so dS^T is the B operand of dQ^T = K^T dS^T, whose A
//     operand K^T is a transposing read of the K tile.
// Scores and dP are recomputed in both (7 products instead of 5), which buys
// determinism and no LDS round trip of P or dS.  All tiles are swizzled and
// copied straight from HBM into LDS, one block ahead.  Both kinds keep
// their register footprint within two waves per SIMD: the MFMAs of one wave
// then overlap the exponential and elementwise work of the other, which the
// hardware arbitrates better than a single wave's own instruction order.
// bwd_grads_kernel runs both kinds in one launch (what fa_bwd uses);
// bwd_dkdv_kernel and bwd_dq_kernel run one kind each.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

// The low and high 16-bit values of a 32-bit word, widened to float.
template <typename E>
__device__ __forceinline__ float lo16(uint32_t w) { return widen16<E>(w & 0xFFFFu); }
template <typename E>
__device__ __forceinline__ float hi16(uint32_t w) { return widen16<E>(w >> 16); }
template <>
__device__ __forceinline__ float hi16<__bf16>(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- D = rowsum(dO * O)
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_dot_kernel(const bf16_t* __restrict__ O,
                                                      const bf16_t* __restrict__ dO,
                                                      float* __restrict__ Dvec, long long rows) {
  constexpr int TPR = D / 8;        // threads per row, one 16-byte chunk each
  constexpr int RPB = 256 / TPR;    // rows per workgroup
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.0f;
  if (row < rows) {
    const uint4 a = *reinterpret_cast<const uint4*>(O + row * D + c * 8);
    const uint4 b = *reinterpret_cast<const uint4*>(dO + row * D + c * 8);
    acc = lo16<E>(a.x) * lo16<E>(b.x) + hi16<E>(a.x) * hi16<E>(b.x) + lo16<E>(a.y) * lo16<E>(b.y) +
          hi16<E>(a.y) * hi16<E>(b.y) + lo16<E>(a.z) * lo16<E>(b.z) + hi16<E>(a.z) * hi16<E>(b.z) +
          lo16<E>(a.w) * lo16<E>(b.w) + hi16<E>(a.w) * hi16<E>(b.w);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && c == 0) Dvec[row] = acc;
}

// ---------------------------------------------------------------- shared tiling
__device__ __forceinline__ void load_rows_as_b(bf16x8* f, const bf16_t* rowp, bool valid, int hi, int nsteps) {
  for (int kk = 0; kk < nsteps; ++kk) {
    if (valid) {
      f[kk] = *reinterpret_cast<const bf16x8*>(rowp + kk * 16 + hi * 8);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) f[kk][j] = (__bf16)0.0f;
    }
  }
}

// A wave's 32 output rows, one per lane (lane l32 holds row l32): accumulator
// set t holds columns 32 t .. 32 t + 31, entry i of it column 32 t + 8 (i/4) +
// 4 hi + i%4 -- written as bf16 through a row-major LDS copy, rows padded by
// 16 bytes: stored directly, each instruction would write 32 rows in 16-byte
// pieces; this way each writes 4 (d = 128) or 8 (d = 64) whole rows.
// `stage` is 32 * (D + 8) idle elements of LDS owned by the wave; rows at
// and past `nrows` are not written.
template <typename E, int D>
__device__ __forceinline__ void store_rows_staged(bf16_t* out0, int nrows, const f32x16* acc, float mul, int lane,
                                                  bf16_t* stage) {
  constexpr int RS = D + 8;
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 w;
      w.x = pack2<E>(acc[t][4 * g + 0] * mul, acc[t][4 * g + 1] * mul);
      w.y = pack2<E>(acc[t][4 * g + 2] * mul, acc[t][4 * g + 3] * mul);
      *reinterpret_cast<uint2*>(stage + l32 * RS + t * 32 + g * 8 + 4 * hi) = w;
    }
  constexpr int LPR = D / 8;  // lanes per row, 16 bytes each
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += 64 / LPR) {
    const int r = r0 + lane / LPR, c = (lane % LPR) * 8;
    if (r < nrows)
      *reinterpret_cast<uint4*>(out0 + (size_t)r * D + c) = *reinterpret_cast<const uint4*>(stage + r * RS + c);
  }
}

// Reads of a swizzled tile: the row-major operand read (row sub*32 + l32,
// chunk 2 kk + hi) and the transposing read (rows sub*32 + ks*16 + 8 r +
// 4 hi + j16/4, column dt*32 + 16 dsub + 4 (j16 % 4)).  Stepping the operand
// read by kk flips byte-offset bits 5 and up (offset(kk) = offset(0) ^
// (kk << 5)), and stepping a transposing read by dt flips bits 6 and up,
// because the chunk index sits above the in-chunk bits and below the row
// bits (the swizzle depends on the row modulo 16 only).  Three offset
// registers replace one per step; fresh() launders them once per block so
// that the XORs are formed there rather than hoisted into registers.
template <int D>
struct TileReaderX {
  uint32_t r0, t0, t1;  // byte offsets: operand row l32 at kk = 0; rows trow, trow + 8 at dt = 0
  __device__ __forceinline__ TileReaderX fresh() const {
    return TileReaderX{(uint32_t)opaque((int)r0), (uint32_t)opaque((int)t0), (uint32_t)opaque((int)t1)};
  }
  __device__ __forceinline__ bf16x8 row8(const bf16_t* tile, int sub, int kk) const {
    const char* base = reinterpret_cast<const char*>(tile + sub * 32 * D);
    return lds_load8(reinterpret_cast<const bf16_t*>(base + (r0 ^ (uint32_t)(kk << 5))));
  }
  __device__ __forceinline__ bf16x8 col8(const bf16_t* tile, int sub, int ks, int dt) const {
    const char* base = reinterpret_cast<const char*>(tile + (sub * 32 + ks * 16) * D);
    return join8(lds_load_tr4(reinterpret_cast<const bf16_t*>(base + (t0 ^ (uint32_t)(dt << 6)))),
                 lds_load_tr4(reinterpret_cast<const bf16_t*>(base + (t1 ^ (uint32_t)(dt << 6)))));
  }
};

template <int D>
__device__ __forceinline__ TileReaderX<D> make_reader_x(int lane) {
  const int l32 = lane & 31, hi = lane >> 5, j16 = lane & 15, dsub = (lane >> 4) & 1;
  const int trow = 4 * hi + (j16 >> 2), tcol = 16 * dsub + 4 * (j16 & 3);
  TileReaderX<D> r;
  r.r0 = 2u * (uint32_t)tile_off<D>(l32, hi * 8);
  r.t0 = 2u * (uint32_t)tile_off<D>(trow, tcol);
  r.t1 = 2u * (uint32_t)tile_off<D>(trow + 8, tcol);
  return r;
}

// dK/dV kernel tiling: the workgroup's 128 K rows stay in one swizzled LDS
// tile for the whole kernel; blocks of 32 query rows of Q and dO (and their
// LSE and D) are copied straight into a ring of two LDS stages.
template <int D>
struct DkdvTile {
  static constexpr int B32 = 128;              // keys per workgroup: 4 waves x 32
  static constexpr int BS = 32;                // query rows per block
  static constexpr int TILE = BS * D;          // one swizzled Q or dO tile (elements)
  static constexpr int NT = 256;
  static constexpr int PER = BS * D / 8 / NT;  // 16-byte copies per lane per tile
  static constexpr int KPER = B32 * D / 8 / NT;
  static constexpr int KTILE_BYTES = B32 * D * 2;
  static constexpr int STAGE_BYTES = 2 * 2 * TILE * 2;     // two stages of (Q, dO)
  static constexpr int LDS_BYTES = KTILE_BYTES + STAGE_BYTES + 2 * 2 * BS * 4;
  static_assert(4 * 32 * (D + 8) * 2 <= LDS_BYTES, "output staging fits the tiles");
};

// ---------------------------------------------------------------- dK, dV
// A workgroup owns 128 keys, 32 per wave.  Per 32-query block a wave forms
// S = Q K^T (K rows from the LDS tile) and dP = dO V^T (V rows in
// registers) in the S layout (rows = queries, lane = key), so P and dS are
// already B operands of dV^T = dO^T P and dK^T = Q^T dS, whose A operands
// dO^T and Q^T come from the swizzled tiles through the transposing LDS read.
// The register footprint allows two waves per SIMD.
template <typename E, int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_wg(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                                        const bf16_t* __restrict__ V, const bf16_t* __restrict__ dO,
                                        const float* __restrict__ LSE, const float* __restrict__ Dvec,
                                        bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int N, float c2,
                                        float scale, int bh, int kb, unsigned char* lds) {
  using T = DkdvTile<D>;
  // LDS: the K tile, two stages of (Q tile, dO tile), two of (LSE, D)
  bf16_t* const ktile = reinterpret_cast<bf16_t*>(lds);
  bf16_t(*const tiles)[2 * T::TILE] = reinterpret_cast<bf16_t(*)[2 * T::TILE]>(lds + T::KTILE_BYTES);
  float(*const vecs)[2 * T::BS] = reinterpret_cast<float(*)[2 * T::BS]>(lds + T::KTILE_BYTES + T::STAGE_BYTES);
  const int k0 = kb * T::B32;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const bf16_t* Qh = Q + hoff;
  const bf16_t* dOh = dO + hoff;
  const float* LSEh = LSE + (size_t)bh * N;
  const float* Dh = Dvec + (size_t)bh * N;

  const int kw0 = k0 + wave * 32;
  const int myk = kw0 + l32;
  const bool wave_live = kw0 < N;

  // This wave's V rows as B operands (n = key, k = d).
  bf16x8 vf[D / 16];
  load_rows_as_b(vf, V + hoff + (size_t)myk * D, myk < N, hi, D / 16);

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    dk[t] = zero16();
    dv[t] = zero16();
  }

  const int q_first = CAUSAL ? k0 : 0;  // earlier queries see none of these keys
  const int qb_first = q_first / T::BS;
  const int qb_last = (N - 1) / T::BS;
  const TileReaderX<D> rdx = make_reader_x<D>(lane);
  int ldoff[T::PER];
  tile_offsets<D, T::BS, T::NT>(ldoff, wave, lane);

  // Copies of block qb into stage stg: the Q and dO tiles, and LSE and D of
  // its rows (LSE by wave 1, D by wave 2, so that no wave carries both on
  // top of its share of the tiles; a block that crosses N takes plain loads
  // and gives the rows past N LSE = +inf, so that their P and dS vanish).
  static_assert(T::NT / 64 >= 3, "waves 1 and 2 copy LSE and D");
  auto issue = [&](int qb, int stg) {
    const int r0 = qb * T::BS;
    load_tile_async<D, T::BS, T::NT>(ldoff, Qh, r0, N, tiles[stg], wave, lane);
    load_tile_async<D, T::BS, T::NT>(ldoff, dOh, r0, N, tiles[stg] + T::TILE, wave, lane);
    if (wave == 1 || wave == 2) {
      const float* src = wave == 1 ? LSEh : Dh;
      float* dst = vecs[stg] + (wave == 1 ? 0 : T::BS);
      if (r0 + T::BS <= N) {
        if (lane < T::BS / 4) dma16(reinterpret_cast<const bf16_t*>(src + r0), lane * 16u, lds_addr(dst));
      } else if (lane < T::BS) {
        const int q = r0 + lane;
        dst[lane] = q < N ? src[q] : (wave == 1 ? __builtin_huge_valf() : 0.0f);
      }
    }
  };
  auto zero_tails = [&](int qb, int stg) {
    zero_tail<D, T::BS, T::NT>(qb * T::BS, N, tiles[stg], wave, lane);
    zero_tail<D, T::BS, T::NT>(qb * T::BS, N, tiles[stg] + T::TILE, wave, lane);
  };

  // One 32-query block: S, dP, then P and dS, then the dV and dK products.
  // Entry i of S is query 8 (i/4) + 4 hi + i%4 of the block, key myk.
  // MASKED: the block may hold queries before some key of the wave.
  auto body = [&](auto masked, bool edge, int qb, int stg) {
    constexpr bool MASKED = decltype(masked)::value;
    const TileReaderX<D> rd = rdx.fresh();
    const bf16_t* Qs = tiles[stg];
    const bf16_t* dOs = tiles[stg] + T::TILE;
    const float* vec = vecs[stg];
    f32x16 sacc = zero16(), dacc = zero16();
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      sacc = mfma<E>(rd.row8(Qs, 0, kk), rd.row8(ktile, wave, kk), sacc);
      dacc = mfma<E>(rd.row8(dOs, 0, kk), vf[kk], dacc);
    }
    // P = 2^(S c - LSE log2 e)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 l4 = *reinterpret_cast<const float4*>(vec + g * 8 + hi * 4);
      const float lv[4] = {l4.x * kLog2e, l4.y * kLog2e, l4.z * kLog2e, l4.w * kLog2e};
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc[4 * g + e] = exp2_fast(__builtin_fmaf(sacc[4 * g + e], c2, -lv[e]));
    }
    // on the diagonal, keys after the query get P = 0: entry i's query
    // offset 8 (i/4) + i%4 below lim is masked (lim = 0 masks nothing)
    if (MASKED) {
      const int lim = edge ? myk - qb * T::BS - hi * 4 : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((i >> 2) * 8 + (i & 3) < lim) sacc[i] = 0.0f;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 d4 = *reinterpret_cast<const float4*>(vec + T::BS + g * 8 + hi * 4);
      const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) dacc[4 * g + e] = sacc[4 * g + e] * (dacc[4 * g + e] - dv4[e]);
    }
    const bf16x8 pb[2] = {pack8<E>(sacc, 0), pack8<E>(sacc, 8)};
    const bf16x8 sb[2] = {pack8<E>(dacc, 0), pack8<E>(dacc, 8)};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        dv[dt] = mfma<E>(rd.col8(dOs, 0, ks, dt), pb[ks], dv[dt]);
        dk[dt] = mfma<E>(rd.col8(Qs, 0, ks, dt), sb[ks], dk[dt]);
      }
  };

  // prologue: the K tile and the first block
  int kofs[T::KPER];
  tile_offsets<D, T::B32, T::NT>(kofs, wave, lane);
  load_tile_async<D, T::B32, T::NT>(kofs, K + hoff, k0, N, ktile, wave, lane);
  issue(qb_first, 0);
  wait_vmem();
  wait_vmem_tracked();
  zero_tail<D, T::B32, T::NT>(k0, N, ktile, wave, lane);
  zero_tails(qb_first, 0);
  __syncthreads();
  auto step = [&](int qb, auto masked) {
    const int stg = (qb - qb_first) & 1;
    if (qb < qb_last) issue(qb + 1, stg ^ 1);
    // a wave skips blocks whose queries all precede its keys
    // blocks on the diagonal mask keys after the query; the rest need no mask
    if (wave_live && !(CAUSAL && qb * T::BS + T::BS - 1 < kw0))
      body(masked, CAUSAL && qb * T::BS < kw0 + 31, qb, stg);
    wait_vmem();
    if (qb < qb_last) zero_tails(qb + 1, stg ^ 1);
    __syncthreads();
  };
  // Causal: the blocks that start before the workgroup's last key sit on
  // the diagonal and run with the mask; the rest run without it.
  const int qb_plain = CAUSAL ? min(qb_last + 1, (k0 + T::B32 - 1 + T::BS - 1) / T::BS) : qb_first;
  int qb = qb_first;
  for (; qb < qb_plain; ++qb) step(qb, std::true_type{});
  for (; qb <= qb_last; ++qb) step(qb, std::false_type{});

  // (the tiles are idle after the loop's last barrier)
  if (wave_live) {
    bf16_t* const stage = reinterpret_cast<bf16_t*>(lds) + wave * 32 * (D + 8);
    const int nrows = min(32, N - kw0);
    store_rows_staged<E, D>(dK + hoff + (size_t)kw0 * D, nrows, dk, scale, lane, stage);
    store_rows_staged<E, D>(dV + hoff + (size_t)kw0 * D, nrows, dv, 1.0f, lane, stage);
  }
}

// dQ kernel tiling: swizzled tiles loaded straight into LDS.
template <int D>
struct DqTile {
  static_assert(4 * 32 * (D + 8) * 2 <= 4 * 64 * D * 2, "output staging fits the tiles");
  static constexpr int B32 = 128;          // queries per workgroup: 4 waves x 32
  static constexpr int BS = 64;            // keys per block (two 32-key subtiles)
  static constexpr int TILE = BS * D;      // one swizzled tile (elements)
  static constexpr int NT = 256;
  static constexpr int PER = BS * D / 8 / NT;  // 16-byte loads per lane per tile
  static constexpr int LDS_BYTES = 4 * TILE * 2;
};

// ---------------------------------------------------------------- dQ
template <typename E, int D, bool CAUSAL>
__device__ __forceinline__ void dq_wg(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                                      const bf16_t* __restrict__ V, const bf16_t* __restrict__ dO,
                                      const float* __restrict__ LSE, const float* __restrict__ Dvec,
                                      bf16_t* __restrict__ dQ, int N, float c2, float scale, int bh, int qb,
                                      unsigned char* lds) {
  using T = DqTile<D>;
  // LDS: a ring of two (K tile, V tile) pairs
  bf16_t* const smem = reinterpret_cast<bf16_t*>(lds);
  const int q0 = qb * T::B32;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hi = lane >> 5;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const bf16_t* Kh = K + hoff;
  const bf16_t* Vh = V + hoff;

  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + (lane & 31);
  const bool wave_live = qw0 < N;
  const int wave_last_q = min(qw0 + 31, N - 1);

  // The workgroup's Q rows are copied in whole rows into the second tile
  // pair (idle until the first prefetch) beside the first K and V tiles, and
  // each wave reads its Q operands from there (loaded straight into
  // registers, they would be fetched in 32-byte pieces of 32 rows per
  // instruction); dO rows go straight to registers.
  static_assert(2 * T::BS == T::B32, "the Q rows fill the second tile pair");
  bf16_t* const qtile = smem + 2 * T::TILE;
  int qoff[T::B32 * D / 8 / T::NT];
  tile_offsets<D, T::B32, T::NT>(qoff, wave, lane);
  load_tile_async<D, T::B32, T::NT>(qoff, Q + hoff, q0, N, qtile, wave, lane);
  bf16x8 qf[D / 16], dof[D / 16];
  load_rows_as_b(dof, dO + hoff + (size_t)myq * D, myq < N, hi, D / 16);
  const float lse2 = myq < N ? LSE[(size_t)bh * N + myq] * kLog2e : __builtin_huge_valf();
  const float dq_d = myq < N ? Dvec[(size_t)bh * N + myq] : 0.0f;

  f32x16 dq[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) dq[t] = zero16();

  const int last_row = min(q0 + T::B32, N) - 1;
  const int n_kblk = CAUSAL ? (last_row / T::BS + 1) : (N + T::BS - 1) / T::BS;
  const int n_wave = !wave_live ? 0 : (CAUSAL ? min(n_kblk, wave_last_q / T::BS + 1) : n_kblk);

  const TileReaderX<D> rdx = make_reader_x<D>(lane);
  int ldoff[T::PER];
  tile_offsets<D, T::BS, T::NT>(ldoff, wave, lane);
  auto ktile = [&](int slot) { return smem + slot * 2 * T::TILE; };
  auto vtile = [&](int slot) { return smem + slot * 2 * T::TILE + T::TILE; };

  // S^T = K Q^T and dP^T = V dO^T for one 32-key subtile (lane = query)
  auto sdp = [&](const TileReaderX<D>& rd, const bf16_t* Ks, const bf16_t* Vs, int sub, f32x16& sacc, f32x16& dacc) {
    sacc = zero16();
    dacc = zero16();
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      sacc = mfma<E>(rd.row8(Ks, sub, kk), qf[kk], sacc);
      dacc = mfma<E>(rd.row8(Vs, sub, kk), dof[kk], dacc);
    }
  };
  // MASKED: the block may hold keys past N or (causal) after some query.
  auto elementwise = [&](auto masked, int kb0, int sub, const f32x16& sacc, const f32x16& dacc, bf16x8* sb,
                         bool edge) {
    // entry i is key kb0 + 32 sub + 4 hi + off(i), off(i) = 8 (i/4) + i%4;
    // on an edge block the keys past N (and, causal, after the query) get
    // P = 0: those with off(i) > lim.  A select per entry, no branch.
    constexpr bool MASKED = decltype(masked)::value;
    const int last_key = CAUSAL ? min(N - 1, myq) : N - 1;
    const int lim = MASKED && edge ? last_key - (kb0 + sub * 32 + hi * 4) : 64;
    f32x16 ds;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float pv = exp2_fast(__builtin_fmaf(sacc[i], c2, -lse2));
      if (MASKED && (i >> 2) * 8 + (i & 3) > lim) pv = 0.0f;
      ds[i] = pv * (dacc[i] - dq_d);
    }
    sb[0] = pack8<E>(ds, 0);
    sb[1] = pack8<E>(ds, 8);
  };
  // dQ^T += K^T dS^T for one subtile
  auto grads = [&](const TileReaderX<D>& rd, const bf16_t* Ks, int sub, const bf16x8* sb) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) dq[dt] = mfma<E>(rd.col8(Ks, sub, ks, dt), sb[ks], dq[dt]);
  };

  load_tile_async<D, T::BS, T::NT>(ldoff, Kh, 0, N, ktile(0), wave, lane);
  load_tile_async<D, T::BS, T::NT>(ldoff, Vh, 0, N, vtile(0), wave, lane);
  wait_vmem();
  wait_vmem_tracked();
  zero_tail<D, T::BS, T::NT>(0, N, ktile(0), wave, lane);
  zero_tail<D, T::BS, T::NT>(0, N, vtile(0), wave, lane);
  zero_tail<D, T::B32, T::NT>(q0, N, qtile, wave, lane);
  __syncthreads();
  {
    const TileReaderX<D> rd = rdx.fresh();
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = rd.row8(qtile, wave, kk);
  }
  __syncthreads();  // every wave holds its Q rows: the second tile pair may take K and V
  // One key block: prefetch the next, compute, then wait for the prefetch.
  auto step = [&](int j, auto masked) {
    const int slot = j & 1;
    if (j + 1 < n_kblk) {
      load_tile_async<D, T::BS, T::NT>(ldoff, Kh, (j + 1) * T::BS, N, ktile(slot ^ 1), wave, lane);
      load_tile_async<D, T::BS, T::NT>(ldoff, Vh, (j + 1) * T::BS, N, vtile(slot ^ 1), wave, lane);
    }
    if (j < n_wave) {
      const bf16_t* Ks = ktile(slot);
      const bf16_t* Vs = vtile(slot);
      const int kb0 = j * T::BS;
      const bool edge = (kb0 + T::BS > N) || (CAUSAL && kb0 + T::BS - 1 > qw0);
      const TileReaderX<D> rd = rdx.fresh();
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        f32x16 s0, d0;
        bf16x8 sb0[2];
        sdp(rd, Ks, Vs, sub, s0, d0);
        elementwise(masked, kb0, sub, s0, d0, sb0, edge);
        grads(rd, Ks, sub, sb0);
      }
    }
    wait_vmem();
    if (j + 1 < n_kblk) {
      zero_tail<D, T::BS, T::NT>((j + 1) * T::BS, N, ktile(slot ^ 1), wave, lane);
      zero_tail<D, T::BS, T::NT>((j + 1) * T::BS, N, vtile(slot ^ 1), wave, lane);
    }
    __syncthreads();
  };
  // The leading blocks hold only keys below N and below the workgroup's
  // first query, so they run without the mask; the rest run with it.
  const int n_plain = min(n_kblk, (CAUSAL ? min(N, q0 + 1) : N) / T::BS);
  int j = 0;
  for (; j < n_plain; ++j) step(j, std::false_type{});
  for (; j < n_kblk; ++j) step(j, std::true_type{});

  // (the tiles are idle after the loop's last barrier)
  if (wave_live)
    store_rows_staged<E, D>(dQ + hoff + (size_t)qw0 * D, min(32, N - qw0), dq, scale, lane,
                            smem + wave * 32 * (D + 8));
}

// Workgroup index -> work item: the hardware hands workgroup i to XCD i % 8;
// the remap gives each XCD a contiguous range of the logical order (heads
// stay within one XCD's L2).
__device__ __forceinline__ int logical_block(int total_blocks, int xcd_remap) {
  const int bid = blockIdx.x;
  return xcd_remap ? (bid & 7) * (total_blocks >> 3) + (bid >> 3) : bid;
}

// dK, dV of one 128-key block per workgroup; causal: the first key blocks
// (the most work) first.
template <typename E, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dvec,
    bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int N, int n_kblk, int total_blocks,
    int xcd_remap, float c2, float scale) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[DkdvTile<D>::LDS_BYTES];
  const int bid = logical_block(total_blocks, xcd_remap);
  const int bh = bid / n_kblk;
  dkdv_wg<E, D, CAUSAL>(Q, K, V, dO, LSE, Dvec, dK, dV, N, c2, scale, bh, bid - bh * n_kblk, lds);
}

// dQ of one 128-query block per workgroup; causal: the last query blocks
// (the most work) first.
template <typename E, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dvec,
    bf16_t* __restrict__ dQ, int N, int n_qblk, int total_blocks, int xcd_remap, float c2,
    float scale) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[DqTile<D>::LDS_BYTES];
  const int bid = logical_block(total_blocks, xcd_remap);
  const int bh = bid / n_qblk;
  dq_wg<E, D, CAUSAL>(Q, K, V, dO, LSE, Dvec, dQ, N, c2, scale, bh, n_qblk - 1 - (bid - bh * n_qblk), lds);
}

// dK/dV and dQ in one launch.  The heads are split into (at most) eight
// groups of G, one per XCD; in each group the dK/dV workgroups (128 keys)
// come first and then the dQ workgroups (128 queries), each kind heaviest
// first, so the dQ work fills the tail of the dK/dV work on the same XCD and
// both read the group's tensors through that XCD's L2.  The two bodies share
// one LDS allocation (a workgroup runs one of them).  Workgroups past the
// last head (when B*H is not a multiple of G) return at once.
template <typename E, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_grads_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dvec,
    bf16_t* __restrict__ dQ, bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int N, int n_blk,
    int total_blocks, int xcd_remap, float c2, float scale, int BH, int G, int chunk) {
  constexpr int B0 = DkdvTile<D>::LDS_BYTES, B1 = DqTile<D>::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char lds[B0 > B1 ? B0 : B1];
  const int bid = logical_block(total_blocks, xcd_remap);
  // Heads in groups of G (one group per XCD), a group's heads in chunks of
  // `chunk` heads (chunk divides G), one chunk after the other, block-major
  // within a chunk (every head's heaviest block first).  chunk = 1 is
  // head-major (a head's blocks together: its tensors stay in L2), chunk = G
  // block-major over the group (the longest workgroups start first).  With
  // chunk = 1 or G a group's dK/dV workgroups come first, then its dQ
  // workgroups; with chunks in between each chunk's dK/dV workgroups are
  // followed by its own dQ workgroups, which find the chunk's tensors still
  // in L2.
  const int per_group = 2 * G * n_blk;
  const int g = bid / per_group;
  const int r = bid - g * per_group;
  const int per_chunk = chunk * n_blk;
  bool is_dq;
  int r2;
  if (chunk > 1 && chunk < G) {
    const int c = r / (2 * per_chunk);
    const int w = r - c * 2 * per_chunk;
    is_dq = w >= per_chunk;
    r2 = c * per_chunk + (is_dq ? w - per_chunk : w);
  } else {
    is_dq = r >= G * n_blk;
    r2 = is_dq ? r - G * n_blk : r;
  }
  const int ck = r2 / per_chunk;
  const int cw = r2 - ck * per_chunk;
  const int bh = g * G + ck * chunk + cw % chunk;
  const int blk = cw / chunk;
  if (bh >= BH) return;
  if (is_dq)
    dq_wg<E, D, CAUSAL>(Q, K, V, dO, LSE, Dvec, dQ, N, c2, scale, bh, n_blk - 1 - blk, lds);
  else
    dkdv_wg<E, D, CAUSAL>(Q, K, V, dO, LSE, Dvec, dK, dV, N, c2, scale, bh, blk, lds);
}

inline int remap_ok(long long total) { return (total % 8 == 0) ? 1 : 0; }

template <typename E, int D>
hipError_t launch_dot_t(const BwdArgs& a, hipStream_t s) {
  const long long rows = (long long)a.B * a.H * a.N;
  constexpr int RPB = 256 / (D / 8);
  const long long blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((bwd_dot_kernel<E, D>), dim3((unsigned)blocks), dim3(256), 0, s, (const bf16_t*)a.o,
                     (const bf16_t*)a.dout, a.dvec, rows);
  return hipGetLastError();
}

template <typename E, int D, bool CAUSAL>
hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t s) {
  const int n_kblk = (a.N + DkdvTile<D>::B32 - 1) / DkdvTile<D>::B32;
  const long long total = (long long)a.B * a.H * n_kblk;
  hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, CAUSAL>), dim3((unsigned)total), dim3(256), 0, s,
                     (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (const bf16_t*)a.dout,
                     a.lse, a.dvec, (bf16_t*)a.dk, (bf16_t*)a.dv, a.N, n_kblk, (int)total,
                     remap_ok(total), scale_log2e(a.scale), a.scale);
  return hipGetLastError();
}

template <typename E, int D, bool CAUSAL>
hipError_t launch_dq_t(const BwdArgs& a, hipStream_t s) {
  const int n_qblk = (a.N + DqTile<D>::B32 - 1) / DqTile<D>::B32;
  const long long total = (long long)a.B * a.H * n_qblk;
  hipLaunchKernelGGL((bwd_dq_kernel<E, D, CAUSAL>), dim3((unsigned)total), dim3(256), 0, s,
                     (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (const bf16_t*)a.dout,
                     a.lse, a.dvec, (bf16_t*)a.dq, a.N, n_qblk, (int)total, remap_ok(total),
                     scale_log2e(a.scale), a.scale);
  return hipGetLastError();
}

// Launches of up to 5.5 rounds of resident workgroups (two per CU at
// d = 128, three at d = 64, 256 CUs), the dQ/dK/dV launch orders each XCD
// group's blocks block-major.  Measured: N=1024 d=64 with 4096 workgroups
// (5.3 rounds) 0.175 -> 0.157 ms against head-major, and 0.155 -> 0.149 ms
// against chunks of four heads; N=1024 d=128 with 4096 workgroups (8
// rounds) 0.3056 -> 0.2985 ms (median) in chunks of four instead; at N=2048
// d=64 (32768 workgroups) block-major is 9% slower than head-major (its
// heads no longer share L2).
constexpr long long kGradsBlockMajorHalfRounds = 11;

template <typename E, int D, bool CAUSAL>
hipError_t launch_grads_t(const BwdArgs& a, hipStream_t s) {
  static_assert(DkdvTile<D>::B32 == DqTile<D>::B32, "one block count for both kinds");
  const int n_blk = (a.N + DkdvTile<D>::B32 - 1) / DkdvTile<D>::B32;
  const int BH = a.B * a.H;
  const int G = (BH + 7) / 8;  // heads per group: one group per XCD
  const long long total = (long long)((BH + G - 1) / G) * 2 * G * n_blk;
  // A launch of a few rounds of workgroups is bound by its longest ones
  // (block-major); longer causal launches go in chunks of four heads, so that
  // the last heads' heaviest workgroups do not start at the very end (bitwise
  // the same gradients; 4x32x4096x128 1.885 -> 1.808 ms, 16x32x1024x128
  // 0.664 -> 0.609, 64x16x2048x64 2.209 -> 2.090, 2x16x8192x128 -1%; chunks
  // of two and eight gave 1.851 and 1.827 at the first), each chunk's dQ
  // workgroups right after its dK/dV ones (a further 1.746 -> 1.715 ms,
  // 0.581 -> 0.556, 2.015 -> 1.963); without the mask every workgroup of a
  // kind costs the same and the order stays head-major.
  const int chunk =
      2 * total <= kGradsBlockMajorHalfRounds * 256LL * (D == 64 ? 3 : 2)
          ? G
          : (CAUSAL ? (G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1)) : 1);
  hipLaunchKernelGGL((bwd_grads_kernel<E, D, CAUSAL>), dim3((unsigned)total), dim3(256), 0, s,
                     (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (const bf16_t*)a.dout,
                     a.lse, a.dvec, (bf16_t*)a.dq, (bf16_t*)a.dk, (bf16_t*)a.dv, a.N, n_blk, (int)total,
                     remap_ok(total), scale_log2e(a.scale), a.scale, BH, G, chunk);
  return hipGetLastError();
}

template <typename E>
hipError_t grads_e(const BwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch_grads_t<E, 64, true>(a, s) : launch_grads_t<E, 64, false>(a, s);
  return a.causal ? launch_grads_t<E, 128, true>(a, s) : launch_grads_t<E, 128, false>(a, s);
}

template <typename E>
hipError_t dot_e(const BwdArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_dot_t<E, 64>(a, s) : launch_dot_t<E, 128>(a, s);
}

template <typename E>
hipError_t dkdv_e(const BwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch_dkdv_t<E, 64, true>(a, s) : launch_dkdv_t<E, 64, false>(a, s);
  return a.causal ? launch_dkdv_t<E, 128, true>(a, s) : launch_dkdv_t<E, 128, false>(a, s);
}

template <typename E>
hipError_t dq_e(const BwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch_dq_t<E, 64, true>(a, s) : launch_dq_t<E, 64, false>(a, s);
  return a.causal ? launch_dq_t<E, 128, true>(a, s) : launch_dq_t<E, 128, false>(a, s);
}

}  // namespace

hipError_t launch_bwd_dot(const BwdArgs& a, hipStream_t s) {
  return a.dtype == kF16 ? dot_e<_Float16>(a, s) : dot_e<__bf16>(a, s);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t s) {
  return a.dtype == kF16 ? dkdv_e<_Float16>(a, s) : dkdv_e<__bf16>(a, s);
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s) {
  return a.dtype == kF16 ? dq_e<_Float16>(a, s) : dq_e<__bf16>(a, s);
}

hipError_t launch_bwd_grads(const BwdArgs& a, hipStream_t s) {
  return a.dtype == kF16 ? grads_e<_Float16>(a, s) : grads_e<__bf16>(a, s);
}

}  // namespace fa
