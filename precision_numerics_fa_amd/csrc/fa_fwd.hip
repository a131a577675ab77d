// Tiled BF16 attention forward for gfx950 (MI355X); the same kernel serves
// IEEE binary16 tensors (the element type E is a template parameter: it
// selects the MFMA and the 16-bit rounding, everything else is shared).
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
// wave; keys arrive in blocks of 128.  K and V tiles (one of each) are
// copied straight from HBM into swizzled LDS tiles (global_load_lds_dwordx4,
// no register staging).
// Scores are formed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16: K
// rows come from LDS as the A operand, the wave's Q rows stay in registers as
// the B operand, and each lane ends up owning one query row (lanes l and l+32
// split its keys).  So the row maximum, the tie detection and the row sum are
// in-lane work plus one exchange with lane l^32, and the BF16 probabilities
// are already laid out as the B operand of O^T = V^T P^T: no LDS round trip
// for P.  V^T is read from the row-major V tile with the gfx950 transposing
// LDS read.  O^T and l stay in registers until the epilogue.
// d = 64 runs the blocks one after the other (V[j] lands during block j's
// scores, K[j+1] during its softmax and products) at three waves per SIMD,
// and the other waves on the SIMD supply the overlap.  d = 128 runs two
// stages per block at two waves per SIMD: the scores of block j+1 beside the
// rescale of O for block j, then block j's product with V beside the softmax
// of block j+1, each stage one basic block with its LDS operand reads
// scheduled a few MFMAs ahead.
//
// Workgroups map to (head, query block) in per-XCD head groups, a group's
// heads taken in chunks, block-major within a chunk (see the kernel's first
// lines).
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
  static constexpr int BQ = kFwdBlockQ;      // query rows per workgroup (4 waves x 32)
  static constexpr int BK = fwd_block_k(D);  // keys per block
  static constexpr int TILE = BK * D;        // one swizzled K or V tile (elements)
  // One K and one V tile at both head sizes.  d = 64, sequential blocks:
  // K[j+1] lands during block j's softmax and products, V[j] during its
  // scores, and the other waves on the SIMD supply the overlap.  d = 128,
  // two stages per block: the scores of block j+1 are formed while O is
  // rescaled for block j, then block j's product with V runs while the
  // softmax of block j+1 is computed.
  static constexpr bool SEQ = D == 64;
  static constexpr int NTILES = 2;
};

// Per-wave softmax state of 32 query rows (one row per lane pair).
struct RowState {
  float m;     // running max of raw scores
  float M;     // current shift, base-2 units
  float l;     // partial row sum over this lane's keys
  bool tied;   // running max attained at least twice
  bool ever;   // the shift was applied at some block
};

// Split-key mode: the partial results of one key range (see fwd_kernel).
struct SplitOut {
  float* obar;  // (splits, B*H, N, d) unnormalised output, fp32
  float* lrow;  // (splits, B*H, N) row sum
  float* mrow;  // (splits, B*H, N) shift M at the end of the range (base-2 units)
  int splits;
};

// SPLIT: the workgroup covers one of `splits` contiguous ranges of its key
// blocks.  It first replays the blocks before its range through the row
// maximum and repeated-maximum bookkeeping only (scores, no exponentials or
// products), so that its own blocks see the same running state, and hence
// the same shift and the same rounding of P, as in one pass; it then writes
// its unnormalised output, row sum and final shift for the merge kernel.
template <typename E, int D, bool CAUSAL, bool STAB, bool DIAG, bool SPLIT>
__global__ __launch_bounds__(256, FwdTile<D>::SEQ ? 3 : 2) void fwd_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    bf16_t* __restrict__ O, float* __restrict__ LSE, uint8_t* __restrict__ row_shifted,
    int N, int n_qblk, int total_blocks, int xcd_remap, float c2, int BH, int G, int chunk, SplitOut sp) {
  using T = FwdTile<D>;
  constexpr int NS = T::BK / 32;   // 32-key subtiles per block
  constexpr int NK = T::BK / 16;   // 16-key MFMA steps per block
  // one K tile and one V tile (direct global -> LDS copies)
  __shared__ __attribute__((aligned(16))) bf16_t smem[T::NTILES * T::TILE];
  bf16_t* const Kbuf = smem;
  bf16_t* const Vbuf = smem + (T::NTILES / 2) * T::TILE;

  // Workgroup -> (head, query block).  The hardware hands workgroup i to XCD
  // i % 8; the remap gives each XCD a contiguous range of the order below.
  // The heaviest (last, for causal) query blocks go first.
  int bid = blockIdx.x;
  int split = 0;
  if (SPLIT) {  // workgroup -> (key range, then head and query block, block-major)
    split = bid % sp.splits;
    bid /= sp.splits;
  } else if (xcd_remap) {
    bid = (bid & 7) * (total_blocks >> 3) + (bid >> 3);
  }
  // The heads are split into groups of G, one per XCD, and a group's heads
  // into chunks of `chunk` heads (chunk divides G), taken one after the
  // other; within a chunk the query blocks go block-major, every head's
  // heaviest block first.  chunk = 1 is head-major (a head's K/V stay in
  // L2), chunk = G block-major over the whole group (the longest workgroups
  // start first).
  const int per_group = G * n_qblk;
  const int g = bid / per_group;
  const int r = bid - g * per_group;
  const int per_chunk = chunk * n_qblk;
  const int ck = r / per_chunk;
  const int cw = r - ck * per_chunk;
  const int bh = g * G + ck * chunk + cw % chunk;
  const int qb = n_qblk - 1 - cw / chunk;
  if (bh >= BH) return;
  const int q0 = qb * T::BQ;

  const int tid = threadIdx.x;
  // wave index as a scalar: every per-wave condition below is then uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const bf16_t* Kh = K + hoff;
  const bf16_t* Vh = V + hoff;

  const int qw0 = q0 + wave * 32;  // first query row of this wave
  const int myq = qw0 + l32;       // this lane's query row
  const bool wave_live = qw0 < N;
  const int wave_last_q = min(qw0 + 31, N - 1);

  const int last_row = min(q0 + T::BQ, N) - 1;
  const int n_kblk = CAUSAL ? (last_row / T::BK + 1) : (N + T::BK - 1) / T::BK;
  // key blocks this wave computes (its causal bound), 0 for a wave past N
  const int n_wave = !wave_live ? 0 : (CAUSAL ? min(n_kblk, wave_last_q / T::BK + 1) : n_kblk);
  // key blocks [jb, je) of this workgroup (all of them unless SPLIT)
  const int jb = SPLIT ? split * n_kblk / sp.splits : 0;
  const int je = SPLIT ? (split + 1) * n_kblk / sp.splits : n_kblk;

  // Q rows of this wave as B operands: element j of step kk is d = 16 kk + 8 hi + j.
  bf16x8 qf[D / 16];

  // LDS byte offsets of the operand reads at step 0.  The K operand of step
  // kk (row t*32 + l32, chunk 2 kk + hi) sits at offset ^ (kk << 5), and the
  // V^T transposing read of d-tile dt (rows ks*16 + 8 r + 4 hi + j16/4,
  // column dt*32 + 16 dsub + 4 (j16 % 4)) at offset ^ (dt << 6): the chunk
  // index lies above the in-chunk bits and below the row bits, so the swizzle
  // and the step combine by XOR.
  const int j16 = lane & 15, dsub = (lane >> 4) & 1;
  const uint32_t kx0 = 2u * (uint32_t)tile_off<D>(l32, hi * 8);
  const uint32_t vx0 = 2u * (uint32_t)tile_off<D>(4 * hi + (j16 >> 2), 16 * dsub + 4 * (j16 & 3));
  const uint32_t vx1 = 2u * (uint32_t)tile_off<D>(8 + 4 * hi + (j16 >> 2), 16 * dsub + 4 * (j16 & 3));

  int ldoff[T::BK * D / 8 / 256];
  tile_offsets<D, T::BK, 256>(ldoff, wave, lane);

  // The workgroup's Q rows are copied in whole rows into the V tile (idle
  // until the first block's V), with the first K block into the K tile
  // (unless a split-key replay needs the K tile first), and each wave reads
  // its operands from there: loading them straight into registers would
  // fetch 32 rows in 32-byte pieces per instruction.  Rows past N are zero.
  static_assert(T::BQ == T::BK, "the Q rows fill one tile");
  const bool k_first = jb < je && (!SPLIT || jb == 0);
  load_tile_async<D, T::BQ, 256>(ldoff, Q + hoff, q0, N, Vbuf, wave, lane);
  if (k_first) load_tile_async<D, T::BK, 256>(ldoff, Kh, jb * T::BK, N, Kbuf, wave, lane);
  wait_vmem();
  zero_tail<D, T::BQ, 256>(q0, N, Vbuf, wave, lane);
  if (k_first) zero_tail<D, T::BK, 256>(jb * T::BK, N, Kbuf, wave, lane);
  __syncthreads();
  {
    const char* qbase = reinterpret_cast<const char*>(Vbuf + wave * 32 * D);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[kk] = lds_load8(reinterpret_cast<const bf16_t*>(qbase + (kx0 ^ (uint32_t)(kk << 5))));
  }
  __syncthreads();  // every wave holds its Q rows: the V tile may take V

  RowState st{kNegInf, kNegInf, 0.0f, false, false};
  f32x16 o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) o[t] = zero16();

  // S^T = K Q^T for one block, raw FP32 dot products.  (The offsets pass an
  // opaque copy per block, so that the XORs are formed here instead of being
  // hoisted out of the block loop into one register per step.)
  auto scores = [&](const bf16_t* Ks, f32x16* s) {
    const uint32_t kx = (uint32_t)opaque((int)kx0);
#pragma unroll
    for (int t = 0; t < NS; ++t) s[t] = zero16();
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        const char* base = reinterpret_cast<const char*>(Ks + t * 32 * D);
        s[t] = mfma<E>(lds_load8(reinterpret_cast<const bf16_t*>(base + (kx ^ (uint32_t)(kk << 5)))), qf[kk],
                            s[t]);
      }
  };

  // Row maximum and repeated-maximum bookkeeping of one block held in s
  // (masked already): updates m (and the tie state) and returns the new shift.
  auto track = [&](const f32x16* s) {
    // block row maximum; stabilised: also the second largest value, two
    // entries at a time: a' = max(a, x, y), b' = max(b, med3(a, x, y))
    // (four entries per step: a = max(m, x, y), t = med3(m, x, y),
    // a' = max(a, z, w), t' = med3(a, z, w), b' = max(b, t, t'): five
    // instructions for four entries)
    float mx = kNegInf, m2 = kNegInf;
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        const float x = s[t][i], y = s[t][i + 1], z = s[t][i + 2], w = s[t][i + 3];
        const float a = __builtin_fmaxf(mx, __builtin_fmaxf(x, y));
        if (STAB) {
          const float t0 = __builtin_amdgcn_fmed3f(mx, x, y);
          const float t1 = __builtin_amdgcn_fmed3f(a, z, w);
          m2 = __builtin_fmaxf(m2, __builtin_fmaxf(t0, t1));
        }
        mx = __builtin_fmaxf(a, __builtin_fmaxf(z, w));
      }
    float mx_lo, mx_hi;
    lane_pair(mx, mx_lo, mx_hi);
    const float bm = __builtin_fmaxf(mx_lo, mx_hi);
    if (STAB) {
      float m2_lo, m2_hi;
      lane_pair(m2, m2_lo, m2_hi);
      const float b2 = __builtin_fmaxf(__builtin_fminf(mx_lo, mx_hi), __builtin_fmaxf(m2_lo, m2_hi));
      const bool btie = (b2 == bm) && (bm > kNegInf);
      // Running count >= 2: a new maximum restarts the count with this
      // block's; an equal maximum adds to it; a smaller one leaves it.
      // (Bitwise, so that no branch splits the block.)
      const bool gt = bm > st.m;
      const bool eq = (bm == st.m) & (bm > kNegInf);
      st.tied = (gt & btie) | (!gt & (eq | st.tied));
    }
    const float m_new = __builtin_fmaxf(st.m, bm);
    const float R = m_new * c2;
    float Mn = R;
    if (STAB) {
      Mn = row_offset<E>(R, st.tied);
      if (DIAG) st.ever = st.ever || st.tied;
    }
    st.m = m_new;
    return Mn;
  };

  // Online softmax of one block held in s (masked already): updates the row
  // state (maximum, tie state, shift, row sum), replaces the scores by the
  // unnormalised FP32 probabilities, and returns the factor alpha by which O
  // must be rescaled before this block's product with V.
  auto online = [&](f32x16* s) {
    const float Mn = track(s);
    const float alpha = exp2_fast(st.M - Mn);  // 0 on the first block (M = -inf)
    st.M = Mn;
    float lsum = 0.0f;
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2_fast(__builtin_fmaf(s[t][i], c2, -Mn));
        s[t][i] = p;
        lsum += p;
      }
    st.l = alpha * st.l + lsum;
    return alpha;
  };
  auto rescale = [&](float alpha) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
  };
  // bf16(P) of the block in s, as the B operands of its product with V
  auto pack = [&](const f32x16* s, bf16x8* pb) {
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) pb[ks] = pack8<E>(s[ks >> 1], (ks & 1) * 8);
  };
  auto softmax = [&](f32x16* s, bf16x8* pb) {
    rescale(online(s));
    pack(s, pb);
  };
  // O^T += V^T bf16(P)^T for one block.
  auto pv = [&](const bf16_t* Vs, const bf16x8* pb) {
    const uint32_t va = (uint32_t)opaque((int)vx0), vb = (uint32_t)opaque((int)vx1);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const char* base = reinterpret_cast<const char*>(Vs + ks * 16 * D);
        const bf16x8 a = join8(lds_load_tr4(reinterpret_cast<const bf16_t*>(base + (va ^ (uint32_t)(dt << 6)))),
                               lds_load_tr4(reinterpret_cast<const bf16_t*>(base + (vb ^ (uint32_t)(dt << 6)))));
        o[dt] = mfma<E>(a, pb[ks], o[dt]);
      }
  };

  auto mask = [&](f32x16* s, int kb0) {
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb0 + t * 32 + (i >> 2) * 8 + hi * 4 + (i & 3);
        if (key >= N || (CAUSAL && key > myq)) s[t][i] = kNegInf;
      }
  };

  f32x16 sa[NS];

  if (SPLIT) {
    // ---- replay of the blocks before this range: scores and the running
    // maximum / repeated-maximum state only, one K tile at a time
    wait_vmem_tracked();
    for (int j = 0; j < jb; ++j) {
      load_tile_async<D, T::BK, 256>(ldoff, Kh, j * T::BK, N, Kbuf, wave, lane);
      wait_vmem();
      zero_tail<D, T::BK, 256>(j * T::BK, N, Kbuf, wave, lane);
      __syncthreads();
      if (j < n_wave) {
        const int kb0 = j * T::BK;
        scores(Kbuf, sa);
        if ((kb0 + T::BK > N) || (CAUSAL && kb0 + T::BK - 1 > qw0)) mask(sa, kb0);
        st.M = track(sa);
      }
      __syncthreads();  // the next copy overwrites the tile just read
    }
  }

  if constexpr (T::SEQ) {
    // ---- sequential blocks: K[j] is in LDS when block j starts
    if (jb < je && !k_first) {
      load_tile_async<D, T::BK, 256>(ldoff, Kh, jb * T::BK, N, Kbuf, wave, lane);
      wait_vmem();
      zero_tail<D, T::BK, 256>(jb * T::BK, N, Kbuf, wave, lane);
      __syncthreads();
    }
    // (on every path into the block loop the compiler must see the
    // prologue's register loads completed, or it waits for them, and with
    // them for the loop's tile copies, inside the loop)
    wait_vmem_tracked();
    constexpr int KPER = T::BK * D / 8 / 256;  // 16-byte copies per lane of one tile
    for (int j = jb; j < je; ++j) {
      const bool live = j < n_wave;
      const int kb0 = j * T::BK;
      // V[j] into the V tile, whose reads of block j-1 ended at its last barrier
      load_tile_async<D, T::BK, 256>(ldoff, Vh, kb0, N, Vbuf, wave, lane);
      if (live) {
        scores(Kbuf, sa);
        if ((kb0 + T::BK > N) || (CAUSAL && kb0 + T::BK - 1 > qw0)) mask(sa, kb0);
      }
      __syncthreads();  // every wave's reads of K[j] are done
      if (j + 1 < je) load_tile_async<D, T::BK, 256>(ldoff, Kh, kb0 + T::BK, N, Kbuf, wave, lane);
      bf16x8 pb[NK];
      if (live) softmax(sa, pb);
      // V[j]'s copies were issued before K[j+1]'s, and loads complete in order
      if (j + 1 < je) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KPER) : "memory");
      } else {
        wait_vmem();
      }
      zero_tail<D, T::BK, 256>(kb0, N, Vbuf, wave, lane);
      __syncthreads();  // V[j] complete for every wave
      if (live) pv(Vbuf, pb);
      wait_vmem();
      if (j + 1 < je) zero_tail<D, T::BK, 256>(kb0 + T::BK, N, Kbuf, wave, lane);
      __syncthreads();  // K[j+1] complete; every wave's reads of V[j] are done
    }
  } else {
    // ---- two stages per block (d = 128).  With P[j] and alpha[j] from the
    // softmax of block j, block j runs
    //   A: S[j+1] = K[j+1] Q^T (MFMA)        with  O *= alpha[j] (VALU)
    //   B: O += V[j]^T P[j]^T  (MFMA)        with  the softmax of block j+1
    // so that each stage pairs matrix work with vector work in one basic
    // block.  P[j+1] overwrites P[j] only after B's products have read it
    // (one P buffer).  The K tile holds K[j+1] during A and receives K[j+2]
    // during B; the V tile receives V[j] during A and holds it during B.  The
    // per-element arithmetic and its order are those of a sequential block:
    // rescale, then the product.
    bf16x8 pb[NK];
    float alpha = 0.0f;
    if (jb < je) {
      // prologue: the scores and softmax of block jb; K[jb+1] lands meanwhile
      if (!k_first) {
        load_tile_async<D, T::BK, 256>(ldoff, Kh, jb * T::BK, N, Kbuf, wave, lane);
        wait_vmem();
        zero_tail<D, T::BK, 256>(jb * T::BK, N, Kbuf, wave, lane);
        __syncthreads();
      }
      const int kb0 = jb * T::BK;
      if (jb < n_wave) {
        scores(Kbuf, sa);
        if ((kb0 + T::BK > N) || (CAUSAL && kb0 + T::BK - 1 > qw0)) mask(sa, kb0);
      }
      __syncthreads();  // every wave's reads of K[jb] are done
      if (jb + 1 < je) load_tile_async<D, T::BK, 256>(ldoff, Kh, kb0 + T::BK, N, Kbuf, wave, lane);
      if (jb < n_wave) {
        alpha = online(sa);
        pack(sa, pb);
      }
      wait_vmem();
      if (jb + 1 < je) zero_tail<D, T::BK, 256>(kb0 + T::BK, N, Kbuf, wave, lane);
      __syncthreads();  // K[jb+1] complete
    }
    // (on every path into the block loop the compiler must see the
    // prologue's register loads completed, or it waits for them, and with
    // them for the loop's tile copies, inside the loop)
    wait_vmem_tracked();
    // The steady stages (every block but the range's last two or three):
    // block j+1 is in the range and needs no mask, V[j] and K[j+2] are whole
    // blocks inside N and K[j+2] is in the range, so each stage is one basic
    // block with no branch.  The schedule of each stage is pinned (operand
    // reads a few products ahead of their MFMA), and nothing moves across a
    // stage boundary: work pulled across would lengthen live ranges past the
    // register budget.
    auto steady = [&](int j) {
      const int kb0 = j * T::BK;
      const int kn0 = kb0 + T::BK;  // first key of block j+1
      // ---- A: V[j] into the V tile (its reads of block j-1 ended at the
      // last barrier); S[j+1] from the K tile; O *= alpha[j]
      load_tile_async<D, T::BK, 256, true>(ldoff, Vh, kb0, N, Vbuf, wave, lane);
      scores(Kbuf, sa);
      rescale(alpha);
      interleave<NS * D / 16, 1, 4, 0>();
      wait_vmem();
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();  // V[j] complete; every wave's reads of K[j+1] are done
      __builtin_amdgcn_sched_barrier(0);
      // ---- B: K[j+2] into the K tile; O += V[j]^T P[j]^T; softmax of block j+1
      load_tile_async<D, T::BK, 256, true>(ldoff, Kh, kn0 + T::BK, N, Kbuf, wave, lane);
      pv(Vbuf, pb);
      alpha = online(sa);
      interleave<NK * D / 32, 2, 3, 0>();
      // P[j+1] replaces P[j] once the products have read it
      __builtin_amdgcn_sched_barrier(0);
      pack(sa, pb);
      wait_vmem();
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();  // K[j+2] complete; every wave's reads of V[j] are done
      __builtin_amdgcn_sched_barrier(0);
    };
    // The same two stages for any block, with every condition at run time:
    // the range's last blocks, and waves past N (copies and barriers only).
    auto general = [&](int j) {
      const int kb0 = j * T::BK;
      const int kn0 = kb0 + T::BK;
      const bool live = j < n_wave;
      const bool next = j + 1 < je && j + 1 < n_wave;
      load_tile_async<D, T::BK, 256>(ldoff, Vh, kb0, N, Vbuf, wave, lane);
      if (next) scores(Kbuf, sa);
      if (live) rescale(alpha);
      wait_vmem();
      zero_tail<D, T::BK, 256>(kb0, N, Vbuf, wave, lane);
      __syncthreads();
      if (j + 2 < je) load_tile_async<D, T::BK, 256>(ldoff, Kh, kn0 + T::BK, N, Kbuf, wave, lane);
      if (live) pv(Vbuf, pb);
      if (next) {
        if ((kn0 + T::BK > N) || (CAUSAL && kn0 + T::BK - 1 > qw0)) mask(sa, kn0);
        alpha = online(sa);
        pack(sa, pb);
      }
      wait_vmem();
      if (j + 2 < je) zero_tail<D, T::BK, 256>(kn0 + T::BK, N, Kbuf, wave, lane);
      __syncthreads();
    };
    // With 128-key blocks and 128-row query blocks a live wave computes every
    // block of the range and only the row's last block can need the mask.
    static_assert(T::BK == T::BQ, "one causal bound per workgroup");
    const int j_steady = n_wave >= je ? max(jb, min(je - 2, N / T::BK - 2)) : jb;
    int j = jb;
    for (; j < j_steady; ++j) steady(j);
    for (; j < je; ++j) general(j);
  }

  // ---- epilogue: O = O_bar / l (as O_bar * (1/l)), LSE = (M + log2 l) ln 2
  float l_lo, l_hi;
  lane_pair(st.l, l_lo, l_hi);
  const float lt = l_lo + l_hi;
  if (SPLIT) {
    // partial results of this range: O_bar and l unnormalised, at shift M
    if (wave_live && myq < N) {
      const size_t prow = ((size_t)split * BH + bh) * (size_t)N + myq;
      float* orow = sp.obar + prow * D;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<float4*>(orow + t * 32 + g4 * 8 + 4 * hi) =
              make_float4(o[t][4 * g4 + 0], o[t][4 * g4 + 1], o[t][4 * g4 + 2], o[t][4 * g4 + 3]);
      if (hi == 0) {
        sp.lrow[prow] = lt;
        sp.mrow[prow] = st.M;
      }
    }
    return;
  }
  // O goes out through LDS (the tiles are idle after the block loop's last
  // barrier): a lane holds 8-byte pieces of one row, so storing them directly
  // would write 32 rows in 16-byte pieces per instruction; staged in a
  // row-major LDS copy of the wave's 32 rows (rows padded by 16 bytes), each
  // store writes 4 (d = 128) or 8 (d = 64) whole rows.
  if (wave_live) {
    constexpr int RS = D + 8;  // staged row stride (elements)
    bf16_t* const stage = smem + wave * 32 * RS;
    const float rinv = 1.0f / lt;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack2<E>(o[t][4 * g + 0] * rinv, o[t][4 * g + 1] * rinv);
        w.y = pack2<E>(o[t][4 * g + 2] * rinv, o[t][4 * g + 3] * rinv);
        *reinterpret_cast<uint2*>(stage + l32 * RS + t * 32 + g * 8 + 4 * hi) = w;
      }
    constexpr int LPR = D / 8;  // lanes per row (16 bytes each)
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += 64 / LPR) {
      const int r = r0 + lane / LPR, c = (lane % LPR) * 8;
      if (qw0 + r < N)
        *reinterpret_cast<uint4*>(O + hoff + (size_t)(qw0 + r) * D + c) =
            *reinterpret_cast<const uint4*>(stage + r * RS + c);
    }
  }
  if (wave_live && myq < N) {
    if (hi == 0) {
      LSE[(size_t)bh * N + myq] = (st.M + __builtin_log2f(lt)) * kLn2;
      if (DIAG) row_shifted[(size_t)bh * N + myq] = st.ever ? 1 : 0;
    }
  }
}

// Launches of up to 5.5 rounds of resident workgroups (two per CU at
// d = 128, three at d = 64, 256 CUs) order each XCD group's query blocks
// block-major (see fwd_kernel).  Measured, causal: N=1024 d=64 with 768 and
// 2048 workgroups 39.1 -> 28.7 us and 82.4 -> 61.2 us, and with 4096
// workgroups (5.3 rounds) 0.129 -> 0.117 ms against chunks of four heads;
// N=4096 and N=1024 d=128 with 4096 workgroups (8 rounds) 0.569 -> 0.596 ms
// and 0.213 -> 0.224 ms, slower block-major than in chunks of four; with 2560
// workgroups (5 rounds, 2x40x4096x128) 0.385 -> 0.367 ms block-major.
constexpr long long kFwdBlockMajorHalfRounds = 11;

template <typename E, int D, bool CAUSAL, bool STAB, bool DIAG>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int n_qblk = (a.N + kFwdBlockQ - 1) / kFwdBlockQ;
  const int BH = a.B * a.H;
  const int G = (BH + 7) / 8;  // heads per group: one group per XCD
  const long long total = (long long)((BH + G - 1) / G) * G * n_qblk;
  const int remap = (total % 8 == 0) ? 1 : 0;
  // Causal, several rounds: chunks of four heads.  Head-major order leaves
  // the group's last head to start its heaviest blocks near the end (a tail
  // of ~8% of the launch); with the last four heads block-major among
  // themselves those start a quarter from the end.  Measured (bitwise the
  // same outputs): 4x32x4096x128 0.600 -> 0.575 ms, 16x32x1024x128 0.238 ->
  // 0.209 ms, 2x16x8192x128 unchanged; without the causal mask, where every
  // block costs the same, chunks of four were 1% slower.
  constexpr long long resident = 256LL * (FwdTile<D>::SEQ ? 3 : 2);
  const int chunk = 2 * total <= kFwdBlockMajorHalfRounds * resident
                        ? G
                        : (CAUSAL ? (G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1)) : 1);
  hipLaunchKernelGGL((fwd_kernel<E, D, CAUSAL, STAB, DIAG, false>), dim3((unsigned)total), dim3(256), 0, stream,
                     (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (bf16_t*)a.o, a.lse,
                     a.row_shifted, a.N, n_qblk, (int)total, remap, scale_log2e(a.scale), BH, G, chunk,
                     SplitOut{});
  return hipGetLastError();
}

// Merge of the key ranges: with M the shift at the end of the last range
// (that of the whole row) and f_s = 2^(M_s - M), O = bf16(sum_s f_s O_bar_s
// * (1 / sum_s f_s l_s)) and LSE = (M + log2 l) ln 2, summed over s in
// order.  One thread per four output columns of a row.
template <int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(const float* __restrict__ obar,
                                                        const float* __restrict__ lrow,
                                                        const float* __restrict__ mrow, bf16_t* __restrict__ O,
                                                        float* __restrict__ LSE, long long rows, int splits) {
  constexpr int TPR = D / 4;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = t / TPR;
  const int c = (int)(t % TPR);
  if (row >= rows) return;
  const float M = mrow[(size_t)(splits - 1) * rows + row];
  float l = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s = 0; s < splits; ++s) {
    const size_t pr = (size_t)s * rows + row;
    const float f = exp2_fast(mrow[pr] - M);  // 0 for a range that saw no key (M_s = -inf)
    l += f * lrow[pr];
    const float4 x = *reinterpret_cast<const float4*>(obar + pr * D + 4 * c);
    acc.x += f * x.x;
    acc.y += f * x.y;
    acc.z += f * x.z;
    acc.w += f * x.w;
  }
  const float rinv = 1.0f / l;
  uint2 w;
  w.x = pack2<__bf16>(acc.x * rinv, acc.y * rinv);
  w.y = pack2<__bf16>(acc.z * rinv, acc.w * rinv);
  *reinterpret_cast<uint2*>(O + row * D + 4 * c) = w;
  if (c == 0) LSE[row] = (M + __builtin_log2f(l)) * kLn2;
}

template <int D, bool CAUSAL, bool STAB>
hipError_t launch_split_t(const FwdArgs& a, const SplitArgs& sa, hipStream_t stream) {
  const int n_qblk = (a.N + kFwdBlockQ - 1) / kFwdBlockQ;
  const int BH = a.B * a.H;
  const long long total = (long long)BH * n_qblk * sa.splits;
  SplitOut sp{sa.obar, sa.lrow, sa.mrow, sa.splits};
  // one group of all heads, block-major (every head's heaviest block first)
  hipLaunchKernelGGL((fwd_kernel<__bf16, D, CAUSAL, STAB, false, true>), dim3((unsigned)total), dim3(256), 0,
                     stream, (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (bf16_t*)a.o, a.lse,
                     nullptr, a.N, n_qblk, (int)total, 0, scale_log2e(a.scale), BH, BH, BH, sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = (long long)BH * a.N;
  const long long threads = rows * (D / 4);
  hipLaunchKernelGGL((fwd_merge_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     sa.obar, sa.lrow, sa.mrow, (bf16_t*)a.o, a.lse, rows, sa.splits);
  return hipGetLastError();
}

template <typename E, int D, bool CAUSAL>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t s) {
  const bool diag = a.row_shifted != nullptr;
  if (a.stabilize)
    return diag ? launch_fwd_t<E, D, CAUSAL, true, true>(a, s) : launch_fwd_t<E, D, CAUSAL, true, false>(a, s);
  return diag ? launch_fwd_t<E, D, CAUSAL, false, true>(a, s) : launch_fwd_t<E, D, CAUSAL, false, false>(a, s);
}

template <typename E>
hipError_t launch_fwd_e(const FwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch_fwd_d<E, 64, true>(a, s) : launch_fwd_d<E, 64, false>(a, s);
  return a.causal ? launch_fwd_d<E, 128, true>(a, s) : launch_fwd_d<E, 128, false>(a, s);
}

}  // namespace

float scale_log2e(float scale) { return (float)((double)scale * 1.4426950408889634); }

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  return a.dtype == kF16 ? launch_fwd_e<_Float16>(a, s) : launch_fwd_e<__bf16>(a, s);
}

hipError_t launch_fwd_split(const FwdArgs& a, const SplitArgs& sa, hipStream_t s) {
  if (a.d == 64) {
    if (a.causal) return a.stabilize ? launch_split_t<64, true, true>(a, sa, s) : launch_split_t<64, true, false>(a, sa, s);
    return a.stabilize ? launch_split_t<64, false, true>(a, sa, s) : launch_split_t<64, false, false>(a, sa, s);
  }
  if (a.causal) return a.stabilize ? launch_split_t<128, true, true>(a, sa, s) : launch_split_t<128, true, false>(a, sa, s);
  return a.stabilize ? launch_split_t<128, false, true>(a, sa, s) : launch_split_t<128, false, false>(a, sa, s);
}

}  // namespace fa
