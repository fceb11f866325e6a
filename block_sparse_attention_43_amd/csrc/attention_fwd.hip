// Fused piecewise sparse attention forward (non-causal, one 64-row query tile per
// workgroup of two waves; each wave owns 32 query rows).
//
// For query t of tile i (PISA paper §3.2 Eq. (3.2), §3.3 and §3.4 phases 1-3;
// Sparse Linear Attention blog, Sparse Linear Attention and PWT sections):
//   Phase 1  exact softmax terms of every key of the selected blocks S_i;
//   Phase 2  one virtual token per unselected block j: logit q·k̄_j + ln n_j + φ_{i,j},
//            value ΣV_j / n_j, scanned densely in groups of 64 centroids with the
//            selected blocks masked out; the weight e^{q·k̄_j + φ} also accumulates
//            into A_t for the first-order term;
//   Phase 3  N_t += A_t H̄ q_t once per tile, then o_t = N_t / D_t.
// All phases update one running max and one denominator (online softmax).
// φ_{i,j} = w̃_{i,j} (or ln(1 + w̃) on request), gated to 0 when w̃ > ln n_j (PWT);
// φ = 0 for PISA. LITERAL replaces phases 2-3 with a pass over the raw unselected
// blocks: per row s = q·k̄_j (row mean of q·k over the block), y_n = q·k_n - s,
// w = ½ mean(y²) = ½ qᵀC_j q, weight n_j e^{s+φ} in the denominator and
// e^{s+φ} Σ_n (1 + y_n) v_n = e^{s+φ}(ΣV_j + H_j q) in the numerator.
//
// Layout on MFMA (v_mfma_f32_32x32x16_bf16, or 32x32x2_f32 for fp32 inputs): the
// scores are computed transposed, Sᵀ = K_tile Qᵀ, so each lane holds 32 keys of one
// query and the row max needs one cross-half exchange; the key rows fed into the A
// operand are permuted so that the Sᵀ accumulator registers are directly the
// B operand of Oᵀ += Vᵀ Pᵀ (Vᵀ comes pre-transposed per block from the statistics
// pass). K / Vᵀ tiles are staged through padded LDS; the next tile's global loads are
// issued before the current tile is computed. Workgroup ids are remapped so that
// neighbouring tiles of one head share an XCD (and its L2).
#include "attention.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace pisa {

// Running-max update shared by every phase (log2 domain), lazy by kTau.
template <int NET>
__device__ __forceinline__ void raise_max(float cand, float& m, float& lsum, float& asum, f32x16 (&acc)[NET]) {
  const bool up = cand > m + kTau;
  if (__any(up)) {
    const float m_new = up ? cand : m;
    const float alpha = fast_exp2(m - m_new);   // 1 where unchanged, 0 from -inf
    m = m_new;
    lsum *= alpha;
    asum *= alpha;
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[et][r] *= alpha;
  }
}

template <class T, int D, int MODE>
__global__ __launch_bounds__(128) void attention_kernel(AttnArgs a) {
  using M = typename MmaFor<T>::type;
  using AB = typename M::AB;
  constexpr int KI = M::KI, KH = M::KH;
  constexpr int EPC = 16 / sizeof(T);       // elements per 16-byte chunk
  constexpr int LDK = D + EPC;              // padded LDS row strides (elements)
  constexpr int LDV = kB + EPC;
  constexpr int NKD = D / KI;               // k-steps over the head dimension
  constexpr int NKB = kB / KI;              // k-steps over the 64 keys of a tile
  constexpr int KPM = 32 / KI;              // k-steps per 32-key m-tile
  constexpr int NET = D / 32;               // 32-row tiles of Oᵀ
  constexpr int CPRK = D / EPC;             // chunks per K row
  constexpr int CPRV = kB / EPC;            // chunks per Vᵀ row
  constexpr int PF = kB * D / EPC / 128;    // chunks per thread per operand tile
  constexpr bool VIRT = (MODE == MODE_PISA || MODE == MODE_PWT || MODE == MODE_PWT_ROW);
  constexpr bool ROWW = MODE == MODE_PWT_ROW;
  constexpr float NEG_INF = -__builtin_huge_valf();

  __shared__ __align__(16) T sK[2][kB * LDK];
  __shared__ __align__(16) T sV[2][D * LDV];
  // σ²_j / 2 of a centroid group (per-row w, bf16; the fp32 tiles leave no LDS for it)
  constexpr bool SIG_LDS = ROWW && sizeof(T) == 2;
  __shared__ __align__(16) T sS[SIG_LDS ? kB * LDK : 1];
  __shared__ float sBias[2][kB], sInvN[2][kB], sLnN[ROWW ? 2 : 1][kB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const uint32_t lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = int(lin / uint32_t(a.nb)), i = int(lin % uint32_t(a.nb));
  const int nb = a.nb;
  int ni = a.block_len ? a.block_len[i] : kB;
  ni = min(max(ni, 1), kB);

  const T* Qh = static_cast<const T*>(a.Q) + size_t(h) * a.L * D;
  const T* Kh = static_cast<const T*>(a.K) + size_t(h) * a.L * D;
  const T* vt = reinterpret_cast<const T*>(a.packed + a.pl.vt) + size_t(h) * nb * D * kB;
  const T* kbp = reinterpret_cast<const T*>(a.packed + a.pl.kbar) + size_t(h) * a.nbp * D;
  const T* vbp = reinterpret_cast<const T*>(a.packed + a.pl.vbar) + size_t(h) * a.nbp * D;
  const T* hbp = reinterpret_cast<const T*>(a.packed + a.pl.hbar) + size_t(h) * D * D;
  const uint32_t* mrow = a.mask ? a.mask + (size_t(h) * nb + i) * a.nw : nullptr;
  const int32_t* irow = a.idx + (size_t(h) * nb + i) * a.K_sel;
  const float* wrow = a.wt ? a.wt + (size_t(h) * nb + i) * nb : nullptr;

  // This lane's query row and its Q fragments (B operand of Sᵀ = K Qᵀ), kept in registers.
  const int qrow = 32 * wave + l32;
  const bool qvalid = qrow < ni;
  AB qf[NKD];
#pragma unroll
  for (int ks = 0; ks < NKD; ++ks)
    qf[ks] = qvalid ? M::load(Qh + (size_t(i) * kB + qrow) * D + KI * ks + KH * g) : M::zero();

  f32x16 acc[NET];
#pragma unroll
  for (int et = 0; et < NET; ++et) acc[et] = zero16();
  float m = NEG_INF, lsum = 0.f, asum = 0.f;

  const int n1 = a.K_sel;
  const int n2 = VIRT ? a.nbp / kB : (MODE == MODE_LITERAL ? nb - a.K_sel : 0);
  const int N = n1 + n2;
  int lit_cursor = 0;

  // Source of tile n: block index (exact / literal) or centroid-group index (virtual);
  // -1 past the end. Called once per tile, in order.
  auto next_source = [&](int n) -> int {
    if (n >= N) return -1;
    if (n < n1) return irow[n];
    if (VIRT) return n - n1;
    int j = lit_cursor;                        // next block whose mask bit is clear
    while (j < nb && ((mrow[j >> 5] >> (j & 31)) & 1u)) ++j;
    lit_cursor = j + 1;
    return j;
  };
  // Valid keys of tile n with source j: n_j for a block (0 if j is out of range), 64 for
  // a centroid group (its padding is masked through the bias).
  auto tile_keys = [&](int n, int j) -> int {
    if (n >= N) return 0;
    if (VIRT && n >= n1) return kB;
    if (j < 0 || j >= nb) return 0;
    const int v = a.block_len ? a.block_len[j] : kB;
    return min(max(v, 1), kB);
  };

  // Packed tiles are in TileLayout order; chunk c below is the natural-order chunk
  // (row c / CPRK of K, row c / CPRV of Vᵀ) that lands in the padded LDS tile.
  using TL = TileLayout<T, D>;
  u32x4 rk[PF], rv[PF];
#define PISA_LOAD_TILE(n_, j_)                                                        \
  do {                                                                               \
    const bool virt_ = VIRT && (n_) >= n1;                                           \
    const T* pk_;                                                                    \
    const T* pv_;                                                                    \
    if (virt_) {                                                                     \
      pk_ = kbp + size_t(j_) * kB * D;                                               \
      pv_ = vbp + size_t(j_) * D * kB;                                               \
    } else {                                                                         \
      const int jj_ = ((j_) >= 0 && (j_) < nb) ? (j_) : 0;                           \
      pk_ = Kh + size_t(jj_) * kB * D;                                               \
      pv_ = vt + size_t(jj_) * D * kB;                                               \
    }                                                                                \
    static_for<0, PF>([&](auto pc) {                                                 \
      constexpr int p = decltype(pc)::value;                                         \
      const int c = tid + 128 * p;                                                   \
      const int kr_ = c / CPRK, kc_ = (c % CPRK) * EPC;                              \
      rk[p] = *reinterpret_cast<const u32x4*>(pk_ + (virt_ ? TL::k(kr_, kc_) : kr_ * D + kc_)); \
      rv[p] = *reinterpret_cast<const u32x4*>(pv_ + TL::v((c % CPRV) * EPC, c / CPRV)); \
    });                                                                              \
  } while (0)
#define PISA_STORE_TILE(buf_)                                                         \
  do {                                                                               \
    static_for<0, PF>([&](auto pc) {                                                 \
      constexpr int p = decltype(pc)::value;                                         \
      const int c = tid + 128 * p;                                                   \
      *reinterpret_cast<u32x4*>(&sK[buf_][(c / CPRK) * LDK + (c % CPRK) * EPC]) = rk[p]; \
      *reinterpret_cast<u32x4*>(&sV[buf_][(c / CPRV) * LDV + (c % CPRV) * EPC]) = rv[p]; \
    });                                                                              \
  } while (0)

  // Raw inputs of one centroid group's bias (threads < 64, centroid 64*grp + tid),
  // loaded one tile ahead; the bias itself is formed when the group is staged.
  uint32_t bw_mask = 0u;
  int bw_len = kB;
  float bw_w = 0.f;
  auto load_bias_raw = [&](int grp) {          // every lane loads (no branch); lanes < 64 use it
    const int jj = min(grp * kB + (tid & 63), nb - 1);
    bw_mask = mrow[jj >> 5];
    bw_len = a.block_len ? a.block_len[jj] : kB;
    if (MODE == MODE_PWT) bw_w = wrow[jj];
  };
  // log2-domain bias ln n_j + φ_{i,j}; -inf for selected blocks and the padding beyond nb.
  // With the per-row w the bias is ln n_j alone and ln n_j is kept for the gate.
  auto store_bias = [&](int buf, int grp) {
    if (tid < kB) {
      const int jj = grp * kB + tid;
      float b = NEG_INF, invn = 0.f, lnn_k = 0.f;
      if (jj < nb && !((bw_mask >> (jj & 31)) & 1u)) {
        const int nj = min(max(bw_len, 1), kB);
        const float lnn = logf(float(nj));
        float phi = 0.f;
        if (MODE == MODE_PWT) {
          float w = bw_w;
          if (a.gate && w > lnn) w = 0.f;
          phi = a.w_linear ? log1pf(w) : w;
        }
        b = (lnn + phi) * kLog2e;
        invn = 1.f / float(nj);
        lnn_k = lnn;
      }
      sBias[buf][tid] = b;
      sInvN[buf][tid] = invn;
      if constexpr (ROWW) sLnN[buf][tid] = lnn_k;
    }
  };

  // Descriptor pipeline: sources of tiles n, n+1, n+2 and key counts of n, n+1 are in
  // registers at the top of iteration n, so no per-tile metadata load is on the
  // critical path.
  int j_c = next_source(0), j_n = next_source(1), j_n2 = next_source(2);
  int k_c = tile_keys(0, j_c), k_n = tile_keys(1, j_n);
  if (N > 0) {
    PISA_LOAD_TILE(0, j_c);
    PISA_STORE_TILE(0);
    if (VIRT && n1 == 0) {
      load_bias_raw(j_c);
      store_bias(0, j_c);
    }
    if (N > 1) {
      PISA_LOAD_TILE(1, j_n);
      if (VIRT && 1 >= n1) load_bias_raw(j_n);
    }
  }
  __syncthreads();

  for (int n = 0; n < N; ++n) {
    const int buf = n & 1;
    const bool second = n >= n1;
    const T* sKb = sK[buf];
    const T* sVb = sV[buf];
    const int nj = k_c;

    // Sᵀ[key][q] for the two 32-key halves of the tile (independent MFMA chains).
    f32x16 s0 = zero16(), s1 = zero16();
    if constexpr (ROWW) {
      if (second) {
        // Per-row diagonal w_{t,j} = ½ Σ_c q_{t,c}² σ²_{j,c} on MFMA (A = σ²_j / 2 rows of
        // the group's centroids, B = q² of this lane's query), gated and mapped in place;
        // the score MFMAs below then accumulate onto φ. The group's σ²/2 rows are staged
        // in LDS first (one coalesced load; zeros past nb), rounded to T as the operand.
        if constexpr (SIG_LDS) {
          __syncthreads();                           // previous group's sS reads done
          for (int c = tid; c < kB * D / 4; c += 128) {
            const int r = c / (D / 4), col = (c % (D / 4)) * 4, jj = j_c * kB + r;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (jj < nb) v = *reinterpret_cast<const float4*>(a.ksig2 + (size_t(h) * nb + jj) * D + col);
            sS[r * LDK + col + 0] = from_f32<T>(0.5f * v.x);
            sS[r * LDK + col + 1] = from_f32<T>(0.5f * v.y);
            sS[r * LDK + col + 2] = from_f32<T>(0.5f * v.z);
            sS[r * LDK + col + 3] = from_f32<T>(0.5f * v.w);
          }
          __syncthreads();
          const T* sr0 = sS + feed_row<M>(l32) * LDK + KH * g;
          const T* sr1 = sr0 + 32 * LDK;
#pragma unroll
          for (int ks = 0; ks < NKD; ++ks) {
            float qv[KH];
            M::unpack(qf[ks], qv);
#pragma unroll
            for (int u = 0; u < KH; ++u) qv[u] *= qv[u];
            const AB b = M::pack(qv);
            s0 = M::mma(M::load(sr0 + KI * ks), b, s0);
            s1 = M::mma(M::load(sr1 + KI * ks), b, s1);
          }
        } else {
          const int j0 = j_c * kB + feed_row<M>(l32), j1 = j0 + 32;
          const float* g0 = a.ksig2 + (size_t(h) * nb + min(j0, nb - 1)) * D + KH * g;
          const float* g1 = a.ksig2 + (size_t(h) * nb + min(j1, nb - 1)) * D + KH * g;
          const float h0 = j0 < nb ? 0.5f : 0.f, h1 = j1 < nb ? 0.5f : 0.f;
#pragma unroll 2
          for (int ks = 0; ks < NKD; ++ks) {
            float qv[KH], v0[KH], v1[KH];
            M::unpack(qf[ks], qv);
#pragma unroll
            for (int u = 0; u < KH; ++u) {
              qv[u] *= qv[u];
              v0[u] = h0 * g0[KI * ks + u];
              v1[u] = h1 * g1[KI * ks + u];
            }
            const AB b = M::pack(qv);
            s0 = M::mma(M::pack(v0), b, s0);
            s1 = M::mma(M::pack(v1), b, s1);
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float l0 = sLnN[buf][acc_key<M>(0, r, g)], l1 = sLnN[buf][acc_key<M>(1, r, g)];
          float w0 = s0[r], w1 = s1[r];
          if (a.gate && w0 > l0) w0 = 0.f;
          if (a.gate && w1 > l1) w1 = 0.f;
          s0[r] = a.w_linear ? log1pf(w0) : w0;
          s1[r] = a.w_linear ? log1pf(w1) : w1;
        }
      }
    }
    {
      const T* kr0 = sKb + feed_row<M>(l32) * LDK + KH * g;
      const T* kr1 = kr0 + 32 * LDK;
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        s0 = M::mma(M::load(kr0 + KI * ks), qf[ks], s0);
        s1 = M::mma(M::load(kr1 + KI * ks), qf[ks], s1);
      }
    }

    if (!second || VIRT) {
      float mx = NEG_INF;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int k0 = acc_key<M>(0, r, g), k1 = acc_key<M>(1, r, g);
        if (second) {
          s0[r] = s0[r] * kLog2e + sBias[buf][k0];
          s1[r] = s1[r] * kLog2e + sBias[buf][k1];
        } else {
          s0[r] = k0 < nj ? s0[r] * kLog2e : NEG_INF;
          s1[r] = k1 < nj ? s1[r] * kLog2e : NEG_INF;
        }
        mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      }
      mx = max_halves(mx);
      raise_max<NET>(mx, m, lsum, asum, acc);
      const float mu = m == NEG_INF ? 0.f : m;
      float ps = 0.f, pa = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = fast_exp2(s0[r] - mu);
        s1[r] = fast_exp2(s1[r] - mu);
        ps += s0[r] + s1[r];
        if (VIRT && second)
          pa += s0[r] * sInvN[buf][acc_key<M>(0, r, g)] + s1[r] * sInvN[buf][acc_key<M>(1, r, g)];
      }
      lsum += ps;
      if (VIRT) asum += pa;
    } else {
      // LITERAL: block-wise first-order weights with the per-row second-order factor.
      const float invn = nj > 0 ? 1.f / float(nj) : 0.f;
      float ssum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (acc_key<M>(0, r, g) < nj) ssum += s0[r];
        if (acc_key<M>(1, r, g) < nj) ssum += s1[r];
      }
      const float mean = sum_halves(ssum) * invn;
      float y2 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float y0 = s0[r] - mean, y1 = s1[r] - mean;
        if (acc_key<M>(0, r, g) < nj) y2 += y0 * y0;
        if (acc_key<M>(1, r, g) < nj) y2 += y1 * y1;
      }
      float w = 0.5f * sum_halves(y2) * invn;
      const float lnn = nj > 0 ? logf(float(nj)) : 0.f;
      if (a.gate && w > lnn) w = 0.f;
      const float phi = a.w_linear ? log1pf(w) : w;
      raise_max<NET>(nj > 0 ? (mean + phi + lnn) * kLog2e : NEG_INF, m, lsum, asum, acc);
      const float mu = m == NEG_INF ? 0.f : m;
      const float cw = nj > 0 ? fast_exp2((mean + phi) * kLog2e - mu) : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = acc_key<M>(0, r, g) < nj ? cw * (1.f + (s0[r] - mean)) : 0.f;
        s1[r] = acc_key<M>(1, r, g) < nj ? cw * (1.f + (s1[r] - mean)) : 0.f;
      }
      lsum += g == 0 ? float(nj) * cw : 0.f;
    }

    // Oᵀ += Vᵀ Pᵀ : the B operand of k-step ks is registers [(ks % KPM) * KH, +KH) of m-tile ks / KPM.
    static_for<0, NKB>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      const AB b = (ks / KPM == 0) ? M::template packv<(ks % KPM) * KH>(s0)
                                   : M::template packv<(ks % KPM) * KH>(s1);
#pragma unroll
      for (int et = 0; et < NET; ++et)
        acc[et] = M::mma(M::load(sVb + (32 * et + l32) * LDV + KI * ks + KH * g), b, acc[et]);
    });

    // Stage tile n + 1 into the other buffer, start loading tile n + 2, advance the
    // descriptor pipeline.
    if (n + 1 < N) {
      PISA_STORE_TILE(buf ^ 1);
      if (VIRT && n + 1 >= n1) store_bias(buf ^ 1, j_n);
      if (n + 2 < N) {
        PISA_LOAD_TILE(n + 2, j_n2);
        if (VIRT && n + 2 >= n1) load_bias_raw(j_n2);
      }
    }
    j_c = j_n;
    k_c = k_n;
    j_n = j_n2;
    k_n = tile_keys(n + 2, j_n2);
    j_n2 = next_source(n + 3);
    __syncthreads();
  }
#undef PISA_LOAD_TILE
#undef PISA_STORE_TILE

  if (VIRT) {
    // Phase 3: Oᵀ += H̄ (A_t q_t)ᵀ with H̄[e][c] as the A operand.
    const float at = sum_halves(asum);
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      float qv[KH];
      M::unpack(qf[ks], qv);
#pragma unroll
      for (int u = 0; u < KH; ++u) qv[u] *= at;
      const AB b = M::pack(qv);
#pragma unroll
      for (int et = 0; et < NET; ++et)
        acc[et] = M::mma(M::load(hbp + size_t(32 * et + l32) * D + KI * ks + KH * g), b, acc[et]);
    }
  }

  const float lt = sum_halves(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const size_t orow = size_t(h) * a.L + size_t(i) * kB + qrow;
  float lse_out = (qvalid && lt > 0.f) ? m * kLn2 + logf(lt) : NEG_INF;
  // Merge with a pass over the other keys whose normalised output and lse are in O and lse
  // (per-row w: the exact tiles ran first in the register-streamed kernel). Softmax over
  // the union: weights e^{lse_x - M} of the two normalised outputs.
  float w_own = 1.f, w_prev = 0.f;
  if (ROWW && a.merge) {
    const float lp = a.lse[orow], M = fmaxf(lp, lse_out);
    w_prev = M > NEG_INF && lp > NEG_INF ? expf(lp - M) : 0.f;
    w_own = M > NEG_INF && lse_out > NEG_INF ? expf(lse_out - M) : 0.f;
    const float den = w_prev + w_own;
    lse_out = den > 0.f ? M + logf(den) : NEG_INF;
    const float id = den > 0.f ? 1.f / den : 0.f;
    w_prev *= id;
    w_own *= id;
  }
  T* sO = sK[0];
  const T* Oprev = static_cast<const T*>(a.O) + orow * D;
#pragma unroll
  for (int et = 0; et < NET; ++et)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = 32 * et + acc_row(r, g);
      float o = acc[et][r] * inv;
      if (ROWW && a.merge) o = w_own * o + w_prev * to_f32(Oprev[e]);
      sO[qrow * LDK + e] = from_f32<T>(qvalid ? o : 0.f);
    }
  if (a.lse && g == 0) a.lse[orow] = lse_out;
  __syncthreads();
  T* Oh = static_cast<T*>(a.O) + (size_t(h) * a.L + size_t(i) * kB) * D;
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int c = tid + 128 * p;
    *reinterpret_cast<u32x4*>(Oh + (c / CPRK) * D + (c % CPRK) * EPC) =
        *reinterpret_cast<const u32x4*>(sO + (c / CPRK) * LDK + (c % CPRK) * EPC);
  }
}

// ---------------------------------------------------------------------------
// Split-key kernel for DROP / PISA / PWT (the timed path).
//
// One 64-row query tile per workgroup of four waves. Wave w owns query rows
// 32*(w & 1) + [0, 32) and the key half 32*(w >> 1) + [0, 32) of every tile it visits,
// with its own running max / sums; the two key halves of each query half are merged
// at the end (flash-decoding style). This keeps 16 score registers and 64 output
// accumulators per lane, so two workgroups (eight waves) fit on a CU and the softmax of
// one wave overlaps the MFMA work of another. Tiles arrive by direct global->LDS loads
// into two stages of swizzled LDS; one barrier per tile.
// ---------------------------------------------------------------------------
template <class T, int D, int MODE>
__global__ __launch_bounds__(256, 2) void attention_split_kernel(AttnArgs a) {
  using M = typename MmaFor<T>::type;
  using AB = typename M::AB;
  constexpr int KI = M::KI, KH = M::KH;
  constexpr int ES = sizeof(T);
  constexpr int KROW = D * ES;                 // bytes per key row
  constexpr int VROW = kB * ES;                // bytes per Vᵀ row (64 keys)
  constexpr int TB = kB * KROW;                // bytes per operand tile
  constexpr int NDMA = TB / 1024;              // 1 KB loads per operand tile
  constexpr int DPW = NDMA / 4;                // ... per wave
  constexpr int NKD = D / KI;                  // k-steps over the head dimension
  constexpr int NKH = 32 / KI;                 // k-steps over a 32-key half
  constexpr int NET = D / 32;                  // 32-row tiles of Oᵀ
  constexpr bool VIRT = (MODE == MODE_PISA || MODE == MODE_PWT);
  constexpr float NEG_INF = -__builtin_huge_valf();
  using KT = SwizzledTile<KROW>;
  using VT = SwizzledTile<VROW>;
  static_assert(NDMA % 4 == 0 && 1024 % KROW == 0 && 1024 % VROW == 0, "tile shape");

  constexpr int DCH = 512;                       // descriptor chunk (exact tiles)
  // Separate objects per stage and operand, so the compiler can see that reading one
  // stage does not depend on the direct loads still landing in the other.
  __shared__ __align__(1024) char sK0[TB], sV0[TB], sK1[TB], sV1[TB];
  __shared__ float sBias[2][kB], sInvN[2][kB];
  __shared__ uint32_t sDesc[2][DCH];             // exact tile -> block | keys << 16

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int qh = wave & 1, kh = wave >> 1;
  const uint32_t lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = int(lin / uint32_t(a.nb)), i = int(lin % uint32_t(a.nb));
  const int nb = a.nb;
  int ni = a.block_len ? a.block_len[i] : kB;
  ni = min(max(ni, 1), kB);

  const T* Qh = static_cast<const T*>(a.Q) + size_t(h) * a.L * D;
  const char* Kh = reinterpret_cast<const char*>(static_cast<const T*>(a.K) + size_t(h) * a.L * D);
  const char* vt = a.packed + a.pl.vt + size_t(h) * nb * TB;
  const char* kbp = a.packed + a.pl.kbar + size_t(h) * a.nbp * KROW;
  const char* vbp = a.packed + a.pl.vbar + size_t(h) * a.nbp * KROW;
  const T* hbp = reinterpret_cast<const T*>(a.packed + a.pl.hbar) + size_t(h) * D * D;
  const uint32_t* mrow = a.mask ? a.mask + (size_t(h) * nb + i) * a.nw : nullptr;
  const int32_t* irow = a.idx + (size_t(h) * nb + i) * a.K_sel;
  const float* wrow = a.wt ? a.wt + (size_t(h) * nb + i) * nb : nullptr;

  const int qrow = 32 * qh + l32;
  const bool qvalid = qrow < ni;
  AB qf[NKD];
#pragma unroll
  for (int ks = 0; ks < NKD; ++ks)
    qf[ks] = qvalid ? M::load(Qh + (size_t(i) * kB + qrow) * D + KI * ks + KH * g) : M::zero();

  f32x16 acc[NET];
#pragma unroll
  for (int et = 0; et < NET; ++et) acc[et] = zero16();
  float m = NEG_INF, lsum = 0.f, asum = 0.f;

  const int n1 = a.K_sel;
  const int N = n1 + (VIRT ? a.nbp / kB : 0);

  // Descriptor of exact tile n: its block (out-of-range indices become block 0 with no
  // valid keys) and the block's valid key count, staged in LDS in chunks of DCH tiles.
  auto fill_desc = [&](int chunk) {
    for (int e = tid; e < DCH; e += 256) {
      const int n = chunk * DCH + e;
      uint32_t d = 0u;
      if (n < n1) {
        const int j = irow[n];
        if (j >= 0 && j < nb) {
          const int v = a.block_len ? a.block_len[j] : kB;
          d = uint32_t(j) | (uint32_t(min(max(v, 1), kB)) << 16);
        }
      }
      sDesc[chunk & 1][e] = d;
    }
  };
  // (source, keys) of tile n: block and n_j for exact tiles, group and 64 for virtual ones.
  auto desc = [&](int n, int& j, int& k) {
    if (n < n1) {
      const uint32_t d = sDesc[(n / DCH) & 1][n % DCH];
      j = int(d & 0xFFFFu);
      k = int(d >> 16);
    } else {
      j = n - n1;
      k = kB;
    }
  };
  // Buffer resources of this head's key tiles, Vᵀ tiles, centroid and mean-value groups;
  // per-lane byte offsets inside a tile are loop-invariant.
  int koff[DPW], voff[DPW];
#pragma unroll
  for (int u = 0; u < DPW; ++u) {
    const int b = (wave * DPW + u) * 1024 + lane * 16;   // byte of the LDS tile this lane fills
    const int rk = b / KROW, rv = b / VROW;
    koff[u] = rk * KROW + ((((b % KROW) >> 4) ^ KT::swz(rk)) << 4);
    voff[u] = rv * VROW + ((((b % VROW) >> 4) ^ VT::swz(rv)) << 4);
  }
  // Direct loads of tile n (source j) into stage ST; this wave's share of both operands.
  auto issue_tile = [&](int n, int j, auto stc) {
    constexpr int ST = decltype(stc)::value;
    char* dk = ST ? sK1 : sK0;
    char* dv = ST ? sV1 : sV0;
    const bool virt = VIRT && n >= n1;
    const int base = __builtin_amdgcn_readfirstlane(((j >= 0 && j < nb) || virt ? j : 0) * TB);
    if (virt) {
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbp, uint32_t(a.nbp) * KROW);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbp, uint32_t(a.nbp) * KROW);
#pragma unroll
      for (int u = 0; u < DPW; ++u) {
        buf_dma16(rk, koff[u], base, dk + (wave * DPW + u) * 1024);
        buf_dma16(rv, voff[u], base, dv + (wave * DPW + u) * 1024);
      }
    } else {
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh, uint32_t(nb) * TB);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vt, uint32_t(nb) * TB);
#pragma unroll
      for (int u = 0; u < DPW; ++u) {
        buf_dma16(rk, koff[u], base, dk + (wave * DPW + u) * 1024);
        buf_dma16(rv, voff[u], base, dv + (wave * DPW + u) * 1024);
      }
    }
  };

  // Raw inputs of a centroid group's bias (threads < 64), loaded one tile ahead.
  uint32_t bw_mask = 0u;
  int bw_len = kB;
  float bw_w = 0.f;
  auto load_bias_raw = [&](int grp) {          // every lane loads (no branch); lanes < 64 use it
    const int jj = min(grp * kB + (tid & 63), nb - 1);
    bw_mask = mrow[jj >> 5];
    bw_len = a.block_len ? a.block_len[jj] : kB;
    if (MODE == MODE_PWT) bw_w = wrow[jj];
  };
  auto store_bias = [&](int st, int grp) {     // log2-domain ln n_j + φ_{i,j}; -inf if excluded
    if (tid < kB) {
      const int jj = grp * kB + tid;
      float b = NEG_INF, invn = 0.f;
      if (jj < nb && !((bw_mask >> (jj & 31)) & 1u)) {
        const int nj = min(max(bw_len, 1), kB);
        const float lnn = logf(float(nj));
        float phi = 0.f;
        if (MODE == MODE_PWT) {
          float w = bw_w;
          if (a.gate && w > lnn) w = 0.f;
          phi = a.w_linear ? log1pf(w) : w;
        }
        b = (lnn + phi) * kLog2e;
        invn = 1.f / float(nj);
      }
      sBias[st][tid] = b;
      sInvN[st][tid] = invn;
    }
  };

  // One tile: Sᵀ for this wave's 32 keys, online softmax, Oᵀ += Vᵀ Pᵀ.
  const bool wave_has_rows = 32 * qh < ni;        // some of this wave's query rows are valid
  auto compute = [&](auto stc, bool second, int nj) {
    constexpr int st = decltype(stc)::value;
    // Nothing to do when all of this wave's rows, or all keys of its half of an exact
    // block, are padding (ragged edge cubes hold 8..32 tokens).
    if (!wave_has_rows || (!second && nj <= 32 * kh)) return;
    const char* sk = st ? sK1 : sK0;
    const char* sv = st ? sV1 : sV0;
    f32x16 s = zero16();
    {
      const int R = 32 * kh + feed_row<M>(l32);
      AB kf[NKD];
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks)
        kf[ks] = M::load(reinterpret_cast<const T*>(sk + KT::offset(R, (KI * ks + KH * g) * ES)));
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) s = M::mma(kf[ks], qf[ks], s);
    }
    // Logits in log2 units: t = s * log2(e) + bias. The max is taken on the same values
    // the exponentials use, so every p <= 2^kTau.
    float mx = NEG_INF;
    if (VIRT && second) {
      // per-key bias / (1 / n_j): keys 32*kh + acc_key(0, r, g) are runs of KH consecutive keys
#pragma unroll
      for (int r = 0; r < 16; r += KH) {
        const int key = 32 * kh + acc_key<M>(0, r, g);
#pragma unroll
        for (int u = 0; u < KH; ++u) s[r + u] = fmaf(s[r + u], kLog2e, sBias[st][key + u]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    } else if (nj >= kB) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx *= kLog2e;
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (32 * kh + acc_key<M>(0, r, g) >= nj) s[r] = NEG_INF;
        mx = fmaxf(mx, s[r]);
      }
      mx *= kLog2e;
    }
    mx = max_halves(mx);
    raise_max<NET>(mx, m, lsum, asum, acc);
    const float mu = m == NEG_INF ? 0.f : m;
    float ps = 0.f, pa = 0.f;
    if (VIRT && second) {
#pragma unroll
      for (int r = 0; r < 16; r += KH) {
        const int key = 32 * kh + acc_key<M>(0, r, g);
#pragma unroll
        for (int u = 0; u < KH; ++u) {
          const float p = fast_exp2(s[r + u] - mu);
          s[r + u] = p;
          ps += p;
          pa = fmaf(p, sInvN[st][key + u], pa);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[r], kLog2e, -mu));
        s[r] = p;
        ps += p;
      }
    }
    lsum += ps;
    if (VIRT) asum += pa;
    static_for<0, NKH>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      const AB b = M::template packv<ks * KH>(s);
      const int kb = (32 * kh + KI * ks + KH * g) * ES;     // byte of this lane's keys in a Vᵀ row
#pragma unroll
      for (int et = 0; et < NET; ++et)
        acc[et] = M::mma(M::load(reinterpret_cast<const T*>(sv + VT::offset(32 * et + l32, kb))), b, acc[et]);
    });
  };

  if (n1 > 0) fill_desc(0);
  if (n1 > DCH) fill_desc(1);
  __syncthreads();
  if (N > 0) {
    int j0, k0;
    desc(0, j0, k0);
    issue_tile(0, j0, std::integral_constant<int, 0>{});
    if (VIRT && n1 == 0) {
      load_bias_raw(j0);
      store_bias(0, j0);
    }
    if (VIRT && N > 1 && 1 >= n1) load_bias_raw(1 - n1);
  }
  // Two stages: even tiles use stage 0, odd tiles stage 1 (unrolled so each LDS read
  // names one stage).
  for (int n = 0; n < N; n += 2) {
    static_for<0, 2>([&](auto hc) {
      constexpr int half = decltype(hc)::value;
      const int t = n + half;
      if (t < N) {
        __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): this wave's loads of tile t landed
        __syncthreads();                         // ... everyone's; stage half ^ 1 is free
        // Refill the descriptor chunk that the tiles just finished used (before any
        // direct load is in flight, so its own waits cost nothing extra).
        if (t % DCH == 0 && t >= DCH && t + DCH < n1) fill_desc(t / DCH + 1);
        if (t + 1 < N) {
          int j1, k1;
          desc(t + 1, j1, k1);
          issue_tile(t + 1, j1, std::integral_constant<int, half ^ 1>{});
          if (VIRT && t + 1 >= n1) store_bias(half ^ 1, j1);
          if (VIRT && t + 2 < N && t + 2 >= n1) load_bias_raw(t + 2 - n1);
        }
        int jc, kc;
        desc(t, jc, kc);
        compute(hc, t >= n1, kc);
      }
    });
  }

  // Merge the two key halves of each query half. Wave (qh, kh) finishes Oᵀ tiles
  // [kh * NET/2, (kh + 1) * NET/2) and hands the other half of its accumulators over.
  constexpr int HE = NET / 2;
  constexpr int XS = HE * 16 + 3;              // floats per lane handed over
  __syncthreads();
  static_assert(XS * 64 * 4 <= TB, "hand-over buffer must fit one stage array");
  auto xbuf = [&](int q, int k) -> float* {      // one array per wave
    char* b = q ? (k ? sV1 : sK1) : (k ? sV0 : sK0);
    return reinterpret_cast<float*>(b);
  };
  {
    float* mine = xbuf(qh, kh) + lane;
#pragma unroll
    for (int u = 0; u < HE; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) mine[(u * 16 + r) * 64] = kh ? acc[u][r] : acc[HE + u][r];
    mine[(HE * 16 + 0) * 64] = m;
    mine[(HE * 16 + 1) * 64] = lsum;
    mine[(HE * 16 + 2) * 64] = asum;
  }
  __syncthreads();
  f32x16 res[HE];
  float mt, lt_part, at_part;
  {
    const float* other = xbuf(qh, 1 - kh) + lane;
    const float mo = other[(HE * 16 + 0) * 64];
    mt = fmaxf(m, mo);
    const float mu = mt == NEG_INF ? 0.f : mt;
    const float f = fast_exp2(m - mu), fo = fast_exp2(mo - mu);
#pragma unroll
    for (int u = 0; u < HE; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) res[u][r] = (kh ? acc[HE + u][r] : acc[u][r]) * f + other[(u * 16 + r) * 64] * fo;
    lt_part = lsum * f + other[(HE * 16 + 1) * 64] * fo;
    at_part = asum * f + other[(HE * 16 + 2) * 64] * fo;
  }
  if (VIRT) {
    // Phase 3: Oᵀ += H̄ (A_t q_t)ᵀ for this wave's Oᵀ tiles, H̄[e][c] as the A operand.
    const float at = sum_halves(at_part);
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      float qv[KH];
      M::unpack(qf[ks], qv);
#pragma unroll
      for (int u = 0; u < KH; ++u) qv[u] *= at;
      const AB b = M::pack(qv);
#pragma unroll
      for (int u = 0; u < HE; ++u)
        res[u] = M::mma(M::load(hbp + size_t(32 * (kh * HE + u) + l32) * D + KI * ks + KH * g), b, res[u]);
    }
  }
  const float lt = sum_halves(lt_part);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (a.lse && kh == 0 && g == 0)
    a.lse[size_t(h) * a.L + size_t(i) * kB + qrow] = (qvalid && lt > 0.f) ? mt * kLn2 + logf(lt) : NEG_INF;
  __syncthreads();                               // hand-over buffer consumed
  // Output tile staged in LDS (swizzled like a key tile) for coalesced 16-byte stores.
  char* sO = sK1;
#pragma unroll
  for (int u = 0; u < HE; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = 32 * (kh * HE + u) + acc_row(r, g);
      *reinterpret_cast<T*>(sO + KT::offset(qrow, e * ES)) = from_f32<T>(qvalid ? res[u][r] * inv : 0.f);
    }
  __syncthreads();
  char* Oh = reinterpret_cast<char*>(static_cast<T*>(a.O) + (size_t(h) * a.L + size_t(i) * kB) * D);
  constexpr int OCH = kB * KROW / 16;            // 16-byte chunks of the output tile
#pragma unroll
  for (int p = 0; p < OCH / 256; ++p) {
    const int c = tid + 256 * p;
    const int row = c / (KROW / 16), cb = (c % (KROW / 16)) * 16;
    *reinterpret_cast<u32x4*>(Oh + size_t(row) * KROW + cb) =
        *reinterpret_cast<const u32x4*>(sO + KT::offset(row, cb));
  }
}

template <class T, int D>
static hipError_t launch_attn_t(int mode, const AttnArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.H) * unsigned(a.nb));
  if (mode == MODE_LITERAL) {
    if (!std::is_same<T, float>::value && a.lse) {
      // bf16 with lse given: the selected blocks as DROP in the fast kernel (writes O,
      // lse), then the unselected blocks in their literal form, merged into O and lse.
      const hipError_t e = launch_attention_frag(MODE_DROP, a, s);
      if (e != hipSuccess) return e;
      return launch_literal_rest(a, s);
    } else {
      hipLaunchKernelGGL((attention_kernel<T, D, MODE_LITERAL>), grid, dim3(128), 0, s, a);
    }
  } else if (mode == MODE_PWT_ROW) {
    if (a.lse) {
      // Two passes: the exact tiles as DROP in the fast kernel (writes O, lse), then the
      // virtual tokens with the per-row w, merged into O and lse.
      if constexpr (std::is_same<T, float>::value) {
        hipLaunchKernelGGL((attention_split_kernel<T, D, MODE_DROP>), grid, dim3(256), 0, s, a);
        AttnArgs v = a;
        v.K_sel = 0;
        v.merge = 1;
        hipLaunchKernelGGL((attention_kernel<T, D, MODE_PWT_ROW>), grid, dim3(128), 0, s, v);
      } else {
        const hipError_t e = launch_attention_frag(MODE_DROP, a, s);
        if (e != hipSuccess) return e;
        return launch_virtual_row(a, s);
      }
    } else {
      hipLaunchKernelGGL((attention_kernel<T, D, MODE_PWT_ROW>), grid, dim3(128), 0, s, a);
    }
  } else if constexpr (std::is_same<T, float>::value) {   // fp32 DROP / PISA / PWT
    switch (mode) {
      case MODE_DROP: hipLaunchKernelGGL((attention_split_kernel<T, D, MODE_DROP>), grid, dim3(256), 0, s, a); break;
      case MODE_PISA: hipLaunchKernelGGL((attention_split_kernel<T, D, MODE_PISA>), grid, dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((attention_split_kernel<T, D, MODE_PWT>), grid, dim3(256), 0, s, a); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_attention(int bf16, int mode, const AttnArgs& a, hipStream_t s) {
  if (bf16 && mode != MODE_LITERAL && mode != MODE_PWT_ROW) return launch_attention_frag(mode, a, s);
  if (bf16) return a.d == 64 ? launch_attn_t<uint16_t, 64>(mode, a, s) : launch_attn_t<uint16_t, 128>(mode, a, s);
  return a.d == 64 ? launch_attn_t<float, 64>(mode, a, s) : launch_attn_t<float, 128>(mode, a, s);
}

}  // namespace pisa
