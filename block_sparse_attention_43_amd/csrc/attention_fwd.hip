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
#include "common.hpp"
#include "internal.hpp"

namespace pisa {

enum { MODE_DROP = 0, MODE_PISA = 1, MODE_PWT = 2, MODE_LITERAL = 3 };

// Key row (within a 32-key m-tile) that the lane with A-row R loads.
template <class M>
__device__ __forceinline__ int feed_row(int R) {
  const int r = 4 * (R >> 3) + (R & 3), gg = (R >> 2) & 1;
  return M::KI * (r / M::KH) + M::KH * gg + (r % M::KH);
}
// Key (within the 64-key tile) held by accumulator register r of m-tile mt in lane half g.
template <class M>
__device__ __forceinline__ int acc_key(int mt, int r, int g) {
  return 32 * mt + M::KI * (r / M::KH) + M::KH * g + (r % M::KH);
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
  constexpr bool VIRT = (MODE == MODE_PISA || MODE == MODE_PWT);
  constexpr float NEG_INF = -__builtin_huge_valf();

  __shared__ __align__(16) T sK[kB * LDK];
  __shared__ __align__(16) T sV[D * LDV];
  __shared__ float sBias[kB], sInvN[kB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const uint32_t lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = int(lin / uint32_t(a.nb)), i = int(lin % uint32_t(a.nb));
  int ni = a.block_len ? a.block_len[i] : kB;
  ni = min(max(ni, 1), kB);

  const T* Qh = static_cast<const T*>(a.Q) + size_t(h) * a.L * D;
  const T* Kh = static_cast<const T*>(a.K) + size_t(h) * a.L * D;
  const T* vt = reinterpret_cast<const T*>(a.packed + a.pl.vt) + size_t(h) * a.nb * D * kB;
  const T* kbp = reinterpret_cast<const T*>(a.packed + a.pl.kbar) + size_t(h) * a.nbp * D;
  const T* vbp = reinterpret_cast<const T*>(a.packed + a.pl.vbar) + size_t(h) * a.nbp * D;
  const T* hbp = reinterpret_cast<const T*>(a.packed + a.pl.hbar) + size_t(h) * D * D;
  const uint32_t* mrow = a.mask ? a.mask + (size_t(h) * a.nb + i) * a.nw : nullptr;
  const int32_t* irow = a.idx + (size_t(h) * a.nb + i) * a.K_sel;

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
  float m = NEG_INF, lsum = 0.f, asum = 0.f;   // running max (log2 units), partial sums

  const int n1 = a.K_sel;
  const int n2 = VIRT ? a.nbp / kB : (MODE == MODE_LITERAL ? a.nb - a.K_sel : 0);
  const int N = n1 + n2;

  int lit_cursor = 0;
  auto source = [&](int n) -> int {
    if (n < n1) return irow[n];
    if (VIRT) return n - n1;
    int j = lit_cursor;                       // next block whose mask bit is clear
    while (j < a.nb && ((mrow[j >> 5] >> (j & 31)) & 1u)) ++j;
    lit_cursor = j + 1;
    return j;
  };
  auto block_n = [&](int j) -> int {          // valid tokens of block j; 0 if j is out of range
    if (j < 0 || j >= a.nb) return 0;
    const int n = a.block_len ? a.block_len[j] : kB;
    return min(max(n, 1), kB);
  };

  uint4 rk[PF], rv[PF];
  auto prefetch = [&](int n, int src) {
    const T* pk;
    const T* pv;
    if (VIRT && n >= n1) {
      pk = kbp + size_t(src) * kB * D;
      pv = vbp + size_t(src) * D * kB;
    } else {
      const int j = (src >= 0 && src < a.nb) ? src : 0;
      pk = Kh + size_t(j) * kB * D;
      pv = vt + size_t(j) * D * kB;
    }
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int c = tid + 128 * p;
      rk[p] = *reinterpret_cast<const uint4*>(pk + (c / CPRK) * D + (c % CPRK) * EPC);
      rv[p] = *reinterpret_cast<const uint4*>(pv + (c / CPRV) * kB + (c % CPRV) * EPC);
    }
  };

  int src = 0;
  if (N > 0) {
    src = source(0);
    prefetch(0, src);
  }
  for (int n = 0; n < N; ++n) {
    const int cur = src;
    const bool second = n >= n1;
    __syncthreads();                          // previous tile fully consumed
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int c = tid + 128 * p;
      *reinterpret_cast<uint4*>(sK + (c / CPRK) * LDK + (c % CPRK) * EPC) = rk[p];
      *reinterpret_cast<uint4*>(sV + (c / CPRV) * LDV + (c % CPRV) * EPC) = rv[p];
    }
    if (VIRT && second && tid < kB) {
      // log2-domain bias ln n_j + φ_{i,j} of the 64 centroids of this group;
      // -inf for selected blocks and for the padding beyond nb.
      const int jj = cur * kB + tid;
      float b = NEG_INF, invn = 0.f;
      if (jj < a.nb && !((mrow[jj >> 5] >> (jj & 31)) & 1u)) {
        const int nj = block_n(jj);
        const float lnn = logf(float(nj));
        float phi = 0.f;
        if (MODE == MODE_PWT) {
          float w = a.wt[(size_t(h) * a.nb + i) * a.nb + jj];
          if (a.gate && w > lnn) w = 0.f;
          phi = a.w_linear ? log1pf(w) : w;
        }
        b = (lnn + phi) * kLog2e;
        invn = 1.f / float(nj);
      }
      sBias[tid] = b;
      sInvN[tid] = invn;
    }
    __syncthreads();
    if (n + 1 < N) {
      src = source(n + 1);
      prefetch(n + 1, src);
    }

    // Sᵀ[key][q] for the two 32-key halves of the tile.
    f32x16 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = zero16();
      const T* krow = sK + (32 * mt + feed_row<M>(l32)) * LDK + KH * g;
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) s[mt] = M::mma(M::load(krow + KI * ks), qf[ks], s[mt]);
    }

    float pr[2][16];
    float mx = NEG_INF;
    if (!second || VIRT) {
      const int nj = second ? kB : block_n(cur);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = acc_key<M>(mt, r, g);
          float t;
          if (second) t = s[mt][r] * kLog2e + sBias[key];
          else t = key < nj ? s[mt][r] * kLog2e : NEG_INF;
          pr[mt][r] = t;
          mx = fmaxf(mx, t);
        }
      mx = max_halves(mx);
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == NEG_INF ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      m = m_new;
      float ps = 0.f, pa = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(pr[mt][r] - m_use);
          pr[mt][r] = p;
          ps += p;
          if (VIRT && second) pa += p * sInvN[acc_key<M>(mt, r, g)];
        }
      lsum = lsum * alpha + ps;
      if (VIRT) asum = asum * alpha + pa;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int et = 0; et < NET; ++et)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[et][r] *= alpha;
      }
    } else {
      // LITERAL: block-wise first-order weights with the per-row second-order factor.
      const int nj = block_n(cur);
      const float invn = nj > 0 ? 1.f / float(nj) : 0.f;
      float ssum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_key<M>(mt, r, g) < nj) ssum += s[mt][r];
      ssum = sum_halves(ssum);
      const float mean = ssum * invn;
      float y2 = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_key<M>(mt, r, g) < nj) {
            const float y = s[mt][r] - mean;
            y2 += y * y;
          }
      y2 = sum_halves(y2);
      float w = 0.5f * y2 * invn;
      const float lnn = nj > 0 ? logf(float(nj)) : 0.f;
      if (a.gate && w > lnn) w = 0.f;
      const float phi = a.w_linear ? log1pf(w) : w;
      const float ell = nj > 0 ? (mean + phi + lnn) * kLog2e : NEG_INF;
      const float m_new = fmaxf(m, ell);
      const float m_use = m_new == NEG_INF ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      m = m_new;
      const float cw = nj > 0 ? fast_exp2((mean + phi) * kLog2e - m_use) : 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pr[mt][r] = acc_key<M>(mt, r, g) < nj ? cw * (1.f + (s[mt][r] - mean)) : 0.f;
      lsum = lsum * alpha + (g == 0 ? float(nj) * cw : 0.f);
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int et = 0; et < NET; ++et)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[et][r] *= alpha;
      }
    }

    // Oᵀ += Vᵀ Pᵀ : the B operand of k-step ks is registers [(ks % KPM) * KH, +KH) of m-tile ks / KPM.
#pragma unroll
    for (int ks = 0; ks < NKB; ++ks) {
      const AB b = M::pack(&pr[ks / KPM][(ks % KPM) * KH]);
#pragma unroll
      for (int et = 0; et < NET; ++et)
        acc[et] = M::mma(M::load(sV + (32 * et + l32) * LDV + KI * ks + KH * g), b, acc[et]);
    }
  }

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
  __syncthreads();
#pragma unroll
  for (int et = 0; et < NET; ++et)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      sK[qrow * LDK + 32 * et + acc_row(r, g)] = from_f32<T>(qvalid ? acc[et][r] * inv : 0.f);
  if (a.lse && g == 0)
    a.lse[size_t(h) * a.L + size_t(i) * kB + qrow] = (qvalid && lt > 0.f) ? m * kLn2 + logf(lt) : NEG_INF;
  __syncthreads();
  T* Oh = static_cast<T*>(a.O) + (size_t(h) * a.L + size_t(i) * kB) * D;
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int c = tid + 128 * p;
    *reinterpret_cast<uint4*>(Oh + (c / CPRK) * D + (c % CPRK) * EPC) =
        *reinterpret_cast<const uint4*>(sK + (c / CPRK) * LDK + (c % CPRK) * EPC);
  }
}

template <class T, int D>
static hipError_t launch_attn_t(int mode, const AttnArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.H) * unsigned(a.nb)), block(128);
  switch (mode) {
    case MODE_DROP: hipLaunchKernelGGL((attention_kernel<T, D, MODE_DROP>), grid, block, 0, s, a); break;
    case MODE_PISA: hipLaunchKernelGGL((attention_kernel<T, D, MODE_PISA>), grid, block, 0, s, a); break;
    case MODE_PWT: hipLaunchKernelGGL((attention_kernel<T, D, MODE_PWT>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((attention_kernel<T, D, MODE_LITERAL>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_attention(int bf16, int mode, const AttnArgs& a, hipStream_t s) {
  if (bf16) return a.d == 64 ? launch_attn_t<uint16_t, 64>(mode, a, s) : launch_attn_t<uint16_t, 128>(mode, a, s);
  return a.d == 64 ? launch_attn_t<float, 64>(mode, a, s) : launch_attn_t<float, 128>(mode, a, s);
}

}  // namespace pisa
