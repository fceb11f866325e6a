// LITERAL for bf16 inputs, second pass: the unselected blocks in their block-wise
// first- and second-order form, merged into the output and lse of a DROP pass over the
// selected blocks (PISA paper §3.2 Eq. (3.2) and its "Practical Challenge": the literal
// per-block compensation, here computed from the raw keys of every unselected block).
//
// For query t of tile i and unselected block j with n_j valid keys: s̄ = mean_n q·k_n,
// y_n = q·k_n - s̄, w = ½ mean_n y_n² (= ½ qᵀC_j q), gated to 0 when w > ln n_j (or taken
// as φ = ln(1 + w) on request). The block adds n_j e^{s̄+φ} to the denominator and
// e^{s̄+φ} Σ_n (1 + y_n) v_n (= e^{s̄+φ}(ΣV_j + H_j q)) to the numerator; everything runs
// under one running max per row and is merged at the end with the DROP pass's
// normalised output and lse (softmax over the union of the two key sets).
//
// Organisation: one workgroup of two waves per 64-row query tile, one wave per SIMD.
// Wave w takes the unselected blocks of index parity w, *both* key halves of each, for
// both query halves, so a block's row statistics (sums over its 64 keys) stay inside one
// wave. K and Vᵀ of a block arrive in MFMA operand order from the statistics call's
// packed tiles (1 KB buffer loads straight into registers); the block is worked key half
// by key half, and each half's K (Vᵀ) registers are refilled with the next block's as
// soon as this block's products with them are issued.
// Scores Sᵀ = K Qᵀ are 32-key x 32-query tiles whose registers, in the packed tiles' key
// order, are directly the B operand of Oᵀ += Vᵀ Pᵀ. At the end wave 1 hands its state to
// wave 0, which merges it with its own and then with the DROP pass.
#include "attention.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace pisa {

namespace {

__device__ __forceinline__ bf16x8 lit_frag(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

template <int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1)))
void literal_rest_kernel(AttnArgs a) {
  constexpr int NKD = D / 16, NET = D / 32, NVF = 2 * NET;
  constexpr int TB = kB * D * 2, HB = TB / 2;
  constexpr float NEG_INF = -__builtin_huge_valf();
  __shared__ __align__(16) float sX[2 * NET * 16 * 64 + 4 * 64];   // hand-over, then output rows
  __shared__ float sW[kB];                                          // weight of the DROP pass per row

  const int lane = threadIdx.x & 63, g = lane >> 5, l32 = lane & 31;
  const int kh = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = a.nb;
  const uint32_t lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = int(lin / uint32_t(nb)), i = int(lin % uint32_t(nb));
  const int m = a.block_len ? min(max(a.block_len[i], 1), kB) : kB;

  const uint16_t* Qh = static_cast<const uint16_t*>(a.Q) + size_t(h) * a.L * D;
  const char* kfh = a.packed + a.pl.kf + size_t(h) * nb * TB;
  const char* vth = a.packed + a.pl.vt + size_t(h) * nb * TB;
  const uint32_t* mrow = a.mask + (size_t(h) * nb + i) * a.nw;

  bf16x8 qf[2][NKD];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 32 * u + l32;
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      bf16x8 v = {};
      if (row < m) v = *reinterpret_cast<const bf16x8*>(Qh + (size_t(i) * kB + row) * D + 16 * ks + 8 * g);
      qf[u][ks] = v;
    }
  }
  f32x16 acc[NET][2];
#pragma unroll
  for (int et = 0; et < NET; ++et) acc[et][0] = acc[et][1] = zero16();
  float mx[2] = {NEG_INF, NEG_INF}, lsum[2] = {0.f, 0.f};

  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kfh, uint32_t(nb) * TB), rv = make_rsrc(vth, uint32_t(nb) * TB);
  bf16x8 kf[2][NKD], vf[2][NVF];
  // One key half's K (or Vᵀ) fragments of block j; a half's registers are refilled for
  // the next block as soon as this block's products with them are issued.
  auto load_k = [&](int j, int hh) {
#pragma unroll
    for (int f = 0; f < NKD; ++f) kf[hh][f] = lit_frag(rk, j * TB + hh * HB + lane * 16 + f * 1024);
  };
  auto load_v = [&](int j, int hh) {
#pragma unroll
    for (int f = 0; f < NVF; ++f) vf[hh][f] = lit_frag(rv, j * TB + hh * HB + lane * 16 + f * 1024);
  };
  // The next unselected block of this wave's parity at or after j (nb when none).
  auto next_block = [&](int j) -> int {
    for (; j < nb; j += 2)
      if (!((mrow[j >> 5] >> (j & 31)) & 1u)) return j;
    return nb;
  };

  int j = next_block(kh);
  if (j < nb) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      load_k(j, hh);
      load_v(j, hh);
    }
  }
  while (j < nb) {
    const int jn = next_block(j + 2);
    const int jl = jn < nb ? jn : j;     // loads past the last block repeat it, unused
    const int nj = a.block_len ? min(max(a.block_len[j], 1), kB) : kB;
    const float invn = __builtin_amdgcn_rcpf(float(nj)), lnn = __logf(float(nj));
    // Sᵀ of key half hh for both query halves; register r of lane half g holds key
    // 32 hh + 16 (r / 8) + 8 g + r % 8 of the block, query 32 u + l32. The packed tiles
    // hold zeros past a block's valid keys (K and Vᵀ alike), so those keys score exactly
    // 0, add nothing to Σ s and Σ s², and their P meets a zero column of Vᵀ: no masks.
    f32x16 s[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x16 t = zero16();
#pragma unroll
        for (int f = 0; f < NKD; ++f) t = MmaBF16::mma(kf[hh][f], qf[u][f], t);
        s[u][hh] = t;
      }
      load_k(jl, hh);
    }
    // Row statistics in one pass: Σ s and Σ s² in four partial sums each (both lane
    // halves end with the same totals); mean(y²) = Σ s² / n - s̄². The cancellation costs
    // a few of fp32's digits at these score magnitudes, far below the bf16 output.
    float cw[2], c0[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float p1[4] = {0.f, 0.f, 0.f, 0.f}, p2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p1[r & 3] += s[u][hh][r];
          p2[r & 3] = fmaf(s[u][hh][r], s[u][hh][r], p2[r & 3]);
        }
      const float mean = sum_halves((p1[0] + p1[1]) + (p1[2] + p1[3])) * invn;
      float w = 0.5f * fmaxf(sum_halves((p2[0] + p2[1]) + (p2[2] + p2[3])) * invn - mean * mean, 0.f);
      if (a.gate && w > lnn) w = 0.f;
      const float phi = a.w_linear ? log1pf(w) : w;
      const float cand = (mean + phi + lnn) * kLog2e;     // log2 of the block's total weight
      if (cand > mx[u]) {                                  // uniform per query
        const float alpha = mx[u] > NEG_INF ? fast_exp2(mx[u] - cand) : 0.f;
        mx[u] = cand;
        lsum[u] *= alpha;
#pragma unroll
        for (int et = 0; et < NET; ++et)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[et][u][r] *= alpha;
      }
      cw[u] = fast_exp2((mean + phi) * kLog2e - mx[u]);
      c0[u] = cw[u] - cw[u] * mean;                        // P = cw (1 + s - s̄) = cw s + c0
      if (g == 0) lsum[u] += float(nj) * cw[u];
    }
    // Oᵀ += Vᵀ Pᵀ, key half by key half
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(fmaf(cw[u], s[u][hh][8 * ks + e], c0[u]));
#pragma unroll
          for (int et = 0; et < NET; ++et) acc[et][u] = MmaBF16::mma(vf[hh][2 * et + ks], pb, acc[et][u]);
        }
      }
      load_v(jl, hh);
    }
    j = jn;
  }

  // Merge the two waves: wave 1 hands its state to wave 0, which finishes alone.
  constexpr int XO = 2 * NET * 16 * 64;
  if (kh == 1) {
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) sX[((et * 2 + u) * 16 + r) * 64 + lane] = acc[et][u][r];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sX[XO + u * 64 + lane] = mx[u];
      sX[XO + (2 + u) * 64 + lane] = lsum[u];
    }
  }
  __syncthreads();
  float lt[2], mt[2];
  if (kh == 0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float mo = sX[XO + u * 64 + lane];
      mt[u] = fmaxf(mx[u], mo);
      const float base = mt[u] > NEG_INF ? mt[u] : 0.f;
      const float f0 = mx[u] > NEG_INF ? fast_exp2(mx[u] - base) : 0.f;
      const float f1 = mo > NEG_INF ? fast_exp2(mo - base) : 0.f;
#pragma unroll
      for (int et = 0; et < NET; ++et)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[et][u][r] = acc[et][u][r] * f0 + sX[((et * 2 + u) * 16 + r) * 64 + lane] * f1;
      lt[u] = sum_halves(lsum[u] * f0 + sX[XO + (2 + u) * 64 + lane] * f1);
    }
  }
  __syncthreads();                                   // hand-over consumed
  if (kh == 0) {
    // Own share w_v / lt per row and the DROP pass's weight w_e, both over their sum; the
    // scaled own output is staged in LDS as fp32 rows [64][D].
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = 32 * u + l32;
      const size_t row = size_t(h) * a.L + size_t(i) * kB + q;
      const float le = a.lse[row];
      const float lv = (q < m && lt[u] > 0.f) ? mt[u] * kLn2 + logf(lt[u]) : NEG_INF;
      const float M = fmaxf(le, lv);
      float we = M > NEG_INF && le > NEG_INF ? expf(le - M) : 0.f;
      float wv = M > NEG_INF && lv > NEG_INF ? expf(lv - M) : 0.f;
      const float den = we + wv, id = den > 0.f ? 1.f / den : 0.f;
      we *= id;
      wv *= id;
      const float sc = lt[u] > 0.f ? wv / lt[u] : 0.f;
#pragma unroll
      for (int et = 0; et < NET; ++et)
#pragma unroll
        for (int r = 0; r < 16; ++r) sX[q * D + 32 * et + acc_row(r, g)] = q < m ? acc[et][u][r] * sc : 0.f;
      if (g == 0) {
        sW[q] = q < m ? we : 0.f;
        a.lse[row] = q < m && den > 0.f ? M + logf(den) : NEG_INF;
      }
    }
  }
  __syncthreads();
  uint16_t* Oh = static_cast<uint16_t*>(a.O) + (size_t(h) * a.L + size_t(i) * kB) * D;
  for (int x = threadIdx.x; x < kB * D / 8; x += 128) {
    const int q = x / (D / 8), c0 = (x % (D / 8)) * 8;
    u32x4 prev = *reinterpret_cast<const u32x4*>(Oh + size_t(q) * D + c0);
    const uint16_t* pe = reinterpret_cast<const uint16_t*>(&prev);
    u32x4 outv;
    uint16_t* po = reinterpret_cast<uint16_t*>(&outv);
    const float we = sW[q];
#pragma unroll
    for (int e = 0; e < 8; ++e) po[e] = f32_to_bf16(sX[q * D + c0 + e] + we * to_f32(pe[e]));
    *reinterpret_cast<u32x4*>(Oh + size_t(q) * D + c0) = outv;
  }
}

template <int D>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((literal_rest_kernel<D>), dim3(unsigned(a.H) * unsigned(a.nb)), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_literal_rest(const AttnArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_t<64>(a, s) : launch_t<128>(a, s);
}

}  // namespace pisa
