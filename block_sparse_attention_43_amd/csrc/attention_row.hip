// Virtual tokens with the per-row diagonal w (PWT_ROW), bf16: the second pass of that mode,
// after a DROP pass over the selected blocks (Sparse Linear Attention blog, PWT section).
#include "attention.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace pisa {
namespace {

__device__ __forceinline__ bf16x8 ld_frag(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

}  // namespace

// ---------------------------------------------------------------------------
// Virtual tokens with the per-row diagonal w (PWT_ROW), bf16, after the selected blocks
// ran as DROP (their normalised output and lse are in O and lse). For query t of tile i
// and every unselected block j: logit q_t·k̄_j + ln n_j + φ(w_{t,j}), w_{t,j} = ½ Σ_c
// q_{t,c}² σ²_{j,c} gated at ln n_j, value ΣV_j / n_j, weight / n_j into A_t; then
// + A_t H̄ q_t; then merged with the DROP pass under one softmax ([SLA] PWT section).
//
// One workgroup of two waves per query tile; wave kh takes key half kh (32 centroids) of
// every 64-centroid group for both query halves, with its own running max, and the halves
// merge at the end. Centroid and v̄ᵀ fragments come in MFMA operand order from the
// statistics pass (packed tiles), σ²/2 fragments are formed from σ² in the same row order,
// so no operand goes through LDS; a group's centroid and v̄ᵀ fragments are loaded into
// their registers as soon as the previous group's last product has read them.
// w = (σ²/2)(q²)ᵀ takes q² and σ²/2 as hi + lo bf16 parts (three products, within ~2^-16
// of fp32): w enters the exponent, q² rounded to bf16 alone moves P by ~3 %, and rows whose
// w lies near the gate's ln n_j flip with an error of 1e-3 in w (a factor n_j in that P).
template <int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1)))
void virtual_row_kernel(AttnArgs a) {
  constexpr int NKD = D / 16, NET = D / 32, NVF = 2 * NET;
  constexpr int TB = kB * D * 2, HB = TB / 2;
  constexpr float NEG_INF = -__builtin_huge_valf();
  __shared__ __align__(16) float sX[2 * NET * 16 * 64 + 6 * 64];   // hand-over, then output staging
  __shared__ float sW[kB];                                          // weight of the DROP pass per row
  __shared__ __align__(16) bf16x8 sSgl[2][D / 16][64];              // lo parts of σ²/2, per wave and lane

  const int lane = threadIdx.x & 63, g = lane >> 5, l32 = lane & 31;
  const int kh = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = a.nb, ngrp = a.nbp / kB;
  const uint32_t lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = int(lin / uint32_t(nb)), i = int(lin % uint32_t(nb));
  const int m = a.block_len ? min(max(a.block_len[i], 1), kB) : kB;

  const uint16_t* Qh = static_cast<const uint16_t*>(a.Q) + size_t(h) * a.L * D;
  const char* kbh = a.packed + a.pl.kbar + size_t(h) * ngrp * TB;
  const char* vbh = a.packed + a.pl.vbar + size_t(h) * ngrp * TB;
  const uint16_t* hbp = reinterpret_cast<const uint16_t*>(a.packed + a.pl.hbar) + size_t(h) * D * D;
  const uint32_t* mrow = a.mask + (size_t(h) * nb + i) * a.nw;
  const float* sig = a.ksig2 + size_t(h) * nb * D;

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
  float mx[2] = {NEG_INF, NEG_INF}, lsum[2] = {0.f, 0.f}, asum[2] = {0.f, 0.f};

  // Operands of group grp for this wave's key half: centroid and σ²/2 fragments (A of the
  // score and w products; lane 32 g + R holds centroid key_of_row(R)), v̄ᵀ fragments.
  bf16x8 kb[NKD], sg[NKD], vb[NVF];             // σ²/2 as hi (sg) + lo (in LDS: registers are full) parts
  uint32_t mword = 0u;
  int blen[16];
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbh, uint32_t(ngrp) * TB), rv = make_rsrc(vbh, uint32_t(ngrp) * TB);
  auto load_k = [&](int grp) {
    const int off = grp * TB + kh * HB + lane * 16;
#pragma unroll
    for (int f = 0; f < NKD; ++f) kb[f] = ld_frag(rk, off + f * 1024, 0);
  };
  auto load_v = [&](int grp) {
    const int off = grp * TB + kh * HB + lane * 16;
#pragma unroll
    for (int f = 0; f < NVF; ++f) vb[f] = ld_frag(rv, off + f * 1024, 0);
  };
  auto load_group = [&](int grp) {
    const int jr = grp * kB + 32 * kh + key_of_row(l32);       // this lane's A row
    const float* sr = sig + size_t(min(jr, nb - 1)) * D + 8 * g;
    const float hv = jr < nb ? 0.5f : 0.f;
#pragma unroll
    for (int f = 0; f < NKD; ++f) {
      const float4 x0 = *reinterpret_cast<const float4*>(sr + 16 * f);
      const float4 x1 = *reinterpret_cast<const float4*>(sr + 16 * f + 4);
      const float v[8] = {hv * x0.x, hv * x0.y, hv * x0.z, hv * x0.w, hv * x1.x, hv * x1.y, hv * x1.z, hv * x1.w};
      sg[f] = MmaBF16::pack(v);
      bf16x8 lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) lo[e] = static_cast<__bf16>(v[e] - static_cast<float>(sg[f][e]));
      sSgl[kh][f][lane] = lo;
    }
    // keys of this lane's score registers: 16 (r / 8) + 8 g + r % 8 of the half
    const int jw = grp * kB + 32 * kh;
    mword = mrow[min(jw, nb - 1) >> 5];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jj = min(jw + 16 * (r >> 3) + 8 * g + (r & 7), nb - 1);
      blen[r] = a.block_len ? a.block_len[jj] : kB;
    }
  };

  load_k(0);
  load_v(0);
  for (int grp = 0; grp < ngrp; ++grp) {
    load_group(grp);
    const int jw = grp * kB + 32 * kh;
    float lnn[16], invn[16];
    bool live[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jj = jw + 16 * (r >> 3) + 8 * g + (r & 7);
      live[r] = jj < nb && !((mword >> (jj & 31)) & 1u);
      const int nn = min(max(blen[r], 1), kB);
      lnn[r] = __logf(float(nn));
      invn[r] = __builtin_amdgcn_rcpf(float(nn));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x16 s = zero16(), w = zero16();
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        // q² as hi + lo parts (w enters the exponent), formed here for every group: the asm
        // keeps the compiler from hoisting all of them out of the loop (registers are full)
        bf16x8 qk = qf[u][ks];
        asm volatile("" : "+v"(qk));
        float qv[8];
        MmaBF16::unpack(qk, qv);
        bf16x8 q2h, q2l;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qv[e] *= qv[e];
          q2h[e] = static_cast<__bf16>(qv[e]);
          q2l[e] = static_cast<__bf16>(qv[e] - static_cast<float>(q2h[e]));
        }
        s = MmaBF16::mma(kb[ks], qf[u][ks], s);
        w = MmaBF16::mma(sg[ks], q2l, w);
        w = MmaBF16::mma(sSgl[kh][ks][lane], q2h, w);
        w = MmaBF16::mma(sg[ks], q2h, w);
      }
      if (u == 1 && grp + 1 < ngrp) load_k(grp + 1);
      float t[16], rmx = NEG_INF;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float wv = w[r];
        if (a.gate && wv > lnn[r]) wv = 0.f;
        const float phi = a.w_linear ? __logf(1.f + wv) : wv;
        t[r] = live[r] ? (s[r] + phi + lnn[r]) * kLog2e : NEG_INF;
        rmx = fmaxf(rmx, t[r]);
      }
      rmx = max_halves(rmx);
      if (rmx > mx[u]) {                             // uniform per query: both halves agree
        const float alpha = mx[u] > NEG_INF ? fast_exp2(mx[u] - rmx) : 0.f;
        mx[u] = rmx;
        lsum[u] *= alpha;
        asum[u] *= alpha;
#pragma unroll
        for (int et = 0; et < NET; ++et)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[et][u][r] *= alpha;
      }
      const float mu = mx[u] > NEG_INF ? mx[u] : 0.f;
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // P in bf16 as the PV product reads it; sums over the same values
        p[r] = to_f32(from_f32<uint16_t>(fast_exp2(t[r] - mu)));
        lsum[u] += p[r];
        asum[u] = fmaf(p[r], invn[r], asum[u]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 pb = MmaBF16::pack(p + 8 * ks);
#pragma unroll
        for (int et = 0; et < NET; ++et) acc[et][u] = MmaBF16::mma(vb[2 * et + ks], pb, acc[et][u]);
      }
      if (u == 1 && grp + 1 < ngrp) load_v(grp + 1);
    }
  }

  // Merge the key halves: wave 1 hands its state to wave 0, which finishes alone.
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
      sX[XO + (0 + u) * 64 + lane] = mx[u];
      sX[XO + (2 + u) * 64 + lane] = lsum[u];
      sX[XO + (4 + u) * 64 + lane] = asum[u];
    }
  }
  __syncthreads();
  float lt[2], at[2], mt[2];
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
      at[u] = sum_halves(asum[u] * f0 + sX[XO + (4 + u) * 64 + lane] * f1);
    }
    // Phase 3: Oᵀ += H̄ (A_t q_t)ᵀ, H̄[e][c] as the A operand.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        float qv[8];
        MmaBF16::unpack(qf[u][ks], qv);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] *= at[u];
        const bf16x8 b = MmaBF16::pack(qv);
#pragma unroll
        for (int et = 0; et < NET; ++et)
          acc[et][u] = MmaBF16::mma(*reinterpret_cast<const bf16x8*>(hbp + size_t(32 * et + l32) * D + 16 * ks + 8 * g), b,
                                    acc[et][u]);
      }
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
static hipError_t launch_vrow_d(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((virtual_row_kernel<D>), dim3(unsigned(a.H) * unsigned(a.nb)), dim3(128), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_virtual_row(const AttnArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_vrow_d<64>(a, s) : launch_vrow_d<128>(a, s);
}

}  // namespace pisa
