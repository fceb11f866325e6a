// Backward of LITERAL (bf16 inputs): the block-wise first order of the PISA paper (§3.2
// Eq. (3.2)) with the per-row second-order weight of the Sparse Linear Attention blog (PWT
// section), differentiated with the selection and the gate's decisions held fixed.
//
// For query t of tile i and key n of block j (x_{t,n} = q_t·k_n over the n_j valid keys):
//   selected j:   P = e^{x - lse_t};  dx = P (dO_t·v_n - Δ_t),  dV weight P
//   unselected j: s̄ = mean_n x, y_n = x_n - s̄, w = ½ mean_n y_n² (gated to 0 when
//                 w > ln n_j), φ = ln(1 + w) or w, E = e^{s̄ + φ - lse_t},
//                 T = Σ_n (1 + y_n) dO_t·v_n,  dℓ = E (T - n_j Δ_t),  dw = φ'(w) dℓ,
//                 dy_n = E dO_t·v_n + dw y_n / n_j,
//                 dx_n = dy_n - mean_m dy_m + dℓ / n_j,  dV weight E (1 + y_n)
// with Δ_t = dO_t·o_t = Σ_sel Σ_n P dO·v_n + Σ_unsel E T. Then dq_t = Σ dx k_n,
// dk_n = Σ_t dx q_t, dv_n = Σ_t (weight) dO_t. The unselected block's part is the
// derivative of E Σ_n (1 + y_n) v_n = e^{s̄ + φ}(ΣV_j + H_j q_t) over the denominator's
// n_j e^{s̄ + φ}, written on the raw keys (no H_j, C_j).
//
// Three launches, every product on bf16 MFMA with fp32 accumulation, operands staged in LDS:
//   literal_bwd_query_kernel<D, 0>   per query tile, all blocks: Δ_t (fp32, exact)
//   literal_bwd_query_kernel<D, 1>   per query tile, all blocks: dQ
//   literal_bwd_key_kernel<D>        per key block, all query tiles: dK, dV
// Each (query tile, key block) step: stage the operand tiles, S = Q Kᵀ and A = dO Vᵀ
// (64 x 64, one 32 x 32 quarter per wave) to LDS in fp32, the per-row pass above (four
// threads per query row, 16 keys each, sums over the block by lane shuffles), dx (and
// the dV weights) in bf16 to LDS, the gradient products. The sums run in a fixed order,
// so repeated runs are bit-identical. Unselected blocks cost as much as selected ones:
// this backward is dense in work, as LITERAL's forward is.
#include "attention.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace pisa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kSS = kB + 1;              // fp32 row stride of the score tiles (odd: no conflicts)
constexpr int kTS = kB + 8;              // bf16 row stride of 64-wide tiles (16-byte rows, spread banks)

// Offset of element k (< 64) within row `row` of a transposed tile written by put_cols:
// groups of eight are XOR-swizzled by row / 8, so the eight rows one thread writes per
// 16-byte chunk (rows eight apart between neighbouring threads) fall in different banks;
// a reader of eight consecutive k from k0 (a multiple of 8) gets them contiguous at
// tpos(row, k0).
__device__ __forceinline__ int tpos(int row, int k) { return k ^ (((row >> 3) & 7) << 3); }

template <int D>
struct LitLds {
  static constexpr int RS = D + 8;       // bf16 row stride of [64][D] tiles
};

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Rows [0, nv) of a [64][D] bf16 block at src (row stride D) into dst (row stride D + 8);
// the other rows zero. Every thread of the workgroup takes part.
template <int D>
__device__ __forceinline__ void stage_rows(uint16_t* dst, const uint16_t* src, int nv) {
  constexpr int CPR = D / 8;
  for (int c = threadIdx.x; c < kB * CPR; c += 256) {
    const int r = c / CPR, col = (c % CPR) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < nv) v = *reinterpret_cast<const u32x4*>(src + size_t(r) * D + col);
    *reinterpret_cast<u32x4*>(dst + r * LitLds<D>::RS + col) = v;
  }
}

// The same staging split in two, so that the next tile's loads run during the current
// tile's products: load_rows takes this thread's 16-byte chunks of rows [0, nv) (zeros
// past nv; every load is in bounds, the block being 64 rows of a padded tensor);
// put_rows writes them as stage_rows does, put_cols as the transpose dst[c][tpos(c, r)] (row
// stride 72).
template <int D>
struct RowRegs {
  static constexpr int CPR = D / 8, N = kB * CPR / 256;
  u32x4 v[N];
};
template <int D>
__device__ __forceinline__ void load_rows(RowRegs<D>& t, const uint16_t* src, int nv) {
#pragma unroll
  for (int k = 0; k < RowRegs<D>::N; ++k) {
    const int c = threadIdx.x + 256 * k, r = c / RowRegs<D>::CPR, col = (c % RowRegs<D>::CPR) * 8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + size_t(r) * D + col);
    t.v[k] = r < nv ? v : u32x4{0u, 0u, 0u, 0u};
  }
}
template <int D>
__device__ __forceinline__ void put_rows(uint16_t* dst, const RowRegs<D>& t) {
#pragma unroll
  for (int k = 0; k < RowRegs<D>::N; ++k) {
    const int c = threadIdx.x + 256 * k, r = c / RowRegs<D>::CPR, col = (c % RowRegs<D>::CPR) * 8;
    *reinterpret_cast<u32x4*>(dst + r * LitLds<D>::RS + col) = t.v[k];
  }
}
template <int D>
__device__ __forceinline__ void put_cols(uint16_t* dst, const RowRegs<D>& t) {
#pragma unroll
  for (int k = 0; k < RowRegs<D>::N; ++k) {
    const int c = threadIdx.x + 256 * k, r = c / RowRegs<D>::CPR, col = (c % RowRegs<D>::CPR) * 8;
    const uint16_t* e = reinterpret_cast<const uint16_t*>(&t.v[k]);
#pragma unroll
    for (int u = 0; u < 8; ++u) dst[(col + u) * kTS + tpos(col + u, r)] = e[u];
  }
}

// S = X Yᵀ for the 32 x 32 quarter (row half qh, column half kh) of two [64][D] LDS tiles,
// written to out[64][65] in fp32.
template <int D>
__device__ __forceinline__ void quarter_product(const uint16_t* X, const uint16_t* Y, float* out, int qh, int kh) {
  const int lane = threadIdx.x & 63, g = lane >> 5, c = lane & 31;
  constexpr int RS = LitLds<D>::RS;
  f32x16 acc = zero16();
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds8(X + (32 * qh + c) * RS + 16 * ks + 8 * g),
                                                  lds8(Y + (32 * kh + c) * RS + 16 * ks + 8 * g), acc, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) out[(32 * qh + acc_row(r, g)) * kSS + 32 * kh + c] = acc[r];
}

// Per-row pass of one (query row, 16-key part): the gradient of the scores (dx) and the dV
// weights of keys [16 p, 16 p + 16), or (DELTA) only this part's share of Σ P dO·v (returned)
// and of the softmax mass Σ P (added to mass). Sums over the block's 64 keys combine the
// four parts of the row (lanes 4 q .. 4 q + 3).
struct RowIn {
  float lse, delta;
  int nj;                                // valid keys of the block
  bool live, sel;                        // row has support; block selected by the tile
  int gate, linear;
};

__device__ __forceinline__ float sum4(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  return v;
}

template <bool DELTA>
__device__ __forceinline__ float row_pass(const float* x, const float* av, const RowIn& in, int p, float* dx, float* wv,
                                          float& mass) {
  float part = 0.f;
  if (in.sel) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const bool ok = in.live && 16 * p + u < in.nj;
      const float P = ok ? __expf(x[u] - in.lse) : 0.f;
      if constexpr (DELTA) {
        part = fmaf(P, av[u], part);
        mass += P;
      } else {
        dx[u] = P * (av[u] - in.delta);
        wv[u] = P;
      }
    }
    return part;
  }
  const float invn = 1.f / float(in.nj);
  float sx = 0.f;
#pragma unroll
  for (int u = 0; u < 16; ++u) sx += (16 * p + u < in.nj) ? x[u] : 0.f;
  const float sbar = sum4(sx) * invn;
  float y[16], syy = 0.f, t = 0.f;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    y[u] = (16 * p + u < in.nj) ? x[u] - sbar : 0.f;
    syy = fmaf(y[u], y[u], syy);
    t += (16 * p + u < in.nj) ? (1.f + y[u]) * av[u] : 0.f;
  }
  float w = 0.5f * sum4(syy) * invn;
  t = sum4(t);
  const bool fired = in.gate && w > __logf(float(in.nj));
  if (fired) w = 0.f;
  const float phi = in.linear ? log1pf(w) : w;
  const float dphi = fired ? 0.f : (in.linear ? 1.f / (1.f + w) : 1.f);
  const float E = in.live ? __expf(sbar + phi - in.lse) : 0.f;
  if constexpr (DELTA) {
    if (p == 0) mass += float(in.nj) * E;
    return (p == 0) ? E * t : 0.f;
  }
  const float dl = E * (t - float(in.nj) * in.delta), dw = dl * dphi;
  float sdy = 0.f;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    dx[u] = (16 * p + u < in.nj) ? fmaf(E, av[u], dw * y[u] * invn) : 0.f;
    sdy += dx[u];
  }
  const float shift = dl * invn - sum4(sdy) * invn;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const bool ok = 16 * p + u < in.nj;
    dx[u] = ok ? dx[u] + shift : 0.f;
    wv[u] = ok ? E * (1.f + y[u]) : 0.f;
  }
  return 0.f;
}

}  // namespace

// PASS 0: Δ of every row of query tile i; PASS 1: its dQ. One workgroup per (head, tile).
// SEL (PASS 0 only): the selected blocks' sums alone, for PWT_ROW, whose unselected blocks
// are virtual tokens handled by rowdiag_bwd_query_kernel.
template <int D, int PASS, bool SEL>
__global__ __launch_bounds__(256) void literal_bwd_query_kernel(BwdArgs a) {
  constexpr int RS = LitLds<D>::RS, NT = D / 64;
  __shared__ __align__(16) uint16_t sQ[kB * RS], sG[kB * RS], sK[kB * RS], sV[kB * RS];
  __shared__ __align__(16) uint16_t sKT[PASS ? D * kTS : 8];
  __shared__ __align__(16) uint16_t sDX[PASS ? kB * kTS : 8];
  __shared__ float sS[kB * kSS], sA[kB * kSS];
  __shared__ float sLse[kB], sDelta[kB];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = tid >> 6, qh = wave >> 1, kh = wave & 1;
  const int nb = a.nb, h = int(blockIdx.x) / nb, i = int(blockIdx.x) % nb;
  auto rows_of = [&](int b) { return a.block_len ? min(max(a.block_len[b], 1), kB) : kB; };
  const int mi = rows_of(i);
  const size_t row0 = size_t(h) * a.L + size_t(i) * kB;
  const uint16_t* Qb = static_cast<const uint16_t*>(a.Q) + row0 * D;
  const uint16_t* Gb = static_cast<const uint16_t*>(a.dO) + row0 * D;
  const uint16_t* Kh = static_cast<const uint16_t*>(a.K) + size_t(h) * a.L * D;
  const uint16_t* Vh = static_cast<const uint16_t*>(a.V) + size_t(h) * a.L * D;
  const uint32_t* mrow = a.mask + (size_t(h) * nb + i) * a.nw;

  stage_rows<D>(sQ, Qb, mi);
  stage_rows<D>(sG, Gb, mi);
  if (tid < kB) {
    sLse[tid] = tid < mi ? (PASS ? a.lse2 : a.lse)[row0 + tid] : kNegInf;
    sDelta[tid] = PASS ? a.delta[row0 + tid] : 0.f;
  }
  __syncthreads();
  const int q = tid >> 2, p = tid & 3;
  f32x16 acc[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) acc[u] = zero16();
  float dpart = 0.f, mpart = 0.f;

  // Blocks visited (SEL: the selected ones only; the same for the whole workgroup); each
  // block's K and V rows are loaded while the previous block's products run.
  auto next_block = [&](int b) {
    ++b;
    if (SEL)
      while (b < nb && !((mrow[b >> 5] >> (b & 31)) & 1u)) ++b;
    return b;
  };
  RowRegs<D> kr, vr;
  int jn = next_block(-1);
  if (jn < nb) {
    load_rows<D>(kr, Kh + size_t(jn) * kB * D, rows_of(jn));
    load_rows<D>(vr, Vh + size_t(jn) * kB * D, rows_of(jn));
  }
  for (int j = jn; j < nb; j = jn) {
    const int nj = rows_of(j);
    jn = next_block(j);
    __syncthreads();                     // previous step's tiles consumed
    put_rows<D>(sK, kr);
    put_rows<D>(sV, vr);
    if constexpr (PASS == 1) put_cols<D>(sKT, kr);
    if (jn < nb) {
      load_rows<D>(kr, Kh + size_t(jn) * kB * D, rows_of(jn));
      load_rows<D>(vr, Vh + size_t(jn) * kB * D, rows_of(jn));
    }
    __syncthreads();
    quarter_product<D>(sQ, sK, sS, qh, kh);
    quarter_product<D>(sG, sV, sA, qh, kh);
    __syncthreads();
    RowIn in;
    in.lse = sLse[q];
    in.delta = sDelta[q];
    in.nj = nj;
    in.live = q < mi && in.lse > kNegInf;
    in.sel = (mrow[j >> 5] >> (j & 31)) & 1u;
    in.gate = a.gate;
    in.linear = a.w_linear;
    float x[16], av[16], dx[16], wv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      x[u] = sS[q * kSS + 16 * p + u];
      av[u] = sA[q * kSS + 16 * p + u];
    }
    if constexpr (PASS == 0) {
      dpart += row_pass<true>(x, av, in, p, dx, wv, mpart);
    } else {
      row_pass<false>(x, av, in, p, dx, wv, mpart);
      bf16x8 lo, hi;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        lo[u] = static_cast<__bf16>(dx[u]);
        hi[u] = static_cast<__bf16>(dx[8 + u]);
      }
      *reinterpret_cast<bf16x8*>(sDX + q * kTS + 16 * p) = lo;
      *reinterpret_cast<bf16x8*>(sDX + q * kTS + 16 * p + 8) = hi;
      __syncthreads();
      // dQ rows [32 qh, +32), columns [64 kh, +64) of d (the NT 32-column tiles) += dx K
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int dt = kh * NT + u;
#pragma unroll
        for (int ks = 0; ks < kB / 16; ++ks)
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds8(sDX + (32 * qh + c) * kTS + 16 * ks + 8 * g),
                                                           lds8(sKT + (32 * dt + c) * kTS + tpos(32 * dt + c, 16 * ks + 8 * g)),
                                                           acc[u], 0, 0, 0);
      }
    }
  }
  if constexpr (PASS == 0) {
    // The forward normalised with the row sums of its bf16 P, so these fp32 P sum to
    // 1 + O(2^-9), and that offset, times the keys' common mean, would reach dQ: the later
    // sweeps take lse' = lse + ln Σ P and Δ = Σ P dO·v / Σ P, so their P sum to 1.
    // SEL leaves the raw sums (Δ part in delta, mass in lse2) for the virtual tokens' sweep.
    const float d = sum4(dpart), m = sum4(mpart);
    const bool live = q < mi && sLse[q] > kNegInf;
    if (p == 0) {
      if (SEL) {
        a.delta[row0 + q] = live ? d : 0.f;
        a.lse2[row0 + q] = live ? m : 0.f;
      } else {
        a.delta[row0 + q] = live ? d / m : 0.f;
        a.lse2[row0 + q] = live ? sLse[q] + logf(m) : kNegInf;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int col = 32 * (kh * NT + u) + c;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * qh + acc_row(r, g);
        a.dQ[(row0 + row) * D + col] = row < mi ? acc[u][r] : 0.f;
      }
    }
  }
}

// dK and dV of key block j over every query tile. One workgroup per (head, block).
template <int D>
__global__ __launch_bounds__(256) void literal_bwd_key_kernel(BwdArgs a) {
  constexpr int RS = LitLds<D>::RS, NT = D / 64;
  __shared__ __align__(16) uint16_t sK[kB * RS], sV[kB * RS], sQ[kB * RS], sG[kB * RS];
  __shared__ __align__(16) uint16_t sQT[D * kTS], sGT[D * kTS];
  __shared__ __align__(16) uint16_t sDXT[kB * kTS], sWT[kB * kTS];
  __shared__ float sS[kB * kSS], sA[kB * kSS];
  __shared__ float sLse[kB], sDelta[kB];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = tid >> 6, qh = wave >> 1, kh = wave & 1;
  const int nb = a.nb, h = int(blockIdx.x) / nb, j = int(blockIdx.x) % nb;
  auto rows_of = [&](int b) { return a.block_len ? min(max(a.block_len[b], 1), kB) : kB; };
  const int nj = rows_of(j);
  const size_t krow0 = size_t(h) * a.L + size_t(j) * kB;
  const uint16_t* Qh = static_cast<const uint16_t*>(a.Q) + size_t(h) * a.L * D;
  const uint16_t* Gh = static_cast<const uint16_t*>(a.dO) + size_t(h) * a.L * D;
  const uint32_t* mh = a.mask + size_t(h) * nb * a.nw;

  stage_rows<D>(sK, static_cast<const uint16_t*>(a.K) + krow0 * D, nj);
  stage_rows<D>(sV, static_cast<const uint16_t*>(a.V) + krow0 * D, nj);
  const int q = tid >> 2, p = tid & 3;
  f32x16 ak[NT], av_[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) ak[u] = av_[u] = zero16();

  // Each query tile's Q and dO rows are loaded once, while the previous tile's products
  // run, and written to LDS both row-major and transposed.
  // The tile's row statistics (lse, Δ; threads below kB) travel with its rows.
  RowRegs<D> qr, gr;
  float rl = 0.f, rd = 0.f;
  auto load_tile = [&](int t) {
    const int mt = rows_of(t);
    load_rows<D>(qr, Qh + size_t(t) * kB * D, mt);
    load_rows<D>(gr, Gh + size_t(t) * kB * D, mt);
    if (tid < kB) {
      const size_t r = size_t(h) * a.L + size_t(t) * kB + tid;
      rl = tid < mt ? a.lse2[r] : kNegInf;
      rd = tid < mt ? a.delta[r] : 0.f;
    }
  };
  load_tile(0);
  for (int i = 0; i < nb; ++i) {
    const int mi = rows_of(i);
    __syncthreads();
    put_rows<D>(sQ, qr);
    put_rows<D>(sG, gr);
    put_cols<D>(sQT, qr);
    put_cols<D>(sGT, gr);
    if (tid < kB) {
      sLse[tid] = rl;
      sDelta[tid] = rd;
    }
    if (i + 1 < nb) load_tile(i + 1);
    __syncthreads();
    quarter_product<D>(sQ, sK, sS, qh, kh);
    quarter_product<D>(sG, sV, sA, qh, kh);
    __syncthreads();
    RowIn in;
    in.lse = sLse[q];
    in.delta = sDelta[q];
    in.nj = nj;
    in.live = q < mi && in.lse > kNegInf;
    in.sel = (mh[size_t(i) * a.nw + (j >> 5)] >> (j & 31)) & 1u;
    in.gate = a.gate;
    in.linear = a.w_linear;
    float x[16], avv[16], dx[16], wv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      x[u] = sS[q * kSS + 16 * p + u];
      avv[u] = sA[q * kSS + 16 * p + u];
    }
    float unused = 0.f;
    row_pass<false>(x, avv, in, p, dx, wv, unused);
    // transposed: [key][query]
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      sDXT[(16 * p + u) * kTS + q] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(dx[u]));
      sWT[(16 * p + u) * kTS + q] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(wv[u]));
    }
    __syncthreads();
    // dK, dV rows [32 kh, +32) (keys), columns [64 qh, +64) of d += dxᵀ Q, (weights)ᵀ dO
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int dt = qh * NT + u;
#pragma unroll
      for (int ks = 0; ks < kB / 16; ++ks) {
        ak[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds8(sDXT + (32 * kh + c) * kTS + 16 * ks + 8 * g),
                                                        lds8(sQT + (32 * dt + c) * kTS + tpos(32 * dt + c, 16 * ks + 8 * g)),
                                                        ak[u], 0, 0, 0);
        av_[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds8(sWT + (32 * kh + c) * kTS + 16 * ks + 8 * g),
                                                         lds8(sGT + (32 * dt + c) * kTS + tpos(32 * dt + c, 16 * ks + 8 * g)),
                                                         av_[u], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int col = 32 * (qh * NT + u) + c;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * kh + acc_row(r, g);
      a.dK[(krow0 + row) * D + col] = row < nj ? ak[u][r] : 0.f;
      a.dV[(krow0 + row) * D + col] = row < nj ? av_[u][r] : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------------------
// PWT_ROW: the virtual tokens with the per-row w_{t,j} = ½ Σ_c q_{t,c}² σ²_{j,c} (Sparse
// Linear Attention blog, PWT section). For query t and unselected block j:
//   P = e^{q·k̄_j + ln n_j + φ(w) - lse_t},  dℓ = P (dO·v̄_j + dO·(H̄ q_t) / n_j - Δ_t),
//   dw = φ'(w) dℓ,  Ā_t = Σ_j P / n_j,
//   dq_t += Σ_j dℓ k̄_j + q_t ∘ Σ_j dw σ²_j + Ā_t H̄ᵀ dO_t,
//   dk̄_j = Σ_t dℓ q_t,  dv̄_j = Σ_t P dO_t,  dσ²_j = ½ Σ_t dw q_t²,
// the statistics' gradients then reaching the tokens as for PWT. The selected blocks' Δ and
// softmax mass come from the LITERAL query kernel restricted to the selection; their dQ,
// dK and dV from the PWT backward's exact sweeps, given the final Δ and lse + ln Σ P.
//
// The virtual kernels keep the 32 x 32 score quarters in registers: the rows of the
// product's A operand are fed in the permuted order that makes accumulator registers
// [8 ks, 8 ks + 8) the B operand of k-step ks of the next product (feed_row), so the
// softmax terms go from one MFMA to the next without LDS. Centroid, v̄ and σ² rows are the
// fp32 statistics rounded to bf16; w enters the exponent and decides the gate, so it is
// formed from hi + lo parts of q² and ½ σ² (three products, within ~2^-16 of fp32), as in
// the forward's virtual_row_kernel.

namespace {

// Rows of centroid group gi (k̄, v̄ = ΣV / n, ½ σ² as hi + lo parts) as bf16 [64][D] tiles,
// zeros past nb; with T also k̄ᵀ and σ²ᵀ as [D][72] tiles.
template <int D, bool T>
__device__ __forceinline__ void stage_group(uint16_t* kb, uint16_t* vb, uint16_t* s2, uint16_t* s2lo, uint16_t* kbt,
                                            uint16_t* s2t, const BwdArgs& a, int h, int gi) {
  constexpr int RS = LitLds<D>::RS, CPR = D / 8;
  for (int x = threadIdx.x; x < kB * CPR; x += 256) {
    const int r = x / CPR, col = (x % CPR) * 8, j = gi * kB + r;
    float k8[8], v8[8], s8[8];
    if (j < a.nb) {
      const size_t o = (size_t(h) * a.nb + j) * D + col;
      const float inv = 1.f / float(min(max(a.block_len ? a.block_len[j] : kB, 1), kB));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        k8[u] = a.kbar[o + u];
        v8[u] = a.vsum[o + u] * inv;
        s8[u] = a.ksig2[o + u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) k8[u] = v8[u] = s8[u] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      kb[r * RS + col + u] = f32_to_bf16(k8[u]);
      vb[r * RS + col + u] = f32_to_bf16(v8[u]);
      const uint16_t hs = f32_to_bf16(0.5f * s8[u]);
      s2[r * RS + col + u] = hs;
      s2lo[r * RS + col + u] = f32_to_bf16(0.5f * s8[u] - bf16_to_f32(hs));
      if constexpr (T) {
        kbt[(col + u) * kTS + r] = f32_to_bf16(k8[u]);
        s2t[(col + u) * kTS + r] = f32_to_bf16(s8[u]);
      }
    }
  }
}

__device__ __forceinline__ bf16x8 square8(bf16x8 v) {
  bf16x8 r;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const float f = static_cast<float>(v[u]);
    r[u] = static_cast<__bf16>(f * f);
  }
  return r;
}

// q² of bf16 q as hi + lo bf16 parts (together exact to 2^-16 relative).
__device__ __forceinline__ void square8_split(bf16x8 v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const float f = static_cast<float>(v[u]) * static_cast<float>(v[u]);
    hi[u] = static_cast<__bf16>(f);
    lo[u] = static_cast<__bf16>(f - static_cast<float>(hi[u]));
  }
}

// φ and φ' of a gated w (the forward's rule), and the virtual token's log-weight offset.
struct PhiOut {
  float phi, dphi;
};
__device__ __forceinline__ PhiOut phi_of(float w, float lnn, int gate, int linear) {
  const bool fired = gate && w > lnn;
  if (fired) w = 0.f;
  return {linear ? log1pf(w) : w, fired ? 0.f : (linear ? 1.f / (1.f + w) : 1.f)};
}

}  // namespace

// Per query tile: PASS 0 adds the virtual tokens' share of Δ_t; PASS 1 adds their share of
// dQ (without Ā H̄ᵀ dO) and writes Ā_t. Wave (kh, x): centroids [32 kh, +32) of each group
// against queries [32 x, +32), Sᵀ, (dO V̄ᵀ)ᵀ and Wᵀ in registers; dQᵀ of the wave's queries
// summed over its centroid half, the halves added at the end.
template <int D, int PASS>
__global__ __launch_bounds__(256) void rowdiag_bwd_query_kernel(BwdArgs a) {
  constexpr int RS = LitLds<D>::RS, NE = D / 32, NKD = D / 16;
  __shared__ __align__(16) uint16_t sQ[kB * RS], sG[kB * RS];
  __shared__ __align__(16) uint16_t sGrp[4 * kB * RS];              // k̄, v̄, ½σ² hi, lo rows; then hand-over
  __shared__ __align__(16) uint16_t sKbT[PASS ? D * kTS : 8], sS2T[PASS ? D * kTS : 8];
  __shared__ float sRow[3][kB], sLnn[kB], sInv[kB], sRed[2][kB];
  __shared__ int sEx[kB];
  uint16_t *sKb = sGrp, *sVb = sGrp + kB * RS, *sS2 = sGrp + 2 * kB * RS, *sS2l = sGrp + 3 * kB * RS;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = tid >> 6, kh = wave & 1, x = wave >> 1;
  const int nb = a.nb, h = int(blockIdx.x) / nb, i = int(blockIdx.x) % nb, ngrp = a.nbp / kB;
  auto rows_of = [&](int b) { return a.block_len ? min(max(a.block_len[b], 1), kB) : kB; };
  const int mi = rows_of(i);
  const size_t row0 = size_t(h) * a.L + size_t(i) * kB;
  stage_rows<D>(sQ, static_cast<const uint16_t*>(a.Q) + row0 * D, mi);
  stage_rows<D>(sG, static_cast<const uint16_t*>(a.dO) + row0 * D, mi);
  if (tid < kB) {
    sRow[0][tid] = tid < mi ? (PASS ? a.lse2 : a.lse)[row0 + tid] : kNegInf;
    sRow[1][tid] = PASS ? a.delta[row0 + tid] : 0.f;
    sRow[2][tid] = a.gu[row0 + tid];
  }
  __syncthreads();
  const int t = 32 * x + c;                                        // this lane's query
  const float lse_t = sRow[0][t], delta_t = sRow[1][t], gu_t = sRow[2][t];
  const bool live = t < mi && lse_t > kNegInf;
  const uint32_t* mrow = a.mask + (size_t(h) * nb + i) * a.nw;
  const int fr = 32 * kh + feed_row<MmaBF16>(c);                   // centroid row fed by this lane
  f32x16 dq[NE], dqw[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) dq[e] = dqw[e] = zero16();
  float dpart = 0.f, mpart = 0.f, apart = 0.f;

  for (int gi = 0; gi < ngrp; ++gi) {
    __syncthreads();                                               // previous group's tiles read
    stage_group<D, PASS == 1>(sKb, sVb, sS2, sS2l, sKbT, sS2T, a, h, gi);
    if (tid < kB) {
      const int j = gi * kB + tid;
      const bool in = j < nb;
      const int n = in ? rows_of(j) : 1;
      sLnn[tid] = __logf(float(n));
      sInv[tid] = 1.f / float(n);
      sEx[tid] = !in || ((mrow[j >> 5] >> (j & 31)) & 1u);
    }
    __syncthreads();
    f32x16 S = zero16(), A = zero16(), W = zero16();
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      const int k0 = 16 * ks + 8 * g;
      const bf16x8 q = lds8(sQ + t * RS + k0);
      bf16x8 qh, ql;
      square8_split(q, qh, ql);
      const bf16x8 sh = lds8(sS2 + fr * RS + k0);
      S = MmaBF16::mma(lds8(sKb + fr * RS + k0), q, S);
      A = MmaBF16::mma(lds8(sVb + fr * RS + k0), lds8(sG + t * RS + k0), A);
      W = MmaBF16::mma(sh, ql, W);
      W = MmaBF16::mma(lds8(sS2l + fr * RS + k0), qh, W);
      W = MmaBF16::mma(sh, qh, W);
    }
    bf16x8 dlb[2], dwb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jl = 32 * kh + 16 * (r >> 3) + 8 * g + (r & 7);    // centroid of register r
      const bool ok = live && !sEx[jl];
      const float lnn = sLnn[jl], inv = sInv[jl];
      const PhiOut ph = phi_of(W[r], lnn, a.gate, a.w_linear);
      const float P = ok ? __expf(S[r] + lnn + ph.phi - lse_t) : 0.f;
      const float dpv = fmaf(gu_t, inv, A[r]);
      if constexpr (PASS == 0) {
        dpart = fmaf(P, dpv, dpart);
        mpart += P;
      } else {
        const float dl = P * (dpv - delta_t);
        apart = fmaf(P, inv, apart);
        dlb[r >> 3][r & 7] = static_cast<__bf16>(dl);
        dwb[r >> 3][r & 7] = static_cast<__bf16>(dl * ph.dphi);
      }
    }
    if constexpr (PASS == 1) {
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int k0 = 32 * kh + 16 * ks + 8 * g;
          dq[e] = MmaBF16::mma(lds8(sKbT + (32 * e + c) * kTS + k0), dlb[ks], dq[e]);
          dqw[e] = MmaBF16::mma(lds8(sS2T + (32 * e + c) * kTS + k0), dwb[ks], dqw[e]);
        }
    }
  }

  __syncthreads();                                                 // group tiles no longer read
  if constexpr (PASS == 0) {
    // add the selected blocks' sums (left by the exact sweep) and renormalise (see there)
    const float v = sum_halves(dpart), m = sum_halves(mpart);
    if (kh == 1 && g == 0) {
      sRed[0][t] = v;
      sRed[1][t] = m;
    }
    __syncthreads();
    if (kh == 0 && g == 0) {
      const float dt = a.delta[row0 + t] + v + sRed[0][t], mt = a.lse2[row0 + t] + m + sRed[1][t];
      a.delta[row0 + t] = live ? dt / mt : 0.f;
      a.lse2[row0 + t] = live ? lse_t + logf(mt) : kNegInf;
    }
  } else {
    const float v = sum_halves(apart);
    if (kh == 1 && g == 0) sRed[1][t] = v;
    // this wave's share of dQ[t][d]: Σ dℓ k̄ + q ∘ Σ dw σ²
    float* hand = reinterpret_cast<float*>(sGrp);                  // [x][e][r][lane] of the kh = 1 waves
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * e + acc_row(r, g);
        const float cv = fmaf(bf16_to_f32(sQ[t * RS + d]), dqw[e][r], dq[e][r]);
        if (kh == 1) hand[((x * NE + e) * 16 + r) * 64 + lane] = cv;
        else dq[e][r] = cv;
      }
    __syncthreads();
    if (kh == 0) {
      if (g == 0) a.abar[row0 + t] = live ? v + sRed[1][t] : 0.f;
      if (t < mi) {
#pragma unroll
        for (int e = 0; e < NE; ++e)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const size_t o = (row0 + t) * D + 32 * e + acc_row(r, g);
            a.dQ[o] += dq[e][r] + hand[((x * NE + e) * 16 + r) * 64 + lane];
          }
      }
    }
  }
}

// dQ += Ā_t H̄ᵀ dO_t for every row: vᵀ = H̄ᵀ dOᵀ on bf16 MFMA with H̄ᵀ as hi + lo bf16 parts
// (dO exact in bf16). One workgroup per (head, 8 query tiles); wave w takes query half w & 1
// and every other 32-row tile of d.
template <int D>
__global__ __launch_bounds__(256) void rowdiag_bwd_hterm_kernel(BwdArgs a) {
  constexpr int RS = LitLds<D>::RS, NE = D / 32, NKD = D / 16, TG = 8;
  __shared__ __align__(16) uint16_t sHh[D * RS], sHl[D * RS];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31, wave = tid >> 6;
  const int h = blockIdx.y, nb = a.nb;
  const float* hT = a.hbarT + size_t(h) * D * D;
  for (int e = tid; e < D * D; e += 256) {                         // H̄ᵀ[c][e'] row-major
    const float f = hT[e];
    const uint16_t hi = f32_to_bf16(f);
    sHh[(e / D) * RS + e % D] = hi;
    sHl[(e / D) * RS + e % D] = f32_to_bf16(f - bf16_to_f32(hi));
  }
  __syncthreads();
  const uint16_t* Gh = static_cast<const uint16_t*>(a.dO);
  for (int i = blockIdx.x * TG; i < min(nb, blockIdx.x * TG + TG); ++i) {
    const int mi = a.block_len ? min(max(a.block_len[i], 1), kB) : kB;
    const size_t row0 = size_t(h) * a.L + size_t(i) * kB;
    const int t = 32 * (wave & 1) + c;
    bf16x8 gf[NKD];
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks)
      gf[ks] = t < mi ? lds8(Gh + (row0 + t) * D + 16 * ks + 8 * g) : MmaBF16::zero();
    const float ab = t < mi ? a.abar[row0 + t] : 0.f;
    for (int e = wave >> 1; e < NE; e += 2) {
      f32x16 v = zero16();
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        const int k0 = 16 * ks + 8 * g;
        v = MmaBF16::mma(lds8(sHh + (32 * e + c) * RS + k0), gf[ks], v);
        v = MmaBF16::mma(lds8(sHl + (32 * e + c) * RS + k0), gf[ks], v);
      }
      if (t < mi && ab != 0.f) {
#pragma unroll
        for (int r = 0; r < 16; ++r) a.dQ[(row0 + t) * D + 32 * e + acc_row(r, g)] += ab * v[r];
      }
    }
  }
}

// Per centroid group (every query tile): dk̄_j = Σ_t dℓ q_t, dv̄_j = Σ_t P dO_t and
// dσ²_j = ½ Σ_t dw q_t² of its unselected pairs. Wave (kh, x): centroids [32 kh, +32) (one per
// lane) against queries [32 x, +32) (fed permuted, so the registers are the B operands of
// the products with Qᵀ, dOᵀ and (q²)ᵀ); the two query halves are added at the end.
template <int D>
__global__ __launch_bounds__(256) void rowdiag_bwd_key_kernel(BwdArgs a) {
  constexpr int RS = LitLds<D>::RS, NE = D / 32, NKD = D / 16;
  __shared__ __align__(16) uint16_t sGrp[4 * kB * RS];
  __shared__ __align__(16) uint16_t sBuf[2 * kB * RS + 2 * D * kTS];   // Q, dO rows, Qᵀ, dOᵀ; then hand-over
  __shared__ float sRow[3][kB];
  uint16_t *sKb = sGrp, *sVb = sGrp + kB * RS, *sS2 = sGrp + 2 * kB * RS, *sS2l = sGrp + 3 * kB * RS;
  uint16_t *sQ = sBuf, *sG = sBuf + kB * RS, *sQT = sBuf + 2 * kB * RS, *sGT = sQT + D * kTS;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = tid >> 6, kh = wave & 1, x = wave >> 1;
  const int nb = a.nb, ngrp = a.nbp / kB, h = int(blockIdx.x) / ngrp, gi = int(blockIdx.x) % ngrp;
  auto rows_of = [&](int b) { return a.block_len ? min(max(a.block_len[b], 1), kB) : kB; };
  stage_group<D, false>(sKb, sVb, sS2, sS2l, nullptr, nullptr, a, h, gi);
  const int jl = 32 * kh + c, j = gi * kB + jl;                    // this lane's centroid
  const bool inj = j < nb;
  const float nj = float(inj ? rows_of(j) : 1), lnn = __logf(nj), inv = 1.f / nj;
  const int fr = 32 * x + feed_row<MmaBF16>(c);                    // query row fed by this lane
  const uint32_t* mh = a.mask + size_t(h) * nb * a.nw;
  f32x16 dkb[NE], dvb[NE], dsg[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) dkb[e] = dvb[e] = dsg[e] = zero16();

  // Each query tile's Q and dO rows are loaded once, while the previous tile's products
  // run, and written to LDS both row-major and transposed.
  // The tile's row statistics (lse, Δ, dO·u; threads below kB) travel with its rows.
  RowRegs<D> qr, gr;
  float r0v = 0.f, r1v = 0.f, r2v = 0.f;
  auto load_tile = [&](int t) {
    const int mt = rows_of(t);
    const size_t rt = size_t(h) * a.L + size_t(t) * kB;
    load_rows<D>(qr, static_cast<const uint16_t*>(a.Q) + rt * D, mt);
    load_rows<D>(gr, static_cast<const uint16_t*>(a.dO) + rt * D, mt);
    if (tid < kB) {
      r0v = tid < mt ? a.lse2[rt + tid] : kNegInf;
      r1v = a.delta[rt + tid];
      r2v = a.gu[rt + tid];
    }
  };
  load_tile(0);
  for (int i = 0; i < nb; ++i) {
    const int mi = rows_of(i);
    __syncthreads();
    put_rows<D>(sQ, qr);
    put_rows<D>(sG, gr);
    put_cols<D>(sQT, qr);
    put_cols<D>(sGT, gr);
    if (tid < kB) {
      sRow[0][tid] = r0v;
      sRow[1][tid] = r1v;
      sRow[2][tid] = r2v;
    }
    if (i + 1 < nb) load_tile(i + 1);
    __syncthreads();
    const bool ex = !inj || ((mh[size_t(i) * a.nw + (j >> 5)] >> (j & 31)) & 1u);
    f32x16 S = zero16(), A = zero16(), W = zero16();
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      const int k0 = 16 * ks + 8 * g;
      const bf16x8 q = lds8(sQ + fr * RS + k0);
      bf16x8 qh, ql;
      square8_split(q, qh, ql);
      const bf16x8 sh = lds8(sS2 + jl * RS + k0);
      S = MmaBF16::mma(q, lds8(sKb + jl * RS + k0), S);
      A = MmaBF16::mma(lds8(sG + fr * RS + k0), lds8(sVb + jl * RS + k0), A);
      W = MmaBF16::mma(ql, sh, W);
      W = MmaBF16::mma(qh, lds8(sS2l + jl * RS + k0), W);
      W = MmaBF16::mma(qh, sh, W);
    }
    bf16x8 pb[2], dlb[2], dwb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tq = 32 * x + 16 * (r >> 3) + 8 * g + (r & 7);     // query of register r
      const float lse = sRow[0][tq];
      const bool ok = !ex && tq < mi && lse > kNegInf;
      const PhiOut ph = phi_of(W[r], lnn, a.gate, a.w_linear);
      const float P = ok ? __expf(S[r] + lnn + ph.phi - lse) : 0.f;
      const float dl = P * (fmaf(sRow[2][tq], inv, A[r]) - sRow[1][tq]);
      pb[r >> 3][r & 7] = static_cast<__bf16>(P);
      dlb[r >> 3][r & 7] = static_cast<__bf16>(dl);
      dwb[r >> 3][r & 7] = static_cast<__bf16>(dl * ph.dphi);
    }
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int k0 = 32 * x + 16 * ks + 8 * g;
        const bf16x8 qt = lds8(sQT + (32 * e + c) * kTS + tpos(32 * e + c, k0));
        dkb[e] = MmaBF16::mma(qt, dlb[ks], dkb[e]);
        dvb[e] = MmaBF16::mma(lds8(sGT + (32 * e + c) * kTS + tpos(32 * e + c, k0)), pb[ks], dvb[e]);
        dsg[e] = MmaBF16::mma(square8(qt), dwb[ks], dsg[e]);
      }
  }

  // add the query halves (x = 1 hands over through LDS, one quantity at a time) and write
  float* hand = reinterpret_cast<float*>(sBuf);                    // [kh][e][r][lane]
  const size_t ob = (size_t(h) * nb + min(j, nb - 1)) * D;
  const size_t op = (size_t(h) * a.nbp + j) * D;                   // chunk 0 of the partial sums
  auto combine = [&](f32x16 (&v)[NE], auto store) {
    __syncthreads();
    if (x == 1) {
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int r = 0; r < 16; ++r) hand[((kh * NE + e) * 16 + r) * 64 + lane] = v[e][r];
    }
    __syncthreads();
    if (x == 0 && inj) {
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int r = 0; r < 16; ++r) store(32 * e + acc_row(r, g), v[e][r] + hand[((kh * NE + e) * 16 + r) * 64 + lane]);
    }
  };
  combine(dkb, [&](int d, float val) { a.dkbar_part[op + d] = val; });
  combine(dvb, [&](int d, float val) { a.dvbar_part[op + d] = val; });
  combine(dsg, [&](int d, float val) { a.dsig2[ob + d] = 0.5f * val; });
}

template <int D>
static hipError_t launch_rowdiag_bwd_d(const BwdArgs& a0, hipStream_t s) {
  BwdArgs a = a0;
  a.nchunk = 1;                          // one partial sum per centroid (rowdiag_bwd_key_kernel)
  a.qsq = nullptr;
  const dim3 tiles(unsigned(a.H) * unsigned(a.nb)), groups(unsigned(a.H) * unsigned(a.nbp / kB));
#define PISA_LAUNCH(...)                       \
  do {                                         \
    hipLaunchKernelGGL(__VA_ARGS__);           \
    hipError_t e_ = hipGetLastError();         \
    if (e_ != hipSuccess) return e_;           \
  } while (0)
  hipError_t e = launch_bwd_rows(a, s);
  if (e != hipSuccess) return e;
  PISA_LAUNCH((literal_bwd_query_kernel<D, 0, true>), tiles, dim3(256), 0, s, a);
  PISA_LAUNCH((rowdiag_bwd_query_kernel<D, 0>), tiles, dim3(256), 0, s, a);
  {
    // the selected keys' dQ and dK, dV: the PWT backward's exact sweeps, with the final Δ
    // and the renormalised lse
    BwdArgs b = a;
    b.lse = a.lse2;
    b.delta_final = 1;
    e = launch_bwd_exact_sweeps(b, s);
    if (e != hipSuccess) return e;
  }
  PISA_LAUNCH((rowdiag_bwd_query_kernel<D, 1>), tiles, dim3(256), 0, s, a);
  PISA_LAUNCH((rowdiag_bwd_hterm_kernel<D>), dim3((a.nb + 7) / 8, a.H), dim3(256), 0, s, a);
  PISA_LAUNCH((rowdiag_bwd_key_kernel<D>), groups, dim3(256), 0, s, a);
#undef PISA_LAUNCH
  return launch_bwd_stats_tail(a, s);
}

hipError_t launch_rowdiag_bwd(const BwdArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_rowdiag_bwd_d<64>(a, s) : launch_rowdiag_bwd_d<128>(a, s);
}

template <int D>
static hipError_t launch_literal_bwd_d(const BwdArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.H) * unsigned(a.nb));
  hipLaunchKernelGGL((literal_bwd_query_kernel<D, 0, false>), grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((literal_bwd_query_kernel<D, 1, false>), grid, dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((literal_bwd_key_kernel<D>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_literal_bwd(const BwdArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_literal_bwd_d<64>(a, s) : launch_literal_bwd_d<128>(a, s);
}

}  // namespace pisa
