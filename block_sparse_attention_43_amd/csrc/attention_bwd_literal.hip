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

// The transpose of the same block: dst[c][r] (row stride 72), zero for rows r >= nv.
template <int D>
__device__ __forceinline__ void stage_cols(uint16_t* dst, const uint16_t* src, int nv) {
  constexpr int CPR = D / 8;
  for (int c = threadIdx.x; c < kB * CPR; c += 256) {
    const int r = c / CPR, col = (c % CPR) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < nv) v = *reinterpret_cast<const u32x4*>(src + size_t(r) * D + col);
    const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
    for (int u = 0; u < 8; ++u) dst[(col + u) * kTS + r] = e[u];
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
// weights of keys [16 p, 16 p + 16), or (DELTA) only this part's share of Δ. Sums over
// the block's 64 keys combine the four parts of the row (lanes 4 q .. 4 q + 3).
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
__device__ __forceinline__ float row_pass(const float* x, const float* av, const RowIn& in, int p, float* dx, float* wv) {
  float part = 0.f;
  if (in.sel) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const bool ok = in.live && 16 * p + u < in.nj;
      const float P = ok ? __expf(x[u] - in.lse) : 0.f;
      if constexpr (DELTA) part = fmaf(P, av[u], part);
      else {
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
  if constexpr (DELTA) return (p == 0) ? E * t : 0.f;
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
template <int D, int PASS>
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
    sLse[tid] = tid < mi ? a.lse[row0 + tid] : kNegInf;
    sDelta[tid] = PASS ? a.delta[row0 + tid] : 0.f;
  }
  const int q = tid >> 2, p = tid & 3;
  f32x16 acc[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) acc[u] = zero16();
  float dpart = 0.f;

  for (int j = 0; j < nb; ++j) {
    const int nj = rows_of(j);
    __syncthreads();                     // previous step's tiles consumed
    stage_rows<D>(sK, Kh + size_t(j) * kB * D, nj);
    stage_rows<D>(sV, Vh + size_t(j) * kB * D, nj);
    if constexpr (PASS == 1) stage_cols<D>(sKT, Kh + size_t(j) * kB * D, nj);
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
      dpart += row_pass<true>(x, av, in, p, dx, wv);
    } else {
      row_pass<false>(x, av, in, p, dx, wv);
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
                                                           lds8(sKT + (32 * dt + c) * kTS + 16 * ks + 8 * g),
                                                           acc[u], 0, 0, 0);
      }
    }
  }
  if constexpr (PASS == 0) {
    const float d = sum4(dpart);
    if (p == 0) a.delta[row0 + q] = (q < mi && sLse[q] > kNegInf) ? d : 0.f;
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

  for (int i = 0; i < nb; ++i) {
    const int mi = rows_of(i);
    const size_t row0 = size_t(h) * a.L + size_t(i) * kB;
    __syncthreads();
    stage_rows<D>(sQ, Qh + size_t(i) * kB * D, mi);
    stage_rows<D>(sG, Gh + size_t(i) * kB * D, mi);
    stage_cols<D>(sQT, Qh + size_t(i) * kB * D, mi);
    stage_cols<D>(sGT, Gh + size_t(i) * kB * D, mi);
    if (tid < kB) {
      sLse[tid] = tid < mi ? a.lse[row0 + tid] : kNegInf;
      sDelta[tid] = tid < mi ? a.delta[row0 + tid] : 0.f;
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
    in.sel = (mh[size_t(i) * a.nw + (j >> 5)] >> (j & 31)) & 1u;
    in.gate = a.gate;
    in.linear = a.w_linear;
    float x[16], avv[16], dx[16], wv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      x[u] = sS[q * kSS + 16 * p + u];
      avv[u] = sA[q * kSS + 16 * p + u];
    }
    row_pass<false>(x, avv, in, p, dx, wv);
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
                                                        lds8(sQT + (32 * dt + c) * kTS + 16 * ks + 8 * g),
                                                        ak[u], 0, 0, 0);
        av_[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds8(sWT + (32 * kh + c) * kTS + 16 * ks + 8 * g),
                                                         lds8(sGT + (32 * dt + c) * kTS + 16 * ks + 8 * g),
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

template <int D>
static hipError_t launch_literal_bwd_d(const BwdArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.H) * unsigned(a.nb));
  hipLaunchKernelGGL((literal_bwd_query_kernel<D, 0>), grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((literal_bwd_query_kernel<D, 1>), grid, dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((literal_bwd_key_kernel<D>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_literal_bwd(const BwdArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_literal_bwd_d<64>(a, s) : launch_literal_bwd_d<128>(a, s);
}

}  // namespace pisa
