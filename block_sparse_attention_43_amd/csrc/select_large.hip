// Block-wise top-K over long rows (more than kSmallNb key blocks) without a score matrix.
//
// The rule is the one of select_topk.hip (PISA paper Fig. 3 prepare phase: the K_sel
// largest q̄_i·k̄_j of each query tile, ties to the lower block index, ascending output,
// plus the routing terms of §3.3 Eq. (7) and of the blog's PWT section); only the way
// the K_sel-th score is found differs. At nb = 20480 a [nb x nb] fp32 score matrix is
// 1.68 GB, so the scores are recomputed instead of stored, and most of them only
// approximately:
//   1. lscore_kernel<0>: every score of a row, approximated on the bf16 matrix cores
//      from hi + lo splits of both factors, is counted into kLBins linear bins that span
//      a bound of the row's range, |q̄_i|·max_j |k̄_j| plus the key-bias range;
//   2. lthresh_kernel: the bin b* holding the K_sel-th largest approximate score, and
//      per key split a slice of the row's candidate list as long as that split's counts
//      in bins b* - 1, b*, b* + 1;
//   3. lscore_kernel<1>: the same approximations again. With ε a bound on how far an
//      approximation lies from the exact fp32 score, a score at least 2ε above the
//      lower edge of bin b* + 1 is selected outright (mask words), one more than 2ε
//      below the lower edge of b* is dropped, and the rest (the scores near b*) are
//      listed by block index;
//   4. lresolve_kernel: the listed scores are computed exactly (exact_score: a
//      fixed-order fp32 dot product), binned again, and b* resolved exactly (radix
//      select on order-preserving keys, ties to the lower index); the mask becomes
//      ascending indices.
// The bin is a monotone function of the score, so every score of a higher bin is larger
// than every score in b*, and the result is the exact top-K of the exact_score values.
// Rows whose lists overflow (many equal scores) or whose exact counts do not reach
// K_sel around b* are redone by lfallback_kernel, which computes the whole row exactly
// into LDS and radix-selects all of it.
#include "common.hpp"
#include "internal.hpp"
#include "select_common.hpp"

namespace pisa {

namespace {

// Per-key bias of the routed scores: ln(M_j + eps) (Eq. (7)), plus ln n_j for the
// predicted-error route (which also adds w̃_{i,j}).
template <int ROUTE>
__device__ __forceinline__ float key_bias(const SelectArgs& a, int h, int j) {
  if constexpr (ROUTE == 0) {
    return 0.f;
  } else {
    float b = logf(a.hnorm[size_t(h) * a.nb + j] + a.route_eps);
    if constexpr (ROUTE == 2) {
      const int n = a.block_len ? min(max(a.block_len[j], 1), kB) : kB;
      b = __fadd_rn(b, logf(float(n)));
    }
    return b;
  }
}

// Final score from the q̄·k̄ product, ½ q̄²·σ² and the key bias, in one fixed order with
// no contraction, as every kernel forms it.
template <int ROUTE>
__device__ __forceinline__ float route_score(float s, float w2, float bias) {
  if constexpr (ROUTE == 2) s = __fadd_rn(s, __fmul_rn(0.5f, w2));
  if constexpr (ROUTE != 0) s = __fadd_rn(s, bias);
  return s;
}

__device__ __forceinline__ int bin_of(float v, float lo, float sc) {
  float t = __fmul_rn(__fsub_rn(v, lo), sc);
  t = fminf(fmaxf(t, 0.f), float(kLBins - 1));
  return int(t);
}

// The smallest float x with bin_of(x) >= b (-inf for b <= 0, +inf past the last bin), by
// bisection over the order-preserving integer image of the floats (bin_of is monotone).
__device__ __forceinline__ float bin_edge(int b, float lo, float sc) {
  if (b <= 0) return -__builtin_huge_valf();
  if (b >= kLBins) return __builtin_huge_valf();
  auto from_key = [](uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); };
  uint32_t below = order_key(-__builtin_huge_valf()), at = order_key(__builtin_huge_valf());
  while (at - below > 1u) {
    const uint32_t mid = below + (at - below) / 2u;
    if (bin_of(from_key(mid), lo, sc) >= b) at = mid;
    else below = mid;
  }
  return from_key(at);
}

// Row parameters from Σ_c q̄_c² (ss), Σ_c q̄²_c (qs, route 2) and the head's key
// statistics: the bins' origin and scale, and the margin 2ε (which lthresh_kernel turns
// into the pass-1 thresholds).
//
// ε bounds |approximate - exact| for one score. The approximation splits each fp32
// factor x into bf16 x_hi + x_lo (within 2^-16 |x|) and sums hi·hi + lo·hi + hi·lo
// (exact products, fp32 sums over at most 3·128 terms): per element within 3.02·2^-16
// of |q_c k_c|, plus at most 384·2^-24 of Σ_c |q_c k_c| for the sums, 2^-13.7 in all;
// exact_score's own rounding adds 2^-19. Σ_c |q_c k_c| ≤ |q̄|·|k̄_j| ≤ R = |q̄|·max_j |k̄_j|
// (Cauchy-Schwarz), and likewise ½ q̄²·σ² ≤ ½ qs·max σ² for route 2, so 2^-11 of that
// scale bounds both with a factor 6 to spare; 2^-20 of the score's magnitude covers the
// fp32 adds of the biases and of the margin itself.
template <int ROUTE>
__device__ __forceinline__ float4 row_param(float ss, float qs, float4 kst) {
  const float R = __fmul_rn(sqrtf(ss), kst.x);
  float lo = __fsub_rn(kst.y, R), hi = __fadd_rn(kst.z, R), m = R;
  if constexpr (ROUTE == 2) {
    const float w = __fmul_rn(__fmul_rn(0.5f, qs), kst.w);
    hi = __fadd_rn(hi, w);
    m = __fadd_rn(m, w);
  }
  const float pad = __fadd_rn(__fmul_rn(__fsub_rn(hi, lo), 1e-6f), 1e-30f);
  lo = __fsub_rn(lo, pad);
  hi = __fadd_rn(hi, pad);
  const float b = fmaxf(fabsf(kst.y), fabsf(kst.z));
  const float eps = __fadd_rn(__fmul_rn(m, 0x1p-11f), __fmul_rn(__fadd_rn(m, b), 0x1p-20f));
  return make_float4(lo, __fdiv_rn(float(kLBins), __fsub_rn(hi, lo)), __fmul_rn(2.f, eps), 0.f);
}

// Head statistics reduced over the lnkp partials by one wave: max |k̄_j|, min and max key
// bias, max σ²_{j,c}. Max and min are exact, so every wave gets the same values.
__device__ __forceinline__ float4 head_stats(const SelectArgs& a, int h) {
  const int lane = threadIdx.x & 63;
  float4 r = make_float4(0.f, __builtin_huge_valf(), -__builtin_huge_valf(), 0.f);
  for (int e = lane; e < a.lnkp; e += 64) {
    const float4 p = a.lkpart[size_t(h) * a.lnkp + e];
    r.x = fmaxf(r.x, p.x);
    r.y = fminf(r.y, p.y);
    r.z = fmaxf(r.z, p.z);
    r.w = fmaxf(r.w, p.w);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    r.x = fmaxf(r.x, __shfl_xor(r.x, o, 64));
    r.y = fminf(r.y, __shfl_xor(r.y, o, 64));
    r.z = fmaxf(r.z, __shfl_xor(r.z, o, 64));
    r.w = fmaxf(r.w, __shfl_xor(r.w, o, 64));
  }
  return r;
}

// Eight fp32 values as bf16 hi + lo (hi = bf16(x), lo = bf16(x - hi); x - hi is exact).
__device__ __forceinline__ void split8(const float (&v)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 x = static_cast<__bf16>(v[e]);
    hi[e] = x;
    lo[e] = static_cast<__bf16>(__fsub_rn(v[e], static_cast<float>(x)));
  }
}

// 32 x 32 tile of approximate X·Bᵀ over the head dimension on v_mfma_f32_32x32x16_bf16:
// at k-step u, lane 32 g + c supplies dimensions g·D/2 + 8u .. + 7 of row c of either
// operand (the same assignment on both sides). Two accumulation chains take turns.
template <int S>
__device__ __forceinline__ f32x16 split_product(const bf16x8 (&Xh)[S], const bf16x8 (&Xl)[S],
                                                const bf16x8 (&Bh)[S], const bf16x8 (&Bl)[S]) {
  f32x16 x = zero16(), y = zero16();
#pragma unroll
  for (int u = 0; u < S; ++u) {
    x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Xh[u], Bh[u], x, 0, 0, 0);
    y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Xl[u], Bh[u], y, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < S; ++u) {
    if (u & 1) y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Xh[u], Bl[u], y, 0, 0, 0);
    else x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Xh[u], Bl[u], x, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = __fadd_rn(x[r], y[r]);
  return x;
}

// The exact score of one (query tile, key block) pair: fp32 dot products in one fixed
// order (four interleaved partial sums, then (s0 + s1) + (s2 + s3)), no contraction.
// q and q2 are the tile's q̄ and q̄² rows (LDS), k and s2 the block's k̄ and σ² rows.
template <int D, int ROUTE>
__device__ __forceinline__ float exact_score(const float* q, const float* q2, const float* k, const float* s2,
                                             float bias) {
  auto dot = [](const float* x, const float* y) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int u = 0; u < D / 4; ++u) {
      const float4 a = reinterpret_cast<const float4*>(x)[u];
      const float4 b = reinterpret_cast<const float4*>(y)[u];
      acc.x = __fmaf_rn(a.x, b.x, acc.x);
      acc.y = __fmaf_rn(a.y, b.y, acc.y);
      acc.z = __fmaf_rn(a.z, b.z, acc.z);
      acc.w = __fmaf_rn(a.w, b.w, acc.w);
    }
    return __fadd_rn(__fadd_rn(acc.x, acc.y), __fadd_rn(acc.z, acc.w));
  };
  const float s = dot(q, k);
  float w2 = 0.f;
  if constexpr (ROUTE == 2) w2 = dot(q2, s2);
  return route_score<ROUTE>(s, w2, bias);
}

// fp32 [H][nb][D] rows as bf16 hi / lo operands in the tiled order of the approximate
// products (SelectArgs::khl): 16-byte unit ((h·tiles + t)·2 + part)·(D/16)·64 + u·64 +
// lane holds part (0 hi, 1 lo) of row 32 t + lane % 32, columns (lane / 32)·D/2 + 8u ..
// + 7, zeros past nb. One contiguous kilobyte per 16-byte load of a wave.
template <int D>
__global__ __launch_bounds__(256) void tile_split_kernel(const float* src, uint4* dst, int nb) {
  constexpr int S = D / 16;
  const int t = blockIdx.x, h = blockIdx.y, tiles = gridDim.x;
  uint4* out = dst + (size_t(h) * tiles + t) * 2 * S * 64;
  for (int e = threadIdx.x; e < S * 64; e += 256) {
    const int u = e / 64, lane = e % 64, row = 32 * t + (lane & 31), col = (lane >> 5) * (D / 2) + 8 * u;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (row < nb) {
      const float4* p = reinterpret_cast<const float4*>(src + (size_t(h) * nb + row) * D + col);
      const float4 x0 = p[0], x1 = p[1];
      v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
      v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
    }
    bf16x8 hi, lo;
    split8(v, hi, lo);
    out[e] = __builtin_bit_cast(uint4, hi);
    out[S * 64 + e] = __builtin_bit_cast(uint4, lo);
  }
}

// Partial head statistics of 256 key blocks (one per thread).
template <int D, int ROUTE>
__global__ __launch_bounds__(256) void lprep_kernel(SelectArgs a) {
  __shared__ float4 red[4];
  const int h = blockIdx.y, tid = threadIdx.x, j = blockIdx.x * 256 + tid, nb = a.nb;
  float4 r = make_float4(0.f, __builtin_huge_valf(), -__builtin_huge_valf(), 0.f);
  if (j < nb) {
    const float4* kr = reinterpret_cast<const float4*>((a.rope_axes ? a.krot : a.kbar) + (size_t(h) * nb + j) * D);
    float ss = 0.f;
#pragma unroll 8
    for (int u = 0; u < D / 4; ++u) {
      const float4 v = kr[u];
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    r.x = sqrtf(ss) * (1.f + 1e-5f);        // above the bound's own rounding
    const float b = key_bias<ROUTE>(a, h, j);
    r.y = r.z = b;
    if constexpr (ROUTE == 2) {
      const float4* sr = reinterpret_cast<const float4*>(a.ksig2 + (size_t(h) * nb + j) * D);
      for (int u = 0; u < D / 4; ++u) {
        const float4 v = sr[u];
        r.w = fmaxf(r.w, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    r.x = fmaxf(r.x, __shfl_xor(r.x, o, 64));
    r.y = fminf(r.y, __shfl_xor(r.y, o, 64));
    r.z = fmaxf(r.z, __shfl_xor(r.z, o, 64));
    r.w = fmaxf(r.w, __shfl_xor(r.w, o, 64));
  }
  if ((tid & 63) == 0) red[tid >> 6] = r;
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) {
      r.x = fmaxf(r.x, red[w].x);
      r.y = fminf(r.y, red[w].y);
      r.z = fmaxf(r.z, red[w].z);
      r.w = fmaxf(r.w, red[w].w);
    }
    a.lkpart[size_t(h) * a.lnkp + blockIdx.x] = r;
  }
}

// The two approximate score passes. Workgroup (row group rg, key split s) of 4 waves:
// wave w owns query tiles rg·128 + 32 w .. + 31 (the A operands, hi and lo, in
// registers: lane 32 g + c holds half g of q̄ of tile c) and streams the 32-block key
// tiles of split s (B operands from SelectArgs::khl), one 32 x 32 score tile per 32
// blocks, prefetched one tile ahead. Split s of every row group runs on XCD s mod 8
// (workgroups are dealt round-robin), so each XCD's L2 holds the centroids of its splits.
template <int D, int PASS, int ROUTE>
__global__ __launch_bounds__(256, 2) void lscore_kernel(SelectArgs a) {
  constexpr int KH = D / 2, S = D / 16;
  __shared__ float4 sp[kLRows];          // PASS 0: row parameters (row_param)
  __shared__ float2 sab[kLRows];         // PASS 1: thresholds A (above) and B (not below)
  __shared__ int sn[kLRows];             // PASS 1: next list slot per row
  __shared__ int s0[kLRows];             // PASS 1: first slot of this split's slice
  __shared__ int se[kLRows];             // PASS 1: end of this split's slice
  __shared__ uint32_t sh[PASS == 0 ? kLRows * (kLBins / 2) : 1];   // PASS 0: histograms
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int ks = a.lks, split = int(blockIdx.x) % ks, rg = int(blockIdx.x) / ks, h = blockIdx.y, nb = a.nb;
  const int tiles = (nb + 31) / 32, t0 = split * tiles / ks, t1 = (split + 1) * tiles / ks;
  const int rl0 = 32 * wave, r0 = rg * kLRows;
  const size_t hn = size_t(h) * nb;
  if constexpr (PASS == 0) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) a.lover[0] = 0;   // the fallback list
    for (int e = tid; e < kLRows * (kLBins / 2); e += 256) sh[e] = 0u;
  }

  // A operands (and q̄² for route 2) as hi / lo, row sums for the bin bounds
  const int arow = min(r0 + rl0 + c, nb - 1);
  bf16x8 Ah[S], Al[S], A2h[ROUTE == 2 ? S : 1], A2l[ROUTE == 2 ? S : 1];
  float ss = 0.f, qs = 0.f;
  {
    const float4* qp = reinterpret_cast<const float4*>(a.qbar + (hn + arow) * D + g * KH);
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const float4 x0 = qp[2 * u], x1 = qp[2 * u + 1];
      const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __fmaf_rn(v[e], v[e], ss);
      split8(v, Ah[u], Al[u]);
    }
    if constexpr (ROUTE == 2) {
      const float4* q2 = reinterpret_cast<const float4*>(a.qsq + (hn + arow) * D + g * KH);
#pragma unroll
      for (int u = 0; u < S; ++u) {
        const float4 x0 = q2[2 * u], x1 = q2[2 * u + 1];
        const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) qs = __fadd_rn(qs, v[e]);
        split8(v, A2h[u], A2l[u]);
      }
    }
  }
  ss = __fadd_rn(ss, __shfl_xor(ss, 32, 64));
  if constexpr (ROUTE == 2) qs = __fadd_rn(qs, __shfl_xor(qs, 32, 64));
  if constexpr (PASS == 0) {
    const float4 kst = head_stats(a, h);
    if (g == 0) {
      const float4 p = row_param<ROUTE>(ss, qs, kst);
      const int row = r0 + rl0 + c;
      sp[rl0 + c] = p;
      if (split == 0 && row < nb) a.lparam[hn + row] = p;
    }
  } else {
    // parameters, b* and this split's slice of each row's list (nothing listed for rows
    // that are out of range or already sent to the fallback)
    if (g == 0) {
      const int row = r0 + rl0 + c;
      float2 ab = make_float2(__builtin_huge_valf(), __builtin_huge_valf());   // nothing above or near
      int slot = 1 << 30, end = 0;
      if (row < nb) {
        const float4 p = a.lparam[hn + row];
        ab = make_float2(p.z, p.w);
        const int4 st = a.lstate[hn + row];
        if (!st.w) {
          slot = a.lcoff[(hn + row) * ks + split];
          end = split + 1 < ks ? a.lcoff[(hn + row) * ks + split + 1] : st.z;
        }
      }
      sab[rl0 + c] = ab;
      sn[rl0 + c] = slot;
      s0[rl0 + c] = slot;
      se[rl0 + c] = end;
    }
  }
  __syncthreads();

  // B operands from the tiled hi / lo copies; tiles past the end (prefetch) read the last
  const uint4* kb = a.khl + size_t(h) * tiles * 2 * S * 64 + lane;
  const uint4* sb2 = a.shl + size_t(h) * tiles * 2 * S * 64 + lane;
  auto load_tile = [&](bf16x8 (&Bh)[S], bf16x8 (&Bl)[S], const uint4* src, int t) {
    const uint4* p = src + size_t(min(t, tiles - 1)) * 2 * S * 64;
#pragma unroll
    for (int u = 0; u < S; ++u) {
      Bh[u] = __builtin_bit_cast(bf16x8, p[u * 64]);
      Bl[u] = __builtin_bit_cast(bf16x8, p[(S + u) * 64]);
    }
  };
  // PASS 1 stores go through buffer descriptors of this head's mask rows and candidate
  // lists; a lane with nothing to store uses an offset past the end, which the hardware
  // drops. Every tile then issues the same number of stores (one mask word per row, one
  // candidate slot per score register), so the compiler's wait before each tile's
  // products needs only that tile's loads, never the previous tile's stores.
  const __amdgpu_buffer_rsrc_t rmask = make_rsrc(a.mask + hn * a.nw, uint32_t(nb) * uint32_t(a.nw) * 4u);
  const __amdgpu_buffer_rsrc_t rcand = make_rsrc(a.lcand + hn * kLCap, uint32_t(nb) * uint32_t(kLCap) * 4u);
  constexpr uint32_t kDrop = 0x80000000u;
  constexpr int kStoresPerTile = 17;
  auto epilogue = [&](const f32x16& acc, const f32x16& acc2, int t) {
    // The row parameters in LDS and the per-row addresses are formed again every tile
    // rather than held in registers across the loop (hoisted, they would not fit): the
    // memory clobber keeps the LDS reads here, the opaque zero the index arithmetic.
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z) :: "memory");
    const int key = 32 * t + c;
    const float bias = key_bias<ROUTE>(a, h, min(key, nb - 1));
    uint32_t word = 0u;                  // PASS 1, lanes of half 0: mask word of row rl0 + c
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = rl0 + acc_row(r, g) + z, row = r0 + rl;
      const bool valid = key < nb && row < nb;
      const float v = route_score<ROUTE>(acc[r], acc2[r], bias);
      if constexpr (PASS == 0) {
        const float4 p = sp[rl];
        const int bin = bin_of(v, p.x, p.y);
        if (valid) atomicAdd(&sh[rl * (kLBins / 2) + (bin >> 1)], 1u << ((bin & 1) * 16));
      } else {
        const float2 ab = sab[rl];
        const bool up = v >= ab.x, near = valid && !up && v >= ab.y;
        const uint64_t above = __ballot(valid && up);
        const uint64_t nearb = __ballot(near);
        if (c == acc_row(r, 0)) word = uint32_t(above);
        if (c == acc_row(r, 1)) word = uint32_t(above >> 32);
        const uint32_t mine = uint32_t(g ? nearb >> 32 : nearb);
        const int slot = sn[rl];
        const int pos = slot + __popc(mine & ((1u << c) - 1u));
        const bool listed = near && pos < se[rl];
        const uint32_t coff = listed ? uint32_t(row * kLCap + pos) * 4u : kDrop;
        __builtin_amdgcn_raw_buffer_store_b32(uint32_t(key), rcand, int(coff), 0, 0);
        if (c == 0) sn[rl] = slot + __popc(mine);
      }
    }
    if constexpr (PASS == 1) {
      const int mrow = r0 + rl0 + c;
      const uint32_t moff = (g == 0 && mrow < nb) ? (uint32_t(mrow) * uint32_t(a.nw) + uint32_t(t)) * 4u : kDrop;
      __builtin_amdgcn_raw_buffer_store_b32(word, rmask, int(moff), 0, 0);
    }
  };

  if constexpr (ROUTE == 2) {
    // ½ q̄²·σ² and q̄·k̄ from one operand buffer, one after the other
    bf16x8 Bh[S], Bl[S];
    for (int t = t0; t < t1; ++t) {
      load_tile(Bh, Bl, sb2, t);
      const f32x16 acc2 = split_product<S>(A2h, A2l, Bh, Bl);
      load_tile(Bh, Bl, kb, t);
      epilogue(split_product<S>(Ah, Al, Bh, Bl), acc2, t);
    }
  } else {
    // Centroids of the next key tile load while this tile's products run (two buffers
    // taking turns). The loads are unconditional (past the split they read the last tile
    // again, unused) and, in PASS 1, the first tile is preceded by as many dropped stores
    // as a tile's epilogue issues: every wait before a product then counts the same
    // operations on every path and waits for that tile's operands only.
    bf16x8 B0h[S], B0l[S], B1h[S], B1l[S];
    load_tile(B0h, B0l, kb, t0);
    if constexpr (PASS == 1) {
#pragma unroll
      for (int e = 0; e < kStoresPerTile; ++e) __builtin_amdgcn_raw_buffer_store_b32(0u, rmask, int(kDrop), 0, 0);
    }
    for (int t = t0; t < t1; t += 2) {
      load_tile(B1h, B1l, kb, t + 1);
      epilogue(split_product<S>(Ah, Al, B0h, B0l), zero16(), t);
      if (t + 1 >= t1) break;
      load_tile(B0h, B0l, kb, t + 2);
      epilogue(split_product<S>(Ah, Al, B1h, B1l), zero16(), t + 1);
    }
  }

  if constexpr (PASS == 0) {
    __syncthreads();
    for (int e = tid; e < kLRows * (kLBins / 2); e += 256) {
      const int row = r0 + e / (kLBins / 2);
      if (row < nb) a.lhist[((hn + row) * ks + split) * (kLBins / 2) + e % (kLBins / 2)] = sh[e];
    }
  } else {
    // how many near scores this split found per row (more than its slice: overflow);
    // each row's counter was last written by a lane of this same wave
    if (g == 0) {
      const int row = r0 + rl0 + c;
      if (row < nb) a.lcnt[(hn + row) * ks + split] = sn[rl0 + c] - s0[rl0 + c];
    }
  }
}

// One wave per row: bin b* of the K_sel-th largest approximate score, and each key
// split's slice of the row's list: as many slots as the split counted in bins b* - 1, b*
// and b* + 1, plus 2. A near score's approximation lies within 2ε of b*, and 2ε is a
// small fraction of a bin, so it falls in one of those bins; splits in key order, so the
// list is in ascending block order. Rows whose list would exceed kLCap go to the fallback.
__global__ __launch_bounds__(256) void lthresh_kernel(SelectArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row_id = static_cast<long long>(blockIdx.x) * 4 + wave;
  if (row_id >= static_cast<long long>(a.H) * a.nb) return;     // whole waves leave together
  const int ks = a.lks, K = a.K_sel, nb = a.nb;
  const uint32_t* hp = a.lhist + size_t(row_id) * ks * (kLBins / 2);
  int c4[4] = {0, 0, 0, 0};              // bins 4 lane .. 4 lane + 3
  for (int s = 0; s < ks; ++s) {
    const uint2 w = reinterpret_cast<const uint2*>(hp + s * (kLBins / 2))[lane];
    c4[0] += int(w.x & 0xFFFFu);
    c4[1] += int(w.x >> 16);
    c4[2] += int(w.y & 0xFFFFu);
    c4[3] += int(w.y >> 16);
  }
  const int tot = c4[0] + c4[1] + c4[2] + c4[3];
  const int incl = wave_inclusive_scan(tot);
  const int total = __shfl(incl, 63, 64);
  int bst;
  if (K >= nb) {
    bst = -1;                            // every bin above: all blocks
  } else if (K <= 0) {
    bst = kLBins;                        // no bin above: none
  } else {
    int found = -1, ab = total - incl;   // scores in the bins of higher lanes
#pragma unroll
    for (int q = 3; q >= 0; --q) {
      if (found < 0 && ab < K && ab + c4[q] >= K) found = 4 * lane + q;
      ab += c4[q];
    }
    const uint64_t who = __ballot(found >= 0);
    const int src = __ffsll(static_cast<unsigned long long>(who)) - 1;
    bst = __shfl(found, src, 64);
  }
  int sz = 0;
  if (bst >= 0 && bst < kLBins && lane < ks) {
#pragma unroll
    for (int db = -1; db <= 1; ++db) {
      const int b = bst + db;
      if (b >= 0 && b < kLBins) {
        const uint32_t w = hp[lane * (kLBins / 2) + (b >> 1)];
        sz += int((b & 1) ? w >> 16 : w & 0xFFFFu);
      }
    }
    sz += 2;
  }
  const int sincl = wave_inclusive_scan(sz);
  const int list = __shfl(sincl, 63, 64);
  if (lane < ks) a.lcoff[size_t(row_id) * ks + lane] = sincl - sz;
  if (lane == 0) {
    const int over = list > kLCap ? 1 : 0;
    a.lstate[row_id] = make_int4(bst, 0, list, over);
    if (over) a.lover[1 + atomicAdd(&a.lover[0], 1)] = int(row_id);
    // pass-1 thresholds: v >= A means the exact score reaches bin b* + 1 (v - ε >=
    // edge(b* + 1) + ε, less the add's rounding, which ε's second term covers); v < B
    // means it stays below bin b*
    const float4 p = a.lparam[row_id];
    const float A = __fadd_rn(bin_edge(bst + 1, p.x, p.y), p.z);
    const float B = __fsub_rn(bin_edge(bst, p.x, p.y), p.z);
    a.lparam[row_id] = make_float4(p.x, p.y, A, B);
  }
}

// Radix select of one wave over P keys per lane: the K-th largest key T and how many keys
// equal to T are taken (0 < K < number of valid keys).
template <int P>
__device__ __forceinline__ void wave_threshold(const uint32_t (&key)[P], const bool (&ok)[P], int K, int* hw,
                                               uint32_t* T, int* take_eq) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0u, pmask = 0u;
  int rem = K;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int q = 0; q < 4; ++q) hw[4 * lane + q] = 0;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (ok[p] && (key[p] & pmask) == prefix) atomicAdd(&hw[(key[p] >> shift) & 255u], 1);
    __builtin_amdgcn_wave_barrier();
    int cq[4], own = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      cq[q] = hw[255 - 4 * lane - q];
      own += cq[q];
    }
    const int inc = wave_inclusive_scan(own);
    int ex = inc - own, dg = -1, rm = 0;
    if (ex < rem && inc >= rem) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (dg < 0 && ex + cq[q] >= rem) {
          dg = 255 - 4 * lane - q;
          rm = rem - ex;
        }
        ex += cq[q];
      }
    }
    const uint64_t who = __ballot(dg >= 0);
    const int src = __ffsll(static_cast<unsigned long long>(who)) - 1;
    dg = __shfl(dg, src, 64);
    rm = __shfl(rm, src, 64);
    prefix |= uint32_t(dg) << shift;
    pmask |= 0xFFu << shift;
    rem = rm;
    __builtin_amdgcn_wave_barrier();
  }
  *T = prefix;
  *take_eq = rem;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// One wave per row. List slot e = 64 p + lane (p < P) holds a near block if it lies in the
// filled part of a split's slice; the filled slots are packed in slot order (which is
// block order) and their exact scores decide: bin above b* joins the pass's mask words,
// bin b* is a candidate, below is dropped. The K_sel - (blocks above) best candidates
// (order key, then lower index) complete the mask, which becomes the row's ascending
// index list. Rows whose slices overflowed or whose exact counts leave b* short or
// over-full go to the fallback. Every load that does not depend on another is issued
// first, so a row costs three memory round trips.
template <int D, int ROUTE>
__global__ __launch_bounds__(256) void lresolve_kernel(SelectArgs a) {
  constexpr int P = kLCap / 64;
  __shared__ int hist[4][256];
  __shared__ uint32_t smask[4][kMaxNb / 32];
  __shared__ int sid[4][kLCap];
  __shared__ __align__(16) float sq[4][D];
  __shared__ __align__(16) float sq2[4][ROUTE == 2 ? D : 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row_id = static_cast<long long>(blockIdx.x) * 4 + wave;
  if (row_id >= static_cast<long long>(a.H) * a.nb) return;     // whole waves leave together
  const int nb = a.nb, h = int(row_id / nb), ks = a.lks, nw = a.nw, K = a.K_sel;
  const uint64_t below = (1ull << lane) - 1ull;

  // independent loads: state, parameters, slices (lane s < ks: split s's first slot,
  // filled count, end), the tile's rows, the pass's mask words
  const int4 st = a.lstate[row_id];
  const float4 prm = a.lparam[row_id];
  int rs = 0, rc = 0, re = 0;
  if (lane < ks) {
    rs = a.lcoff[size_t(row_id) * ks + lane];
    rc = a.lcnt[size_t(row_id) * ks + lane];
    re = lane + 1 < ks ? a.lcoff[size_t(row_id) * ks + lane + 1] : st.z;
  }
  for (int e = lane; e < D; e += 64) {
    sq[wave][e] = a.qbar[size_t(row_id) * D + e];
    if constexpr (ROUTE == 2) sq2[wave][e] = a.qsq[size_t(row_id) * D + e];
  }
  uint32_t* s = smask[wave];
  uint32_t* mrow = a.mask + size_t(row_id) * nw;
  int n_mask = 0;
  for (int w = lane; w < nw; w += 64) {
    const uint32_t x = mrow[w];
    s[w] = x;
    n_mask += __popc(x);
  }
  if (st.w) return;                      // already with the fallback
  auto to_fallback = [&]() {
    if (lane == 0) a.lover[1 + atomicAdd(&a.lover[0], 1)] = int(row_id);
  };
  if (__ballot(lane < ks && rc > re - rs)) {
    to_fallback();
    return;
  }
  const int bst = st.x;

  // the filled slots' block indices, packed in slot order
  int first[kMaxKs], count[kMaxKs];      // every slice (empty past ks: lanes >= ks hold 0, 0)
#pragma unroll
  for (int k = 0; k < kMaxKs; ++k) {
    first[k] = __shfl(rs, k, 64);
    count[k] = __shfl(rc, k, 64);
  }
  int nf = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int e = 64 * p + lane;
    bool filled = false;
#pragma unroll
    for (int k = 0; k < kMaxKs; ++k) filled = filled || (e >= first[k] && e < first[k] + count[k]);
    const uint64_t fb = __ballot(filled);
    if (filled) sid[wave][nf + __popcll(fb & below)] = min(int(a.lcand[size_t(row_id) * kLCap + e]), nb - 1);
    nf += __popcll(fb);
  }
  __builtin_amdgcn_wave_barrier();

  // exact scores of the packed candidates: lane takes positions 64 q + lane
  const float* kbase = (a.rope_axes ? a.krot : a.kbar) + size_t(h) * nb * D;
  const float* sbase = ROUTE == 2 ? a.ksig2 + size_t(h) * nb * D : nullptr;
  const int nq = (nf + 63) / 64;
  uint32_t key[P];
  int id[P];
  bool ok[P], up[P];
  int n_up = 0, n_in = 0;
#pragma unroll
  for (int q = 0; q < P; ++q) {
    key[q] = 0u;
    id[q] = 0;
    ok[q] = up[q] = false;
    if (q < nq && 64 * q + lane < nf) {
      const int j = sid[wave][64 * q + lane];
      const float v = exact_score<D, ROUTE>(sq[wave], sq2[wave], kbase + size_t(j) * D, sbase + size_t(j) * D,
                                            key_bias<ROUTE>(a, h, j));
      const int eb = bin_of(v, prm.x, prm.y);
      id[q] = j;
      up[q] = eb > bst;
      ok[q] = eb == bst;
      key[q] = order_key(v);
      n_up += up[q] ? 1 : 0;
      n_in += ok[q] ? 1 : 0;
    }
  }
  const int above = wave_sum(n_mask + n_up), in_bin = wave_sum(n_in), need = K - above;
  if (need < 0 || need > in_bin) {
    to_fallback();
    return;
  }
#pragma unroll
  for (int q = 0; q < P; ++q)
    if (up[q]) atomicOr(&s[id[q] >> 5], 1u << (id[q] & 31));
  if (need > 0) {
    uint32_t T = 0u;
    int take_eq = 0;
    const bool all = need == in_bin;
    if (!all) wave_threshold<P>(key, ok, need, hist[wave], &T, &take_eq);
    // equal keys in packed order (64 q + lane), which is block order
    int eq_seen = 0;
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const bool eq = ok[q] && key[q] == T;
      const uint64_t eqb = __ballot(eq);
      const int rank = eq_seen + __popcll(eqb & below);
      eq_seen += __popcll(eqb);
      const bool take = ok[q] && (all || key[q] > T || (eq && rank < take_eq));
      if (take) atomicOr(&s[id[q] >> 5], 1u << (id[q] & 31));
    }
  }
  __builtin_amdgcn_wave_barrier();
  // the mask row and the ascending indices, 64 mask words per round: output slot o of a
  // round belongs to the last word whose prefix count is <= o, and is that word's
  // (o - prefix)-th set bit, so every lane writes consecutive slots
  int32_t* out = a.idx + size_t(row_id) * K;
  int* pre = hist[wave];                 // [0, 64): prefix counts, [64, 128): the words
  int base = 0;
  for (int w0 = 0; w0 < nw; w0 += 64) {
    const int w = w0 + lane;
    const uint32_t x = w < nw ? s[w] : 0u;
    if (w < nw) mrow[w] = x;
    const int c = __popc(x);
    const int incl = wave_inclusive_scan(c);
    const int total = __shfl(incl, 63, 64);
    pre[lane] = incl - c;
    pre[64 + lane] = int(x);
    __builtin_amdgcn_wave_barrier();
    for (int o = lane; o < total; o += 64) {
      int l = 0;
#pragma unroll
      for (int step = 32; step > 0; step >>= 1)
        if (pre[l + step] <= o) l += step;
      int k = o - pre[l], b = 0;
      uint32_t bits = uint32_t(pre[64 + l]);
#pragma unroll
      for (int step = 16; step > 0; step >>= 1) {
        const int lowc = __popc(bits & ((1u << step) - 1u));
        if (k >= lowc) {
          k -= lowc;
          bits >>= step;
          b += step;
        }
      }
      if (base + o < K) out[base + o] = 32 * (w0 + l) + b;   // holds by construction; kept as a guard
    }
    base += total;
    __builtin_amdgcn_wave_barrier();
  }
}

// Rows sent to the fallback: the whole row's exact scores into LDS (one block per thread
// in turn), radix-selected by the workgroup: four 8-bit passes over order-preserving keys,
// lower index first at equal keys.
template <int D, int ROUTE>
__global__ __launch_bounds__(256) void lfallback_kernel(SelectArgs a) {
  constexpr int P = kMaxNb / 256;
  __shared__ float sS[kMaxNb];
  __shared__ int hist[256];
  __shared__ int scan_sh[8];
  __shared__ uint32_t s_digit;
  __shared__ int s_rem;
  __shared__ uint32_t smask[kMaxNb / 32];
  __shared__ __align__(16) float sq[D];
  __shared__ __align__(16) float sq2[ROUTE == 2 ? D : 4];
  const int tid = threadIdx.x;
  const int nb = a.nb, K = a.K_sel, nw = a.nw;
  const int nrows = __hip_atomic_load(&a.lover[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int e = blockIdx.x; e < nrows; e += gridDim.x) {
    const int row_id = a.lover[1 + e];
    const int h = row_id / nb;
    const size_t hn = size_t(h) * nb;
    for (int c = tid; c < D; c += 256) {
      sq[c] = a.qbar[size_t(row_id) * D + c];
      if constexpr (ROUTE == 2) sq2[c] = a.qsq[size_t(row_id) * D + c];
    }
    __syncthreads();
    const float* kb = (a.rope_axes ? a.krot : a.kbar) + hn * D;
    const float* s2 = a.ksig2 + hn * D;
    for (int j = tid; j < nb; j += 256)
      sS[j] = exact_score<D, ROUTE>(sq, sq2, kb + size_t(j) * D, s2 + size_t(j) * D, key_bias<ROUTE>(a, h, j));
    __syncthreads();

    // radix select over the LDS row: thread t owns blocks [t P, t P + P)
    const int base = tid * P;
    uint32_t key[P];
#pragma unroll
    for (int p = 0; p < P; ++p) key[p] = (base + p < nb) ? order_key(sS[base + p]) : 0u;
    uint32_t T = 0u;
    int take_eq = 0;
    const bool all = K >= nb;
    if (K > 0 && !all) {
      uint32_t prefix = 0u, pmask = 0u;
      int rem = K;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        hist[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int p = 0; p < P; ++p)
          if (base + p < nb && (key[p] & pmask) == prefix) atomicAdd(&hist[(key[p] >> shift) & 255u], 1);
        __syncthreads();
        const int b = 255 - tid;
        const int v = hist[b];
        int tot;
        const int excl = block_exclusive_scan_256(v, scan_sh, &tot);
        if (excl < rem && excl + v >= rem) {
          s_digit = uint32_t(b);
          s_rem = rem - excl;
        }
        __syncthreads();
        prefix |= s_digit << shift;
        pmask |= 0xFFu << shift;
        rem = s_rem;
        __syncthreads();
      }
      T = prefix;
      take_eq = rem;
    }
    int eq_local = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) eq_local += (base + p < nb && key[p] == T) ? 1 : 0;
    int tot;
    const int eq_start = block_exclusive_scan_256(eq_local, scan_sh, &tot);
    auto selected = [&](int p, int& eqc) -> bool {
      if (base + p >= nb) return false;
      if (all) return true;
      if (K == 0) return false;
      if (key[p] > T) return true;
      if (key[p] == T) return eqc++ < take_eq;
      return false;
    };
    int cnt = 0;
    {
      int eqc = eq_start;
#pragma unroll
      for (int p = 0; p < P; ++p) cnt += selected(p, eqc) ? 1 : 0;
    }
    int pos = block_exclusive_scan_256(cnt, scan_sh, &tot);
    for (int w = tid; w < nw; w += 256) smask[w] = 0u;
    __syncthreads();
    int32_t* out = a.idx + size_t(row_id) * K;
    {
      int eqc = eq_start;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if (selected(p, eqc)) {
          if (pos < K) out[pos] = base + p;
          ++pos;
          atomicOr(&smask[(base + p) >> 5], 1u << ((base + p) & 31));
        }
      }
    }
    __syncthreads();
    uint32_t* mo = a.mask + size_t(row_id) * nw;
    for (int w = tid; w < nw; w += 256) mo[w] = smask[w];
    __syncthreads();                     // LDS reused by the next row
  }
}

template <int D, int ROUTE>
hipError_t launch_large_r(const SelectArgs& a, hipStream_t s) {
  const int nrg = (a.nb + kLRows - 1) / kLRows;
  const unsigned rows4 = unsigned((static_cast<long long>(a.H) * a.nb + 3) / 4);
  const dim3 tg((a.nb + 31) / 32, a.H);
  hipLaunchKernelGGL((tile_split_kernel<D>), tg, dim3(256), 0, s, a.rope_axes ? a.krot : a.kbar, a.khl, a.nb);
  if constexpr (ROUTE == 2) hipLaunchKernelGGL((tile_split_kernel<D>), tg, dim3(256), 0, s, a.ksig2, a.shl, a.nb);
  hipLaunchKernelGGL((lprep_kernel<D, ROUTE>), dim3(a.lnkp, a.H), dim3(256), 0, s, a);
  hipLaunchKernelGGL((lscore_kernel<D, 0, ROUTE>), dim3(nrg * a.lks, a.H), dim3(256), 0, s, a);
  hipLaunchKernelGGL(lthresh_kernel, dim3(rows4), dim3(256), 0, s, a);
  hipLaunchKernelGGL((lscore_kernel<D, 1, ROUTE>), dim3(nrg * a.lks, a.H), dim3(256), 0, s, a);
  hipLaunchKernelGGL((lresolve_kernel<D, ROUTE>), dim3(rows4), dim3(256), 0, s, a);
  const long long rows = static_cast<long long>(a.H) * a.nb;
  hipLaunchKernelGGL((lfallback_kernel<D, ROUTE>), dim3(unsigned(rows < 256 ? rows : 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select_large(const SelectArgs& a, hipStream_t s) {
  if (a.d == 64) {
    if (a.route == 0) return launch_large_r<64, 0>(a, s);
    if (a.route == 1) return launch_large_r<64, 1>(a, s);
    return launch_large_r<64, 2>(a, s);
  }
  if (a.route == 0) return launch_large_r<128, 0>(a, s);
  if (a.route == 1) return launch_large_r<128, 1>(a, s);
  return launch_large_r<128, 2>(a, s);
}

}  // namespace pisa
