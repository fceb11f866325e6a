// Block-wise top-K over long rows (more than kSmallNb key blocks) without a score matrix.
//
// The rule is the one of select_topk.hip (PISA paper Fig. 3 prepare phase: the K_sel
// largest q̄_i·k̄_j of each query tile, ties to the lower block index, ascending output,
// plus the routing terms of §3.3 Eq. (7) and of the blog's PWT section); only the way
// the K_sel-th score is found differs. At nb = 20480 a [nb x nb] fp32 score matrix is
// 1.68 GB, so the scores are recomputed on the fp32 matrix cores instead of stored:
//   1. lscore_kernel<0>: every score of a row is counted into kLBins linear bins that
//      span a bound of the row's range, |q̄_i|·max_j |k̄_j| plus the key-bias range;
//   2. lthresh_kernel: the bin b* holding the K_sel-th largest score, per row;
//   3. lscore_kernel<1>: the scores again; bins above b* are selected outright (mask
//      words), the scores inside b* are listed with their block index;
//   4. lresolve_kernel: the list is resolved exactly (radix select on order-preserving
//      keys, ties to the lower index) and the mask turned into ascending indices.
// A score's bin is a monotone function of its fp32 value, so every score of a higher bin
// is larger than every score in b*: the result is the exact top-K of the fp32 scores.
// Both score passes run the same instructions on the same inputs, so they agree bit for
// bit. A row whose b* holds more than kLCap scores (many exactly equal scores) is redone
// by lfallback_kernel, which recomputes the row into LDS and radix-selects all of it.
#include "common.hpp"
#include "internal.hpp"
#include "select_common.hpp"

namespace pisa {

namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
// no contraction, as every pass computes it.
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

// Bin parameters (lo, scale) of a row from Σ_c q̄_c² (ss), Σ_c q̄²_c (qs, route 2) and
// the head's key statistics; the same expression in both score passes.
template <int ROUTE>
__device__ __forceinline__ float2 row_bins(float ss, float qs, float4 kst) {
  const float R = __fmul_rn(sqrtf(ss), kst.x);
  float lo = __fsub_rn(kst.y, R), hi = __fadd_rn(kst.z, R);
  if constexpr (ROUTE == 2) hi = __fadd_rn(hi, __fmul_rn(__fmul_rn(0.5f, qs), kst.w));
  const float pad = __fadd_rn(__fmul_rn(__fsub_rn(hi, lo), 1e-6f), 1e-30f);
  lo = __fsub_rn(lo, pad);
  hi = __fadd_rn(hi, pad);
  return make_float2(lo, __fdiv_rn(float(kLBins), __fsub_rn(hi, lo)));
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

// 32 x 32 tile of X·Bᵀ over the head dimension on v_mfma_f32_32x32x2f32 (lane 32 g + c
// holds half g of row c of each operand). Two accumulation chains (even and odd k-pairs)
// summed at the end, so the matrix core alternates between them instead of waiting for
// each result in turn; every score of this path is formed in exactly this order.
template <int KH>
__device__ __forceinline__ f32x16 pair_product(const float (&X)[KH], const float (&B)[KH]) {
  f32x16 e = zero16(), o = zero16();
#pragma unroll
  for (int m = 0; m < KH; m += 2) {
    e = __builtin_amdgcn_mfma_f32_32x32x2f32(X[m], B[m], e, 0, 0, 0);
    o = __builtin_amdgcn_mfma_f32_32x32x2f32(X[m + 1], B[m + 1], o, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) e[r] = __fadd_rn(e[r], o[r]);
  return e;
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

// The two score passes. Workgroup (row group rg, key split s) of 4 waves: wave w owns
// query tiles rg·128 + 32 w .. + 31 (A operand of v_mfma_f32_32x32x2f32 in registers:
// lane 32 g + c holds half g of q̄ of tile c) and streams the 32-block key tiles of split
// s (B operand: half g of k̄ of block c), one 32 x 32 score tile per 32 blocks, prefetched
// one tile ahead. Split s of every row group runs on XCD s mod 8 (workgroups are dealt
// round-robin), so each XCD's L2 holds the centroids of its splits only.
template <int D, int PASS, int ROUTE>
__global__ __launch_bounds__(256, 2) void lscore_kernel(SelectArgs a) {
  constexpr int KH = D / 2;
  __shared__ float2 sp[kLRows];          // row bin parameters
  __shared__ int sb[kLRows];             // PASS 1: b* per row
  __shared__ int sn[kLRows];             // PASS 1: next candidate slot per row
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

  // A operand (and ½-less q̄² for route 2), row sums for the bin bounds
  const int arow = min(r0 + rl0 + c, nb - 1);
  float A[KH], A2[ROUTE == 2 ? KH : 1];
  {
    const float4* qp = reinterpret_cast<const float4*>(a.qbar + (hn + arow) * D + g * KH);
#pragma unroll
    for (int u = 0; u < KH / 4; ++u) {
      const float4 v = qp[u];
      A[4 * u] = v.x; A[4 * u + 1] = v.y; A[4 * u + 2] = v.z; A[4 * u + 3] = v.w;
    }
    if constexpr (ROUTE == 2) {
      const float4* sp2 = reinterpret_cast<const float4*>(a.qsq + (hn + arow) * D + g * KH);
#pragma unroll
      for (int u = 0; u < KH / 4; ++u) {
        const float4 v = sp2[u];
        A2[4 * u] = v.x; A2[4 * u + 1] = v.y; A2[4 * u + 2] = v.z; A2[4 * u + 3] = v.w;
      }
    }
  }
  {
    float ss = 0.f, qs = 0.f;
#pragma unroll
    for (int m = 0; m < KH; ++m) ss = __fmaf_rn(A[m], A[m], ss);
    ss = __fadd_rn(ss, __shfl_xor(ss, 32, 64));
    if constexpr (ROUTE == 2) {
#pragma unroll
      for (int m = 0; m < KH; ++m) qs = __fadd_rn(qs, A2[m]);
      qs = __fadd_rn(qs, __shfl_xor(qs, 32, 64));
    }
    const float4 kst = head_stats(a, h);
    if (g == 0) sp[rl0 + c] = row_bins<ROUTE>(ss, qs, kst);
  }
  if constexpr (PASS == 1) {
    // b* and the next list slot of each row (past the list: out of range or overflowing)
    if (g == 0) {
      const int row = r0 + rl0 + c;
      int b = kLBins, slot = 1 << 30;
      if (row < nb) {
        const int4 st = a.lstate[hn + row];
        b = st.x;
        if (!st.w) slot = a.lcoff[(hn + row) * ks + split];
      }
      sb[rl0 + c] = b;
      sn[rl0 + c] = slot;
    }
  }
  __syncthreads();

  // B operands from the tiled copies (SelectArgs::ktile): each 16-byte load of the wave
  // reads one contiguous kilobyte; tiles past the end (prefetch) read the last tile.
  const float4* kb = reinterpret_cast<const float4*>(a.ktile) + size_t(h) * tiles * (KH / 4) * 64 + lane;
  const float4* sb2 = reinterpret_cast<const float4*>(a.stile) + size_t(h) * tiles * (KH / 4) * 64 + lane;
  auto load_rows = [&](float (&B)[KH], const float4* src, int t) {
    const float4* p = src + size_t(min(t, tiles - 1)) * (KH / 4) * 64;
#pragma unroll
    for (int u = 0; u < KH / 4; ++u) {
      const float4 v = p[u * 64];
      B[4 * u] = v.x; B[4 * u + 1] = v.y; B[4 * u + 2] = v.z; B[4 * u + 3] = v.w;
    }
  };
  auto product = [&](const float (&X)[KH], const float (&B)[KH]) { return pair_product<KH>(X, B); };
  // PASS 1 stores go through buffer descriptors of this head's mask rows and candidate
  // lists; a lane with nothing to store uses an offset past the end, which the hardware
  // drops. Every tile then issues the same number of stores (one mask word per row, one
  // candidate slot per score register), so the compiler's wait before each tile's
  // products needs only that tile's loads, never the previous tile's stores. (Staging the
  // output in LDS and writing it in bursts instead measured 6 % slower: more work per
  // score register than the dropped stores cost.)
  const __amdgpu_buffer_rsrc_t rmask = make_rsrc(a.mask + hn * a.nw, uint32_t(nb) * uint32_t(a.nw) * 4u);
  const __amdgpu_buffer_rsrc_t rcand = make_rsrc(a.lcand + hn * kLCap, uint32_t(nb) * uint32_t(kLCap) * 8u);
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
      const float2 p = sp[rl];
      const int bin = bin_of(v, p.x, p.y);
      if constexpr (PASS == 0) {
        if (valid) atomicAdd(&sh[rl * (kLBins / 2) + (bin >> 1)], 1u << ((bin & 1) * 16));
      } else {
        const int bst = sb[rl];
        const uint64_t above = __ballot(valid && bin > bst);
        const uint64_t inbin = __ballot(valid && bin == bst);
        if (c == acc_row(r, 0)) word = uint32_t(above);
        if (c == acc_row(r, 1)) word = uint32_t(above >> 32);
        const uint32_t mine = uint32_t(g ? inbin >> 32 : inbin);
        const int slot = sn[rl];
        const int pos = slot + __popc(mine & ((1u << c) - 1u));
        const bool listed = valid && bin == bst && pos < kLCap;
        const uint32_t coff = listed ? uint32_t(row * kLCap + pos) * 8u : kDrop;
        const u32x2 ent = {order_key(v), uint32_t(key)};
        __builtin_amdgcn_raw_buffer_store_b64(ent, rcand, int(coff), 0, 0);
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
    float B[KH];
    for (int t = t0; t < t1; ++t) {
      load_rows(B, sb2, t);
      const f32x16 acc2 = product(A2, B);
      load_rows(B, kb, t);
      epilogue(product(A, B), acc2, t);
    }
  } else {
    // Centroids of the next key tile load while this tile's products run (two buffers
    // taking turns). The loads are unconditional (past the split they read the last tile
    // again, unused) and, in PASS 1, the first tile is preceded by as many dropped stores
    // as a tile's epilogue issues: every wait before a product then counts the same
    // operations on every path and waits for that tile's operands only.
    float B0[KH], B1[KH];
    load_rows(B0, kb, t0);
    if constexpr (PASS == 1) {
#pragma unroll
      for (int e = 0; e < kStoresPerTile; ++e) __builtin_amdgcn_raw_buffer_store_b32(0u, rmask, int(kDrop), 0, 0);
    }
    for (int t = t0; t < t1; t += 2) {
      load_rows(B1, kb, t + 1);
      epilogue(product(A, B0), zero16(), t);
      if (t + 1 >= t1) break;
      load_rows(B0, kb, t + 2);
      epilogue(product(A, B1), zero16(), t + 1);
    }
  }

  if constexpr (PASS == 0) {
    __syncthreads();
    for (int e = tid; e < kLRows * (kLBins / 2); e += 256) {
      const int row = r0 + e / (kLBins / 2);
      if (row < nb) a.lhist[((hn + row) * ks + split) * (kLBins / 2) + e % (kLBins / 2)] = sh[e];
    }
  }
}

// One wave per row: bin b* of the K_sel-th largest score, the blocks still needed from it,
// and each key split's first slot in the row's candidate list (splits in key order, so
// the list is in ascending block order). Rows whose b* holds more than kLCap scores go to
// the fallback list.
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
  int bst, need = 0, cnt = 0;
  if (K >= nb) {
    bst = -1;                            // every bin above: all blocks
  } else if (K <= 0) {
    bst = kLBins;                        // no bin above: none
  } else {
    int found = -1, nd = 0, cn = 0, ab = total - incl;   // scores in the bins of higher lanes
#pragma unroll
    for (int q = 3; q >= 0; --q) {
      if (found < 0 && ab < K && ab + c4[q] >= K) {
        found = 4 * lane + q;
        nd = K - ab;
        cn = c4[q];
      }
      ab += c4[q];
    }
    const uint64_t who = __ballot(found >= 0);
    const int src = __ffsll(static_cast<unsigned long long>(who)) - 1;
    bst = __shfl(found, src, 64);
    need = __shfl(nd, src, 64);
    cnt = __shfl(cn, src, 64);
  }
  int cs = 0;
  if (bst >= 0 && bst < kLBins && lane < ks) {
    const uint32_t w = hp[lane * (kLBins / 2) + (bst >> 1)];
    cs = int((bst & 1) ? w >> 16 : w & 0xFFFFu);
  }
  const int excl = wave_inclusive_scan(cs) - cs;
  if (lane < ks) a.lcoff[size_t(row_id) * ks + lane] = excl;
  if (lane == 0) {
    const int over = cnt > kLCap ? 1 : 0;
    a.lstate[row_id] = make_int4(bst, need, cnt, over);
    if (over) a.lover[1 + atomicAdd(&a.lover[0], 1)] = int(row_id);
  }
}

// Radix select of one wave over P keys per lane (lane order = block order): the K-th
// largest key T and how many keys equal to T are taken (0 < K < number of valid keys).
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

// One wave per row: the need best candidates of b* (order key, then lower index) join the
// mask words of the bins above, and the row's mask becomes its ascending index list.
__global__ __launch_bounds__(256) void lresolve_kernel(SelectArgs a) {
  constexpr int P = kLCap / 64;
  __shared__ int hist[4][256];
  __shared__ uint32_t smask[4][kMaxNb / 32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row_id = static_cast<long long>(blockIdx.x) * 4 + wave;
  if (row_id >= static_cast<long long>(a.H) * a.nb) return;
  const int4 st = a.lstate[row_id];
  if (st.w) return;                      // overflowing rows: lfallback_kernel
  const int n = st.z, need = st.y, nw = a.nw, K = a.K_sel;
  uint32_t key[P];
  int id[P];
  bool ok[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int e = P * lane + p;
    ok[p] = e < n;
    key[p] = 0u;
    id[p] = 0;
    if (ok[p]) {
      const uint2 v = a.lcand[size_t(row_id) * kLCap + e];
      key[p] = v.x;
      id[p] = int(v.y);
    }
  }
  uint32_t T = 0u;
  int take_eq = 0;
  const bool all = need >= n;
  if (need > 0 && !all) wave_threshold<P>(key, ok, need, hist[wave], &T, &take_eq);

  uint32_t* s = smask[wave];
  uint32_t* mrow = a.mask + size_t(row_id) * nw;
  for (int w = lane; w < nw; w += 64) s[w] = mrow[w];
  __builtin_amdgcn_wave_barrier();
  if (need > 0) {
    int eq_local = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) eq_local += (ok[p] && key[p] == T) ? 1 : 0;
    int eqc = wave_inclusive_scan(eq_local) - eq_local;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      bool take = false;
      if (ok[p]) {
        if (all || key[p] > T) take = true;
        else if (key[p] == T) take = eqc++ < take_eq;
      }
      if (take) atomicOr(&s[id[p] >> 5], 1u << (id[p] & 31));
    }
  }
  __builtin_amdgcn_wave_barrier();
  // ascending indices: lane l takes words [l W, l W + W)
  const int W = (nw + 63) / 64, w0 = lane * W, w1 = min(w0 + W, nw);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(s[w]);
  int pos = wave_inclusive_scan(cnt) - cnt;
  int32_t* out = a.idx + size_t(row_id) * K;
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = s[w];
    mrow[w] = bits;
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1u;
      if (pos < K) out[pos] = 32 * w + b;   // holds by construction; kept as a guard
      ++pos;
    }
  }
}

// Rows whose threshold bin overflowed the list: the whole row is recomputed into LDS with
// the same products (A holds the one query tile in all 32 rows) and radix-selected by a
// workgroup, as select_topk.hip's topk_kernel does from a stored row.
template <int D, int ROUTE>
__global__ __launch_bounds__(256) void lfallback_kernel(SelectArgs a) {
  constexpr int KH = D / 2, P = kMaxNb / 256;
  __shared__ float sS[kMaxNb];
  __shared__ int hist[256];
  __shared__ int scan_sh[8];
  __shared__ uint32_t s_digit;
  __shared__ int s_rem;
  __shared__ uint32_t smask[kMaxNb / 32];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int nb = a.nb, K = a.K_sel, nw = a.nw, tiles = (nb + 31) / 32;
  const int nrows = __hip_atomic_load(&a.lover[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int e = blockIdx.x; e < nrows; e += gridDim.x) {
    const int row_id = a.lover[1 + e];
    const int h = row_id / nb;
    const size_t hn = size_t(h) * nb;
    float A[KH], A2[ROUTE == 2 ? KH : 1];
    {
      const float4* qp = reinterpret_cast<const float4*>(a.qbar + size_t(row_id) * D + g * KH);
#pragma unroll
      for (int u = 0; u < KH / 4; ++u) {
        const float4 v = qp[u];
        A[4 * u] = v.x; A[4 * u + 1] = v.y; A[4 * u + 2] = v.z; A[4 * u + 3] = v.w;
      }
      if constexpr (ROUTE == 2) {
        const float4* q2 = reinterpret_cast<const float4*>(a.qsq + size_t(row_id) * D + g * KH);
#pragma unroll
        for (int u = 0; u < KH / 4; ++u) {
          const float4 v = q2[u];
          A2[4 * u] = v.x; A2[4 * u + 1] = v.y; A2[4 * u + 2] = v.z; A2[4 * u + 3] = v.w;
        }
      }
    }
    const float* kb = (a.rope_axes ? a.krot : a.kbar) + hn * D + g * KH;
    for (int t = wave; t < tiles; t += 4) {
      const int key = 32 * t + c, kc = min(key, nb - 1);
      float B[KH];
      const float4* p = reinterpret_cast<const float4*>(kb + size_t(kc) * D);
#pragma unroll
      for (int u = 0; u < KH / 4; ++u) {
        const float4 v = p[u];
        B[4 * u] = v.x; B[4 * u + 1] = v.y; B[4 * u + 2] = v.z; B[4 * u + 3] = v.w;
      }
      const f32x16 acc = pair_product<KH>(A, B);
      f32x16 acc2 = zero16();
      if constexpr (ROUTE == 2) {
        const float4* q = reinterpret_cast<const float4*>(a.ksig2 + (hn + kc) * D + g * KH);
#pragma unroll
        for (int u = 0; u < KH / 4; ++u) {
          const float4 v = q[u];
          B[4 * u] = v.x; B[4 * u + 1] = v.y; B[4 * u + 2] = v.z; B[4 * u + 3] = v.w;
        }
        acc2 = pair_product<KH>(A2, B);
      }
      const float v = route_score<ROUTE>(acc[0], acc2[0], key_bias<ROUTE>(a, h, kc));
      if (g == 0 && key < nb) sS[key] = v;
    }
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
  hipLaunchKernelGGL((lprep_kernel<D, ROUTE>), dim3(a.lnkp, a.H), dim3(256), 0, s, a);
  hipLaunchKernelGGL((lscore_kernel<D, 0, ROUTE>), dim3(nrg * a.lks, a.H), dim3(256), 0, s, a);
  hipLaunchKernelGGL(lthresh_kernel, dim3(rows4), dim3(256), 0, s, a);
  hipLaunchKernelGGL((lscore_kernel<D, 1, ROUTE>), dim3(nrg * a.lks, a.H), dim3(256), 0, s, a);
  hipLaunchKernelGGL(lresolve_kernel, dim3(rows4), dim3(256), 0, s, a);
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
