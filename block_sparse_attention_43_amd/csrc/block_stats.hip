// Prepare phase, part 1: per-block key/value statistics of every head.
//
// For key block j with n_j valid tokens (PISA paper §3.4 prepare phase and Fig. 3;
// Sparse Linear Attention blog, notation and PWT sections):
//   k̄_j = (1/n_j) Σ k_i,   ΣV_j = Σ v_i,   σ²_{j,c} = (1/n_j) Σ (k_{i,c} - k̄_{j,c})²,
//   H̄ᵀ = (1/nb) Σ_j Σ_i (k_i - k̄_j) v_iᵀ,
// optionally H_j (stored [e][c]) and C_j = (1/n_j) Σ (k_i - k̄_j)(k_i - k̄_j)ᵀ.
//
// One pass over K and V (HBM-bound). A workgroup of 4 waves streams G consecutive
// blocks through LDS; the d x d cross term K_jᵀV_j runs on MFMA with exact bf16
// products and fp32 accumulation, and the per-block centring k̄_j ΣV_jᵀ is removed in
// fp32 before the block is added to the workgroup's partial sum. Partials are reduced
// in a fixed order by a second kernel, so repeated runs are bit-identical.
// The same pass writes the attention kernel's operands in the storage type, as 64-key
// tiles in TileLayout order: Vᵀ per block (and, for bf16, K per block, so that the
// attention kernel streams both straight into MFMA operand registers), centroids and
// mean values ΣV_j / n_j per group of 64 blocks, and H̄[e][c]. Padding keys are zero.
#include "common.hpp"
#include "internal.hpp"

namespace pisa {

template <class T, int D, bool PER_BLOCK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PER_BLOCK ? 1 : 2)))
void block_stats_kernel(StatsArgs a, unsigned flags) {
  using M = typename MmaFor<T>::type;
  constexpr int KI = M::KI, KH = M::KH;
  constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
  constexpr int LDR = D + EPC;             // row stride of the row-major K tile (elements)
  constexpr int LDT = kB + EPC;            // row stride of the transposed tiles
  constexpr int CPR = D / EPC;             // chunks per token row
  constexpr int CPT = kB * CPR / 256;      // chunks per thread per operand
  constexpr int NT = D / 32;               // 32-wide output tiles per side of d x d
  constexpr int TPW = NT * NT / 4;         // output tiles per wave
  // K row-major (source of the operand-order K tile) and Kᵀ, Vᵀ (XOR-swizzled, see tix):
  // the column statistics, the Vᵀ tile and both MFMA operands read 16-byte chunks of the
  // transposed tiles.
  __shared__ __align__(16) T sK[kB * LDR];
  __shared__ __align__(16) T sKt[D * LDT];
  __shared__ __align__(16) T sVt[D * LDT];
  __shared__ float sKbar[D], sVsum[D];

  const int h = blockIdx.y, grp = blockIdx.x;
  const int j0 = grp * a.G;
  const int j1 = min(a.nb, j0 + a.G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int ct = (wave * TPW) / NT;        // row tile (c) of this wave; its tiles share it

  const T* Kh = static_cast<const T*>(a.K) + size_t(h) * a.L * D;
  const T* Vh = static_cast<const T*>(a.V) + size_t(h) * a.L * D;
  using TL = TileLayout<T, D>;
  constexpr int TE = kB * D;               // elements per 64-key tile
  T* vt = reinterpret_cast<T*>(a.packed + a.pl.vt) + size_t(h) * a.nb * TE;
  T* kf = reinterpret_cast<T*>(a.packed + a.pl.kf) + size_t(h) * a.nb * TE;
  T* kbp = reinterpret_cast<T*>(a.packed + a.pl.kbar) + size_t(h) * a.nbp * D;
  T* vbp = reinterpret_cast<T*>(a.packed + a.pl.vbar) + size_t(h) * a.nbp * D;

  // Running Σ_j Σ_i (k_i - k̄_j) v_iᵀ of this workgroup's blocks, as [c][e] MFMA tiles.
  f32x16 run[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) run[u] = zero16();

  // Block j's K and V rows, 16-byte chunks, held in registers one block ahead.
  u32x4 rk[CPT], rv[CPT];
  auto load_block = [&](int j) {
#pragma unroll
    for (int p = 0; p < CPT; ++p) {
      const int c = tid + 256 * p;
      const int row = c / CPR, col = (c % CPR) * EPC;
      rk[p] = *reinterpret_cast<const u32x4*>(Kh + size_t(j * kB + row) * D + col);
      rv[p] = *reinterpret_cast<const u32x4*>(Vh + size_t(j * kB + row) * D + col);
    }
  };
  if (j0 < j1) load_block(j0);

  for (int j = j0; j < j1; ++j) {
    int n = a.block_len ? a.block_len[j] : kB;
    n = min(max(n, 1), kB);
    const float invn = 1.f / float(n);

    __syncthreads();                       // previous block's LDS reads done
#pragma unroll
    for (int p = 0; p < CPT; ++p) {        // stage K_j (row-major and transposed), V_jᵀ; rows >= n_j as zeros
      const int c = tid + 256 * p;
      const int row = c / CPR, col = (c % CPR) * EPC;
      const u32x4 z = {0u, 0u, 0u, 0u};
      const u32x4 kv = row < n ? rk[p] : z, vv = row < n ? rv[p] : z;
      *reinterpret_cast<u32x4*>(sK + row * LDR + col) = kv;
      const T* ek = reinterpret_cast<const T*>(&kv);
      const T* ev = reinterpret_cast<const T*>(&vv);
#pragma unroll
      for (int u = 0; u < EPC; ++u) {
        sKt[tix<T, LDT>(col + u, row)] = ek[u];
        sVt[tix<T, LDT>(col + u, row)] = ev[u];
      }
    }
    if (j + 1 < j1) load_block(j + 1);     // in flight while this block is reduced
    __syncthreads();

    // Column statistics: threads [0, D) own key columns, [128, 128 + D) value columns; each
    // reads its column as 64 / EPC chunks of the transposed tile.
    if (tid < D) {
      float s = 0.f;
      for (int q = 0; q < kB / EPC; ++q) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(sKt + tix<T, LDT>(tid, q * EPC));
        const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
        for (int u = 0; u < EPC; ++u) s += to_f32(e[u]);
      }
      const float mean = s * invn;
      float ss = 0.f;
      for (int q = 0; q < kB / EPC; ++q) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(sKt + tix<T, LDT>(tid, q * EPC));
        const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
        for (int u = 0; u < EPC; ++u) {
          const float dv = to_f32(e[u]) - mean;
          ss += q * EPC + u < n ? dv * dv : 0.f;
        }
      }
      const size_t o = (size_t(h) * a.nb + j) * D + tid;
      a.kbar[o] = mean;
      a.ksig2[o] = ss * invn;
      sKbar[tid] = mean;
      kbp[size_t(j / kB) * TE + TL::k(j % kB, tid)] = from_f32<T>(mean);
    } else if (tid >= 128 && tid < 128 + D) {
      const int c = tid - 128;
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < kB / EPC; ++q) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(sVt + tix<T, LDT>(c, q * EPC));
        const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
        for (int u = 0; u < EPC; ++u) s += to_f32(e[u]);
      }
      a.vsum[(size_t(h) * a.nb + j) * D + c] = s;
      sVsum[c] = s;
      vbp[size_t(j / kB) * TE + TL::v(j % kB, c)] = from_f32<T>(s * invn);
    }

    // Vᵀ tile of the block (and the K tile for bf16), one 16-byte chunk per thread and
    // step in storage order, so the stores are coalesced.
    for (int x = tid; x < TE / EPC; x += 256) {
      int i0 = 0, e = 0;
      TL::vchunk(x, i0, e);
      *reinterpret_cast<u32x4*>(vt + size_t(j) * TE + x * EPC) =
          *reinterpret_cast<const u32x4*>(sVt + tix<T, LDT>(e, i0));
      if constexpr (sizeof(T) == 2) {
        int key = 0, c0 = 0;
        TL::kchunk(x, key, c0);
        *reinterpret_cast<u32x4*>(kf + size_t(j) * TE + x * EPC) =
            *reinterpret_cast<const u32x4*>(sK + key * LDR + c0);
      }
    }
    __syncthreads();                       // sKbar / sVsum visible

    // Cross term on MFMA, accumulated straight into the running sum:
    // run[c][e] += Σ_i K[i][c] V[i][e] (A = Kᵀ, B = V, k = token), then the centring
    // term k̄_j[c] ΣV_j[e] is removed for this block.
    f32x16 blk[PER_BLOCK ? TPW : 1];
#pragma unroll
    for (int u = 0; u < (PER_BLOCK ? TPW : 1); ++u) blk[u] = zero16();
#pragma unroll
    for (int ks = 0; ks < kB / KI; ++ks) {
      const typename M::AB A = M::load(sKt + tix<T, LDT>(32 * ct + l32, KI * ks + KH * g));
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int et = (wave * TPW + u) % NT;
        const typename M::AB Bv = M::load(sVt + tix<T, LDT>(32 * et + l32, KI * ks + KH * g));
        if constexpr (PER_BLOCK) blk[u] = M::mma(A, Bv, blk[u]);
        else run[u] = M::mma(A, Bv, run[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int et = (wave * TPW + u) % NT;
      const int e = 32 * et + l32;
      const float ve = sVsum[e];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * ct + acc_row(r, g);
        if constexpr (PER_BLOCK) {
          const float hv = blk[u][r] - sKbar[c] * ve;
          run[u][r] += hv;
          if (flags & 1u) a.hblk[((size_t(h) * a.nb + j) * D + e) * D + c] = hv;
        } else {
          run[u][r] = fmaf(-sKbar[c], ve, run[u][r]);
        }
      }
    }
    if constexpr (PER_BLOCK) {
      if (flags & 2u) {
        // C_j[c][c'] = (1/n) Σ_i K[i][c] K[i][c'] - k̄_c k̄_c'
        f32x16 cb[TPW];
#pragma unroll
        for (int u = 0; u < TPW; ++u) cb[u] = zero16();
#pragma unroll
        for (int ks = 0; ks < kB / KI; ++ks) {
          const typename M::AB A = M::load(sKt + tix<T, LDT>(32 * ct + l32, KI * ks + KH * g));
#pragma unroll
          for (int u = 0; u < TPW; ++u) {
            const int et = (wave * TPW + u) % NT;
            cb[u] = M::mma(A, M::load(sKt + tix<T, LDT>(32 * et + l32, KI * ks + KH * g)), cb[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          const int et = (wave * TPW + u) % NT;
          const int c2 = 32 * et + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 32 * ct + acc_row(r, g);
            a.cblk[((size_t(h) * a.nb + j) * D + c) * D + c2] = cb[u][r] * invn - sKbar[c] * sKbar[c2];
          }
        }
      }
    }
  }

  float* part = a.part + (size_t(h) * a.ngroups + grp) * D * D;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int et = (wave * TPW + u) % NT;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 32 * ct + acc_row(r, g);
      part[size_t(c) * D + 32 * et + l32] = run[u][r];
    }
  }
}

// Fixed-order reduction of the per-workgroup partials into H̄ᵀ (fp32) and H̄[e][c]
// (storage type); also zeroes the padding rows of the packed centroid / mean-value
// tiles beyond nb so the attention kernel reads finite zeros there.
//
// Workgroup = 16 elements of H̄; thread (sub, xi) sums the group partials q ≡ sub (mod 16)
// of element xi in increasing q, and the 16 partial sums are added in sub order: a fixed
// order, so reruns are bit-identical, with 16 times the parallelism and 1/16 the chain
// length of one sum per element (the long sequences have a thousand partials per head).
template <class T, int D>
__global__ __launch_bounds__(256) void hbar_reduce_kernel(StatsArgs a) {
  __shared__ float red[16][17];
  const int h = blockIdx.y, tid = threadIdx.x, xi = tid & 15, sub = tid >> 4;
  const int x = blockIdx.x * 16 + xi;
  const float* part = a.part + size_t(h) * a.ngroups * D * D + x;
  float ps = 0.f;
  for (int q = sub; q < a.ngroups; q += 16) ps += part[size_t(q) * D * D];
  red[sub][xi] = ps;
  __syncthreads();
  if (sub != 0) return;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += red[k][xi];
  const int c = x / D, e = x % D;
  const float hb = s / float(a.nb);
  a.hbarT[size_t(h) * D * D + x] = hb;
  T* hbp = reinterpret_cast<T*>(a.packed + a.pl.hbar) + size_t(h) * D * D;
  hbp[size_t(e) * D + c] = from_f32<T>(hb);

  const int pad = a.nbp - a.nb;
  if (pad > 0 && x < pad * D) {
    using TL = TileLayout<T, D>;
    const size_t last = size_t(a.nb / kB) * kB * D;       // first element of the last group
    const int key = a.nb % kB + x / D, col = x % D;
    T* kbp = reinterpret_cast<T*>(a.packed + a.pl.kbar) + size_t(h) * a.nbp * D;
    T* vbp = reinterpret_cast<T*>(a.packed + a.pl.vbar) + size_t(h) * a.nbp * D;
    kbp[last + TL::k(key, col)] = from_f32<T>(0.f);
    vbp[last + TL::v(key, col)] = from_f32<T>(0.f);
  }
}

// Block heterogeneity M_j = ||H_j - H̄||_F (PISA paper §3.3: the error bound of replacing
// every H_j by the global H̄ grows with max_j ||H_j - H̄||, and covariance-aware selection
// takes its log as a routing prior; the Frobenius norm bounds the spectral one). H̄ is
// only known once every block has been reduced, so this is a second pass over K and V
// with the first pass's layout: G blocks per workgroup through LDS, K_jᵀV_j on MFMA,
// centring with the first pass's k̄_j and ΣV_j, H̄ᵀ held in registers in accumulator
// order. Squares are summed per lane, then across lanes and waves in a fixed order.
template <class T, int D>
__global__ __launch_bounds__(256) void heterogeneity_kernel(StatsArgs a) {
  using M = typename MmaFor<T>::type;
  constexpr int KI = M::KI, KH = M::KH;
  constexpr int EPC = 16 / sizeof(T), LDT = kB + EPC, CPR = D / EPC, CPT = kB * CPR / 256;
  constexpr int NT = D / 32, TPW = NT * NT / 4;
  __shared__ __align__(16) T sKt[D * LDT];      // K_jᵀ, V_jᵀ, XOR-swizzled (see tix)
  __shared__ __align__(16) T sVt[D * LDT];
  __shared__ float sKbar[D], sVsum[D], sPart[4];

  const int h = blockIdx.y, j0 = blockIdx.x * a.G, j1 = min(a.nb, j0 + a.G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int ct = (wave * TPW) / NT;
  const T* Kh = static_cast<const T*>(a.K) + size_t(h) * a.L * D;
  const T* Vh = static_cast<const T*>(a.V) + size_t(h) * a.L * D;

  f32x16 hb[TPW];                          // H̄ᵀ[c][e] at this lane's accumulator slots
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int e = 32 * ((wave * TPW + u) % NT) + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) hb[u][r] = a.hbarT[(size_t(h) * D + 32 * ct + acc_row(r, g)) * D + e];
  }

  u32x4 rk[CPT], rv[CPT];
  auto load_block = [&](int j) {
#pragma unroll
    for (int p = 0; p < CPT; ++p) {
      const int c = tid + 256 * p, row = c / CPR, col = (c % CPR) * EPC;
      rk[p] = *reinterpret_cast<const u32x4*>(Kh + size_t(j * kB + row) * D + col);
      rv[p] = *reinterpret_cast<const u32x4*>(Vh + size_t(j * kB + row) * D + col);
    }
  };
  if (j0 < j1) load_block(j0);

  for (int j = j0; j < j1; ++j) {
    int n = a.block_len ? a.block_len[j] : kB;
    n = min(max(n, 1), kB);
    __syncthreads();                       // previous block's LDS reads done
#pragma unroll
    for (int p = 0; p < CPT; ++p) {
      const int c = tid + 256 * p, row = c / CPR, col = (c % CPR) * EPC;
      const u32x4 z = {0u, 0u, 0u, 0u};
      const u32x4 kv = row < n ? rk[p] : z, vv = row < n ? rv[p] : z;
      const T* ek = reinterpret_cast<const T*>(&kv);
      const T* ev = reinterpret_cast<const T*>(&vv);
#pragma unroll
      for (int u = 0; u < EPC; ++u) {
        sKt[tix<T, LDT>(col + u, row)] = ek[u];
        sVt[tix<T, LDT>(col + u, row)] = ev[u];
      }
    }
    const size_t o = (size_t(h) * a.nb + j) * D;
    if (tid < D) sKbar[tid] = a.kbar[o + tid];
    else if (tid >= 128 && tid < 128 + D) sVsum[tid - 128] = a.vsum[o + tid - 128];
    if (j + 1 < j1) load_block(j + 1);
    __syncthreads();

    f32x16 blk[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) blk[u] = zero16();
#pragma unroll
    for (int ks = 0; ks < kB / KI; ++ks) {
      const typename M::AB A = M::load(sKt + tix<T, LDT>(32 * ct + l32, KI * ks + KH * g));
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int et = (wave * TPW + u) % NT;
        blk[u] = M::mma(A, M::load(sVt + tix<T, LDT>(32 * et + l32, KI * ks + KH * g)), blk[u]);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const float ve = sVsum[32 * ((wave * TPW + u) % NT) + l32];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dv = blk[u][r] - sKbar[32 * ct + acc_row(r, g)] * ve - hb[u][r];
        ss = fmaf(dv, dv, ss);
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    if (lane == 0) sPart[wave] = ss;
    __syncthreads();
    if (tid == 0) a.hnorm[size_t(h) * a.nb + j] = sqrtf((sPart[0] + sPart[1]) + (sPart[2] + sPart[3]));
  }
}

// Launch order of the query tiles for the bf16 attention kernels: tiles of more than 32
// valid rows (two query halves per tile), then the others, each ascending. Entry
// tile * 128 + rows after the two counts; one workgroup, each thread a contiguous chunk.
__global__ __launch_bounds__(256) void tile_order_kernel(StatsArgs a) {
  __shared__ int sh[8];
  int32_t* out = reinterpret_cast<int32_t*>(a.packed + a.pl.tiles);
  const int nb = a.nb, C = (nb + 255) / 256, t0 = min(int(threadIdx.x) * C, nb), t1 = min(t0 + C, nb);
  auto rows = [&](int t) { return a.block_len ? min(max(a.block_len[t], 1), kB) : kB; };
  int full = 0;
  for (int t = t0; t < t1; ++t) full += rows(t) > 32;
  int total;
  const int before = block_exclusive_scan_256(full, sh, &total);
  int pf = before, pr = total + (t0 - before);
  for (int t = t0; t < t1; ++t) {
    const int r = rows(t);
    out[2 + (r > 32 ? pf++ : pr++)] = t * 128 + r;
  }
  if (threadIdx.x == 0) {
    out[0] = total;
    out[1] = nb - total;
  }
}

template <class T, int D>
static hipError_t launch_stats_t(const StatsArgs& a, unsigned flags, hipStream_t s) {
  dim3 g1(a.ngroups, a.H), g2(D * D / 16, a.H);
  if (flags & 3u) hipLaunchKernelGGL((block_stats_kernel<T, D, true>), g1, dim3(256), 0, s, a, flags);
  else hipLaunchKernelGGL((block_stats_kernel<T, D, false>), g1, dim3(256), 0, s, a, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((hbar_reduce_kernel<T, D>), g2, dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (flags & 4u) {
    hipLaunchKernelGGL((heterogeneity_kernel<T, D>), g1, dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(tile_order_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_block_stats(int bf16, const StatsArgs& a, unsigned flags, hipStream_t s) {
  if (bf16) return a.d == 64 ? launch_stats_t<uint16_t, 64>(a, flags, s) : launch_stats_t<uint16_t, 128>(a, flags, s);
  return a.d == 64 ? launch_stats_t<float, 64>(a, flags, s) : launch_stats_t<float, 128>(a, flags, s);
}

}  // namespace pisa
