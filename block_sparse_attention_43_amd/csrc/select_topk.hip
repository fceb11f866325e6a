// Prepare phase, part 2: pooled-query block scores, the second-order matrix and
// block-wise top-K selection.
//
// q̄_i = mean of the valid rows of query tile i, \overline{q²}_i = mean of their squares
// (PISA paper Fig. 3 prepare phase; Sparse Linear Attention blog, PWT section: square
// first, then average). Scores s_{i,j} = q̄_i·k̄_j (MoBA-style block-mean scoring,
// blog Sparse Attention section) and w̃_{i,j} = ½ Σ_c \overline{q²}_{i,c} σ²_{j,c}, the
// [query block x key block] matrix that PWT computes once before the attention kernel.
// S_i keeps the K_sel largest scores, ties to the lower block index, emitted in
// ascending block order plus a bitmask of the selected blocks. Covariance-aware routing
// (PISA paper §3.3, Eq. (7)) adds ln(M_j + eps) of the block heterogeneity to every score
// of key block j; the row softmax of Eq. (7) keeps the order, so the top-K is taken on
// the sum. Routing by predicted truncation error (Sparse Linear Attention blog, PWT
// section: mass times heterogeneity) adds w̃_{i,j} + ln n_j on top.
//
// Scores are fp32 (matrix-core fp32 products and sums) with one fixed summation order per
// element, so identical centroids score identically. Top-K is an exact radix select on
// order-preserving 32-bit keys held in registers (256 threads, up to 128 keys each), with
// the tie rule resolved by block-wide prefix counts in index order.
#include "common.hpp"
#include "internal.hpp"

namespace pisa {

template <class T, int D>
__global__ __launch_bounds__(256) void pool_kernel(SelectArgs a) {
  // Thread t reads 16-byte chunks (EPC columns) of rows t / CPR + RG * p; column sums and
  // sums of squares are reduced over the RG row groups through LDS.
  constexpr int EPC = 16 / sizeof(T);
  constexpr int CPR = D / EPC;             // chunks per row
  constexpr int RG = 256 / CPR;            // row groups
  __shared__ float s1[RG][D], s2[RG][D];
  const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  int n = a.block_len ? a.block_len[i] : kB;
  n = min(max(n, 1), kB);
  const int ch = tid % CPR, rg = tid / CPR;
  const T* Qt = static_cast<const T*>(a.Q) + (size_t(h) * a.L + size_t(i) * kB) * D;
  float sum[EPC], sq[EPC];
#pragma unroll
  for (int u = 0; u < EPC; ++u) sum[u] = sq[u] = 0.f;
#pragma unroll
  for (int p = 0; p < kB / RG; ++p) {
    const int r = rg + RG * p;
    if (r < n) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(Qt + size_t(r) * D + ch * EPC);
      const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
      for (int u = 0; u < EPC; ++u) {
        const float x = to_f32(e[u]);
        sum[u] += x;
        sq[u] += x * x;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < EPC; ++u) {
    s1[rg][ch * EPC + u] = sum[u];
    s2[rg][ch * EPC + u] = sq[u];
  }
  __syncthreads();
  if (tid < D) {
    float t1 = 0.f, t2 = 0.f;
    for (int q = 0; q < RG; ++q) {
      t1 += s1[q][tid];
      t2 += s2[q][tid];
    }
    const float invn = 1.f / float(n);
    a.qbar[(size_t(h) * a.nb + i) * D + tid] = t1 * invn;
    a.qsq[(size_t(h) * a.nb + i) * D + tid] = t2 * invn;
  }
}

// RoPE-aware centroids (Sparse Linear Attention (2) blog, Selection Error): the mean of
// the valid pre-rotation rows of block i (queries for blockIdx.z = 0, keys for 1), turned
// by the rotary embedding at the block centre c_i = mean position of its valid tokens, so
// that q̄·k̄ of two turned means depends on c_j - c_i only. Column means as in pool_kernel;
// the centre and the angles c_a · base^(-2f/width_a) are taken in fp64, the turn in fp32.
template <class T, int D>
__global__ __launch_bounds__(256) void rope_pool_kernel(SelectArgs a) {
  constexpr int EPC = 16 / sizeof(T), CPR = D / EPC, RG = 256 / CPR;
  __shared__ float s1[RG][D];
  __shared__ float mean[D];
  __shared__ double centre[3];
  const int i = blockIdx.x, h = blockIdx.y, keys = blockIdx.z, tid = threadIdx.x;
  int n = a.block_len ? a.block_len[i] : kB;
  n = min(max(n, 1), kB);
  const int ch = tid % CPR, rg = tid / CPR;
  const T* X = static_cast<const T*>(keys ? a.K_pre : a.Q_pre) + (size_t(h) * a.L + size_t(i) * kB) * D;
  float sum[EPC];
#pragma unroll
  for (int u = 0; u < EPC; ++u) sum[u] = 0.f;
#pragma unroll
  for (int p = 0; p < kB / RG; ++p) {
    const int r = rg + RG * p;
    if (r < n) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(X + size_t(r) * D + ch * EPC);
      const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
      for (int u = 0; u < EPC; ++u) sum[u] += to_f32(e[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < EPC; ++u) s1[rg][ch * EPC + u] = sum[u];
  if (tid < a.rope_axes) {
    double c = 0.0;
    for (int r = 0; r < n; ++r) c += double(a.pos[(size_t(i) * kB + r) * a.rope_axes + tid]);
    centre[tid] = c / double(n);
  }
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
    for (int q = 0; q < RG; ++q) t += s1[q][tid];
    mean[tid] = t * (1.f / float(n));
  }
  __syncthreads();
  if (tid < D / 2) {                         // pair tid: axis ax, frequency f
    int ax = 0, off = 0, f = tid;
    while (ax + 1 < a.rope_axes && f >= a.rope_width[ax] / 2) {
      f -= a.rope_width[ax] / 2;
      off += a.rope_width[ax];
      ++ax;
    }
    const int w = a.rope_width[ax];
    const int i0 = a.rope_pairs ? off + f : off + 2 * f;
    const int i1 = a.rope_pairs ? i0 + w / 2 : i0 + 1;
    const double ang = centre[ax] * pow(double(a.rope_base), -2.0 * f / w);
    double sd, cd;
    sincos(ang, &sd, &cd);
    const float cs = float(cd), sn = float(sd), x0 = mean[i0], x1 = mean[i1];
    float* out = (keys ? a.krot : a.qbar) + (size_t(h) * a.nb + i) * D;
    out[i0] = x0 * cs - x1 * sn;
    out[i1] = x0 * sn + x1 * cs;
  }
}

// S = Q̄ K̄ᵀ and W = ½ Q̄² Σ²ᵀ per head on the fp32 matrix cores: a 64x64 output tile per
// workgroup, each of its four waves a 32x32 quarter (v_mfma_f32_32x32x2f32 over the head
// dimension). The 64 query and 64 key rows are staged in LDS with coalesced 16-byte loads.
// MFMA step m pairs column m (lane half 0) with column m + D/2 (lane half 1), so each
// lane reads one contiguous half row per operand. Every output element is accumulated
// in the same order whatever its position, so identical centroids score identically.
template <int D>
__global__ __launch_bounds__(256) void score_kernel(SelectArgs a) {
  constexpr int KH = D / 2;                // MFMA steps
  constexpr int RS = D + 4;                // LDS row stride in floats (staggers the banks)
  constexpr int CPR = D / 4, NCH = 64 * CPR / 256;
  __shared__ __align__(16) float sA[64 * RS], sB[64 * RS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
  // Workgroups are dealt round-robin to the XCDs: remap so that the tiles of one head run
  // on one XCD and read its centroids from that XCD's L2.
  const uint32_t nt = gridDim.x, lin = xcd_remap(blockIdx.x + nt * (blockIdx.y + nt * blockIdx.z), nt * nt * gridDim.z);
  const int h = int(lin / (nt * nt)), i0 = int(lin / nt % nt) * 64, j0 = int(lin % nt) * 64, nb = a.nb;
  const int wi = (wave >> 1) * 32, wj = (wave & 1) * 32;
  const int col = j0 + wj + c;
  auto product = [&](const float* A, const float* B) {
#pragma unroll
    for (int p = 0; p < NCH; ++p) {          // rows past nb read a valid row, not stored
      const int q = tid + 256 * p, r = q / CPR, cc = 4 * (q % CPR);
      const float4 va = *reinterpret_cast<const float4*>(A + (size_t(h) * nb + min(i0 + r, nb - 1)) * D + cc);
      const float4 vb = *reinterpret_cast<const float4*>(B + (size_t(h) * nb + min(j0 + r, nb - 1)) * D + cc);
      *reinterpret_cast<float4*>(&sA[r * RS + cc]) = va;
      *reinterpret_cast<float4*>(&sB[r * RS + cc]) = vb;
    }
    __syncthreads();
    const float* pa = &sA[(wi + c) * RS + KH * g];
    const float* pb = &sB[(wj + c) * RS + KH * g];
    f32x16 acc = zero16();
#pragma unroll
    for (int u = 0; u < KH / 4; ++u) {
      const float4 x = *reinterpret_cast<const float4*>(pa + 4 * u);
      const float4 y = *reinterpret_cast<const float4*>(pb + 4 * u);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x.x, y.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x.y, y.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x.z, y.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x.w, y.w, acc, 0, 0, 0);
    }
    __syncthreads();                         // LDS reused by the next product
    return acc;
  };
  auto store = [&](float* out, const f32x16& v) {
    if (col >= nb) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = i0 + wi + acc_row(r, g);
      if (row < nb) out[(size_t(h) * nb + row) * nb + col] = v[r];
    }
  };
  f32x16 w = zero16();
  if (a.wt || a.route == 2) {
    w = product(a.qsq, a.ksig2);
#pragma unroll
    for (int r = 0; r < 16; ++r) w[r] *= 0.5f;
    if (a.wt) store(a.wt, w);
  }
  f32x16 s = product(a.qbar, a.rope_axes ? a.krot : a.kbar);
  if (a.route != 0 && col < nb) {
    // per key block: ln(M_j + eps) (Eq. (7)), plus ln n_j and w̃ for the predicted-error route
    float bias = logf(a.hnorm[size_t(h) * nb + col] + a.route_eps);
    if (a.route == 2) {
      const int n = a.block_len ? min(max(a.block_len[col], 1), kB) : kB;
      bias += logf(float(n));
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = (a.route == 2 ? s[r] + w[r] : s[r]) + bias;
  }
  store(a.scores, s);
}

__device__ __forceinline__ uint32_t order_key(float s) {
  s = s + 0.0f;                                   // -0 -> +0 so equal scores tie
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup per (query tile, head). Thread t owns block indices [t*P, t*P + P).
template <int P>
__global__ __launch_bounds__(256) void topk_kernel(SelectArgs a) {
  __shared__ int hist[256];
  __shared__ int scan_sh[8];
  __shared__ uint32_t s_digit;
  __shared__ int s_rem;
  __shared__ uint32_t smask[1024];
  const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int nb = a.nb, K = a.K_sel;
  const float* row = a.scores + (size_t(h) * nb + i) * nb;
  const int base = tid * P;

  uint32_t key[P];
#pragma unroll
  for (int p = 0; p < P; ++p) key[p] = (base + p < nb) ? order_key(row[base + p]) : 0u;

  // Threshold key T (the K-th largest) and how many keys equal to T are taken.
  uint32_t T = 0u;
  int take_eq = 0;
  bool all = (K >= nb);
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
      const int b = 255 - tid;                 // scan from the highest digit down
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

  // Selected flags in index order: key > T, or key == T among the first take_eq such.
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
  int32_t* out = a.idx + (size_t(h) * nb + i) * K;
  if (a.mask) {
    for (int w = tid; w < a.nw; w += 256) smask[w] = 0u;
    __syncthreads();
  }
  {
    int eqc = eq_start;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (selected(p, eqc)) {
        if (pos < K) out[pos] = base + p;   // bound holds by construction; kept as a guard
        ++pos;
        if (a.mask) atomicOr(&smask[(base + p) >> 5], 1u << ((base + p) & 31));
      }
    }
  }
  if (a.mask) {
    __syncthreads();
    uint32_t* mo = a.mask + (size_t(h) * nb + i) * a.nw;
    for (int w = tid; w < a.nw; w += 256) mo[w] = smask[w];
  }
}

// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// One wave per (query tile, head), four rows per workgroup, for nb <= 64 P: lane l owns
// block indices [l P, l P + P), so index order is lane order and the tie rule is a lane
// prefix. The same radix select as topk_kernel with wave-private histograms in LDS and
// wave scans instead of block barriers.
template <int P>
__global__ __launch_bounds__(256) void topk_wave_kernel(SelectArgs a) {
  __shared__ int hist[4][256];
  __shared__ uint32_t smask[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = a.nb, K = a.K_sel;
  const int row_id = blockIdx.x * 4 + wave;          // h * nb + i
  if (row_id >= a.H * nb) return;                     // whole waves leave together
  const float* row = a.scores + size_t(row_id) * nb;
  const int base = lane * P;
  int* hw = hist[wave];

  uint32_t key[P];
#pragma unroll
  for (int p = 0; p < P; ++p) key[p] = (base + p < nb) ? order_key(row[base + p]) : 0u;

  uint32_t Tk = 0u;
  int take_eq = 0;
  const bool all = K >= nb;
  if (K > 0 && !all) {
    uint32_t prefix = 0u, pmask = 0u;
    int rem = K;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
#pragma unroll
      for (int q = 0; q < 4; ++q) hw[4 * lane + q] = 0;
#pragma unroll
      for (int p = 0; p < P; ++p)
        if (base + p < nb && (key[p] & pmask) == prefix) atomicAdd(&hw[(key[p] >> shift) & 255u], 1);
      // lane l takes digits 255 - 4l .. 252 - 4l (high digits first)
      int c[4], own = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = hw[255 - 4 * lane - q];
        own += c[q];
      }
      const int incl = wave_inclusive_scan(own);
      int excl = incl - own;
      // the lane whose digits reach rem finds the digit; broadcast it
      int dg = -1, rm = 0;
      if (excl < rem && incl >= rem) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (dg < 0 && excl + c[q] >= rem) {
            dg = 255 - 4 * lane - q;
            rm = rem - excl;
          }
          excl += c[q];
        }
      }
      const uint64_t who = __ballot(dg >= 0);
      const int src = __ffsll(static_cast<unsigned long long>(who)) - 1;
      dg = __shfl(dg, src, 64);
      rm = __shfl(rm, src, 64);
      prefix |= uint32_t(dg) << shift;
      pmask |= 0xFFu << shift;
      rem = rm;
    }
    Tk = prefix;
    take_eq = rem;
  }

  int eq_local = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) eq_local += (base + p < nb && key[p] == Tk) ? 1 : 0;
  const int eq_start = wave_inclusive_scan(eq_local) - eq_local;
  auto selected = [&](int p, int& eqc) -> bool {
    if (base + p >= nb) return false;
    if (all) return true;
    if (K == 0) return false;
    if (key[p] > Tk) return true;
    if (key[p] == Tk) return eqc++ < take_eq;
    return false;
  };
  int cnt = 0;
  {
    int eqc = eq_start;
#pragma unroll
    for (int p = 0; p < P; ++p) cnt += selected(p, eqc) ? 1 : 0;
  }
  int pos = wave_inclusive_scan(cnt) - cnt;
  int32_t* out = a.idx + size_t(row_id) * K;
  uint32_t* sm = smask[wave];
  if (a.mask) sm[lane] = 0u;
  {
    int eqc = eq_start;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (selected(p, eqc)) {
        if (pos < K) out[pos] = base + p;   // bound holds by construction; kept as a guard
        ++pos;
        if (a.mask) atomicOr(&sm[(base + p) >> 5], 1u << ((base + p) & 31));
      }
    }
  }
  if (a.mask) {
    uint32_t* mo = a.mask + size_t(row_id) * a.nw;
    if (lane < a.nw) mo[lane] = sm[lane];
  }
}

template <class T, int D>
static hipError_t launch_select_t(const SelectArgs& a, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (a.rope_axes == 0 || a.wt) {            // RoPE-aware scores read Q only for w̃
    hipLaunchKernelGGL((pool_kernel<T, D>), dim3(a.nb, a.H), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.rope_axes > 0) {                     // after pool_kernel: replaces q̄
    hipLaunchKernelGGL((rope_pool_kernel<T, D>), dim3(a.nb, a.H, 2), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nt = (a.nb + 63) / 64;
  hipLaunchKernelGGL((score_kernel<D>), dim3(nt, nt, a.H), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.nb <= 64 * 32) {
    const int pw = (a.nb + 63) / 64;
    const dim3 gw(unsigned((size_t(a.H) * a.nb + 3) / 4));
    if (pw <= 4) hipLaunchKernelGGL((topk_wave_kernel<4>), gw, dim3(256), 0, s, a);
    else if (pw <= 8) hipLaunchKernelGGL((topk_wave_kernel<8>), gw, dim3(256), 0, s, a);
    else if (pw <= 12) hipLaunchKernelGGL((topk_wave_kernel<12>), gw, dim3(256), 0, s, a);
    else if (pw <= 16) hipLaunchKernelGGL((topk_wave_kernel<16>), gw, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((topk_wave_kernel<32>), gw, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int per = (a.nb + 255) / 256;
  const dim3 g(a.nb, a.H);
  if (per <= 1) hipLaunchKernelGGL((topk_kernel<1>), g, dim3(256), 0, s, a);
  else if (per <= 2) hipLaunchKernelGGL((topk_kernel<2>), g, dim3(256), 0, s, a);
  else if (per <= 4) hipLaunchKernelGGL((topk_kernel<4>), g, dim3(256), 0, s, a);
  else if (per <= 8) hipLaunchKernelGGL((topk_kernel<8>), g, dim3(256), 0, s, a);
  else if (per <= 16) hipLaunchKernelGGL((topk_kernel<16>), g, dim3(256), 0, s, a);
  else if (per <= 32) hipLaunchKernelGGL((topk_kernel<32>), g, dim3(256), 0, s, a);
  else if (per <= 64) hipLaunchKernelGGL((topk_kernel<64>), g, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((topk_kernel<128>), g, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(int bf16, const SelectArgs& a, hipStream_t s) {
  if (bf16) return a.d == 64 ? launch_select_t<uint16_t, 64>(a, s) : launch_select_t<uint16_t, 128>(a, s);
  return a.d == 64 ? launch_select_t<float, 64>(a, s) : launch_select_t<float, 128>(a, s);
}

}  // namespace pisa
