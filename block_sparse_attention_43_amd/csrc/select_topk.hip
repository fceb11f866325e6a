// Prepare phase, part 2: pooled-query block scores, the second-order matrix and
// block-wise top-K selection.
//
// q̄_i = mean of the valid rows of query tile i, \overline{q²}_i = mean of their squares
// (PISA paper Fig. 3 prepare phase; Sparse Linear Attention blog, PWT section: square
// first, then average). Scores s_{i,j} = q̄_i·k̄_j (MoBA-style block-mean scoring,
// blog Sparse Attention section); the matrix w̃_{i,j} = ½ Σ_c \overline{q²}_{i,c} σ²_{j,c}
// that PWT reads in the attention call is written by pooled_w.hip. S_i keeps the K_sel largest scores, ties to the lower block index, emitted in
// ascending block order plus a bitmask of the selected blocks. Covariance-aware routing
// (PISA paper §3.3, Eq. (7)) adds ln(M_j + eps) of the block heterogeneity to every score
// of key block j; the row softmax of Eq. (7) keeps the order, so the top-K is taken on
// the sum. Routing by predicted truncation error (Sparse Linear Attention blog, PWT
// section: mass times heterogeneity) adds w̃_{i,j} + ln n_j on top.
//
// Scores are fp32 (matrix-core fp32 products and sums) with one fixed summation order per
// element, so identical centroids score identically. Rows of at most kSmallNb blocks are
// stored and selected here (linear bins over the row's range, then a radix select on
// order-preserving 32-bit keys within the threshold bin, the tie rule by prefix counts in
// index order); longer rows go to select_large.hip, which recomputes the scores instead
// of storing them.
#include "common.hpp"
#include "internal.hpp"
#include "select_common.hpp"

namespace pisa {

// One wave per query tile, four tiles per workgroup. Lane l reads 16-byte chunk l % CPR of
// rows l / CPR + RPL·p (RPL = 64 / CPR rows per wave-wide load, all loads issued before
// any sum), so each load instruction covers RPL whole rows; the lanes holding the same
// chunk then add their column sums and sums of squares with lane exchanges, in a fixed
// order. No LDS and no workgroup barrier.
template <class T, int D>
__global__ __launch_bounds__(256) void pool_kernel(SelectArgs a) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int CPR = D / EPC;             // chunks per row
  static_assert(CPR <= 64 && 64 % CPR == 0, "a row fits one wave-wide load");
  constexpr int RPL = 64 / CPR;            // rows per wave-wide load
  constexpr int NL = kB / RPL;             // loads per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = blockIdx.x * 4 + wave, h = blockIdx.y;
  if (i >= a.nb) return;                   // whole waves leave together
  int n = a.block_len ? a.block_len[i] : kB;
  n = min(max(n, 1), kB);
  const int ch = lane % CPR, r0 = lane / CPR;
  const T* Qt = static_cast<const T*>(a.Q) + (size_t(h) * a.L + size_t(i) * kB) * D;
  u32x4 v[NL];
#pragma unroll
  for (int p = 0; p < NL; ++p) {
    const int r = r0 + RPL * p;
    v[p] = r < n ? *reinterpret_cast<const u32x4*>(Qt + size_t(r) * D + ch * EPC) : u32x4{0u, 0u, 0u, 0u};
  }
  float sum[EPC], sq[EPC];
#pragma unroll
  for (int u = 0; u < EPC; ++u) sum[u] = sq[u] = 0.f;
#pragma unroll
  for (int p = 0; p < NL; ++p) {
    const T* e = reinterpret_cast<const T*>(&v[p]);
#pragma unroll
    for (int u = 0; u < EPC; ++u) {
      const float x = to_f32(e[u]);
      sum[u] += x;
      sq[u] += x * x;
    }
  }
#pragma unroll
  for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
    for (int u = 0; u < EPC; ++u) {
      sum[u] += __shfl_xor(sum[u], o, 64);
      sq[u] += __shfl_xor(sq[u], o, 64);
    }
  if (lane < CPR) {
    const float invn = 1.f / float(n);
    float* qb = a.qbar + (size_t(h) * a.nb + i) * D + ch * EPC;
    float* qs = a.qsq + (size_t(h) * a.nb + i) * D + ch * EPC;
#pragma unroll
    for (int u = 0; u < EPC; u += 4) {
      *reinterpret_cast<float4*>(qb + u) = make_float4(sum[u] * invn, sum[u + 1] * invn, sum[u + 2] * invn, sum[u + 3] * invn);
      *reinterpret_cast<float4*>(qs + u) = make_float4(sq[u] * invn, sq[u + 1] * invn, sq[u + 2] * invn, sq[u + 3] * invn);
    }
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

// S = Q̄ K̄ᵀ per head (plus W = ½ Q̄² Σ²ᵀ for the predicted-error route) on the fp32
// matrix cores: a 64x64 output tile per workgroup, each of its four waves a 32x32 quarter
// (v_mfma_f32_32x32x2f32 over the head dimension). The 64 query and 64 key rows are staged in LDS with coalesced 16-byte loads.
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
  if (a.route == 2) {                        // predicted-error route: w̃ enters the score
    w = product(a.qsq, a.ksig2);
#pragma unroll
    for (int r = 0; r < 16; ++r) w[r] *= 0.5f;
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

// One wave per (query tile, head), four rows per workgroup, for nb <= 64 P: lane l owns
// block indices [l P, l P + P), so index order is lane order and the tie rule is a lane
// prefix.
//
// The row reaches the lanes through LDS: the wave reads it with coalesced 16-byte loads
// into a per-wave buffer padded by one word every 32 (a lane's P words then sit in
// distinct banks) and each lane takes its own range from there.
//
// Selection is exact in two stages. First, 256 linear bins over the row's value range
// [lo, hi]: bin(x) = min(255, ⌊(x - lo)·256 / (hi - lo)⌋) in fp32, a non-decreasing
// function of x, so every key in a higher bin is at least every key in a lower one and
// equal scores share a bin; the histogram gives the bin b* that holds the K-th largest
// score and how many of the K fall in it. Scores spread over many bins, so the LDS
// counters see little contention (an 8-bit radix digit of the raw key puts most of a
// row's scores in a handful of exponent digits). Second, the 4-pass 8-bit radix select
// on order-preserving keys, over the keys of bin b* only, fixes the threshold key and how
// many keys equal to it are taken, lowest indices first. A row whose range is not finite
// puts every key in bin 0, which is the plain radix select.
template <int P>
__global__ __launch_bounds__(256) void topk_wave_kernel(SelectArgs a) {
  constexpr int NBIN = 256;
  constexpr int RW = 64 * P + 2 * P;         // padded row words per wave (one pad word per 32)
  __shared__ int hist[4][NBIN];
  __shared__ uint32_t smask[4][64];
  __shared__ float srow[4][RW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = a.nb, K = a.K_sel;
  const int row_id = blockIdx.x * 4 + wave;          // h * nb + i
  if (row_id >= a.H * nb) return;                     // whole waves leave together
  const float* row = a.scores + size_t(row_id) * nb;
  const int base = lane * P;
  int* hw = hist[wave];
  float* rs = srow[wave];
  auto pad = [](int e) { return e + (e >> 5); };

  // Coalesced staging: 16-byte chunks where the row allows (rows start at a multiple of
  // nb floats, so only nb % 4 == 0 keeps every chunk aligned), single words otherwise.
  // All loads are issued before the first LDS write, so one memory latency covers the row.
  if ((nb & 3) == 0) {
    constexpr int NC = (P + 3) / 4;                 // 16-byte chunks per lane
    float4 v[NC];
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      const int c = min(lane + 64 * q, nb / 4 - 1);  // clamped in bounds; the extra chunks are not stored
      v[q] = *reinterpret_cast<const float4*>(row + 4 * c);
    }
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      const int c = lane + 64 * q;
      if (4 * c < nb) {
        rs[pad(4 * c)] = v[q].x; rs[pad(4 * c + 1)] = v[q].y; rs[pad(4 * c + 2)] = v[q].z; rs[pad(4 * c + 3)] = v[q].w;
      }
    }
  } else {
    float v[P];
#pragma unroll
    for (int q = 0; q < P; ++q) v[q] = row[min(lane + 64 * q, nb - 1)];
#pragma unroll
    for (int q = 0; q < P; ++q)
      if (lane + 64 * q < nb) rs[pad(lane + 64 * q)] = v[q];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  uint32_t key[P];
  float x[P];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const bool v = base + p < nb;
    x[p] = v ? rs[pad(base + p)] + 0.0f : 0.f;      // -0 -> +0 so equal scores tie
    key[p] = v ? order_key(x[p]) : 0u;
    if (v) {
      kmin = min(kmin, key[p]);
      kmax = max(kmax, key[p]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, uint32_t(__shfl_xor(int(kmin), o, 64)));
    kmax = max(kmax, uint32_t(__shfl_xor(int(kmax), o, 64)));
  }
  auto key_value = [](uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); };
  const float lo = key_value(kmin), hi = key_value(kmax);
  const float span = hi - lo;
  const float scale = float(NBIN) / span;
  const bool lin = __builtin_isfinite(lo) && __builtin_isfinite(hi) && span > 0.f && __builtin_isfinite(span) &&
                   __builtin_isfinite(scale) && scale > 0.f;
  int bn[P];
#pragma unroll
  for (int p = 0; p < P; ++p) bn[p] = lin ? min(NBIN - 1, int((x[p] - lo) * scale)) : 0;

  // Finds the digit (0..255, high first) whose count reaches rem; returns it and the rank
  // left within it. Lane l holds the counts of digits 255 - 4l .. 252 - 4l.
  auto find_digit = [&](int rem, int& rm) -> int {
    int c[4], own = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = hw[255 - 4 * lane - q];
      own += c[q];
    }
    const int incl = wave_inclusive_scan(own);
    int excl = incl - own;
    int dg = -1, r = 0;
    if (excl < rem && incl >= rem) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (dg < 0 && excl + c[q] >= rem) {
          dg = 255 - 4 * lane - q;
          r = rem - excl;
        }
        excl += c[q];
      }
    }
    const uint64_t who = __ballot(dg >= 0);
    const int src = __ffsll(static_cast<unsigned long long>(who)) - 1;
    rm = __shfl(r, src, 64);
    return __shfl(dg, src, 64);
  };

  int bstar = -1;                               // threshold bin; keys above it are all taken
  uint32_t Tk = 0u;
  int take_eq = 0;
  const bool all = K >= nb;
  if (K > 0 && !all) {
#pragma unroll
    for (int q = 0; q < 4; ++q) hw[4 * lane + q] = 0;
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (base + p < nb) atomicAdd(&hw[bn[p]], 1);
    int rem = 0;
    bstar = find_digit(K, rem);
    // The keys of bin b* (usually a few dozen) are gathered into the wave's LDS buffer,
    // which the row no longer needs, at most CM per lane; the radix passes then visit
    // those instead of all P keys of every lane. A larger bin keeps the keys in place.
    constexpr int CM = 4;
    int cl = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) cl += (base + p < nb && bn[p] == bstar) ? 1 : 0;
    const int cincl = wave_inclusive_scan(cl);
    const int ctot = __shfl(cincl, 63, 64);
    uint32_t prefix = 0u, pmask = 0u;
    auto radix = [&](auto count_keys) {
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
#pragma unroll
        for (int q = 0; q < 4; ++q) hw[4 * lane + q] = 0;
        count_keys(shift, pmask, prefix);
        int rm = 0;
        const int dg = find_digit(rem, rm);
        prefix |= uint32_t(dg) << shift;
        pmask |= 0xFFu << shift;
        rem = rm;
      }
    };
    if (ctot <= 64 * CM) {
      uint32_t* cbuf = reinterpret_cast<uint32_t*>(rs);
      int w = cincl - cl;
#pragma unroll
      for (int p = 0; p < P; ++p)
        if (base + p < nb && bn[p] == bstar) cbuf[w++] = key[p];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      uint32_t ck[CM];
#pragma unroll
      for (int m = 0; m < CM; ++m) ck[m] = lane + 64 * m < ctot ? cbuf[lane + 64 * m] : 0u;
      radix([&](int shift, uint32_t pm, uint32_t pf) {
#pragma unroll
        for (int m = 0; m < CM; ++m)
          if (lane + 64 * m < ctot && (ck[m] & pm) == pf) atomicAdd(&hw[(ck[m] >> shift) & 255u], 1);
      });
    } else {
      radix([&](int shift, uint32_t pm, uint32_t pf) {
#pragma unroll
        for (int p = 0; p < P; ++p)
          if (base + p < nb && bn[p] == bstar && (key[p] & pm) == pf) atomicAdd(&hw[(key[p] >> shift) & 255u], 1);
      });
    }
    Tk = prefix;
    take_eq = rem;
  }

  // Taken: every key of a bin above b*; in b*, keys above Tk and the first take_eq keys
  // equal to Tk in index order.
  int eq_local = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) eq_local += (base + p < nb && bn[p] == bstar && key[p] == Tk) ? 1 : 0;
  const int eq_start = wave_inclusive_scan(eq_local) - eq_local;
  auto selected = [&](int p, int& eqc) -> bool {
    if (base + p >= nb) return false;
    if (all) return true;
    if (K == 0) return false;
    if (bn[p] > bstar) return true;
    if (bn[p] < bstar) return false;
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

// fp32 [H][nb][D] rows into the tiled order of the w̃ products (SelectArgs::stile):
// float4 ((h·tiles + t)·(D/8) + u)·64 + lane is row 32 t + lane % 32, columns
// (lane / 32)·D/2 + 4u .. + 3, zeros past nb. Writes are coalesced; the source is small.
template <int D>
__global__ __launch_bounds__(256) void tile_rows_kernel(const float* src, float* dst, int nb) {
  constexpr int U = D / 8;
  const int t = blockIdx.x, h = blockIdx.y, tiles = gridDim.x;
  float4* out = reinterpret_cast<float4*>(dst) + (size_t(h) * tiles + t) * U * 64;
  for (int e = threadIdx.x; e < U * 64; e += 256) {
    const int u = e / 64, lane = e % 64, row = 32 * t + (lane & 31), col = (lane >> 5) * (D / 2) + 4 * u;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < nb) v = *reinterpret_cast<const float4*>(src + (size_t(h) * nb + row) * D + col);
    out[e] = v;
  }
}

hipError_t launch_tile_rows(const float* src, float* dst, int H, int nb, int d, hipStream_t s) {
  const dim3 g((nb + 31) / 32, H);
  if (d == 64) hipLaunchKernelGGL((tile_rows_kernel<64>), g, dim3(256), 0, s, src, dst, nb);
  else hipLaunchKernelGGL((tile_rows_kernel<128>), g, dim3(256), 0, s, src, dst, nb);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_select_t(const SelectArgs& a, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (a.rope_axes == 0 || a.wt) {            // RoPE-aware scores read Q only for w̃
    hipLaunchKernelGGL((pool_kernel<T, D>), dim3((a.nb + 3) / 4, a.H), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.rope_axes > 0) {                     // after pool_kernel: replaces q̄
    hipLaunchKernelGGL((rope_pool_kernel<T, D>), dim3(a.nb, a.H, 2), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.wt) {                                // σ² in the tiled order of the w̃ products
    e = launch_tile_rows(a.ksig2, a.stile, a.H, a.nb, D, s);
    if (e != hipSuccess) return e;
  }
  e = launch_pooled_w(a, s);                 // w̃ (when asked for), after the pooled q²
  if (e != hipSuccess) return e;
  const int nt = (a.nb + 63) / 64;
  if (a.nb > kSmallNb) return launch_select_large(a, s);   // no score matrix: recomputed scores
  hipLaunchKernelGGL((score_kernel<D>), dim3(nt, nt, a.H), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  static_assert(kSmallNb <= 64 * 32, "one wave per row covers every stored row");
  const int pw = (a.nb + 63) / 64;
  const dim3 gw(unsigned((size_t(a.H) * a.nb + 3) / 4));
  if (pw <= 4) hipLaunchKernelGGL((topk_wave_kernel<4>), gw, dim3(256), 0, s, a);
  else if (pw <= 8) hipLaunchKernelGGL((topk_wave_kernel<8>), gw, dim3(256), 0, s, a);
  else if (pw <= 12) hipLaunchKernelGGL((topk_wave_kernel<12>), gw, dim3(256), 0, s, a);
  else if (pw <= 16) hipLaunchKernelGGL((topk_wave_kernel<16>), gw, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((topk_wave_kernel<32>), gw, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(int bf16, const SelectArgs& a, hipStream_t s) {
  if (bf16) return a.d == 64 ? launch_select_t<uint16_t, 64>(a, s) : launch_select_t<uint16_t, 128>(a, s);
  return a.d == 64 ? launch_select_t<float, 64>(a, s) : launch_select_t<float, 128>(a, s);
}

}  // namespace pisa
