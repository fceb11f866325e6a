// The pooled second-order weight of PWT (Sparse Linear Attention blog, PWT section):
// w̃_{i,j} = ½ Σ_c \overline{q²}_{i,c} σ²_{j,c} for every query tile i and key block j,
// where \overline{q²}_i is the mean of the squared valid query rows of tile i and σ²_j the
// per-dimension variance of key block j. One [nb x d]·[d x nb] product per head, written
// as the [H][nb][nb] fp32 matrix the attention call reads one row of per query tile.
//
// Both factors are non-negative, so the product has no cancellation and its relative
// error is that of each term. The fp32 factors are split into bf16 pairs x = x_hi + x_lo
// (x_hi = bf16(x), x_lo = bf16(x - x_hi), together within 2^-18 |x|), and the three
// products hi·hi + hi·lo + lo·hi run on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16,
// exact products, fp32 sums): every term within 3·2^-18 of its fp32 value, at a fifth of
// the fp32 matrix core time, so the call is bound by writing the matrix.
#include "common.hpp"
#include "internal.hpp"

namespace pisa {

namespace {

// The k-slots of the products: at k-step s, lane half g supplies dimensions
// g·D/2 + 8s .. + 7 (the same for both operands; any one-to-one assignment gives the same
// sum of products, and this one matches the tiled rows of SelectArgs::stile).
// Half g of one fp32 row, as hi and lo bf16 operands of every k-step.
template <int D>
__device__ __forceinline__ void split_row(const float* row, bf16x8 (&hi)[D / 16], bf16x8 (&lo)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const float4 x0 = *reinterpret_cast<const float4*>(row + 8 * s);
    const float4 x1 = *reinterpret_cast<const float4*>(row + 8 * s + 4);
    const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 h = static_cast<__bf16>(v[e]);
      hi[s][e] = h;
      lo[s][e] = static_cast<__bf16>(v[e] - static_cast<float>(h));
    }
  }
}

// Workgroup (row group of 128 query tiles, key split) of 4 waves: wave w keeps the split
// \overline{q²} rows of its 32 tiles in registers and streams 32-block tiles of σ² rows of
// the split, one 32 x 32 block of w̃ per key tile. Stores go through a buffer descriptor;
// out-of-range elements take an offset past the end, which the hardware drops, so every
// tile issues the same stores and the wait before a tile's products covers its loads only.
template <int D>
__global__ __launch_bounds__(256, 2) void pooled_w_kernel(SelectArgs a, int ks) {
  constexpr int NS = D / 16;
  constexpr uint32_t kDrop = 0x80000000u;
  constexpr int kNonTemporal = 2;        // streaming store: the matrix is not re-read here
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int split = int(blockIdx.x) % ks, rg = int(blockIdx.x) / ks, h = blockIdx.y, nb = a.nb;
  const int tiles = (nb + 31) / 32, t0 = split * tiles / ks, t1 = (split + 1) * tiles / ks;
  const size_t hn = size_t(h) * nb;
  const int rl0 = rg * 128 + 32 * wave;
  bf16x8 ahi[NS], alo[NS];
  split_row<D>(a.qsq + (hn + min(rl0 + c, nb - 1)) * D + g * (D / 2), ahi, alo);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.wt + hn * nb, uint32_t(nb) * uint32_t(nb) * 4u);
  // σ² from the tiled copy: one contiguous kilobyte per 16-byte load of the wave
  const float4* s2 = reinterpret_cast<const float4*>(a.stile) + size_t(h) * tiles * (D / 8) * 64 + lane;

  auto load = [&](float4 (&B)[2 * NS], int t) {
    const float4* p = s2 + size_t(min(t, tiles - 1)) * (D / 8) * 64;
#pragma unroll
    for (int u = 0; u < 2 * NS; ++u) B[u] = p[u * 64];
  };
  auto tile = [&](const float4 (&B)[2 * NS], int t) {
    f32x16 acc = zero16();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float v[8] = {B[2 * s].x, B[2 * s].y, B[2 * s].z, B[2 * s].w,
                          B[2 * s + 1].x, B[2 * s + 1].y, B[2 * s + 1].z, B[2 * s + 1].w};
      bf16x8 bh, bl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 x = static_cast<__bf16>(v[e]);
        bh[e] = x;
        bl[e] = static_cast<__bf16>(v[e] - static_cast<float>(x));
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[s], bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[s], bl, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[s], bh, acc, 0, 0, 0);
    }
    const int key = 32 * t + c;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rl0 + acc_row(r, g);
      const uint32_t off = (row < nb && key < nb) ? (uint32_t(row) * uint32_t(nb) + uint32_t(key)) * 4u : kDrop;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(0.5f * acc[r]), rw, int(off), 0, kNonTemporal);
    }
  };

  // σ² rows of the next key tile load while this tile's products run (two buffers taking
  // turns, loads unconditional: past the split they read clamped, valid rows that go
  // unused); the first tile is preceded by as many dropped stores as a tile issues, so the
  // waits count the same operations on every path
  float4 B0[2 * NS], B1[2 * NS];
  load(B0, t0);
#pragma unroll
  for (int e = 0; e < 16; ++e) __builtin_amdgcn_raw_buffer_store_b32(0u, rw, int(kDrop), 0, 0);
  for (int t = t0; t < t1; t += 2) {
    load(B1, t + 1);
    tile(B0, t);
    if (t + 1 >= t1) break;
    load(B0, t + 2);
    tile(B1, t + 1);
  }
}

template <int D>
hipError_t launch_t(const SelectArgs& a, hipStream_t s) {
  const int nrg = (a.nb + 127) / 128, tiles = (a.nb + 31) / 32;
  int ks = 1;
  while (ks < 16 && static_cast<long long>(nrg) * a.H * ks < 2048 && tiles / (2 * ks) >= 2) ks *= 2;
  hipLaunchKernelGGL((pooled_w_kernel<D>), dim3(nrg * ks, a.H), dim3(256), 0, s, a, ks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pooled_w(const SelectArgs& a, hipStream_t s) {
  if (!a.wt) return hipSuccess;
  return a.d == 64 ? launch_t<64>(a, s) : launch_t<128>(a, s);
}

}  // namespace pisa
