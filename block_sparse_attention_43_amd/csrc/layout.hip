// Layout step: natural token order <-> block order (Sparse Linear Attention blog, notation:
// tokens are cut into blocks of B; video latents are grouped into 3D cubes so that a block
// is a compact neighbourhood). Pure data movement, HBM-bound: one thread per 16-byte chunk
// of a row, rows gathered (to blocks) or scattered (back) through a slot -> token table.
#include "common.hpp"
#include "internal.hpp"

namespace pisa {

// dst[h][s] = perm[s] >= 0 ? src[h][perm[s]] : 0, rows of `row_bytes` bytes.
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* src, char* dst, const int32_t* perm,
                                                          int L_nat, int L_pad, int row_bytes) {
  const int cpr = row_bytes / 16;
  const size_t x = size_t(blockIdx.x) * 256 + threadIdx.x;
  const size_t total = size_t(L_pad) * cpr;
  if (x >= total) return;
  const int h = blockIdx.y;
  const int s = int(x / cpr), c = int(x % cpr);
  const int t = perm[s];
  u32x4 v = {0u, 0u, 0u, 0u};
  if (t >= 0 && t < L_nat) v = *reinterpret_cast<const u32x4*>(src + (size_t(h) * L_nat + t) * row_bytes + c * 16);
  *reinterpret_cast<u32x4*>(dst + (size_t(h) * L_pad + s) * row_bytes + c * 16) = v;
}

// dst[h][perm[s]] = src[h][s] for every slot with perm[s] in [0, L_nat).
__global__ __launch_bounds__(256) void scatter_rows_kernel(const char* src, char* dst, const int32_t* perm,
                                                           int L_nat, int L_pad, int row_bytes) {
  const int cpr = row_bytes / 16;
  const size_t x = size_t(blockIdx.x) * 256 + threadIdx.x;
  const size_t total = size_t(L_pad) * cpr;
  if (x >= total) return;
  const int h = blockIdx.y;
  const int s = int(x / cpr), c = int(x % cpr);
  const int t = perm[s];
  if (t < 0 || t >= L_nat) return;
  *reinterpret_cast<u32x4*>(dst + (size_t(h) * L_nat + t) * row_bytes + c * 16) =
      *reinterpret_cast<const u32x4*>(src + (size_t(h) * L_pad + s) * row_bytes + c * 16);
}

hipError_t launch_layout(bool to_blocks, const void* src, void* dst, const int32_t* perm, int H, int L_nat,
                         int L_pad, int row_bytes, hipStream_t s) {
  const size_t total = size_t(L_pad) * (row_bytes / 16);
  const dim3 grid(unsigned((total + 255) / 256), unsigned(H));
  if (to_blocks)
    hipLaunchKernelGGL(gather_rows_kernel, grid, dim3(256), 0, s, static_cast<const char*>(src),
                       static_cast<char*>(dst), perm, L_nat, L_pad, row_bytes);
  else
    hipLaunchKernelGGL(scatter_rows_kernel, grid, dim3(256), 0, s, static_cast<const char*>(src),
                       static_cast<char*>(dst), perm, L_nat, L_pad, row_bytes);
  return hipGetLastError();
}

}  // namespace pisa
