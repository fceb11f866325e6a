// Device-side helpers shared by the gfx950 kernels: element types, MFMA operand
// traits, wave reductions and the XCD-aware workgroup remap.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pisa {

// Compile-time loop: f(std::integral_constant<int, I>) for I in [I0, N).
template <int I0, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < N) {
    f(std::integral_constant<int, I0>{});
    static_for<I0 + 1, N>(f);
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte chunk

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = static_cast<__bf16>(x);  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

// Storage element <-> float.
template <class T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }
template <class T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) { return f32_to_bf16(v); }

// ---------------------------------------------------------------------------
// MFMA operand traits for the 32x32 output shape.
//
// For v_mfma_f32_32x32x{KI}: lane l supplies KH = KI/2 consecutive k-values of
// row (l % 32) of A and of column (l % 32) of B, at k = KH*(l/32) + [0, KH).
// Accumulator register r of lane l holds D[8*(r/4) + 4*(l/32) + r%4][l % 32].
// ---------------------------------------------------------------------------
struct MmaBF16 {
  using T = uint16_t;                // storage element
  using AB = bf16x8;                 // one lane's operand
  static constexpr int KI = 16;      // k per instruction
  static constexpr int KH = 8;       // k per lane
  __device__ __forceinline__ static AB load(const T* p) {
    return *reinterpret_cast<const AB*>(p);         // 16 bytes, 16-byte aligned
  }
  __device__ __forceinline__ static AB pack(const float* v) {
    AB r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(v[i]);
    return r;
  }
  __device__ __forceinline__ static AB zero() {
    AB r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(0.f);
    return r;
  }
  __device__ __forceinline__ static void unpack(AB a, float* v) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = static_cast<float>(a[i]);
  }
  __device__ __forceinline__ static f32x16 mma(AB a, AB b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Operand from 8 consecutive accumulator registers [OFF, OFF + 8).
  template <int OFF>
  __device__ __forceinline__ static AB packv(const f32x16& v) {
    AB r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(v[OFF + i]);
    return r;
  }
};

struct MmaF32 {
  using T = float;
  using AB = float;
  static constexpr int KI = 2;
  static constexpr int KH = 1;
  __device__ __forceinline__ static AB load(const T* p) { return *p; }
  __device__ __forceinline__ static AB pack(const float* v) { return v[0]; }
  __device__ __forceinline__ static AB zero() { return 0.f; }
  __device__ __forceinline__ static void unpack(AB a, float* v) { v[0] = a; }
  __device__ __forceinline__ static f32x16 mma(AB a, AB b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  template <int OFF>
  __device__ __forceinline__ static AB packv(const f32x16& v) { return v[OFF]; }
};

template <class T> struct MmaFor;
template <> struct MmaFor<uint16_t> { using type = MmaBF16; };
template <> struct MmaFor<float> { using type = MmaF32; };

// ---------------------------------------------------------------------------
// Element order of a 64-key tile (64 keys x D columns) in the packed buffers.
//
// fp32: K-type tiles are plain rows [key][c], V-type tiles plain Vᵀ rows [e][key].
// bf16: MFMA operand order for v_mfma_f32_32x32x16_bf16, so that one 16-byte load per
// lane, 1 KB per wave, is exactly one operand. The tile is two 32-key halves; in a half,
//   K-type (A operand of Sᵀ = K Qᵀ), fragment ks < D/16: lane 32g + R holds
//     K[key_of_row(R)][16 ks + 8 g + u], u < 8;
//   V-type (A operand of Oᵀ += Vᵀ Pᵀ), fragment (et < D/32, ks < 2): lane 32g + l holds
//     V[16 ks + 8 g + u][32 et + l], u < 8.
// key_of_row permutes the 32 keys of a half so that Sᵀ accumulator register r of lane
// half g holds key 16 (r / 8) + 8 g + r % 8: registers [8 ks, 8 ks + 8) are then the
// B operand (P) of k-step ks of Oᵀ += Vᵀ Pᵀ without any data movement.
// In both layouts the fastest index runs over 16 bytes of consecutive c (K-type) or
// consecutive keys (V-type), so a 16-byte chunk is contiguous in either.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int key_of_row(int R) {        // A row R -> key within the half
  return 16 * ((4 * (R >> 3) + (R & 3)) >> 3) + 8 * ((R >> 2) & 1) + ((4 * (R >> 3) + (R & 3)) & 7);
}
__host__ __device__ constexpr int row_of_key(int k) {        // inverse of key_of_row
  return 8 * ((8 * (k >> 4) + (k & 7)) >> 2) + 4 * ((k >> 3) & 1) + ((8 * (k >> 4) + (k & 7)) & 3);
}

template <class T, int D> struct TileLayout;
template <int D> struct TileLayout<float, D> {
  __host__ __device__ static constexpr int k(int key, int c) { return key * D + c; }
  __host__ __device__ static constexpr int v(int key, int e) { return e * 64 + key; }
  // 16-byte chunk x of a V-type tile in storage order -> (first key, e) it holds
  __host__ __device__ static constexpr void vchunk(int x, int& key0, int& e) {
    e = x / 16;
    key0 = (x % 16) * 4;
  }
};
template <int D> struct TileLayout<uint16_t, D> {
  __host__ __device__ static constexpr int k(int key, int c) {
    return ((((key >> 5) * (D / 16) + (c >> 4)) * 64 + 32 * ((c >> 3) & 1) + row_of_key(key & 31)) << 3) + (c & 7);
  }
  __host__ __device__ static constexpr int v(int key, int e) {
    return (((((key >> 5) * (D / 32) + (e >> 5)) * 2 + ((key >> 4) & 1)) * 64 + 32 * ((key >> 3) & 1) + (e & 31)) << 3) +
           (key & 7);
  }
  __host__ __device__ static constexpr void vchunk(int x, int& key0, int& e) {
    const int lane = x & 63, f = x >> 6;
    const int half = f / (D / 16), et = (f % (D / 16)) >> 1, ks = f & 1;
    e = 32 * et + (lane & 31);
    key0 = 32 * half + 16 * ks + 8 * (lane >> 5);
  }
  // 16-byte chunk x of a K-type tile in storage order -> (key, first c) it holds
  __host__ __device__ static constexpr void kchunk(int x, int& key, int& c0) {
    const int lane = x & 63, f = x >> 6;
    key = 32 * (f / (D / 16)) + key_of_row(lane & 31);
    c0 = 16 * (f % (D / 16)) + 8 * (lane >> 5);
  }
};

// Element (row e, column c) of a transposed [rows][64] LDS tile with row stride LDT: the
// 16-byte chunks of a row are XOR-swizzled by the row's chunk index, so the column-wise
// stores of a transpose spread over the LDS banks; a chunk stays contiguous for 16-byte
// operand reads.
template <class T, int LDT>
__device__ __forceinline__ int tix(int e, int c) {
  constexpr int EPC = 16 / sizeof(T), NCH = 64 / EPC;
  return e * LDT + ((((c / EPC) ^ ((e / EPC) % NCH)) * EPC) + c % EPC);
}

// Row index -> accumulator row of the 32x32 output:  row(r, g) = 8*(r/4) + 4*g + r%4.
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Combine a value with the one held by lane l ^ 32 (the other half of the wave).
// v_permlane32_swap with the same register as both operands returns the low half's
// values in one result and the high half's in the other, on every lane; combining the
// two is symmetric, so both halves end with bit-identical results.
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// LDS tiles staged by direct global->LDS loads (global_load_lds_dwordx4).
//
// One such load writes 16 bytes per lane at (LDS base + 16 * lane), i.e. a wave fills
// 1 KB of LDS contiguously. A tile of `rows` rows of ROW bytes is kept unpadded; the
// 16-byte chunks of row r are stored in XOR-permuted order (chunk c at position
// c ^ swz(r)) so that the MFMA operand reads, which take the same logical chunk from
// many rows, spread over all banks.
// ---------------------------------------------------------------------------
template <int ROW>
struct SwizzledTile {
  static constexpr int kChunks = ROW / 16;                          // chunks per row
  static constexpr int kRowsPerLine = ROW >= 256 ? 1 : 256 / ROW;   // rows sharing 256 bytes
  static constexpr int kMask = (kChunks < 16 ? kChunks : 16) - 1;
  __device__ __forceinline__ static int swz(int r) { return (r / kRowsPerLine) & kMask; }
  // byte offset of (row r, byte b within the logical row)
  __device__ __forceinline__ static int offset(int r, int b) {
    return r * ROW + (((b >> 4) ^ swz(r)) << 4) + (b & 15);
  }
};

__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src,
      (__attribute__((address_space(3))) void*)(lds_wave_base), 16, 0, 0);
}

// Buffer-addressed variant: byte address = base(rsrc) + soff (scalar) + voff (per lane);
// reads past `bytes` of the resource return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}
__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t r, int voff, int soff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_wave_base),
                                           16, voff, soff, 0, 0);
}

// Workgroups are dealt round-robin to the 8 XCDs; remap so that consecutive logical
// ids (neighbouring query tiles of one head) run on the same XCD and share its L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t n) {
  constexpr uint32_t kX = 8;
  uint32_t q = n / kX, rmd = n % kX;
  uint32_t x = b % kX, slot = b / kX;
  uint32_t base = x < rmd ? x * (q + 1) : rmd * (q + 1) + (x - rmd) * q;
  return base + slot;
}

// Block-wide exclusive scan of one int per thread (blockDim.x = 256).
__device__ __forceinline__ int block_exclusive_scan_256(int v, int* sh /*[8]*/, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int s = sh[w];
    if (w < wave) off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

}  // namespace pisa
