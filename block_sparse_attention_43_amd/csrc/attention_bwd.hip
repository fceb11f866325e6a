// Backward of the piecewise attention (DROP, PISA, PWT) with the selection and the gate's
// decisions held fixed, the way sparse fine-tuning trains through the block statistics
// (Sparse Linear Attention blog, PWT section: gradients flow through k̄_j, H_j (here H̄)
// and σ²_j, the routing is detached).
//
// For query t of tile i: P_{t,k} = e^{x_{t,k} - lse_t} (exact keys), P_{t,j} = e^{ℓ_{t,j} - lse_t}
// (virtual tokens, ℓ = q·k̄_j + φ_{i,j} + ln n_j), Δ_t = dO_t·O_t, u_t = H̄ q_t,
// Ā_t = Σ_j P_{t,j} / n_j. The softmax rule gives
//   dx_{t,k} = P_{t,k}(dO_t·v_k - Δ_t),   dℓ_{t,j} = P_{t,j}(dO_t·v̄_j + dO_t·u_t / n_j - Δ_t)
// and
//   dq_t = Σ_k dx k_k + Σ_j dℓ k̄_j + Ā_t H̄ᵀ dO_t + (2/m_i) q_t ∘ ½ Σ_j dw̃_{i,j} σ²_j
//   dk_k, dv_k (exact) = Σ_t dx_{t,k} q_t, Σ_t P_{t,k} dO_t
//   dk̄_j = Σ_t dℓ q_t, dv̄_j = Σ_t P_{t,j} dO_t, dH̄ = Σ_t Ā_t dO_t q_tᵀ,
//   dw̃_{i,j} = φ'(w̃_{i,j}) Σ_{t in i} dℓ_{t,j},  dσ²_j = ½ Σ_i dw̃_{i,j} \overline{q²}_i
// then every token of block j receives
//   dk += dk̄_j / n_j + (2/n_j)(k - k̄_j) ∘ dσ²_j + (1/nb) dH̄ᵀ (v - v̄_j),
//   dv += dv̄_j / n_j + (1/nb) dH̄ (k - k̄_j).
//
// Kernels, in launch order (all sums in a fixed order: repeated runs are bit-identical):
//   bwd_rows_kernel      per query tile: dO_t·u_t, the pooled \overline{q²}_i
//   bwd_delta_kernel     (forward output given) Δ_O = dO_t·O_t per row, corrected to Δ_t
//                        in the dQ sweep
//   csr_count/scan/fill  per key block: the query tiles that selected it, ascending
//   bwd_query_kernel     per query tile, one sweep: dQ from the exact and virtual tiles and
//                        H̄ᵀ, Ā_t, and (no forward output given) Δ_t = Σ P dP
//   bwd_key_kernel       per key block: dK, dV of its exact keys over the tiles that
//                        selected it; per centroid group and chunk of query tiles: dk̄, dv̄
//                        and (PWT) dw̃
//   bwd_dh_kernel + bwd_dh_reduce_kernel: dH̄
//   bwd_wprod_kernel     the products with dw̃: dqsq_i and dσ²_j
//   bwd_qsq_kernel       dQ += the pooled-q² term
//   bwd_chain_kernel     per key block: the statistics' gradients onto its tokens
// The 64 x 64 products run on MFMA with operands staged in LDS (bf16 MFMA with fp32
// accumulation for bf16 inputs; P and dS enter their products in bf16, as the forward
// pass's P does); scores are computed with the rows fed in the order that lets the
// accumulators serve directly as the B operand of the following product.
#include "attention.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace pisa {

namespace {

constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float POS_INF = __builtin_huge_valf();

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <class T>
__device__ __forceinline__ u32x4 zero_chunk() {
  return u32x4{0u, 0u, 0u, 0u};
}

// Workgroup barrier that waits for this wave's LDS operations and for all but its newest VM
// vector memory loads (direct loads of tiles issued later than the one about to be read).
// __syncthreads would also drain those: its release fence covers the direct loads' LDS
// writes. The "memory" clobber keeps the compiler from moving memory accesses across it.
template <int VM>
__device__ __forceinline__ void barrier_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x70);   // vmcnt(VM) expcnt(7) lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// LDS address (offset in the workgroup's LDS) of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(p)));
}

// Reads of LDS that direct loads fill, written as inline asm whose block also waits for
// them: the compiler does not track which LDS object a direct load writes and would make
// any LDS read it sees wait for every direct load still in flight. Outputs are
// early-clobber, so no destination shares a register with an address still to be used.
template <int OFF>
__device__ __forceinline__ void lds_read4x16(u32x4 (&o)[4], const uint32_t (&ad)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n\t"
      "ds_read_b128 %1, %5 offset:%8\n\t"
      "ds_read_b128 %2, %6 offset:%8\n\t"
      "ds_read_b128 %3, %7 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void lds_read8x16(u32x4 (&o)[8], const uint32_t (&ad)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%16\n\t"
      "ds_read_b128 %1, %9 offset:%16\n\t"
      "ds_read_b128 %2, %10 offset:%16\n\t"
      "ds_read_b128 %3, %11 offset:%16\n\t"
      "ds_read_b128 %4, %12 offset:%16\n\t"
      "ds_read_b128 %5, %13 offset:%16\n\t"
      "ds_read_b128 %6, %14 offset:%16\n\t"
      "ds_read_b128 %7, %15 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]),
        "i"(OFF));
}
template <int N, int OFF>
__device__ __forceinline__ void lds_read_x16(u32x4 (&o)[N], const uint32_t (&ad)[N]) {
  static_assert(N == 4 || N == 8, "read block size");
  if constexpr (N == 4) lds_read4x16<OFF>(o, ad);
  else lds_read8x16<OFF>(o, ad);
}
// Eight 16-byte reads at one address plus the offsets O0..O7.
template <int O0, int O1, int O2, int O3, int O4, int O5, int O6, int O7>
__device__ __forceinline__ void lds_read8_at(u32x4 (&o)[8], uint32_t ad) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%9\n\t"
      "ds_read_b128 %1, %8 offset:%10\n\t"
      "ds_read_b128 %2, %8 offset:%11\n\t"
      "ds_read_b128 %3, %8 offset:%12\n\t"
      "ds_read_b128 %4, %8 offset:%13\n\t"
      "ds_read_b128 %5, %8 offset:%14\n\t"
      "ds_read_b128 %6, %8 offset:%15\n\t"
      "ds_read_b128 %7, %8 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(ad), "i"(O0), "i"(O1), "i"(O2), "i"(O3), "i"(O4), "i"(O5), "i"(O6), "i"(O7));
}
// Eight LDS transpose reads (ds_read_b64_tr_b16, gfx950): within each group of 16 lanes,
// lane 4a + b receives element b of the 8-byte rows addressed by lanes a, a + 4, a + 8 and
// a + 12 of the group; if lane 4u + a addresses row r0 + u at column c0 + 4a of a bf16 tile,
// lane t gets rows r0 .. r0 + 3 of column c0 + t, i.e. a transposed operand from row-major
// data. Waits for its reads like the blocks above.
__device__ __forceinline__ void lds_read8_tr16(u32x2 (&o)[8], const uint32_t (&ad)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]));
}
__device__ __forceinline__ void lds_write_u32(uint32_t ad, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(ad), "v"(v) : "memory");
}
// Barrier after this wave's LDS operations, leaving its vector memory loads in flight.
__device__ __forceinline__ void barrier_lgkm() {
  __builtin_amdgcn_s_waitcnt(0xC07F);              // vmcnt(63) expcnt(7) lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}
__device__ __forceinline__ uint32_t lds_read_u32(uint32_t ad) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(ad));
  return v;
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Per query tile: gu_t = dO_t·(H̄ q_t) for valid rows with support (0 otherwise) and, for
// PWT, the tile's pooled \overline{q²}_i. Uᵀ = H̄ Qᵀ on the fp32 matrix cores (A = H̄ rows
// read from H̄ᵀ, B = the staged Q rows), so each lane holds one query's column and the
// dot with dO needs no cross-lane sum; wave w takes query half w & 1 and every other
// 32-row tile of e.
// bf16 inputs: ROWS_G query tiles per workgroup share H̄ staged once in LDS as hi + lo bf16
// parts; u = H̄ q on bf16 MFMA (q exact in bf16, so the products lose nothing), gu = dO·u.
constexpr int ROWS_G = 8;
template <int D>
__device__ __forceinline__ void rows_bf16(const BwdArgs& a) {
  constexpr int NE = D / 32, NKD = D / 16, LDH = D + 8;
  __shared__ __align__(16) uint16_t sHh[D * LDH], sHl[D * LDH];
  __shared__ float part[4][32];
  const int h = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const float* hT = a.hbarT + size_t(h) * D * D;
  for (int x = tid; x < D * D; x += 256) {         // H̄[e][c] = H̄ᵀ[c][e]
    const int c = x / D, e = x % D;
    const float f = hT[x];
    const uint16_t hi = from_f32<uint16_t>(f);
    sHh[e * LDH + c] = hi;
    sHl[e * LDH + c] = from_f32<uint16_t>(f - to_f32(hi));
  }
  __syncthreads();
  const uint16_t* Qh = static_cast<const uint16_t*>(a.Q);
  const uint16_t* Gh = static_cast<const uint16_t*>(a.dO);
  const int tq = wave & 1, t = 32 * tq + l32;
  for (int i = blockIdx.x * ROWS_G; i < min(a.nb, blockIdx.x * ROWS_G + ROWS_G); ++i) {
    const int m = min(max(a.block_len ? a.block_len[i] : kB, 1), kB);
    const size_t row0 = size_t(h) * a.L + size_t(i) * kB;
    if (a.qsq && tid < D) {
      float s = 0.f;
#pragma unroll 8
      for (int r = 0; r < m; ++r) {
        const float q = to_f32(Qh[(row0 + r) * D + tid]);
        s = fmaf(q, q, s);
      }
      a.qsq[(size_t(h) * a.nb + i) * D + tid] = s / float(m);
    }
    bf16x8 qf[NKD];
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks)
      qf[ks] = t < m ? *reinterpret_cast<const bf16x8*>(Qh + (row0 + t) * D + 16 * ks + 8 * g) : MmaBF16::zero();
    float gu = 0.f;
    for (int et = wave >> 1; et < NE; et += 2) {
      f32x16 u = zero16();
      const uint16_t* hr = sHh + (32 * et + l32) * LDH + 8 * g;
      const uint16_t* lr = sHl + (32 * et + l32) * LDH + 8 * g;
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        u = MmaBF16::mma(*reinterpret_cast<const bf16x8*>(hr + 16 * ks), qf[ks], u);
        u = MmaBF16::mma(*reinterpret_cast<const bf16x8*>(lr + 16 * ks), qf[ks], u);
      }
      if (t < m) {
        // dO[t][e] for e = 32 et + acc_row(r, g): four runs of four
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint2 w = *reinterpret_cast<const uint2*>(Gh + (row0 + t) * D + 32 * et + 8 * q4 + 4 * g);
          const float d0 = __uint_as_float(w.x << 16), d1 = __uint_as_float(w.x & 0xFFFF0000u);
          const float d2 = __uint_as_float(w.y << 16), d3 = __uint_as_float(w.y & 0xFFFF0000u);
          gu = fmaf(d0, u[4 * q4 + 0], gu);
          gu = fmaf(d1, u[4 * q4 + 1], gu);
          gu = fmaf(d2, u[4 * q4 + 2], gu);
          gu = fmaf(d3, u[4 * q4 + 3], gu);
        }
      }
    }
    gu = sum_halves(gu);
    __syncthreads();                               // previous tile's part[] read
    if (g == 0) part[wave][l32] = gu;
    __syncthreads();
    if (tid < kB) {
      const float l = a.lse[row0 + tid];
      const bool live = tid < m && l > NEG_INF;
      const int q = tid >> 5, r = tid & 31;
      a.gu[row0 + tid] = live ? part[q][r] + part[q + 2][r] : 0.f;
    }
  }
}

template <class T, int D>
__global__ __launch_bounds__(256) void bwd_rows_kernel(BwdArgs a) {
  if constexpr (sizeof(T) == 2) {
    rows_bf16<D>(a);
  } else {
    constexpr int NE = D / 32;
    __shared__ float sq[kB][D + 1], sg[kB][D + 1];
    __shared__ float part[4][32];
    const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
    int m = a.block_len ? a.block_len[i] : kB;
    m = min(max(m, 1), kB);
    const size_t row0 = size_t(h) * a.L + size_t(i) * kB;
    const T* Qt = static_cast<const T*>(a.Q) + row0 * D;
    const T* Gt = static_cast<const T*>(a.dO) + row0 * D;
    for (int x = tid; x < kB * D; x += 256) {
      const bool ok = (x / D) < m;
      sq[x / D][x % D] = ok ? to_f32(Qt[x]) : 0.f;
      sg[x / D][x % D] = ok ? to_f32(Gt[x]) : 0.f;
    }
    __syncthreads();
    if (a.qsq && tid < D) {
      float s = 0.f;
      for (int r = 0; r < m; ++r) s = fmaf(sq[r][tid], sq[r][tid], s);
      a.qsq[(size_t(h) * a.nb + i) * D + tid] = s / float(m);
    }
    const float* hT = a.hbarT + size_t(h) * D * D;
    const int tq = wave & 1, t = 32 * tq + l32;
    float gu = 0.f;
    for (int et = wave >> 1; et < NE; et += 2) {
      f32x16 u = zero16();
#pragma unroll 8
      for (int ks = 0; ks < D / 2; ++ks) {
        const int c = 2 * ks + g;
        u = __builtin_amdgcn_mfma_f32_32x32x2f32(hT[size_t(c) * D + 32 * et + l32], sq[t][c], u, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) gu = fmaf(sg[t][32 * et + acc_row(r, g)], u[r], gu);
    }
    gu = sum_halves(gu);
    if (g == 0) part[wave][l32] = gu;
    __syncthreads();
    if (tid < kB) {
      const float l = a.lse[row0 + tid];
      const bool live = tid < m && l > NEG_INF;
      const int q = tid >> 5, r = tid & 31;
      a.gu[row0 + tid] = live ? part[q][r] + part[q + 2][r] : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Operand tiles that are not rows of the inputs, in the input type (centroid tiles rounded
// from fp32 as the forward's are), zeros past the valid rows: kind 0, block i: Kᵀ [d][64];
// kind 1, query tile i: Qᵀ and dOᵀ; kind 2, centroid group i: k̄ rows [64][d], k̄ᵀ [d][64]
// and v̄ = ΣV / n rows [64][d]. The sweeps move them, with the rows of Q, K, V and dO
// themselves, into LDS by direct loads; the bf16 sweeps form the transposed operands from
// rows with LDS transpose reads and use kind 1 only for dH̄.
template <class T, int D>
__global__ __launch_bounds__(256) void bwd_pack_kernel(BwdArgs a) {
  constexpr int EPC = 16 / sizeof(T), LDT = kB + EPC, CPR = D / EPC, CPT = kB / EPC;
  constexpr size_t TE = size_t(kB) * D;
  __shared__ __align__(16) T sXt[D * LDT];
  const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int nb = a.nb, ngrp = a.nbp / kB;
  // Transpose of the valid rows of a 64-row block of src into sXt.
  auto stage_t = [&](const T* src, int valid) {
    for (int c = tid; c < kB * CPR; c += 256) {
      const int r = c / CPR, col = (c % CPR) * EPC;
      const u32x4 v = r < valid ? *reinterpret_cast<const u32x4*>(src + size_t(r) * D + col) : zero_chunk<T>();
      const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
      for (int u = 0; u < EPC; ++u) sXt[tix<T, LDT>(col + u, r)] = e[u];
    }
  };
  auto write_t = [&](T* out) {
    for (int c = tid; c < D * CPT; c += 256) {
      const int e = c / CPT, k0 = (c % CPT) * EPC;
      *reinterpret_cast<u32x4*>(out + e * kB + k0) = *reinterpret_cast<const u32x4*>(&sXt[tix<T, LDT>(e, k0)]);
    }
  };
  // bf16 forms Kᵀ and k̄ᵀ operands with LDS transpose reads: its launch starts at z = 1
  const int kind = int(blockIdx.z) + (sizeof(T) == 2 ? 1 : 0);
  T* out;
  if (kind < 2) {
    const int valid = min(max(a.block_len ? a.block_len[i] : kB, 1), kB);
    const size_t row0 = (size_t(h) * a.L + size_t(i) * kB) * D, to = (size_t(h) * nb + i) * TE;
    if (kind == 0) {
      stage_t(static_cast<const T*>(a.K) + row0, valid);
      out = reinterpret_cast<T*>(a.kt) + to;
    } else {
      stage_t(static_cast<const T*>(a.Q) + row0, valid);
      __syncthreads();
      write_t(reinterpret_cast<T*>(a.qt) + to);
      __syncthreads();
      stage_t(static_cast<const T*>(a.dO) + row0, valid);
      out = reinterpret_cast<T*>(a.gt) + to;
    }
  } else {
    if (i >= ngrp) return;
    const int j0 = i * kB, valid = min(kB, nb - j0);
    const size_t to = (size_t(h) * ngrp + i) * TE;
    T* kr = reinterpret_cast<T*>(a.kbr) + to;
    T* vr = reinterpret_cast<T*>(a.vbr) + to;
    for (int x = tid; x < kB * D; x += 256) {
      const int r = x / D, c = x % D;
      float fk = 0.f, fv = 0.f;
      if (r < valid) {
        const size_t o = (size_t(h) * nb + j0 + r) * D + c;
        fk = a.kbar[o];
        fv = a.vsum[o] * (1.f / float(min(max(a.block_len ? a.block_len[j0 + r] : kB, 1), kB)));
      }
      const T tk = from_f32<T>(fk);
      kr[x] = tk;
      vr[x] = from_f32<T>(fv);
      sXt[tix<T, LDT>(c, r)] = tk;
    }
    out = reinterpret_cast<T*>(a.kbt) + to;
  }
  __syncthreads();
  write_t(out);
}

// ---------------------------------------------------------------------------------------
// Log2-domain bias of every virtual token of query tile i, (ln n_j + φ_ij) log2 e, -inf for
// the selected blocks and the padding past nb (φ as in the forward: gated w̃, or ln(1 + w̃)),
// with φ'(w̃) (0 where excluded or gated, and for PISA); and, once, 1 / n_j (0 past nb).
template <int MODE>
__global__ __launch_bounds__(256) void bwd_bias_kernel(BwdArgs a) {
  constexpr float NEG_INF = -__builtin_huge_valf();
  const int i = blockIdx.x, h = blockIdx.y, nb = a.nb;
  const uint32_t* mrow = a.mask + (size_t(h) * nb + i) * a.nw;
  const float* wrow = MODE == MODE_PWT ? a.wt + (size_t(h) * nb + i) * nb : nullptr;
  float* out = a.vbias + (size_t(h) * nb + i) * a.nbp;
  for (int jj = threadIdx.x; jj < a.nbp; jj += 256) {
    const int nn = jj < nb ? min(max(a.block_len ? a.block_len[jj] : kB, 1), kB) : 0;
    float b = NEG_INF, dphi = 0.f;
    if (jj < nb && !((mrow[jj >> 5] >> (jj & 31)) & 1u)) {
      const float lnn = logf(float(nn));
      float phi = 0.f;
      if (MODE == MODE_PWT) {
        float w = wrow[jj];
        const bool fired = a.gate && w > lnn;
        if (fired) w = 0.f;
        phi = a.w_linear ? log1pf(w) : w;
        dphi = fired ? 0.f : (a.w_linear ? 1.f / (1.f + w) : 1.f);
      }
      b = (lnn + phi) * kLog2e;
    }
    out[jj] = b;
    a.vdphi[(size_t(h) * nb + i) * a.nbp + jj] = dphi;
    if (h == 0 && i == 0) a.vinvn[jj] = nn > 0 ? 1.f / float(nn) : 0.f;
  }
}

// ---------------------------------------------------------------------------------------
// Query tiles that selected key block j (from the membership bitmask), ascending: counts,
// per-head exclusive scan, fill. One thread per (head, block) for count and fill.
__global__ __launch_bounds__(256) void csr_count_kernel(BwdArgs a) {
  const int j = blockIdx.x * 256 + threadIdx.x, h = blockIdx.y;
  if (j >= a.nb) return;
  const uint32_t* mh = a.mask + size_t(h) * a.nb * a.nw;
  int c = 0;
  for (int i = 0; i < a.nb; ++i) c += (mh[size_t(i) * a.nw + (j >> 5)] >> (j & 31)) & 1u;
  a.csr_off[size_t(h) * (a.nb + 1) + j + 1] = c;
}

__global__ __launch_bounds__(256) void csr_scan_kernel(BwdArgs a) {
  __shared__ int sh[8];
  const int h = blockIdx.x, tid = threadIdx.x;
  int* off = a.csr_off + size_t(h) * (a.nb + 1);
  const int C = (a.nb + 255) / 256, j0 = min(tid * C, a.nb), j1 = min(j0 + C, a.nb);
  int s = 0;
  for (int j = j0; j < j1; ++j) s += off[j + 1];
  int total;
  int run = block_exclusive_scan_256(s, sh, &total);
  __syncthreads();
  const int cap = a.nb * a.K_sel;                  // list capacity (a mask with more bits is cut)
  for (int j = j0; j < j1; ++j) {
    const int c = off[j + 1];
    off[j + 1] = min(run + c, cap);
    run += c;
  }
  if (tid == 0) off[0] = 0;
}

__global__ __launch_bounds__(256) void csr_fill_kernel(BwdArgs a) {
  const int j = blockIdx.x * 256 + threadIdx.x, h = blockIdx.y;
  if (j >= a.nb) return;
  const uint32_t* mh = a.mask + size_t(h) * a.nb * a.nw;
  const int* off = a.csr_off + size_t(h) * (a.nb + 1);
  const int o0 = off[j], len = off[j + 1] - o0;
  int* out = a.csr_list + size_t(h) * a.nb * a.K_sel + o0;
  int c = 0;
  for (int i = 0; i < a.nb && c < len; ++i)
    if ((mh[size_t(i) * a.nw + (j >> 5)] >> (j & 31)) & 1u) out[c++] = i;
}

// ---------------------------------------------------------------------------------------
// Δ_t = dO_t·O_t from the forward output, in fp32, for rows with support (valid slot,
// finite lse); 0 elsewhere, as the single-sweep form writes it. LPR lanes per row, each
// one 16-byte chunk of O and of dO, summed across the row's lanes.
template <class T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  constexpr int EPL = 16 / int(sizeof(T)), LPR = D / EPL, RPB = 256 / LPR;
  static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "lanes per row");
  const size_t rows = size_t(a.H) * a.L;
  const size_t r = size_t(blockIdx.x) * RPB + threadIdx.x / LPR;
  const int c = int(threadIdx.x % LPR);
  float s = 0.f;
  bool live = false;
  if (r < rows) {
    const int t = int(r % size_t(a.L)), blk = t / kB;
    const int m = min(max(a.block_len ? a.block_len[blk] : kB, 1), kB);
    live = (t % kB) < m && a.lse[r] > NEG_INF;
    if (live) {
      const size_t off = r * D + size_t(c) * EPL;
      const u32x4 vo = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.O) + off);
      const u32x4 vg = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.dO) + off);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (sizeof(T) == 2) {
          s = fmaf(__uint_as_float(vo[k] << 16), __uint_as_float(vg[k] << 16), s);
          s = fmaf(__uint_as_float(vo[k] & 0xFFFF0000u), __uint_as_float(vg[k] & 0xFFFF0000u), s);
        } else {
          s = fmaf(__uint_as_float(vo[k]), __uint_as_float(vg[k]), s);
        }
      }
    }
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (r < rows && c == 0) a.delta[r] = live ? s : 0.f;
}

// ---------------------------------------------------------------------------------------
// Per query tile: dQ over its exact tiles and centroid groups, then + Ā_t H̄ᵀ dO_t.
// Wave (wk, wq) computes Sᵀ and dPᵀ for key half wk and query half wq (keys fed through
// feed_row, so registers are the B operands of the products with Kᵀ); the two key halves
// are merged at the end.
// DIR (Δ_O = dO·O from bwd_delta_kernel): dS = P∘(dP - Δ_O) and P enter one product each
// with Kᵀ, in the input type, and the sweep sums ε = Σ dS in fp32 (= Δ - Δ_O: O's
// rounding, which Σ P k would otherwise amplify), then forms dQ = Kᵀ dSᵀ - ε kp and hands
// Δ = Δ_O + ε to the key sweep.
// Otherwise one sweep without Δ: dQ is linear in Δ, dq_t = Σ P dP k - Δ_t Σ P k, so the
// sweep accumulates dQ₀ = Kᵀ (P∘dP)ᵀ, kp = Kᵀ Pᵀ and Δ_t = Σ P dP (the definition of
// dO_t·o_t, in fp32 from the recomputed P and dP) and forms dQ₀ - Δ kp at the end. P∘dP
// and P enter their products as hi + lo bf16 pairs, so the cancellation in the difference
// costs no bf16 rounding.
// Each tile's operands (K or k̄ rows, V or v̄ rows, Kᵀ or k̄ᵀ, and a virtual tile's biases
// and 1 / n_j) arrive by direct global->LDS loads into a ring of NST stages, NST - 1 tiles
// ahead of use, each stage its own LDS object (so the compiler sees that reading one stage
// does not wait for the loads landing in another); tiles are swizzled rows (SwizzledTile).
template <class T, int D, int MODE, bool DIR>
__global__ __launch_bounds__(256) void bwd_query_kernel(BwdArgs a) {
  using M = typename MmaFor<T>::type;
  using AB = typename M::AB;
  constexpr int KI = M::KI, KH = M::KH;
  constexpr int ES = sizeof(T);
  constexpr int NKD = D / KI, NKH = 32 / KI, NET = D / 32;
  constexpr bool VIRT = MODE != MODE_DROP;
  constexpr bool SPLIT = sizeof(T) == 2;            // hi + lo operands for bf16
  constexpr int KROW = D * ES, TROW = kB * ES;      // bytes per key row; per Kᵀ row
  constexpr int TB = kB * KROW;                     // bytes per operand tile
  constexpr int DPW = TB / 4096;                    // 1 KB direct loads per wave and operand
  // Stage: K (or k̄) rows, V (or v̄) rows, for fp32 also Kᵀ (bf16 forms the transposed
  // operand from the rows with LDS transpose reads), then 4 x 64-float rows.
  constexpr int NTILE = SPLIT ? 2 : 3;
  constexpr int RB = NTILE * TB;
  constexpr int SB = RB + 4 * kB * 4;               // bytes per stage
  constexpr int BUDGET = 152 * 1024;
  constexpr int NST = 4 * SB <= BUDGET ? 4 : (3 * SB <= BUDGET ? 3 : (2 * SB <= BUDGET ? 2 : 1));
  constexpr int PT = NTILE * DPW + 1;               // direct loads per wave and tile
  constexpr int DCH = 256;                          // descriptor chunk (exact tiles)
  using KT = SwizzledTile<KROW>;
  using TT = SwizzledTile<TROW>;
  static_assert(DPW >= 1 && TB % 4096 == 0, "tile shape");
  __shared__ __align__(1024) char sS0[SB];
  __shared__ __align__(1024) char sS1[NST > 1 ? SB : 16];
  __shared__ __align__(1024) char sS2[NST > 2 ? SB : 16];
  __shared__ __align__(1024) char sS3[NST > 3 ? SB : 16];
  __shared__ float sDel[2][kB];
  __shared__ uint32_t sDesc[2][DCH];                // exact tile -> block | valid keys << 16

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // kept scalar
  const int wk = wave >> 1, wq = wave & 1;
  const uint32_t lin = xcd_remap(blockIdx.x, gridDim.x);
  const int h = int(lin / uint32_t(a.nb)), i = int(lin % uint32_t(a.nb));
  const int nb = a.nb, ngrp = a.nbp / kB;
  int m = a.block_len ? a.block_len[i] : kB;
  m = min(max(m, 1), kB);
  const size_t row0 = size_t(h) * a.L + size_t(i) * kB;
  const int qrow = 32 * wq + l32;
  const float lse = a.lse[row0 + qrow];
  const bool qvalid = qrow < m && lse > NEG_INF;
  const float lse2 = qvalid ? lse * kLog2e : POS_INF;   // P = 0 on rows without support
  const float gu = a.gu[row0 + qrow];
  const float dl = DIR && qvalid ? a.delta[row0 + qrow] : 0.f;

  const T* Qh = static_cast<const T*>(a.Q) + size_t(h) * a.L * D;
  const T* Gh = static_cast<const T*>(a.dO) + size_t(h) * a.L * D;
  AB qf[NKD], gf[NKD];
#pragma unroll
  for (int ks = 0; ks < NKD; ++ks) {
    qf[ks] = qvalid ? M::load(Qh + (size_t(i) * kB + qrow) * D + KI * ks + KH * g) : M::zero();
    gf[ks] = qvalid ? M::load(Gh + (size_t(i) * kB + qrow) * D + KI * ks + KH * g) : M::zero();
  }
  f32x16 dqt[NET], kpt[NET];
#pragma unroll
  for (int et = 0; et < NET; ++et) dqt[et] = kpt[et] = zero16();
  float abar = 0.f, dsum = 0.f;

  // Let the fragment loads land before the first direct loads are issued, so that later
  // waits for those (counted from the newest) never have to cover them.
  __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)

  const int32_t* irow = a.idx + (size_t(h) * nb + i) * a.K_sel;
  const int n1 = a.K_sel, N = n1 + (VIRT ? ngrp : 0);
  const int R = 32 * wk + feed_row<M>(l32);       // key row this lane feeds

  auto fill_desc = [&](int chunk) {
    for (int e = tid; e < DCH; e += 256) {
      const int n = chunk * DCH + e;
      uint32_t d = 0u;
      if (n < n1) {
        const int j = irow[n];
        if (j >= 0 && j < nb) d = uint32_t(j) | (uint32_t(min(max(a.block_len ? a.block_len[j] : kB, 1), kB)) << 16);
      }
      sDesc[chunk & 1][e] = d;
    }
  };
  auto desc = [&](int t) -> uint32_t {
    return __builtin_amdgcn_readfirstlane(lds_read_u32(lds_addr(&sDesc[(t / DCH) & 1][t % DCH])));
  };

  // Per-lane source offsets inside a tile of the 16-byte chunk each direct load of this
  // lane fills (swizzled order), for the row tiles (rows of KROW bytes) and Kᵀ tiles.
  int koff[DPW], krow[DPW], toff[DPW];
#pragma unroll
  for (int u = 0; u < DPW; ++u) {
    const int b = (wave * DPW + u) * 1024 + lane * 16;
    const int rk = b / KROW, rt = b / TROW;
    krow[u] = rk;
    koff[u] = rk * KROW + ((((b % KROW) >> 4) ^ KT::swz(rk)) << 4);
    toff[u] = rt * TROW + ((((b % TROW) >> 4) ^ TT::swz(rt)) << 4);
  }
  // Direct loads of tile t into stage S. Rows of an exact block past its valid count are
  // loaded from row 0 instead (finite values; their keys are masked). Wave 0 loads a
  // virtual tile's biases, wave 1 its 1 / n_j; every wave issues the same PT loads.
  const char* Kb = reinterpret_cast<const char*>(static_cast<const T*>(a.K) + size_t(h) * a.L * D);
  const char* Vb = reinterpret_cast<const char*>(static_cast<const T*>(a.V) + size_t(h) * a.L * D);
  auto issue = [&](int t, auto sc) {
    constexpr int S = decltype(sc)::value;
    char* st = S == 0 ? sS0 : (S == 1 ? sS1 : (S == 2 ? sS2 : sS3));
    const char *pk, *pv, *pt, *pr;
    int nrows;
    if (VIRT && t >= n1) {
      const size_t go = (size_t(h) * ngrp + (t - n1)) * TB;
      pk = a.kbr + go;
      pv = a.vbr + go;
      pt = a.kbt + go;
      nrows = kB;
      pr = wave == 0 ? reinterpret_cast<const char*>(a.vbias + (size_t(h) * nb + i) * a.nbp + (t - n1) * kB)
                     : reinterpret_cast<const char*>(a.vinvn + (t - n1) * kB);
    } else {
      const uint32_t d = desc(t);
      const int j = int(d & 0xFFFFu);
      nrows = int(d >> 16);
      pk = Kb + size_t(j) * TB;
      pv = Vb + size_t(j) * TB;
      pt = a.kt + (size_t(h) * nb + j) * TB;
      pr = reinterpret_cast<const char*>(a.vinvn ? a.vinvn : a.lse);   // unused values
    }
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(pk, TB), rv = make_rsrc(pv, TB), rt = make_rsrc(pt, TB);
#pragma unroll
    for (int u = 0; u < DPW; ++u) {
      const int ko = krow[u] < nrows ? koff[u] : koff[u] - krow[u] * KROW;
      buf_dma16(rk, ko, 0, st + (wave * DPW + u) * 1024);
      buf_dma16(rv, ko, 0, st + TB + (wave * DPW + u) * 1024);
      if constexpr (!SPLIT) buf_dma16(rt, toff[u], 0, st + 2 * TB + (wave * DPW + u) * 1024);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(pr, kB * 4), (__attribute__((address_space(3))) void*)(st + RB + wave * kB * 4),
                                             4, lane * 4, 0, 0, 0);
  };

  // LDS byte offsets inside a stage of this lane's operand fragments: K (and V, one tile
  // further) rows for the scores, Kᵀ rows for dQ₀ and kp, and this lane's first bias.
  constexpr int NT = NET * NKH;
  uint32_t kad[NKD], tad[NT];
#pragma unroll
  for (int ks = 0; ks < NKD; ++ks) kad[ks] = KT::offset(R, (KI * ks + KH * g) * ES);
#pragma unroll
  for (int et = 0; et < NET; ++et)
#pragma unroll
    for (int ks = 0; ks < NKH; ++ks)
      tad[et * NKH + ks] = 2 * TB + TT::offset(32 * et + l32, (32 * wk + KI * ks + KH * g) * ES);
  const int key0 = 32 * wk + acc_key<M>(0, 0, g);
  // transpose reads: lane 16 G + 4 u + a addresses key row 32 wk + 8 (G / 2) + u (+ the
  // fragment's k offset) at column 16 (G % 2) + 4 a (+ the fragment's column tile)
  const int trow = 32 * wk + 8 * (lane >> 5) + ((lane & 15) >> 2), tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // One tile from stage S: Sᵀ, dPᵀ, P and P∘dP (hi + lo), dQ₀ and kp.
  auto compute = [&](int t, auto sc) {
    constexpr int S = decltype(sc)::value;
    const char* sk = S == 0 ? sS0 : (S == 1 ? sS1 : (S == 2 ? sS2 : sS3));
    const bool virt = VIRT && t >= n1;
    const int nj = virt ? kB : int(desc(t) >> 16);
    if (nj == 0) return;                           // uniform: out-of-range index
    // bf16 operands are read ahead into registers; fp32 ones (four times as many
    // registers) where the products use them.
    constexpr int NA = SPLIT ? NKD : 1, NTA = SPLIT ? NT : 1;
    AB ka[NA], va[NA], ta[NTA];
    float bias[16], invn[16];
    f32x16 s = zero16(), p = zero16();
    if constexpr (SPLIT) {
      // bf16: every operand in three blocks of 16-byte reads, the rows' biases in a fourth.
      // DIR: the V rows are read while the Sᵀ products run, the Kᵀ fragments and biases
      // while the dPᵀ products run (the fences keep the products between the read blocks).
      static_assert(NKD == 4 || NKD == 8, "fragments per block");
      const uint32_t base = lds_addr(sk);
      uint32_t ad[NKD];
      u32x4 rk[NKD], rv[NKD];
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) ad[ks] = base + kad[ks];
      lds_read_x16<NKD, 0>(rk, ad);
      if constexpr (DIR) {
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks) s = M::mma(__builtin_bit_cast(AB, rk[ks]), qf[ks], s);
        __builtin_amdgcn_sched_barrier(0);
        lds_read_x16<NKD, TB>(rv, ad);
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks) p = M::mma(__builtin_bit_cast(AB, rv[ks]), gf[ks], p);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        lds_read_x16<NKD, TB>(rv, ad);
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks) {
          ka[ks] = __builtin_bit_cast(AB, rk[ks]);
          va[ks] = __builtin_bit_cast(AB, rv[ks]);
        }
      }
      // Kᵀ fragments from the K rows by transpose reads: fragment x = (et, ks) is two
      // reads (keys +0..3, +4..7 of its k range).
      static_assert(2 * NT % 8 == 0, "transpose read blocks");
#pragma unroll
      for (int b8 = 0; b8 < 2 * NT / 8; ++b8) {
        uint32_t adr[8];
        u32x2 o[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int y = 8 * b8 + v, x = y >> 1, rr = y & 1;
          const int et = x / NKH, ks = x % NKH;
          adr[v] = base + KT::offset(trow + KI * ks + 4 * rr, (32 * et + tcol) * ES);
        }
        lds_read8_tr16(o, adr);
#pragma unroll
        for (int v = 0; v < 8; v += 2)
          ta[(8 * b8 + v) >> 1] = __builtin_bit_cast(AB, u32x4{o[v][0], o[v][1], o[v + 1][0], o[v + 1][1]});
      }
      if (virt) {
        // keys key0 + {0..7, 16..23}: biases at +0, +64 bytes, 1 / n_j one row (256 bytes) on
        u32x4 rb[8];
        lds_read8_at<0, 16, 64, 80, 256, 272, 320, 336>(rb, base + RB + key0 * 4);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          bias[r] = __uint_as_float(rb[(r >> 3) * 2 + ((r >> 2) & 1)][r & 3]);
          invn[r] = __uint_as_float(rb[4 + (r >> 3) * 2 + ((r >> 2) & 1)][r & 3]);
        }
      }
    } else {
      const float* sbias = reinterpret_cast<const float*>(sk + RB);
      if (virt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * wk + acc_key<M>(0, r, g);
          bias[r] = sbias[key];
          invn[r] = sbias[kB + key];
        }
      }
    }
    if (!virt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        bias[r] = 32 * wk + acc_key<M>(0, r, g) < nj ? 0.f : NEG_INF;
        invn[r] = 0.f;
      }
    }
    if constexpr (!(SPLIT && DIR)) {
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        s = M::mma(SPLIT ? ka[ks % NA] : M::load(reinterpret_cast<const T*>(sk + kad[ks])), qf[ks], s);
        p = M::mma(SPLIT ? va[ks % NA] : M::load(reinterpret_cast<const T*>(sk + TB + kad[ks])), gf[ks], p);
      }
    }
    f32x16 slo, plo;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float P = fast_exp2(fmaf(s[r], kLog2e, bias[r]) - lse2);
      float dp = p[r];
      if (virt) {
        dp = fmaf(gu, invn[r], dp);
        abar = fmaf(P, invn[r], abar);
      }
      if constexpr (DIR) {
        const float ds = P * (dp - dl);
        dsum += ds;                                // ε
        s[r] = ds;
        p[r] = P;
        continue;
      }
      const float pd = P * dp;
      dsum += pd;
      s[r] = pd;                                   // P∘dP, then its hi part
      p[r] = P;                                    // P, then its hi part
      if constexpr (SPLIT) {
        const float sh = to_f32(from_f32<T>(pd)), ph = to_f32(from_f32<T>(P));
        slo[r] = pd - sh;
        plo[r] = P - ph;
        s[r] = sh;
        p[r] = ph;
      }
    }
    static_for<0, NKH>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      const AB bs = M::template packv<ks * KH>(s);
#pragma unroll
      for (int et = 0; et < NET; ++et) {
        const AB kt = SPLIT ? ta[(et * NKH + ks) % NTA] : M::load(reinterpret_cast<const T*>(sk + tad[et * NKH + ks]));
        dqt[et] = M::mma(kt, bs, dqt[et]);
        kpt[et] = M::mma(kt, M::template packv<ks * KH>(p), kpt[et]);
        if constexpr (SPLIT && !DIR) {
          dqt[et] = M::mma(kt, M::template packv<ks * KH>(slo), dqt[et]);
          kpt[et] = M::mma(kt, M::template packv<ks * KH>(plo), kpt[et]);
        }
      }
    });
  };

  if (n1 > 0) fill_desc(0);
  if (n1 > DCH) fill_desc(1);
  __syncthreads();
  // Prologue: tiles [0, NST - 1) in flight (tile 0 with a single stage).
  static_for<0, (NST > 1 ? NST - 1 : 1)>([&](auto sc) {
    if (decltype(sc)::value < N) issue(decltype(sc)::value, sc);
  });
  // NST tiles per iteration so every stage index is static.
  for (int n = 0; n < N; n += NST) {
    static_for<0, NST>([&](auto sc) {
      constexpr int S = decltype(sc)::value;
      const int t = n + S;
      if (t < N) {
        // This wave's loads of tile t have landed once at most the loads of the tiles
        // issued after it (NST - 2 of them, fewer at the end) are outstanding; after the
        // barrier everyone's have, and the stage of tile t - 1 is free.
        if constexpr (NST >= 4) {
          if (t + 2 < N) barrier_vm<2 * PT>();
          else if (t + 1 < N) barrier_vm<PT>();
          else barrier_vm<0>();
        } else if constexpr (NST == 3) {
          if (t + 1 < N) barrier_vm<PT>();
          else barrier_vm<0>();
        } else {
          barrier_vm<0>();
        }
        if (t % DCH == 0 && t >= DCH && t + DCH < n1) fill_desc(t / DCH + 1);
        if (NST > 1 && t + NST - 1 < N) issue(t + NST - 1, std::integral_constant<int, (S + NST - 1) % NST>{});
        compute(t, sc);
        if (NST == 1) {
          __syncthreads();
          if (t + 1 < N) issue(t + 1, sc);
        }
      }
    });
  }

  // Δ (DIR: ε) of this lane's query over both key halves, then this wave's share of
  // dQ₀ - Δ kp (DIR: Kᵀ dSᵀ - ε kp); Δ (DIR: Δ_O + ε) for the key sweep.
  dsum = sum_halves(dsum);
  if (g == 0) sDel[wk][qrow] = dsum;
  __syncthreads();
  // (DIR with a final Δ, a.delta_final: dS already used the row's Δ; no correction)
  const float delta = qvalid && !(DIR && a.delta_final) ? sDel[0][qrow] + sDel[1][qrow] : 0.f;
  if (wk == 0 && g == 0 && !(DIR && a.delta_final)) a.delta[row0 + qrow] = qvalid ? dl + delta : 0.f;
#pragma unroll
  for (int et = 0; et < NET; ++et)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqt[et][r] = fmaf(-delta, kpt[et][r], dqt[et][r]);

  // Merge the key halves: wave (1, wq) hands its partial dQᵀ and Ā to wave (0, wq).
  constexpr int XF = (NET * 16 + 1) * 64;          // floats handed over per wave
  static_assert(2 * XF * 4 <= SB, "hand-over buffer");
  if (wk == 1) {
    float* mine = reinterpret_cast<float*>(sS0) + wq * XF + lane;
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 16; ++r) mine[(et * 16 + r) * 64] = dqt[et][r];
    mine[NET * 16 * 64] = abar;
  }
  __syncthreads();
  if (wk == 1) return;
  {
    const float* other = reinterpret_cast<const float*>(sS0) + wq * XF + lane;
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqt[et][r] += other[(et * 16 + r) * 64];
    abar = sum_halves(abar + other[NET * 16 * 64]);
  }
  if (VIRT) {
    // dQᵀ[c][q] += Σ_e H̄ᵀ[c][e] (Ā_q dO_q)[e]: A = H̄ᵀ rows (fp32 → T), B = Ā·dO fragments.
    const float* hT = a.hbarT + size_t(h) * D * D;
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      float gv[KH];
      M::unpack(gf[ks], gv);
#pragma unroll
      for (int u = 0; u < KH; ++u) gv[u] *= abar;
      const AB b = M::pack(gv);
#pragma unroll
      for (int et = 0; et < NET; ++et) {
        float hv[KH];
#pragma unroll
        for (int u = 0; u < KH; ++u) hv[u] = hT[size_t(32 * et + l32) * D + KI * ks + KH * g + u];
        dqt[et] = M::mma(M::pack(hv), b, dqt[et]);
      }
    }
  }
  float* dq = a.dQ + (row0 + qrow) * D;
#pragma unroll
  for (int et = 0; et < NET; ++et)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[32 * et + acc_row(r, g)] = qvalid ? dqt[et][r] : 0.f;
  if (g == 0) a.abar[row0 + qrow] = qvalid ? abar : 0.f;
}

// ---------------------------------------------------------------------------------------
// Per key block (exact: over the query tiles that selected it) or per centroid group and
// chunk of query tiles (virtual): dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS. Wave (wq, wk) computes
// S and dP for query half wq and key half wk (queries fed through feed_row, so P and dS
// in registers are the B operands); the two query halves are merged at the end.
// Each query tile's Q and dO rows, Qᵀ and dOᵀ, row statistics and (centroid groups) the
// tile's biases and φ' arrive by direct loads into a ring of NST stages, read through
// inline-asm blocks (bf16) as in bwd_query_kernel.
template <class T, int D, int MODE, bool GROUP>
__global__ __launch_bounds__(256) void bwd_key_kernel(BwdArgs a) {
  using M = typename MmaFor<T>::type;
  using AB = typename M::AB;
  constexpr int KI = M::KI, KH = M::KH;
  constexpr int ES = sizeof(T);
  constexpr int NKD = D / KI, NKH = 32 / KI, NET = D / 32, NT = NET * NKH;
  constexpr bool SPLIT = sizeof(T) == 2;
  constexpr int KROW = D * ES, TROW = kB * ES, TB = kB * KROW;
  constexpr int DPW = TB / 4096;                    // 1 KB direct loads per wave and operand
  // Stage: Q and dO rows, for fp32 also Qᵀ and dOᵀ (bf16 forms the transposed operands
  // from the rows with LDS transpose reads), then the rows lse, Δ, gu, bias, φ', 3 unused.
  constexpr int NTILE = SPLIT ? 2 : 4;
  constexpr int RB = NTILE * TB;
  constexpr int SB = RB + 8 * kB * 4;               // bytes per stage
  constexpr int BUDGET = 152 * 1024;
  constexpr int NST = 4 * SB <= BUDGET ? 4 : (3 * SB <= BUDGET ? 3 : (2 * SB <= BUDGET ? 2 : 1));
  constexpr int PT = NTILE * DPW + 2;               // direct loads per wave and tile
  constexpr int DCH = 256;
  using KT = SwizzledTile<KROW>;
  using TT = SwizzledTile<TROW>;
  static_assert(DPW >= 1 && TB % 4096 == 0, "tile shape");
  __shared__ __align__(1024) char sS0[SB];
  __shared__ __align__(1024) char sS1[NST > 1 ? SB : 16];
  __shared__ __align__(1024) char sS2[NST > 2 ? SB : 16];
  __shared__ __align__(1024) char sS3[NST > 3 ? SB : 16];
  __shared__ float sCol[2][kB];
  __shared__ uint32_t sDesc[2][DCH];                // tile -> query tile | valid rows << 16

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // kept scalar
  const int wq = wave >> 1, wk = wave & 1;
  const int nb = a.nb;
  const int ngrp = a.nbp / kB;
  int h, j, chunk = 0;
  {
    const uint32_t units = GROUP ? uint32_t(ngrp) * a.nchunk : uint32_t(nb);
    const uint32_t lin = xcd_remap(blockIdx.x, gridDim.x);
    h = int(lin / units);
    const int u = int(lin % units);
    j = GROUP ? u / a.nchunk : u;
    chunk = GROUP ? u % a.nchunk : 0;
  }
  const int kcol = 32 * wk + l32;                  // this lane's key (column of S)
  int nj = 0, jj = 0;
  float invn = 0.f;
  bool kvalid;
  if (!GROUP) {
    nj = min(max(a.block_len ? a.block_len[j] : kB, 1), kB);
    kvalid = kcol < nj;
  } else {
    jj = j * kB + kcol;
    kvalid = jj < nb;
    if (kvalid) invn = 1.f / float(min(max(a.block_len ? a.block_len[jj] : kB, 1), kB));
  }
  // K and V rows of this lane's key as B operands (T; centroid groups rounded from fp32).
  AB kf[NKD], vf[NKD];
  {
    const T* Kh = static_cast<const T*>(a.K) + size_t(h) * a.L * D;
    const T* Vh = static_cast<const T*>(a.V) + size_t(h) * a.L * D;
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      if (!kvalid) {
        kf[ks] = M::zero();
        vf[ks] = M::zero();
      } else if (!GROUP) {
        kf[ks] = M::load(Kh + (size_t(j) * kB + kcol) * D + KI * ks + KH * g);
        vf[ks] = M::load(Vh + (size_t(j) * kB + kcol) * D + KI * ks + KH * g);
      } else {
        float kv[KH], vv[KH];
        const float* kb = a.kbar + (size_t(h) * nb + jj) * D + KI * ks + KH * g;
        const float* vs = a.vsum + (size_t(h) * nb + jj) * D + KI * ks + KH * g;
#pragma unroll
        for (int u = 0; u < KH; ++u) {
          kv[u] = to_f32(from_f32<T>(kb[u]));
          vv[u] = to_f32(from_f32<T>(vs[u] * invn));
        }
        kf[ks] = M::pack(kv);
        vf[ks] = M::pack(vv);
      }
    }
  }
  f32x16 dvt[NET], dkt[NET];
#pragma unroll
  for (int et = 0; et < NET; ++et) dvt[et] = dkt[et] = zero16();

  // Query tiles visited: the CSR list of block j, or chunk `chunk` of all tiles.
  int t0, t1;
  const int* list = nullptr;
  if (!GROUP) {
    const int* off = a.csr_off + size_t(h) * (nb + 1);
    t0 = off[j];
    t1 = off[j + 1];
    list = a.csr_list + size_t(h) * nb * a.K_sel;
  } else {
    const int per = (nb + a.nchunk - 1) / a.nchunk;
    t0 = min(nb, chunk * per);
    t1 = min(nb, t0 + per);
  }
  const int N = t1 - t0;
  // Let the operand loads land before the first direct loads are issued, so that later
  // waits for those (counted from the newest) never have to cover them.
  __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)

  auto fill_desc = [&](int c) {
    for (int e = tid; e < DCH; e += 256) {
      const int n = c * DCH + e;
      uint32_t d = 0u;
      if (n < N) {
        const int i = GROUP ? t0 + n : list[t0 + n];
        d = uint32_t(i) | (uint32_t(min(max(a.block_len ? a.block_len[i] : kB, 1), kB)) << 16);
      }
      sDesc[c & 1][e] = d;
    }
  };
  auto desc = [&](int n) -> uint32_t {
    return __builtin_amdgcn_readfirstlane(lds_read_u32(lds_addr(&sDesc[(n / DCH) & 1][n % DCH])));
  };

  // Per-lane source offsets (swizzled order) of the chunks this lane's direct loads fill.
  int roff[DPW], rrow[DPW], toff[DPW];
#pragma unroll
  for (int u = 0; u < DPW; ++u) {
    const int b = (wave * DPW + u) * 1024 + lane * 16;
    const int rk = b / KROW, rt = b / TROW;
    rrow[u] = rk;
    roff[u] = rk * KROW + ((((b % KROW) >> 4) ^ KT::swz(rk)) << 4);
    toff[u] = rt * TROW + ((((b % TROW) >> 4) ^ TT::swz(rt)) << 4);
  }
  const char* Qb = reinterpret_cast<const char*>(static_cast<const T*>(a.Q) + size_t(h) * a.L * D);
  const char* Gb = reinterpret_cast<const char*>(static_cast<const T*>(a.dO) + size_t(h) * a.L * D);
  // Direct loads of tile n into stage S. Query rows past the tile's valid count are loaded
  // from row 0 (finite values; those queries get P = 0). Every wave issues PT loads: its
  // share of the four tiles and two 256-byte rows (wave 0: lse, Δ; wave 1: gu, bias;
  // wave 2: φ'; the others repeat the lse row into unused slots).
  auto issue = [&](int n, auto sc) {
    constexpr int S = decltype(sc)::value;
    char* st = S == 0 ? sS0 : (S == 1 ? sS1 : (S == 2 ? sS2 : sS3));
    const uint32_t d = desc(n);
    const int i = int(d & 0xFFFFu), m = int(d >> 16);
    const size_t rowb = size_t(h) * a.L + size_t(i) * kB;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qb + size_t(i) * TB, TB), rg = make_rsrc(Gb + size_t(i) * TB, TB);
    const __amdgpu_buffer_rsrc_t rqt = make_rsrc(a.qt + (size_t(h) * nb + i) * TB, TB);
    const __amdgpu_buffer_rsrc_t rgt = make_rsrc(a.gt + (size_t(h) * nb + i) * TB, TB);
#pragma unroll
    for (int u = 0; u < DPW; ++u) {
      const int ro = rrow[u] < m ? roff[u] : roff[u] - rrow[u] * KROW;
      const int lb = (wave * DPW + u) * 1024;
      buf_dma16(rq, ro, 0, st + lb);
      buf_dma16(rg, ro, 0, st + TB + lb);
      if constexpr (!SPLIT) {
        buf_dma16(rqt, toff[u], 0, st + 2 * TB + lb);
        buf_dma16(rgt, toff[u], 0, st + 3 * TB + lb);
      }
    }
    const float* lse_row = a.lse + rowb;
    const float* r0 = lse_row;
    const float* r1 = lse_row;
    if (wave == 0) {
      r1 = a.delta + rowb;
    } else if (wave == 1) {
      r0 = a.gu + rowb;
      if (GROUP) r1 = a.vbias + (size_t(h) * nb + i) * a.nbp + j * kB;
    } else if (wave == 2) {
      if (GROUP && MODE == MODE_PWT) r0 = a.vdphi + (size_t(h) * nb + i) * a.nbp + j * kB;
    }
    auto row_dma = [&](const float* src, int slot) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(src, kB * 4),
                                               (__attribute__((address_space(3))) void*)(st + RB + slot * kB * 4),
                                               4, lane * 4, 0, 0, 0);
    };
    row_dma(r0, 2 * wave);
    row_dma(r1, 2 * wave + 1);
  };

  // LDS byte offsets inside a stage of this lane's operand fragments and first query.
  uint32_t rad[NKD], tad[NT];
  const int Rq = 32 * wq + feed_row<M>(l32);       // query row this lane feeds
#pragma unroll
  for (int ks = 0; ks < NKD; ++ks) rad[ks] = KT::offset(Rq, (KI * ks + KH * g) * ES);
#pragma unroll
  for (int et = 0; et < NET; ++et)
#pragma unroll
    for (int ks = 0; ks < NKH; ++ks)
      tad[et * NKH + ks] = TT::offset(32 * et + l32, (32 * wq + KI * ks + KH * g) * ES);
  const int q0 = 32 * wq + acc_key<M>(0, 0, g);
  // transpose reads: lane 16 G + 4 u + a addresses query row 32 wq + 8 (G / 2) + u (+ the
  // fragment's k offset) at column 16 (G % 2) + 4 a (+ the fragment's column tile)
  const int trow = 32 * wq + 8 * (lane >> 5) + ((lane & 15) >> 2), tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  auto compute = [&](int n, auto sc) {
    constexpr int S = decltype(sc)::value;
    const char* sk = S == 0 ? sS0 : (S == 1 ? sS1 : (S == 2 ? sS2 : sS3));
    const int m = int(desc(n) >> 16);
    constexpr int NA = SPLIT ? NKD : 1, NTA = SPLIT ? NT : 1;
    AB qa[NA], ga[NA], qta[NTA], gta[NTA];
    float lse[16], del[16], gu[16], bias, dphi = 0.f;
    const uint32_t base = lds_addr(sk);
    // Row statistics of this lane's queries q0 + {0..7, 16..23} (lse, Δ, gu) and this
    // lane's key's bias and φ'. Centroid groups read them while the score products run
    // (fenced there, measured faster); exact blocks before them.
    auto read_rows = [&]() {
      if constexpr (SPLIT) {
        u32x4 rb[8], rc[8];
        lds_read8_at<0, 16, 64, 80, 256, 272, 320, 336>(rb, base + RB + q0 * 4);
        lds_read8_at<512, 528, 576, 592, 768, 784, 1024, 1040>(rc, base + RB + q0 * 4);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int v = (r >> 3) * 2 + ((r >> 2) & 1);
          lse[r] = __uint_as_float(rb[v][r & 3]);
          del[r] = __uint_as_float(rb[4 + v][r & 3]);
          gu[r] = __uint_as_float(rc[v][r & 3]);
        }
        bias = GROUP ? __uint_as_float(lds_read_u32(base + RB + 3 * kB * 4 + kcol * 4)) : 0.f;
        if (GROUP && MODE == MODE_PWT) dphi = __uint_as_float(lds_read_u32(base + RB + 4 * kB * 4 + kcol * 4));
      } else {
        const float* rows = reinterpret_cast<const float*>(sk + RB);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = 32 * wq + acc_key<M>(0, r, g);
          lse[r] = rows[q];
          del[r] = rows[kB + q];
          gu[r] = rows[2 * kB + q];
        }
        bias = GROUP ? rows[3 * kB + kcol] : 0.f;
        if (GROUP && MODE == MODE_PWT) dphi = rows[4 * kB + kcol];
      }
    };
    constexpr bool LATE = SPLIT && GROUP;
    if constexpr (SPLIT) {
      static_assert(NKD == 4 || NKD == 8, "fragments per block");
      uint32_t ad[NKD];
      u32x4 r4[NKD], rv[NKD];
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) ad[ks] = base + rad[ks];
      lds_read_x16<NKD, 0>(r4, ad);
      lds_read_x16<NKD, TB>(rv, ad);
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        qa[ks] = __builtin_bit_cast(AB, r4[ks]);
        ga[ks] = __builtin_bit_cast(AB, rv[ks]);
      }
    }
    if constexpr (!LATE) read_rows();
    auto qfrag = [&](int ks) { return SPLIT ? qa[ks % NA] : M::load(reinterpret_cast<const T*>(sk + rad[ks])); };
    auto gfrag = [&](int ks) { return SPLIT ? ga[ks % NA] : M::load(reinterpret_cast<const T*>(sk + TB + rad[ks])); };
    f32x16 s = zero16(), p = zero16();
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      s = M::mma(qfrag(ks), kf[ks], s);
      p = M::mma(gfrag(ks), vf[ks], p);
    }
    if constexpr (LATE) {
      // read_rows written out: through the lambda this instance spills (measured)
      __builtin_amdgcn_sched_barrier(0);
      u32x4 rb[8], rc[8];
      lds_read8_at<0, 16, 64, 80, 256, 272, 320, 336>(rb, base + RB + q0 * 4);
      lds_read8_at<512, 528, 576, 592, 768, 784, 1024, 1040>(rc, base + RB + q0 * 4);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = (r >> 3) * 2 + ((r >> 2) & 1);
        lse[r] = __uint_as_float(rb[v][r & 3]);
        del[r] = __uint_as_float(rb[4 + v][r & 3]);
        gu[r] = __uint_as_float(rc[v][r & 3]);
      }
      bias = __uint_as_float(lds_read_u32(base + RB + 3 * kB * 4 + kcol * 4));
      if (MODE == MODE_PWT) dphi = __uint_as_float(lds_read_u32(base + RB + 4 * kB * 4 + kcol * 4));
      __builtin_amdgcn_sched_barrier(0);
    }
    (void)dphi;
    if (!GROUP) bias = kvalid ? 0.f : NEG_INF;
    f32x16 pr;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = 32 * wq + acc_key<M>(0, r, g);
      const float L2 = (q < m && lse[r] > NEG_INF) ? lse[r] * kLog2e : POS_INF;
      const float P = fast_exp2(fmaf(s[r], kLog2e, bias) - L2);
      float dp = p[r];
      if (GROUP) dp = fmaf(gu[r], invn, dp);
      pr[r] = P;
      s[r] = P * (dp - del[r]);
    }
    if constexpr (GROUP && MODE == MODE_PWT) {
      // dw̃_{i,j} = φ'(w̃_{i,j}) Σ_{t in tile i} dℓ_{t,j}: column sums of dS over both query
      // halves, exchanged through LDS (asm accesses and a barrier that keeps the ring's
      // loads in flight).
      float cs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) cs += s[r];
      cs = sum_halves(cs);
      if (g == 0) lds_write_u32(lds_addr(&sCol[wq][kcol]), __float_as_uint(cs));
      barrier_lgkm();
      if (wave == 0) {
        const float c0 = __uint_as_float(lds_read_u32(lds_addr(&sCol[0][lane])));
        const float c1 = __uint_as_float(lds_read_u32(lds_addr(&sCol[1][lane])));
        const float dph = SPLIT ? __uint_as_float(lds_read_u32(base + RB + 4 * kB * 4 + lane * 4))
                                : reinterpret_cast<const float*>(sk + RB)[4 * kB + lane];
        const int x = GROUP ? t0 + n : 0;
        if (j * kB + lane < nb) a.dwt[(size_t(h) * nb + x) * nb + j * kB + lane] = dph * (c0 + c1);
      }
    }
    // dS enters dKᵀ in the input type, as P enters dVᵀ: Σ_t dS q_t has no cancellation
    // that would amplify its rounding (unlike Σ_k dS k in the dQ sweep).
    if constexpr (SPLIT) {
      // Qᵀ and dOᵀ fragments from the Q and dO rows by transpose reads, once the score
      // operands are dead: fragment x = (et, ks) is two reads (rows +0..3, +4..7).
      static_assert(2 * NT % 8 == 0, "transpose read blocks");
#pragma unroll
      for (int op = 0; op < 2; ++op) {
#pragma unroll
        for (int b8 = 0; b8 < 2 * NT / 8; ++b8) {
          uint32_t ad[8];
          u32x2 o[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            const int y = 8 * b8 + v, x = y >> 1, rr = y & 1;
            const int et = x / NKH, ks = x % NKH;
            ad[v] = base + op * TB + KT::offset(trow + KI * ks + 4 * rr, (32 * et + tcol) * ES);
          }
          lds_read8_tr16(o, ad);
#pragma unroll
          for (int v = 0; v < 8; v += 2) {
            const int x = (8 * b8 + v) >> 1;
            const AB f = __builtin_bit_cast(AB, u32x4{o[v][0], o[v][1], o[v + 1][0], o[v + 1][1]});
            if (op == 0) qta[x] = f;
            else gta[x] = f;
          }
        }
      }
    }
    static_for<0, NKH>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      const AB bp = M::template packv<ks * KH>(pr);
      const AB bs = M::template packv<ks * KH>(s);
#pragma unroll
      for (int et = 0; et < NET; ++et) {
        const int x = et * NKH + ks;
        const AB ga_t = SPLIT ? gta[x % NTA] : M::load(reinterpret_cast<const T*>(sk + 3 * TB + tad[x]));
        const AB qa_t = SPLIT ? qta[x % NTA] : M::load(reinterpret_cast<const T*>(sk + 2 * TB + tad[x]));
        dvt[et] = M::mma(ga_t, bp, dvt[et]);
        dkt[et] = M::mma(qa_t, bs, dkt[et]);
      }
    });
  };

  if (N > 0) fill_desc(0);
  if (N > DCH) fill_desc(1);
  __syncthreads();
  // Prologue: tiles [0, NST - 1) in flight (tile 0 with a single stage).
  static_for<0, (NST > 1 ? NST - 1 : 1)>([&](auto sc) {
    if (decltype(sc)::value < N) issue(decltype(sc)::value, sc);
  });
  for (int n0 = 0; n0 < N; n0 += NST) {
    static_for<0, NST>([&](auto sc) {
      constexpr int S = decltype(sc)::value;
      const int n = n0 + S;
      if (n < N) {
        // Tile n has landed once at most the loads issued after it are outstanding (the
        // next tile's, and a dw̃ store); after the barrier everyone's have, and the stage
        // of tile n - 1 is free.
        if constexpr (NST >= 4) {
          if (n + 2 < N) barrier_vm<2 * PT>();
          else if (n + 1 < N) barrier_vm<PT>();
          else barrier_vm<0>();
        } else if constexpr (NST == 3) {
          if (n + 1 < N) barrier_vm<PT>();
          else barrier_vm<0>();
        } else {
          barrier_vm<0>();
        }
        if (n % DCH == 0 && n >= DCH && n + DCH < N) fill_desc(n / DCH + 1);
        if (NST > 1 && n + NST - 1 < N) issue(n + NST - 1, std::integral_constant<int, (S + NST - 1) % NST>{});
        compute(n, sc);
        if (NST == 1) {
          __syncthreads();
          if (n + 1 < N) issue(n + 1, sc);
        }
      }
    });
  }

  // Merge the query halves: wave (1, wk) hands over to wave (0, wk).
  constexpr int XF = 2 * NET * 16 * 64;            // floats handed over per wave
  // one stage array per handing wave (or both in the single stage)
  static_assert(NST >= 2 ? XF * 4 <= SB : 2 * XF * 4 <= SB, "hand-over buffer");
  char* const hbuf = NST >= 2 ? (wk ? sS1 : sS0) : sS0 + wk * XF * 4;
  __syncthreads();
  if (wq == 1) {
    float* mine = reinterpret_cast<float*>(hbuf) + lane;
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        mine[(et * 16 + r) * 64] = dvt[et][r];
        mine[((NET + et) * 16 + r) * 64] = dkt[et][r];
      }
  }
  __syncthreads();
  if (wq == 1) return;
  const float* other = reinterpret_cast<const float*>(hbuf) + lane;
#pragma unroll
  for (int et = 0; et < NET; ++et)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dvt[et][r] += other[(et * 16 + r) * 64];
      dkt[et][r] += other[((NET + et) * 16 + r) * 64];
    }
  // dVᵀ / dKᵀ accumulators: row e = 32 et + acc_row(r, g), column = this lane's key.
  float *dk, *dv;
  if (!GROUP) {
    const size_t o = (size_t(h) * a.L + size_t(j) * kB + kcol) * D;
    dk = a.dK + o;
    dv = a.dV + o;
  } else {
    if (!kvalid) return;
    const size_t o = ((size_t(h) * a.nchunk + chunk) * a.nbp + jj) * D;
    dk = a.dkbar_part + o;
    dv = a.dvbar_part + o;
  }
#pragma unroll
  for (int et = 0; et < NET; ++et)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = 32 * et + acc_row(r, g);
      dk[e] = dkt[et][r];
      dv[e] = dvt[et][r];
    }
}

// ---------------------------------------------------------------------------------------
// dH̄[e][c] = Σ_t Ā_t dO_t[e] q_t[c]: per (head, chunk of query tiles) a d x d partial on the
// fp32 matrix cores (A = (Ā dO)ᵀ, B = Q, contraction over the rows; wave w owns every
// fourth 32 x 32 output tile), then a fixed-order reduction over the chunks.
// bf16 inputs: bf16 MFMA over the packed dOᵀ and Qᵀ tiles, the contraction over the tile's
// 64 rows; A = (Ā dO)ᵀ formed in fp32 and entered as hi + lo bf16 parts, B = Qᵀ (exact), so
// the sums lose nothing to the bf16 operands. Operands come straight from global memory,
// the next tile's in flight while the current one is multiplied.
template <int D>
__device__ __forceinline__ void dh_bf16(const BwdArgs& a) {
  constexpr int NE = D / 32, NTW = NE * NE / 4, NKS = kB / 16;
  constexpr int NA = 1, NB = NTW;                  // one A row tile and NTW column tiles per wave
  static_assert(NTW <= NE && NE % NTW == 0, "wave tiling");
  const int h = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int per = (a.nb + a.nhch - 1) / a.nhch;
  const int i0 = min(a.nb, ch * per), i1 = min(a.nb, i0 + per);
  // output tiles of this wave: (et, ct) = (ea + x, cb + y), x < NA, y < NB
  const int ea = (wave * NTW) / NE, cb = (wave * NTW) % NE;
  f32x16 acc[NA][NB];
#pragma unroll
  for (int x = 0; x < NA; ++x)
#pragma unroll
    for (int y = 0; y < NB; ++y) acc[x][y] = zero16();
  const size_t TE = size_t(kB) * D;
  const uint16_t* gt = reinterpret_cast<const uint16_t*>(a.gt) + size_t(h) * a.nb * TE;
  const uint16_t* qt = reinterpret_cast<const uint16_t*>(a.qt) + size_t(h) * a.nb * TE;
  u32x4 ga[2][NKS][NA], qb[2][NKS][NB];
  float4 ab[2][NKS][2];
  auto load = [&](int i, int buf) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int t = 16 * ks + 8 * g;
#pragma unroll
      for (int x = 0; x < NA; ++x)
        ga[buf][ks][x] = *reinterpret_cast<const u32x4*>(gt + size_t(i) * TE + size_t(32 * (ea + x) + l32) * kB + t);
#pragma unroll
      for (int y = 0; y < NB; ++y)
        qb[buf][ks][y] = *reinterpret_cast<const u32x4*>(qt + size_t(i) * TE + size_t(32 * (cb + y) + l32) * kB + t);
      const float4* ap = reinterpret_cast<const float4*>(a.abar + size_t(h) * a.L + size_t(i) * kB + t);
      ab[buf][ks][0] = ap[0];
      ab[buf][ks][1] = ap[1];
    }
  };
  if (i0 < i1) load(i0, 0);
  for (int i = i0; i < i1; i += 2) {
    static_for<0, 2>([&](auto bc) {
      constexpr int B = decltype(bc)::value;
      if (i + B < i1) {
        if (i + B + 1 < i1) load(i + B + 1, B ^ 1);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const float av[8] = {ab[B][ks][0].x, ab[B][ks][0].y, ab[B][ks][0].z, ab[B][ks][0].w,
                               ab[B][ks][1].x, ab[B][ks][1].y, ab[B][ks][1].z, ab[B][ks][1].w};
#pragma unroll
          for (int x = 0; x < NA; ++x) {
            const uint16_t* gv = reinterpret_cast<const uint16_t*>(&ga[B][ks][x]);
            float hi[8], lo[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const float f = av[u] * to_f32(gv[u]);
              hi[u] = to_f32(from_f32<uint16_t>(f));
              lo[u] = f - hi[u];
            }
            const bf16x8 ah = MmaBF16::pack(hi), al = MmaBF16::pack(lo);
#pragma unroll
            for (int y = 0; y < NB; ++y) {
              const bf16x8 bq = __builtin_bit_cast(bf16x8, qb[B][ks][y]);
              acc[x][y] = MmaBF16::mma(ah, bq, acc[x][y]);
              acc[x][y] = MmaBF16::mma(al, bq, acc[x][y]);
            }
          }
        }
      }
    });
  }
  float* out = a.dh_part + (size_t(h) * a.nhch + ch) * D * D;
#pragma unroll
  for (int x = 0; x < NA; ++x)
#pragma unroll
    for (int y = 0; y < NB; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) out[(32 * (ea + x) + acc_row(r, g)) * D + 32 * (cb + y) + l32] = acc[x][y][r];
}

template <class T, int D>
__global__ __launch_bounds__(256) void bwd_dh_kernel(BwdArgs a) {
  if constexpr (sizeof(T) == 2) {
    dh_bf16<D>(a);
  } else {
    constexpr int NE = D / 32, NTW = NE * NE / 4;
    __shared__ float sg[kB][D + 1], sq[kB][D + 1];
    const int h = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
    const int per = (a.nb + a.nhch - 1) / a.nhch;
    const int i0 = min(a.nb, ch * per), i1 = min(a.nb, i0 + per);
    f32x16 acc[NTW];
#pragma unroll
    for (int u = 0; u < NTW; ++u) acc[u] = zero16();
    for (int i = i0; i < i1; ++i) {
      const size_t row0 = size_t(h) * a.L + size_t(i) * kB;
      __syncthreads();
      for (int x = tid; x < kB * D; x += 256) {
        const int r = x / D, c = x % D;
        const float ab = a.abar[row0 + r];
        sg[r][c] = ab * to_f32(static_cast<const T*>(a.dO)[(row0 + r) * D + c]);
        sq[r][c] = ab != 0.f ? to_f32(static_cast<const T*>(a.Q)[(row0 + r) * D + c]) : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < NTW; ++u) {
        const int tile = wave * NTW + u, et = tile / NE, ct = tile % NE;
#pragma unroll 8
        for (int ks = 0; ks < kB / 2; ++ks) {
          const int t = 2 * ks + g;
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(sg[t][32 * et + l32], sq[t][32 * ct + l32], acc[u], 0, 0, 0);
        }
      }
    }
    float* out = a.dh_part + (size_t(h) * a.nhch + ch) * D * D;
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
      const int tile = wave * NTW + u, et = tile / NE, ct = tile % NE;
#pragma unroll
      for (int r = 0; r < 16; ++r) out[(32 * et + acc_row(r, g)) * D + 32 * ct + l32] = acc[u][r];
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_dh_reduce_kernel(BwdArgs a) {
  const int h = blockIdx.y, x = blockIdx.x * 256 + threadIdx.x;
  if (x >= D * D) return;
  float s = 0.f;
  for (int c = 0; c < a.nhch; ++c) s += a.dh_part[(size_t(h) * a.nhch + c) * D * D + x];
  a.dh[size_t(h) * D * D + x] = s;
}

// ---------------------------------------------------------------------------------------
// PWT: the two products with dw̃ [nb x nb], on the fp32 matrix cores, one 64-row by d
// output block per workgroup (4 waves, contraction over 64-wide chunks staged in LDS):
//   TRANS = false: dqsq_i = ½ Σ_j dw̃_{i,j} σ²_j (applied to dQ by bwd_qsq_kernel)
//   TRANS = true:  dσ²_j = ½ Σ_i dw̃_{i,j} \overline{q²}_i
template <class T, int D, bool TRANS>
__global__ __launch_bounds__(256) void bwd_wprod_kernel(BwdArgs a) {
  constexpr int NE = D / 32, NTW = 2 * NE / 4;     // 32 x 32 output tiles per wave
  __shared__ float sA[kB][kB + 1], sB[kB][D + 1];
  __shared__ float sOut[kB][D + 1];
  const int h = blockIdx.y, r0 = blockIdx.x * kB, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int nb = a.nb;
  const float* W = a.dwt + size_t(h) * nb * nb;
  const float* Bm = (TRANS ? a.qsq : a.ksig2) + size_t(h) * nb * D;
  f32x16 acc[NTW];
#pragma unroll
  for (int u = 0; u < NTW; ++u) acc[u] = zero16();
  for (int k0 = 0; k0 < nb; k0 += kB) {
    __syncthreads();
    for (int x = tid; x < kB * kB; x += 256) {     // sA[r][k] = dw̃ (or its transpose), 0 outside
      const int r = x / kB, k = x % kB, row = r0 + r, col = k0 + k;
      float v = 0.f;
      if (row < nb && col < nb) v = TRANS ? W[size_t(col) * nb + row] : W[size_t(row) * nb + col];
      sA[r][k] = v;
    }
    for (int x = tid; x < kB * D; x += 256) {
      const int k = x / D, c = x % D;
      sB[k][c] = k0 + k < nb ? Bm[size_t(k0 + k) * D + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
      const int tile = wave * NTW + u, rt = tile / NE, ct = tile % NE;
#pragma unroll 8
      for (int ks = 0; ks < kB / 2; ++ks) {
        const int k = 2 * ks + g;
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(sA[32 * rt + l32][k], sB[k][32 * ct + l32], acc[u], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NTW; ++u) {
    const int tile = wave * NTW + u, rt = tile / NE, ct = tile % NE;
#pragma unroll
    for (int r = 0; r < 16; ++r) sOut[32 * rt + acc_row(r, g)][32 * ct + l32] = 0.5f * acc[u][r];
  }
  __syncthreads();
  float* out = TRANS ? a.dsig2 : a.dqsq;
  for (int x = tid; x < kB * D; x += 256) {
    const int r = x / D, c = x % D;
    if (r0 + r < nb) out[(size_t(h) * nb + r0 + r) * D + c] = sOut[r][c];
  }
}

// dq_t += (2/m_i) q_t ∘ dqsq_i on the valid rows of every query tile (PWT), four elements
// per thread.
template <class T, int D>
__global__ __launch_bounds__(256) void bwd_qsq_kernel(BwdArgs a) {
  const size_t x = (size_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  const size_t total = size_t(a.H) * a.L * D;
  if (x >= total) return;
  const size_t row = x / D;                        // h * L + token
  const int c = int(x % D);
  const int h = int(row / size_t(a.L)), tok = int(row % size_t(a.L));
  const int i = tok / kB, r = tok % kB;
  const int m = min(max(a.block_len ? a.block_len[i] : kB, 1), kB);
  if (r >= m) return;
  const float sc = 2.f / float(m);
  const float4 w = *reinterpret_cast<const float4*>(a.dqsq + (size_t(h) * a.nb + i) * D + c);
  float q[4];
  if constexpr (sizeof(T) == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.Q) + x);
    q[0] = __uint_as_float(v.x << 16);
    q[1] = __uint_as_float(v.x & 0xFFFF0000u);
    q[2] = __uint_as_float(v.y << 16);
    q[3] = __uint_as_float(v.y & 0xFFFF0000u);
  } else {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(a.Q) + x);
    q[0] = v.x; q[1] = v.y; q[2] = v.z; q[3] = v.w;
  }
  float4* dq = reinterpret_cast<float4*>(a.dQ + x);
  float4 d = *dq;
  d.x += sc * w.x * q[0];
  d.y += sc * w.y * q[1];
  d.z += sc * w.z * q[2];
  d.w += sc * w.w * q[3];
  *dq = d;
}

constexpr int CHAIN_G = 8;                         // key blocks per workgroup of bwd_chain_kernel

// ---------------------------------------------------------------------------------------
// bf16 inputs: G = dH̄ / nb staged once per workgroup as hi + lo bf16 parts, in both
// orientations; the products run on bf16 MFMA with the token rows (exact in bf16) as A
// operands straight from memory, and the block means enter as per-block vectors:
//   dK[t][c] += Σ_e v_t[e] G[e][c] - (v̄ᵀ G)[c],   dV[t][e] += Σ_c k_t[c] G[e][c] - (G k̄)[e].
template <int D, int MODE>
__device__ __forceinline__ void chain_bf16(const BwdArgs& a) {
  constexpr int NE = D / 32, NKD = D / 16, LDG = D + 8, CT = NE / 2;
  __shared__ __align__(16) uint16_t sGh[D * LDG], sGl[D * LDG];   // G[e][c]
  __shared__ __align__(16) uint16_t sTh[D * LDG], sTl[D * LDG];   // Gᵀ[c][e]
  __shared__ float sdk[D], sdv[D], sdsig[D], skb[D], svb[D], scv[D], sck[D];
  const int h = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int nb = a.nb;
  const float invnb = 1.f / float(nb);
  for (int x = tid; x < D * D; x += 256) {
    const int e = x / D, c = x % D;
    const float f = a.dh[size_t(h) * D * D + x] * invnb;
    const uint16_t hi = from_f32<uint16_t>(f), lo = from_f32<uint16_t>(f - to_f32(hi));
    sGh[e * LDG + c] = hi;
    sGl[e * LDG + c] = lo;
    sTh[c * LDG + e] = hi;
    sTl[c * LDG + e] = lo;
  }
  const uint16_t* Kb = static_cast<const uint16_t*>(a.K);
  const uint16_t* Vb = static_cast<const uint16_t*>(a.V);
  const int tt = wave & 1, cp = wave >> 1;          // token half; column tiles cp CT .. cp CT + CT - 1
  const int t = 32 * tt + l32;                      // A row of this lane
  for (int j = blockIdx.x * CHAIN_G; j < min(nb, blockIdx.x * CHAIN_G + CHAIN_G); ++j) {
    const int n = min(max(a.block_len ? a.block_len[j] : kB, 1), kB);
    const float invn = 1.f / float(n);
    const size_t row0 = size_t(h) * a.L + size_t(j) * kB;
    __syncthreads();                                // G staged; previous block's vectors read
    if (tid < D) {
      float dk = 0.f, dv = 0.f;
      for (int c = 0; c < a.nchunk; ++c) {
        const size_t o = ((size_t(h) * a.nchunk + c) * a.nbp + j) * D + tid;
        dk += a.dkbar_part[o];
        dv += a.dvbar_part[o];
      }
      const size_t o = (size_t(h) * nb + j) * D + tid;
      sdk[tid] = dk * invn;
      sdv[tid] = dv * invn;
      sdsig[tid] = MODE == MODE_PWT ? a.dsig2[o] * 2.f * invn : 0.f;
      skb[tid] = a.kbar[o];
      svb[tid] = a.vsum[o] * invn;
    }
    // this lane's token rows as A operands (zeros on padding rows)
    bf16x8 va[NKD], ka[NKD];
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      const size_t o = (row0 + t) * D + 16 * ks + 8 * g;
      va[ks] = t < n ? *reinterpret_cast<const bf16x8*>(Vb + o) : MmaBF16::zero();
      ka[ks] = t < n ? *reinterpret_cast<const bf16x8*>(Kb + o) : MmaBF16::zero();
    }
    __syncthreads();
    if (tid < D) {                                  // (v̄ᵀ G)[c]
      float sv = 0.f;
      for (int e = 0; e < D; ++e) sv = fmaf(svb[e], to_f32(sGh[e * LDG + tid]) + to_f32(sGl[e * LDG + tid]), sv);
      scv[tid] = sv;
    } else if (tid >= 128 && tid < 128 + D) {       // (G k̄)[e]
      const int e = tid - 128;
      float sk = 0.f;
      for (int c = 0; c < D; ++c) sk = fmaf(to_f32(sTh[c * LDG + e]) + to_f32(sTl[c * LDG + e]), skb[c], sk);
      sck[e] = sk;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < CT; ++u) {
      const int col = 32 * (cp * CT + u) + l32;
      f32x16 ak = zero16(), av = zero16();
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        const int kk = 16 * ks + 8 * g;
        // dK: B(k = e, col c) = G[e][c] = Gᵀ[c][e];  dV: B(k = c, col e) = G[e][c]
        const bf16x8 th = *reinterpret_cast<const bf16x8*>(sTh + col * LDG + kk);
        const bf16x8 tl = *reinterpret_cast<const bf16x8*>(sTl + col * LDG + kk);
        const bf16x8 gh = *reinterpret_cast<const bf16x8*>(sGh + col * LDG + kk);
        const bf16x8 gl = *reinterpret_cast<const bf16x8*>(sGl + col * LDG + kk);
        ak = MmaBF16::mma(va[ks], th, ak);
        ak = MmaBF16::mma(va[ks], tl, ak);
        av = MmaBF16::mma(ka[ks], gh, av);
        av = MmaBF16::mma(ka[ks], gl, av);
      }
      const float dkc = sdk[col], dvc = sdv[col], dsc = sdsig[col], kbc = skb[col];
      const float cvc = scv[col], ckc = sck[col];
      // Branch-free, so all loads of the update are in flight together; padding rows
      // (zeros from the key sweep) are written back unchanged.
      float xk[16], xv[16], kt[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const size_t o = (row0 + 32 * tt + acc_row(r, g)) * D + col;
        xk[r] = a.dK[o];
        xv[r] = a.dV[o];
        kt[r] = to_f32(Kb[o]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = 32 * tt + acc_row(r, g);
        const size_t o = (row0 + tr) * D + col;
        const float uk = xk[r] + (dkc + (kt[r] - kbc) * dsc + (ak[r] - cvc));
        const float uv = xv[r] + (dvc + (av[r] - ckc));
        a.dK[o] = tr < n ? uk : xk[r];
        a.dV[o] = tr < n ? uv : xv[r];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Per key block: the statistics' gradients onto its valid tokens (adds to dK, dV). The two
// d x d products run on the fp32 matrix cores with dH̄ / nb and the centred tokens staged in
// LDS: dK[t][c] += Σ_e (v_t - v̄)[e] dH̄[e][c], dV[t][e] += Σ_c (k_t - k̄)[c] dH̄[e][c]; the
// output columns run along the lanes, so the updates of dK and dV are row-contiguous.
template <class T, int D, int MODE>
__global__ __launch_bounds__(256) void bwd_chain_kernel(BwdArgs a) {
  if constexpr (sizeof(T) == 2) {
    chain_bf16<D, MODE>(a);
  } else {
    constexpr int NE = D / 32;
    __shared__ float sH[D][D + 1];                   // dH̄[e][c] / nb
    __shared__ float sKd[kB][D + 1], sVd[kB][D + 1]; // k - k̄, v - v̄ (0 on padding)
    __shared__ float sdk[D], sdv[D], sdsig[D], skb[D], svb[D];
    const int h = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
    const int nb = a.nb;
    const float invnb = 1.f / float(nb);
    for (int x = tid; x < D * D; x += 256) sH[x / D][x % D] = a.dh[size_t(h) * D * D + x] * invnb;
    // CHAIN_G consecutive blocks per workgroup share the staged dH̄.
    for (int j = blockIdx.x * CHAIN_G; j < min(nb, blockIdx.x * CHAIN_G + CHAIN_G); ++j) {
    const int n = min(max(a.block_len ? a.block_len[j] : kB, 1), kB);
    const float invn = 1.f / float(n);
    __syncthreads();                                 // previous block's reads done
    if (tid < D) {
      float dk = 0.f, dv = 0.f;
      for (int c = 0; c < a.nchunk; ++c) {
        const size_t o = ((size_t(h) * a.nchunk + c) * a.nbp + j) * D + tid;
        dk += a.dkbar_part[o];
        dv += a.dvbar_part[o];
      }
      const size_t o = (size_t(h) * nb + j) * D + tid;
      sdk[tid] = dk * invn;
      sdv[tid] = dv * invn;
      sdsig[tid] = MODE == MODE_PWT ? a.dsig2[o] * 2.f * invn : 0.f;
      skb[tid] = a.kbar[o];
      svb[tid] = a.vsum[o] * invn;
    }
    __syncthreads();
    const size_t row0 = size_t(h) * a.L + size_t(j) * kB;
    const T* Kb = static_cast<const T*>(a.K) + row0 * D;
    const T* Vb = static_cast<const T*>(a.V) + row0 * D;
    for (int x = tid; x < kB * D; x += 256) {
      const int t = x / D, c = x % D;
      const bool ok = t < n;
      sKd[t][c] = ok ? to_f32(Kb[x]) - skb[c] : 0.f;
      sVd[t][c] = ok ? to_f32(Vb[x]) - svb[c] : 0.f;
    }
    __syncthreads();
    // wave: token half tt (rows 32 tt + [0, 32)), output column tiles xt = wave / 2, + 2
    const int tt = wave & 1;
    for (int xt = wave >> 1; xt < NE; xt += 2) {
      f32x16 ak = zero16(), av = zero16();
      const int col = 32 * xt + l32;
#pragma unroll 8
      for (int ks = 0; ks < D / 2; ++ks) {
        const int k = 2 * ks + g;
        // dK: A(row t, k = e) = (v - v̄)[t][e], B(k = e, col c) = dH̄[e][c]
        // dV: A(row t, k = c) = (k - k̄)[t][c], B(k = c, col e) = dH̄[e][c]
        ak = __builtin_amdgcn_mfma_f32_32x32x2f32(sVd[32 * tt + l32][k], sH[k][col], ak, 0, 0, 0);
        av = __builtin_amdgcn_mfma_f32_32x32x2f32(sKd[32 * tt + l32][k], sH[col][k], av, 0, 0, 0);
      }
      const float dkc = sdk[col], dvc = sdv[col], dsc = sdsig[col];
      // Branch-free, so all 32 loads of the update are in flight together; padding rows
      // (zeros from the key sweep) receive + 0.
      float xk[16], xv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const size_t o = (row0 + 32 * tt + acc_row(r, g)) * D + col;
        xk[r] = a.dK[o];
        xv[r] = a.dV[o];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * tt + acc_row(r, g);
        const bool on = t < n;
        const size_t o = (row0 + t) * D + col;
        const float uk = xk[r] + (dkc + sKd[t][col] * dsc + ak[r]), uv = xv[r] + (dvc + av[r]);
        a.dK[o] = on ? uk : xk[r];
        a.dV[o] = on ? uv : xv[r];
      }
    }
    }
  }
}

// ---------------------------------------------------------------------------------------
template <class T, int D, int MODE>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  const dim3 tiles(a.nb, a.H), blocks((a.nb + 255) / 256, a.H);
#define PISA_CHECK()                             \
  do {                                           \
    hipError_t e_ = hipGetLastError();           \
    if (e_ != hipSuccess) return e_;             \
  } while (0)
  const dim3 rows_grid(sizeof(T) == 2 ? unsigned((a.nb + ROWS_G - 1) / ROWS_G) : unsigned(a.nb), unsigned(a.H));
  hipLaunchKernelGGL((bwd_rows_kernel<T, D>), rows_grid, dim3(256), 0, s, a);
  PISA_CHECK();
  // Kinds of packed tiles read: fp32 Kᵀ (0) and Qᵀ, dOᵀ (1, key sweep); bf16 Qᵀ, dOᵀ for
  // dH̄ only (not in DROP); centroid groups (2) unless DROP.
  {
    const unsigned kinds = sizeof(T) == 2 ? (MODE == MODE_DROP ? 0u : 2u) : (MODE == MODE_DROP ? 2u : 3u);
    if (kinds > 0) {
      hipLaunchKernelGGL((bwd_pack_kernel<T, D>), dim3(a.nb, a.H, kinds), dim3(256), 0, s, a);
      PISA_CHECK();
    }
  }
  if (MODE != MODE_DROP) {
    hipLaunchKernelGGL((bwd_bias_kernel<MODE>), dim3(a.nb, a.H), dim3(256), 0, s, a);
    PISA_CHECK();
  }
  hipLaunchKernelGGL(csr_count_kernel, blocks, dim3(256), 0, s, a);
  PISA_CHECK();
  hipLaunchKernelGGL(csr_scan_kernel, dim3(a.H), dim3(256), 0, s, a);
  PISA_CHECK();
  hipLaunchKernelGGL(csr_fill_kernel, blocks, dim3(256), 0, s, a);
  PISA_CHECK();
  if (a.O) {
    constexpr unsigned RPB = 256u / (D * sizeof(T) / 16u);
    const size_t rows = size_t(a.H) * size_t(a.L);
    hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3(unsigned((rows + RPB - 1) / RPB)), dim3(256), 0, s, a);
    PISA_CHECK();
    hipLaunchKernelGGL((bwd_query_kernel<T, D, MODE, true>), dim3(unsigned(a.H) * unsigned(a.nb)), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((bwd_query_kernel<T, D, MODE, false>), dim3(unsigned(a.H) * unsigned(a.nb)), dim3(256), 0, s, a);
  }
  PISA_CHECK();
  hipLaunchKernelGGL((bwd_key_kernel<T, D, MODE, false>), dim3(unsigned(a.H) * unsigned(a.nb)), dim3(256), 0, s, a);
  PISA_CHECK();
  if (MODE != MODE_DROP) {
    const unsigned groups = unsigned(a.nbp / kB) * unsigned(a.nchunk);
    hipLaunchKernelGGL((bwd_key_kernel<T, D, MODE, true>), dim3(unsigned(a.H) * groups), dim3(256), 0, s, a);
    PISA_CHECK();
    hipLaunchKernelGGL((bwd_dh_kernel<T, D>), dim3(a.nhch, a.H), dim3(256), 0, s, a);
    PISA_CHECK();
    hipLaunchKernelGGL((bwd_dh_reduce_kernel<D>), dim3((D * D + 255) / 256, a.H), dim3(256), 0, s, a);
    PISA_CHECK();
    if (MODE == MODE_PWT) {
      const dim3 wgrid((a.nb + kB - 1) / kB, a.H);
      hipLaunchKernelGGL((bwd_wprod_kernel<T, D, false>), wgrid, dim3(256), 0, s, a);
      PISA_CHECK();
      const size_t quads = size_t(a.H) * a.L * D / 4;
      hipLaunchKernelGGL((bwd_qsq_kernel<T, D>), dim3(unsigned((quads + 255) / 256)), dim3(256), 0, s, a);
      PISA_CHECK();
      hipLaunchKernelGGL((bwd_wprod_kernel<T, D, true>), wgrid, dim3(256), 0, s, a);
      PISA_CHECK();
    }
    hipLaunchKernelGGL((bwd_chain_kernel<T, D, MODE>), dim3((a.nb + CHAIN_G - 1) / CHAIN_G, a.H), dim3(256), 0, s, a);
    PISA_CHECK();
  }
#undef PISA_CHECK
  return hipSuccess;
}

template <class T, int D>
static hipError_t launch_bwd_d(int mode, const BwdArgs& a, hipStream_t s) {
  switch (mode) {
    case MODE_DROP: return launch_bwd_t<T, D, MODE_DROP>(a, s);
    case MODE_PISA: return launch_bwd_t<T, D, MODE_PISA>(a, s);
    default: return launch_bwd_t<T, D, MODE_PWT>(a, s);
  }
}

// Pieces shared with the PWT_ROW backward (attention_bwd_literal.hip): dO·(H̄ q) per row,
// and after its sweeps dH̄ from Ā and the statistics' gradients onto the tokens (with dσ²).
hipError_t launch_bwd_rows(const BwdArgs& a, hipStream_t s) {
  const dim3 grid(unsigned((a.nb + ROWS_G - 1) / ROWS_G), unsigned(a.H));
  if (a.d == 64) hipLaunchKernelGGL((bwd_rows_kernel<uint16_t, 64>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((bwd_rows_kernel<uint16_t, 128>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_stats_tail_d(const BwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bwd_pack_kernel<uint16_t, D>), dim3(a.nb, a.H, 1), dim3(256), 0, s, a);   // Qᵀ, dOᵀ for dH̄
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dh_kernel<uint16_t, D>), dim3(a.nhch, a.H), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dh_reduce_kernel<D>), dim3((D * D + 255) / 256, a.H), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_chain_kernel<uint16_t, D, MODE_PWT>), dim3((a.nb + CHAIN_G - 1) / CHAIN_G, a.H), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_stats_tail(const BwdArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_bwd_stats_tail_d<64>(a, s) : launch_bwd_stats_tail_d<128>(a, s);
}

template <int D>
static hipError_t launch_bwd_exact_sweeps_d(const BwdArgs& a, hipStream_t s) {
  const dim3 tiles(unsigned(a.H) * unsigned(a.nb)), blocks((a.nb + 255) / 256, a.H);
  hipLaunchKernelGGL((bwd_query_kernel<uint16_t, D, MODE_DROP, true>), tiles, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(csr_count_kernel, blocks, dim3(256), 0, s, a);
  hipLaunchKernelGGL(csr_scan_kernel, dim3(a.H), dim3(256), 0, s, a);
  hipLaunchKernelGGL(csr_fill_kernel, blocks, dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_key_kernel<uint16_t, D, MODE_DROP, false>), tiles, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_exact_sweeps(const BwdArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_bwd_exact_sweeps_d<64>(a, s) : launch_bwd_exact_sweeps_d<128>(a, s);
}

hipError_t launch_attention_bwd(int bf16, int mode, const BwdArgs& a, hipStream_t s) {
  if (bf16) return a.d == 64 ? launch_bwd_d<uint16_t, 64>(mode, a, s) : launch_bwd_d<uint16_t, 128>(mode, a, s);
  return a.d == 64 ? launch_bwd_d<float, 64>(mode, a, s) : launch_bwd_d<float, 128>(mode, a, s);
}

}  // namespace pisa
