// Register-streamed attention forward for bf16 inputs, modes DROP / PISA / PWT.
//
// Same computation as the LDS-staged kernels of attention_fwd.hip (PISA paper §3.2
// Eq. (3.2), §3.3 and §3.4 phases 1-3; Sparse Linear Attention blog, Sparse Linear
// Attention and PWT sections): exact softmax terms of every key of the selected blocks,
// one virtual token per unselected block (logit q·k̄_j + ln n_j + φ_ij, value ΣV_j / n_j,
// its weight e^{q·k̄_j + φ} also summed into A_t), then N_t += A_t H̄ q_t and
// o_t = N_t / D_t, all under one softmax.
//
// Organisation, chosen for gfx950:
// * One workgroup of two waves per 64-row query tile. Wave w takes key half w (32 keys)
//   of every tile, for all 64 queries: the scores Sᵀ (32 keys x 64 queries, two
//   v_mfma_f32_32x32x16_bf16 output tiles) and the output Oᵀ (D x 64) are each computed
//   once, and the two halves' softmax states are merged at the end.
// * K, Vᵀ, centroid and mean-value tiles are stored in MFMA operand order (TileLayout),
//   so a wave streams its 8 KB + 8 KB of a tile with 1 KB buffer loads straight into
//   operand registers, two steps ahead of use. The main loop has no barrier.
// * One wave per SIMD holds Q (both query halves), the D x 64 accumulators and two tiles
//   of operands. MFMA and VALU work overlap inside the wave by software pipelining over
//   units u = (tile u / 2, query half u % 2): step k issues the score MFMAs of unit k + 1
//   and the PV MFMAs of unit k - 1 while the VALU runs the softmax of unit k.
// * Everything that depends on the key alone enters the scores through the accumulator
//   input of the first score MFMA: 0 / -inf for the valid / padding keys of exact tiles,
//   ln n_j + φ_ij (or -inf for selected blocks) for virtual tokens. These 32-key rows
//   live in LDS (a fixed table of masks, and per wave a ring of virtual-tile rows filled
//   ahead of use) and are read one step before the scores that add them, so the softmax
//   is the same short sequence of exp2, bf16 packing and v_dot2 sums for every tile.
// * Exact-tile descriptors (block index, valid keys) are staged in LDS per wave and read
//   one issue ahead of use.
// * No rescaling and no running max inside the loop: each row's exponentials are taken
//   against a fixed reference, the max of the row's first unit (each wave its own). Any
//   exponential above 2^60 leaves the row's sum above 2^60; a wave with such a row (or
//   one whose first unit had no valid key and whose sum fell below 2^-60) computes the
//   true row max in a score-only pass and runs its tiles again against it, which bounds
//   every exponential by 1. The accumulators are therefore touched by MFMA only.
#include "attention.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace pisa {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 ld_frag(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

template <int I>
using ic = std::integral_constant<int, I>;

// Sums beyond these bounds send a wave to the second pass (see above).
constexpr float kSumHi = 0x1p60f, kSumLo = 0x1p-60f;

}  // namespace

template <int D, int MODE, int UPT>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attention_frag_kernel(AttnArgs a) {
  constexpr int NKD = D / 16;            // K fragments per half tile (score k-steps)
  constexpr int NET = D / 32;            // 32-row tiles of Oᵀ
  constexpr int NVF = 2 * NET;           // Vᵀ fragments per half tile
  constexpr int HE = NET / 2;            // Oᵀ tiles finalised by each wave
  constexpr int TB = kB * D * 2;         // bytes per tile
  constexpr int HB = TB / 2;             // bytes per half tile
  constexpr bool VIRT = MODE == MODE_PISA || MODE == MODE_PWT;
  constexpr float NEG_INF = -__builtin_huge_valf();
  constexpr int kDead = 0x40000000;      // tile offset past every buffer: loads return zeros
  constexpr int XS = HE * 32 + 8;        // floats per lane handed over in the merge
  // Tiles of K / Vᵀ operands held in registers (loads run NS - 1 tiles ahead); d = 128
  // has room for two.
  constexpr int NS = D == 128 ? 2 : 3;
  // Bias rows: 33 mask rows (row nk: keys < nk get 0, the others -inf), then per wave a
  // ring of VR virtual-tile rows (32 fp32 biases ln n_j + φ, then 32 bf16 weights 1 / n_j):
  // the first VR filled before the loop, VH at a time, later ones one per loading step.
  constexpr int VR = 32, VH = 16, MROWS = 33;
  using KT = SwizzledTile<D * 2>;
  static_assert(2 * XS * 64 * 4 >= kB * D * 2, "output staging must fit the hand-over buffer");

  __shared__ __align__(16) float sX[2 * XS * 64];
  __shared__ __align__(16) float sRow[MROWS + (VIRT ? 2 * VR : 0)][64];

  const int lane = threadIdx.x & 63, g = lane >> 5, l32 = lane & 31;
  const int kh = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, kept scalar
  const int nb = a.nb, ngrp = a.nbp / kB;
  // Query tiles of more than 32 rows run with two units per tile, the others with one
  // (their second query half is all padding); each kind has its own launch over the
  // statistics call's tile order (that kind's tiles first), and the workgroups past the
  // kind's count leave at once.
  const int32_t* order = reinterpret_cast<const int32_t*>(a.packed + a.pl.tiles);
  const uint32_t cnt = uint32_t(order[UPT == 2 ? 0 : 1]), work = uint32_t(a.H) * cnt;
  if (blockIdx.x >= work) return;
  const uint32_t lin = xcd_remap(blockIdx.x, work);
  const int h = int(lin / cnt);
  const int ent = order[2 + (UPT == 2 ? 0 : order[0]) + int(lin % cnt)];
  const int i = ent >> 7, ni = ent & 127;

  const uint16_t* Qh = static_cast<const uint16_t*>(a.Q) + size_t(h) * a.L * D;
  const char* kfh = a.packed + a.pl.kf + size_t(h) * nb * TB;
  const char* vth = a.packed + a.pl.vt + size_t(h) * nb * TB;
  const char* kbh = a.packed + a.pl.kbar + size_t(h) * ngrp * TB;
  const char* vbh = a.packed + a.pl.vbar + size_t(h) * ngrp * TB;
  const uint16_t* hbp = reinterpret_cast<const uint16_t*>(a.packed + a.pl.hbar) + size_t(h) * D * D;
  const uint32_t* mrow = VIRT ? a.mask + (size_t(h) * nb + i) * a.nw : nullptr;
  const float* wrow = MODE == MODE_PWT ? a.wt + (size_t(h) * nb + i) * nb : nullptr;

  // Q fragments, B operand of Sᵀ = K Qᵀ, for query halves 0 and 1; padding rows (all of
  // half 1 with one unit per tile) are zero.
  bf16x8 qf[2][NKD];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int row = 32 * qt + l32;
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      bf16x8 v = {};
      if ((UPT == 2 || qt == 0) && row < ni) v = *reinterpret_cast<const bf16x8*>(Qh + (size_t(i) * kB + row) * D + 16 * ks + 8 * g);
      qf[qt][ks] = v;
    }
  }

  // Mask rows, written in full by each wave (the same values), so no barrier is needed.
  for (int e = lane; e < MROWS * 32; e += 64) sRow[e >> 5][e & 31] = (e & 31) < (e >> 5) ? 0.f : NEG_INF;

  f32x16 acc[NET][2];
  // Per query half: the exponent reference (log2 units), Σ p and Σ p / n_j over virtual
  // tokens (A_t), each over this lane's 16 keys.
  float mu[2] = {0.f, 0.f}, lsum[2], asum[2];

  // Exact tiles of this wave. Descriptors (block j | key half << 16 | valid keys << 17)
  // are staged in a wave-private LDS table that lives in this wave's own hand-over
  // region (written only after its loop); each issue reads the next descriptor one issue
  // ahead, so the loop never waits on memory for them.
  //
  // When the whole selection fits the table, each wave keeps only useful work: its own
  // key half of every full block, and half 0 of every other block of at most 32 tokens
  // (ragged blocks alternate between the waves); out-of-range indices are dropped. The
  // two partial softmax states are merged at the end, so any split of the keys is exact.
  // Larger selections are staged DCAP tiles at a time, every block with half kh.
  constexpr int DCAP = XS * 64;
  uint32_t* dtab = reinterpret_cast<uint32_t*>(sX + kh * XS * 64);
  const int32_t* irow = a.idx + (size_t(h) * nb + i) * a.K_sel;
  const bool compact = a.K_sel <= DCAP;
  int n1 = a.K_sel;                      // exact tiles of this wave
  int N = n1 + (VIRT ? ngrp : 0);        // all tiles of this wave
  int dbase = 0;
  auto block_keys = [&](int j) -> int { return a.block_len ? min(max(a.block_len[j], 1), kB) : kB; };
  // jf: this lane's entry of the first 64, loaded by the caller ahead of other work.
  auto build_list = [&](int jf) -> int {  // compact table; returns its length
    const uint64_t below = (uint64_t(1) << lane) - 1u;
    int written = 0, ragged = 0;
    for (int s0 = 0; s0 < a.K_sel; s0 += 64) {
      const int e = s0 + lane;
      const int j = s0 == 0 ? jf : e < a.K_sel ? irow[e] : -1;
      const bool valid = j >= 0 && j < nb;
      const int v = valid ? block_keys(j) : 0;
      const bool rag = valid && v <= 32;
      const uint64_t rmask = __ballot(rag);
      const int rank = ragged + __popcll(rmask & below);
      const bool mine = valid && (!rag || (rank & 1) == kh);
      const uint64_t mmask = __ballot(mine);
      if (mine) {
        const uint32_t half = rag ? 0u : uint32_t(kh);
        dtab[written + __popcll(mmask & below)] = uint32_t(j) | (half << 16) | (uint32_t(v) << 17);
      }
      written += __popcll(mmask);
      ragged += __popcll(rmask);
    }
    return written;
  };
  auto fill = [&](int t0) {              // uncompacted table of tiles [t0, t0 + DCAP)
    const int cnt = min(DCAP, n1 - t0);
    for (int e = lane; e < cnt; e += 64) {
      const int j = irow[t0 + e];
      const bool valid = j >= 0 && j < nb;
      dtab[e] = valid ? uint32_t(j) | (uint32_t(kh) << 16) | (uint32_t(block_keys(j)) << 17) : uint32_t(kh) << 16;
    }
    dbase = t0;
  };
  auto read_desc = [&](int t) -> uint32_t {   // t < n1, t >= dbase
    if (!compact && t - dbase >= DCAP) fill(t);
    return dtab[t - dbase];
  };

  // Virtual-tile rows of tiles [t0, t0 + cnt) into the ring (slot (t - n1) mod VR): lane
  // half g takes every other tile, lane l32 one key of this wave's half of the group.
  auto vrow = [&](int t) { return MROWS + kh * VR + ((t - n1) & (VR - 1)); };
  // Row of virtual tile t from this lane's inputs (mask word, block length, w̃ of key jj =
  // its key of the group): lane l32 writes key l32 of this wave's half.
  auto write_vrow = [&](int t, uint32_t mw, int blv, float wv) {
    const int jj = (t - n1) * kB + 32 * kh + l32;
    float bias = NEG_INF, inv = 0.f;
    if (jj < nb && !((mw >> (jj & 31)) & 1u)) {
      // Hardware log (v_log_f32, within 1 ulp): w >= 0 keeps ln(1 + w) accurate to
      // ~1e-7 absolute, far below the logit's own rounding.
      const int nj = min(max(blv, 1), kB);
      const float lnn = __logf(float(nj));
      float phi = 0.f;
      if constexpr (MODE == MODE_PWT) {
        float w = wv;
        if (a.gate && w > lnn) w = 0.f;
        phi = a.w_linear ? __logf(1.f + w) : w;
      }
      bias = lnn + phi;
      inv = __builtin_amdgcn_rcpf(float(nj));
    }
    sRow[vrow(t)][l32] = bias;
    reinterpret_cast<__bf16*>(&sRow[vrow(t)][32])[l32] = static_cast<__bf16>(inv);
  };
  // Inputs of key l32 of virtual tile t (clamped in bounds; unused past the last tile).
  auto vin_jj = [&](int t) { return min((t - n1) * kB + 32 * kh + l32, nb - 1); };
  // Rows of tiles [t0, t0 + cnt), cnt <= VH, lane half g taking every other tile; all
  // inputs are loaded first, so one memory latency covers the fill.
  auto vfill = [&](int t0, int cnt) {
    constexpr int VI = VH / 2;
    uint32_t mw[VI];
    int bl[VI];
    float wv[VI];
#pragma unroll
    for (int q = 0; q < VI; ++q) {
      const int jj = vin_jj(t0 + 2 * q + g);
      mw[q] = mrow[jj >> 5];
      bl[q] = a.block_len ? a.block_len[jj] : kB;
      wv[q] = MODE == MODE_PWT ? wrow[jj] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < VI; ++q)
      if (2 * q + g < cnt) write_vrow(t0 + 2 * q + g, mw[q], bl[q], wv[q]);
  };
  // The 16 biases of a row this lane adds, in Sᵀ accumulator order: register r of lane
  // half g holds key 16 (r / 8) + 8 g + r % 8.
  auto read_row = [&](int row) -> f32x16 {
    const float4* p = reinterpret_cast<const float4*>(&sRow[row][8 * g]);
    const float4 x0 = p[0], x1 = p[1], x2 = p[4], x3 = p[5];
    f32x16 c;
    c[0] = x0.x; c[1] = x0.y; c[2] = x0.z; c[3] = x0.w;
    c[4] = x1.x; c[5] = x1.y; c[6] = x1.z; c[7] = x1.w;
    c[8] = x2.x; c[9] = x2.y; c[10] = x2.z; c[11] = x2.w;
    c[12] = x3.x; c[13] = x3.y; c[14] = x3.z; c[15] = x3.w;
    return c;
  };
  // The matching 1 / n_j weights of a virtual row, as the bf16 pairs of P.
  auto read_inv = [&](int row, bf16x8 (&w)[2]) {
    const bf16x8* p = reinterpret_cast<const bf16x8*>(&sRow[row][32 + 4 * g]);
    w[0] = p[0];
    w[1] = p[2];
  };

  uint32_t dnext = 0u;                   // descriptor of the next exact tile to issue
  // Operand ring: the K and Vᵀ registers of NS tiles. Stage s holds tiles t with t % NS == s.
  bf16x8 kst[NS][NKD], vst[NS][NVF];
  int toff[NS], crow[NS];
  uint32_t pv_m = 0u;                    // inputs of the next progressively written virtual row
  int pv_b = 0;
  float pv_w = 0.f;

  // Tile t's source (stage P = t % NS): fragment offset and bias row from its descriptor,
  // and the descriptor pipeline advanced. The fragment loads themselves are spread over
  // the step.
  auto issue_desc = [&](int t, auto pc) {
    constexpr int P = decltype(pc)::value;
    int off = kDead, row = 0;
    if (t < N) {
      if (VIRT && t >= n1) {
        off = (t - n1) * TB + kh * HB;
        row = vrow(t);
      } else {
        const uint32_t d = __builtin_amdgcn_readfirstlane(dnext);
        const int half = int((d >> 16) & 1u);
        off = int(d & 0xFFFFu) * TB + half * HB;
        row = min(max(int(d >> 17) - 32 * half, 0), 32);   // valid keys from this half's first
        if (t + 1 < n1) dnext = read_desc(t + 1);
      }
    }
    toff[P] = off;
    crow[P] = row;
    __builtin_amdgcn_sched_barrier(0);
  };
  // Buffer resource and lane offset of tile t's K (or Vᵀ) fragments in stage P.
  auto krsrc = [&](int t) { return VIRT && t >= n1 ? make_rsrc(kbh, uint32_t(ngrp) * TB) : make_rsrc(kfh, uint32_t(nb) * TB); };
  auto vrsrc = [&](int t) { return VIRT && t >= n1 ? make_rsrc(vbh, uint32_t(ngrp) * TB) : make_rsrc(vth, uint32_t(nb) * TB); };
  auto frag_at = [&](__amdgpu_buffer_rsrc_t r, int vo, int f) { return ld_frag(r, vo + (f & 3) * 1024, (f >> 2) * 4096); };
  // Exponent reference from one unit's scores: its row max in log2 units, 0 if empty.
  auto ref_of = [&](const f32x16& s) -> float {
    float x = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) x = fmaxf(x, s[r]);
    x = max_halves(x);
    return x > NEG_INF ? x * kLog2e : 0.f;
  };

  f32x16 sb[2];
  f32x16 c0;                             // bias row of the tile whose scores come next
  bf16x8 pb[2][2];
  const bf16x2 one2 = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

  // One pipeline step k, ST = k % (2 NS). With UPT = 2 units per tile, unit k is
  // (tile k / 2, query half k % 2); query tiles of at most 32 rows use UPT = 1, one unit
  // (query half 0) per tile, and skip the all-padding half.
  //
  // The step's matrix work (score MFMAs of unit k + 1, PV MFMAs of unit k - 1,
  // alternating) and its VALU work (softmax of unit k) are laid out as NM groups: MFMA c,
  // then one fragment load (steps that start a tile's loads) and a slice of the softmax,
  // fenced so that the in-order wave always has VALU work to issue while an MFMA runs.
  constexpr int NM = NKD + NVF;                  // MFMAs per step
  // Vᵀ fragment read by the PV MFMA of group 2 v.
  auto vfrag = [](int v) constexpr { return 2 * (v % NET) + v / NET; };
  auto step = [&](int k, auto stc) {
    constexpr int ST = decltype(stc)::value;
    constexpr int BP = ST & 1, BO = BP ^ 1;                  // buffer of unit k; of units k -+ 1
    constexpr int QT = UPT == 2 ? BP : 0, QO = UPT == 2 ? BO : 0;   // query halves of the same
    constexpr int TP = (ST / UPT) % NS;                      // stage of unit k's tile
    constexpr int SK = ((ST + 1) / UPT) % NS;                // K stage read by the scores of unit k + 1
    constexpr int SV = ((ST + UPT * NS - 1) / UPT) % NS;     // V stage read by the PV of unit k - 1
    constexpr bool LOADS = UPT == 1 || (ST & 1);             // steps that stream a tile's operands
    constexpr int VL = UPT == 2 ? NS - 1 : NS - 2;           // Vᵀ runs VL tiles ahead, K NS
    constexpr int LV = (TP + VL) % NS;                       // stage receiving Vᵀ
    // Steps whose score MFMAs are the last to add the current bias row load the next one
    // (tile n + 1, or n + 2 with one unit per tile) once the first score MFMA has read it.
    constexpr bool CLOAD = UPT == 1 || (ST & 1) == 0;
    constexpr int CT = UPT == 2 ? 1 : 2;
    constexpr int CS = (ST / UPT + CT) % NS;
    const int n = k / UPT;
    f32x16& sc = sb[BP];
    f32x16& sn = sb[BO];
    // K of tile n + NS goes into the stage that tile n just left, Vᵀ of tile n + VL into
    // the one that tile n + VL - NS left.
    const int vov = lane * 16 + toff[LV];       // read before the K issue may reuse the slot
    if constexpr (LOADS) issue_desc(n + NS, ic<TP>{});
    if constexpr (VIRT && LOADS) {
      // Virtual rows past the prologue's VR: the inputs of tile n + NS + 2 are loaded here
      // and its row written at the next loading step, a step or more before its bias
      // row is read (tile n + NS + 1, loaded at the previous one, is written now).
      const int tp = n + NS + 1, tq = n + NS + 2;
      if (tp < N && tp - n1 >= VR) write_vrow(tp, pv_m, pv_b, pv_w);
      if (tq < N && tq - n1 >= VR) {
        const int jj = vin_jj(tq);
        pv_m = mrow[jj >> 5];
        pv_b = a.block_len ? a.block_len[jj] : kB;
        pv_w = MODE == MODE_PWT ? wrow[jj] : 0.f;
      }
    }
    const int crw = crow[CS];
    const __amdgpu_buffer_rsrc_t rk = krsrc(n + NS), rv = vrsrc(n + VL);   // used when LOADS
    const int vok = lane * 16 + toff[TP];
    const float nmu = -mu[QT];
    // Softmax of unit k against the row's fixed reference: element r's exponential at
    // group r NM / 16, each pair packed to bf16 two slots later and summed (v_dot2, the
    // same bf16 values the PV MFMA reads) one slot after that.
    auto pack = [&](auto dc) {
      constexpr int dd = decltype(dc)::value;
      pb[BP][dd >> 2][2 * (dd & 3)] = static_cast<__bf16>(sc[2 * dd]);
      pb[BP][dd >> 2][2 * (dd & 3) + 1] = static_cast<__bf16>(sc[2 * dd + 1]);
    };
    auto total = [&](auto dc) {
      constexpr int dd = decltype(dc)::value;
      const bf16x2 pr = {pb[BP][dd >> 2][2 * (dd & 3)], pb[BP][dd >> 2][2 * (dd & 3) + 1]};
      lsum[QT] = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, lsum[QT], false);
    };
    static_for<0, NM>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      if constexpr (c & 1) {                     // score MFMA f of unit k + 1
        constexpr int f = c >> 1;
        sn = MmaBF16::mma(kst[SK][f], qf[QO][f], f == 0 ? c0 : sn);
      } else {                                   // PV MFMA v of unit k - 1
        constexpr int v = c >> 1, et = v % NET, ks = v / NET;
        acc[et][QO] = MmaBF16::mma(vst[SV][2 * et + ks], pb[BO][ks], acc[et][QO]);
      }
      // Each group loads the fragment that the same group of a later step consumes, so
      // every fragment has the same lead.
      if constexpr (LOADS) {
        if constexpr (c & 1) kst[TP][c >> 1] = frag_at(rk, vok, c >> 1);
        else vst[LV][vfrag(c >> 1)] = frag_at(rv, vov, vfrag(c >> 1));
      }
      if constexpr (CLOAD && c == 4) c0 = read_row(crw);
      static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        if constexpr (r * NM / 16 == c) sc[r] = fast_exp2(fmaf(sc[r], kLog2e, nmu));
      });
      static_for<0, 8>([&](auto dc) {
        constexpr int dd = decltype(dc)::value;
        if constexpr ((2 * dd + 2) * NM / 16 == c) pack(dc);
        if constexpr ((2 * dd + 3) * NM / 16 == c) total(dc);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<0, 8>([&](auto dc) {
      constexpr int dd = decltype(dc)::value;
      if constexpr ((2 * dd + 2) * NM / 16 >= NM) pack(dc);
      if constexpr ((2 * dd + 3) * NM / 16 >= NM) total(dc);
    });
    // P of unit k is used by the next step's MFMAs and the sums only after the loop;
    // keep them computed here rather than sunk next to those uses.
    asm volatile("" ::"v"(pb[BP][0]), "v"(pb[BP][1]), "v"(lsum[QT]));

    if (VIRT && n >= n1) {            // A_t: Σ p / n_j over this lane's virtual tokens
      bf16x8 iw[2];
      read_inv(vrow(n), iw);
      float pa = asum[QT];
      static_for<0, 8>([&](auto dc) {
        constexpr int dd = decltype(dc)::value, x = dd >> 2, y = 2 * (dd & 3);
        const bf16x2 pr = {pb[BP][x][y], pb[BP][x][y + 1]}, wr = {iw[x][y], iw[x][y + 1]};
        pa = __builtin_amdgcn_fdot2_f32_bf16(pr, wr, pa, false);
      });
      asum[QT] = pa;
    }
  };
  // After the last step: PV of the last unit (its step index mod 2 NS is STL).
  auto finish = [&](auto stlc) {
    constexpr int STL = decltype(stlc)::value;
    constexpr int SV = (STL / UPT) % NS, BL = STL & 1, QL = UPT == 2 ? BL : 0;
    static_for<0, 2>([&](auto kc) {
      constexpr int ks = decltype(kc)::value;
#pragma unroll
      for (int et = 0; et < NET; ++et) acc[et][QL] = MmaBF16::mma(vst[SV][2 * et + ks], pb[BL][ks], acc[et][QL]);
    });
  };

  // Score-only pass over this wave's tiles: the true max of every row (log2 units) as the
  // new reference. Taken only after an out-of-range sum, so it is kept simple.
  auto max_pass = [&]() {
    float mt[2] = {NEG_INF, NEG_INF};
    if (!compact && n1 > 0) fill(0);
    for (int t = 0; t < N; ++t) {
      int off, row;
      __amdgpu_buffer_rsrc_t r;
      if (VIRT && t >= n1) {
        if (((t - n1) & (VH - 1)) == 0) vfill(t, min(VH, N - t));
        off = (t - n1) * TB + kh * HB;
        row = vrow(t);
        r = make_rsrc(kbh, uint32_t(ngrp) * TB);
      } else {
        const uint32_t d = __builtin_amdgcn_readfirstlane(read_desc(t));
        const int half = int((d >> 16) & 1u);
        off = int(d & 0xFFFFu) * TB + half * HB;
        row = min(max(int(d >> 17) - 32 * half, 0), 32);
        r = make_rsrc(kfh, uint32_t(nb) * TB);
      }
      bf16x8 kk[NKD];
#pragma unroll
      for (int f = 0; f < NKD; ++f) kk[f] = frag_at(r, lane * 16 + off, f);
      const f32x16 cb = read_row(row);
#pragma unroll
      for (int qt = 0; qt < UPT; ++qt) {
        f32x16 s = cb;
#pragma unroll
        for (int f = 0; f < NKD; ++f) s = MmaBF16::mma(kk[f], qf[qt][f], s);
        float x = s[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) x = fmaxf(x, s[e]);
        mt[qt] = fmaxf(mt[qt], max_halves(x));
      }
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) mu[qt] = mt[qt] > NEG_INF ? mt[qt] * kLog2e : 0.f;
  };

  // The tile loop for UPT units per tile; a wave with an out-of-range row sum runs it
  // again against the rows' true maxima.
  auto run = [&]() {
    constexpr int VL = UPT == 2 ? NS - 1 : NS - 2;
    for (int pass = 0;; ++pass) {
#pragma unroll
      for (int et = 0; et < NET; ++et) acc[et][0] = acc[et][1] = zero16();
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) lsum[qt] = asum[qt] = 0.f;
      if (N == 0) break;
      // Prologue: descriptors, virtual rows, K of tiles [0, NS), Vᵀ of tiles [0, VL),
      // scores of unit 0, issued as the loading steps of tiles -NS .. -1 would issue them
      // (the loop's memory waits then hold from its first step on). Vᵀ stage NS - 1 and
      // P of "unit -1" are zero, so step 0's PV adds nothing.
      // The first chunk of the selection is loaded before the first virtual rows are
      // filled (their rows depend on the virtual index only), so the two memory
      // latencies overlap.
      const int jf = compact && lane < a.K_sel ? irow[lane] : -1;
      if constexpr (VIRT) {
        if (ngrp > 0) vfill(n1, min(VH, ngrp));
      }
      if (a.K_sel > 0) {
        if (compact) {
          n1 = build_list(jf);
          N = n1 + (VIRT ? ngrp : 0);
        } else {
          fill(0);
        }
        if (n1 > 0) dnext = read_desc(0);
      }
      if (N == 0) break;
      if constexpr (VIRT) {
        if (N > n1 + VH) vfill(n1 + VH, min(VH, N - n1 - VH));
      }
      pb[1][0] = pb[1][1] = bf16x8{};
      static_for<0, NS>([&](auto pc) {
        constexpr int P = decltype(pc)::value, TV = P - NS + VL, LVP = (P + VL) % NS;
        issue_desc(P, pc);
        const __amdgpu_buffer_rsrc_t rk = krsrc(P), rv = vrsrc(TV < 0 ? 0 : TV);
        const int vok = lane * 16 + toff[P];
        const int vov = lane * 16 + (TV < 0 ? kDead : toff[TV < 0 ? 0 : TV % NS]);   // tile < 0: zeros
        static_for<0, NM>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          if constexpr (c & 1) kst[P][c >> 1] = frag_at(rk, vok, c >> 1);
          else vst[LVP][vfrag(c >> 1)] = frag_at(rv, vov, vfrag(c >> 1));
          __builtin_amdgcn_sched_barrier(0);
        });
      });
      c0 = read_row(crow[0]);
      sb[0] = MmaBF16::mma(kst[0][0], qf[0][0], c0);
      static_for<1, NKD>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        sb[0] = MmaBF16::mma(kst[0][f], qf[0][f], sb[0]);
      });
      if (pass == 0) {
        mu[0] = ref_of(sb[0]);
        if constexpr (UPT == 2) {
          f32x16 s1 = MmaBF16::mma(kst[0][0], qf[1][0], c0);
          static_for<1, NKD>([&](auto fc) {
            constexpr int f = decltype(fc)::value;
            s1 = MmaBF16::mma(kst[0][f], qf[1][f], s1);
          });
          mu[1] = ref_of(s1);
        }
      }
      if constexpr (UPT == 1) c0 = read_row(crow[1]);

      // 2 NS steps per iteration so every stage and buffer index is static; the last
      // steps run after the loop (a single loop exit keeps the register assignment
      // simple), then the PV of the last unit.
      const int last = UPT * N;
      int k = 0;
      for (; k + 2 * NS <= last; k += 2 * NS)
        static_for<0, 2 * NS>([&](auto sc) { step(k + decltype(sc)::value, sc); });
      static_for<0, 2 * NS / UPT>([&](auto rc) {
        constexpr int R = decltype(rc)::value * UPT;       // steps left
        if (last - k == R) {
          static_for<0, R>([&](auto sc) { step(k + decltype(sc)::value, sc); });
          finish(ic<(R + 2 * NS - 1) % (2 * NS)>{});
        }
      });
      if (pass > 0) break;
      bool over = false;
#pragma unroll
      for (int qt = 0; qt < UPT; ++qt) {
        const float l = sum_halves(lsum[qt]);
        over |= !(l >= kSumLo && l <= kSumHi);
      }
      if (!__any(over)) break;
      max_pass();
    }
  };
  run();


  // Merge the two key halves. Each lane's sums cover its own 16 keys; both lane halves
  // hold the same reference. Wave kh finalises Oᵀ tiles [kh HE, kh HE + HE) of both query
  // halves and hands the partner's tiles over through LDS.
  {
    float* mine = sX + kh * XS * 64 + lane;
    auto hand_over = [&](auto oc) {
      constexpr int O = decltype(oc)::value;      // first tile the partner finalises
#pragma unroll
      for (int u = 0; u < HE; ++u)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int r = 0; r < 16; ++r) mine[((u * 2 + qt) * 16 + r) * 64] = acc[O + u][qt][r];
    };
    if (kh == 0) hand_over(ic<HE>{});
    else hand_over(ic<0>{});
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      mine[(HE * 32 + qt) * 64] = mu[qt];
      mine[(HE * 32 + 2 + qt) * 64] = lsum[qt];
      mine[(HE * 32 + 4 + qt) * 64] = asum[qt];
    }
  }
  __syncthreads();
  f32x16 res[HE][2];
  float mt[2], lt[2], at[2];
  {
    const float* oth = sX + (1 - kh) * XS * 64 + lane;
    auto combine = [&](auto oc) {
      constexpr int O = decltype(oc)::value;      // first tile this wave finalises
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float mo = oth[(HE * 32 + qt) * 64];
        mt[qt] = fmaxf(mu[qt], mo);
        const float f = fast_exp2(mu[qt] - mt[qt]), fo = fast_exp2(mo - mt[qt]);
#pragma unroll
        for (int u = 0; u < HE; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) res[u][qt][r] = acc[O + u][qt][r] * f + oth[((u * 2 + qt) * 16 + r) * 64] * fo;
        lt[qt] = lsum[qt] * f + oth[(HE * 32 + 2 + qt) * 64] * fo;
        at[qt] = asum[qt] * f + oth[(HE * 32 + 4 + qt) * 64] * fo;
      }
    };
    if (kh == 0) combine(ic<0>{});
    else combine(ic<HE>{});
  }
  if constexpr (VIRT) {
    // Phase 3: Oᵀ += H̄ (A_t q_t)ᵀ for this wave's Oᵀ tiles, H̄[e][c] as the A operand.
    bf16x8 hf[HE][NKD];
#pragma unroll
    for (int u = 0; u < HE; ++u)
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks)
        hf[u][ks] = *reinterpret_cast<const bf16x8*>(hbp + size_t(32 * (kh * HE + u) + l32) * D + 16 * ks + 8 * g);
#pragma unroll
    for (int qt = 0; qt < UPT; ++qt) {
      const float A = sum_halves(at[qt]);
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        bf16x8 b;
#pragma unroll
        for (int u = 0; u < 8; ++u) b[u] = static_cast<__bf16>(static_cast<float>(qf[qt][ks][u]) * A);
#pragma unroll
        for (int u = 0; u < HE; ++u) res[u][qt] = MmaBF16::mma(hf[u][ks], b, res[u][qt]);
      }
    }
  }
  float inv[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float l = sum_halves(lt[qt]);
    inv[qt] = l > 0.f ? 1.f / l : 0.f;
    const int q = 32 * qt + l32;
    if (a.lse && kh == 0 && g == 0)
      a.lse[size_t(h) * a.L + size_t(i) * kB + q] = (q < ni && l > 0.f) ? mt[qt] * kLn2 + logf(l) : NEG_INF;
  }
  __syncthreads();                                  // hand-over buffers consumed
  // Output tile staged in LDS (swizzled rows) for coalesced 16-byte stores.
  char* so = reinterpret_cast<char*>(sX);
#pragma unroll
  for (int u = 0; u < HE; ++u)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int q = 32 * qt + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = 32 * (kh * HE + u) + acc_row(r, g);
        *reinterpret_cast<uint16_t*>(so + KT::offset(q, e * 2)) = f32_to_bf16(q < ni ? res[u][qt][r] * inv[qt] : 0.f);
      }
    }
  __syncthreads();
  char* Oh = reinterpret_cast<char*>(static_cast<uint16_t*>(a.O) + (size_t(h) * a.L + size_t(i) * kB) * D);
  constexpr int OCH = kB * D * 2 / 16;             // 16-byte chunks of the output tile
#pragma unroll
  for (int p = 0; p < OCH / 128; ++p) {
    const int c = threadIdx.x + 128 * p;
    const int row = c / (D * 2 / 16), cb = (c % (D * 2 / 16)) * 16;
    *reinterpret_cast<u32x4*>(Oh + size_t(row) * D * 2 + cb) = *reinterpret_cast<const u32x4*>(so + KT::offset(row, cb));
  }
}

template <int D, int MODE>
static hipError_t launch_frag_m(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.H) * unsigned(a.nb));
  hipLaunchKernelGGL((attention_frag_kernel<D, MODE, 2>), grid, dim3(128), 0, s, a);
  // The tile counts come from the statistics call's tile order on the device, so the
  // short-tile launch always runs; its workgroups leave at once when there are none.
  hipLaunchKernelGGL((attention_frag_kernel<D, MODE, 1>), grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_frag_d(int mode, const AttnArgs& a, hipStream_t s) {
  switch (mode) {
    case MODE_DROP: return launch_frag_m<D, MODE_DROP>(a, s);
    case MODE_PISA: return launch_frag_m<D, MODE_PISA>(a, s);
    default: return launch_frag_m<D, MODE_PWT>(a, s);
  }
}

hipError_t launch_attention_frag(int mode, const AttnArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_frag_d<64>(mode, a, s) : launch_frag_d<128>(mode, a, s);
}

}  // namespace pisa
