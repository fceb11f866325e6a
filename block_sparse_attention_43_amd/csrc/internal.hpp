// Host-side interface between the C ABI (abi.hip) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pisa {

constexpr int kB = 64;  // block / tile size handled by the kernels

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Byte offsets inside the packed (kernel-layout) statistics buffer. Every region but
// H̄ is a sequence of 64-key tiles of 64 * d elements; the element order inside a tile
// is TileLayout<T, d> (common.hpp): plain K rows / Vᵀ rows for fp32, MFMA operand order
// for bf16. The bf16 layout also carries an operand-order copy of K per block.
struct PackedLayout {
  size_t kf, vt, kbar, vbar, hbar, tiles, total;
  int nb, nbp;
};

inline PackedLayout packed_layout(size_t elem, int H, int L, int d) {
  PackedLayout p;
  p.nb = L / kB;
  p.nbp = (p.nb + kB - 1) / kB * kB;
  const size_t tile = size_t(kB) * d * elem;
  size_t o = 0;
  p.kf = o;   o = align256(o + (elem == 2 ? size_t(H) * p.nb * tile : 0));  // [H][nb] K tiles (bf16)
  p.vt = o;   o = align256(o + size_t(H) * p.nb * tile);                    // [H][nb] Vᵀ tiles
  p.kbar = o; o = align256(o + size_t(H) * (p.nbp / kB) * tile);            // [H][nbp/64] centroid tiles
  p.vbar = o; o = align256(o + size_t(H) * (p.nbp / kB) * tile);            // [H][nbp/64] (ΣV/n)ᵀ tiles
  p.hbar = o; o = align256(o + size_t(H) * d * d * elem);                   // [H][d][d]   H̄[e][c]
  p.tiles = o; o = align256(o + (2 + size_t(p.nb)) * 4);                    // query-tile order
  p.total = o;
  return p;
}

// Blocks reduced per workgroup in the statistics kernel (sets its workspace size).
inline int stats_group(int H, int nb) {
  long long g = (static_cast<long long>(H) * nb + 1023) / 1024;
  if (g < 1) g = 1;
  if (g > 64) g = 64;
  return static_cast<int>(g);
}

struct StatsArgs {
  const void* K;
  const void* V;
  const int32_t* block_len;
  float* kbar;
  float* vsum;
  float* ksig2;
  float* hbarT;
  float* hblk;
  float* cblk;
  float* hnorm;    // [H][nb] or null
  char* packed;
  float* part;     // [H][ngroups][d][d]
  int H, L, d, nb, nbp, G, ngroups;
  PackedLayout pl;
};

struct SelectArgs {
  const void* Q;
  const float* kbar;
  const float* ksig2;
  const float* hnorm;  // [H][nb] M_j (routes 1, 2)
  float route_eps;
  int route;           // 0 block mean, 1 + ln(M_j + eps), 2 + w̃ + ln n_j + ln(M_j + eps)
  // RoPE-aware centroids (rope_axes > 0): pre-rotation Q and K pooled per block and turned
  // at the block centre; the turned key centroids go to krot (workspace), queries to qbar.
  const void* Q_pre;
  const void* K_pre;
  const float* pos;    // [L][rope_axes]
  float* krot;         // [H][nb][d] workspace
  int rope_axes, rope_pairs;
  int rope_width[3];
  float rope_base;
  const int32_t* block_len;
  float* qbar;     // [H][nb][d]   workspace
  float* qsq;      // [H][nb][d]   workspace
  float* scores;   // [H][nb][nb]  workspace (nb <= kSmallNb only)
  float* wt;       // [H][nb][nb]  or null
  int32_t* idx;    // [H][nb][K_sel]
  uint32_t* mask;  // [H][nb][nw]  or null (the caller's, else workspace for nb > kSmallNb)
  int H, L, d, nb, K_sel, nw;
  // nb > kSmallNb: histogram-threshold selection without the score matrix (workspace)
  uint32_t* lhist;  // [H][nb][lks][kLBins / 2] per key split, bin counts as u16 pairs
  int4* lstate;     // [H][nb] threshold bin b*, -, list length, sent to the fallback
  int* lcoff;       // [H][nb][lks] first list slot of each key split's slice
  int* lcnt;        // [H][nb][lks] near scores each key split found
  uint32_t* lcand;  // [H][nb][kLCap] near block indices (ascending within the list)
  float4* lparam;   // [H][nb] bin origin, bin scale, margin 2ε per row
  float4* lkpart;   // [H][lnkp] max |k̄_j|, min and max key bias, max σ²_{j,c} per 256 blocks
  int* lover;       // [1 + H nb] rows for the fallback: count, rows
  int lks, lnkp;
  // bf16 hi / lo operands of the approximate score products (select_large.hip): 16-byte
  // unit ((h·tiles + t)·2 + part)·(d/16)·64 + u·64 + lane = part of row 32 t + lane % 32,
  // columns (lane / 32)·d/2 + 8u .. + 7, so each 16-byte load of a wave reads 1 KB.
  uint4* khl;       // k̄ (or the turned key centroids)
  uint4* shl;       // σ² (predicted-error route)
  // fp32 σ² rows in the tiled order of the w̃ products (tile_rows in select_topk.hip):
  // float4 ((h·tiles + t)·(d/8) + u)·64 + lane = row 32 t + lane % 32, columns
  // (lane / 32)·d/2 + 4u .. + 3.
  float* stile;
};

// Selection over many key blocks: rows of at most kSmallNb blocks keep the whole score
// row in registers; longer rows go through a linear-bin histogram of the recomputed scores.
constexpr int kSmallNb = 2048;
constexpr int kLBins = 256;   // linear bins per row
constexpr int kLCap = 1024;   // list slots per row (scores near the threshold bin)
constexpr int kMaxKs = 16;    // key splits of the score passes, at most
constexpr int kLRows = 128;   // query tiles per workgroup of the score passes
constexpr int kMaxNb = 32768; // longest row the selection handles (128 KB of fp32 in LDS)

struct SelectLayout {
  size_t qbar, qsq, krot, stile, khl, shl, scores, lhist, lstate, lcoff, lcnt, lcand, lparam, lkpart, lover, lmask,
      total;
  int lks, lnkp;
};

inline SelectLayout select_layout(int H, int nb, int d) {
  SelectLayout w{};
  const size_t Hs = size_t(H), f = sizeof(float), hnd = Hs * nb * d * f;
  const size_t tiled = Hs * ((size_t(nb) + 31) / 32) * 32 * d * f;
  size_t o = 0;
  w.qbar = o; o += hnd;
  w.qsq = o;  o += hnd;
  w.krot = o; o = align256(o + hnd);
  w.stile = o; o = align256(o + tiled);
  if (nb <= kSmallNb) {
    w.scores = o; o = align256(o + Hs * nb * nb * f);
    w.total = o;
    return w;
  }
  const int nrg = (nb + kLRows - 1) / kLRows, tiles = (nb + 31) / 32;
  int ks = 1;
  while (ks < kMaxKs && static_cast<long long>(nrg) * H * ks < 2048 && tiles / (2 * ks) >= 4) ks *= 2;
  w.lks = ks;
  w.lnkp = (nb + 255) / 256;
  const size_t nw = size_t(tiles);
  w.khl = o;    o = align256(o + tiled);
  w.shl = o;    o = align256(o + tiled);
  w.lhist = o;  o = align256(o + Hs * nb * ks * (kLBins / 2) * 4);
  w.lstate = o; o = align256(o + Hs * nb * 16);
  w.lcoff = o;  o = align256(o + Hs * nb * ks * 4);
  w.lcnt = o;   o = align256(o + Hs * nb * ks * 4);
  w.lcand = o;  o = align256(o + Hs * nb * kLCap * 4);
  w.lparam = o; o = align256(o + Hs * nb * 16);
  w.lkpart = o; o = align256(o + Hs * w.lnkp * 16);
  w.lover = o;  o = align256(o + (1 + Hs * nb) * 4);
  w.lmask = o;  o = align256(o + Hs * nb * nw * 4);
  w.total = o;
  return w;
}

struct AttnArgs {
  const void* Q;
  const void* K;
  const char* packed;
  const int32_t* block_len;
  const int32_t* idx;
  const uint32_t* mask;
  const float* wt;
  const float* ksig2;  // [H][nb][d] σ²_j (per-row diagonal w only)
  void* O;
  float* lse;
  int H, L, d, nb, nbp, K_sel, nw;
  int w_linear;    // phi(w) = ln(1 + w) instead of w
  int gate;        // zero w when w > ln n_j
  int merge;       // O, lse already hold another pass over other keys: combine with it
  PackedLayout pl;
};

// Backward of the attention call (DROP / PISA / PWT); workspace regions as laid out by
// bwd_layout below.
struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* dO;
  const void* O;     // [H][L][d] the forward output, or null (Δ then formed in the dQ sweep)
  const float* lse;
  const int32_t* block_len;
  const int32_t* idx;
  const uint32_t* mask;
  const float* wt;
  const float* kbar;
  const float* vsum;
  const float* ksig2;
  const float* hbarT;
  float* dQ;
  float* dK;
  float* dV;
  float* delta;      // [H][L]   Δ_t = dO_t·o_t: dO·O from O, else formed as Σ P dP
  float* lse2;       // [H][L]   LITERAL / PWT_ROW: lse + ln Σ P (the sweeps' P then sum to 1)
  float* gu;         // [H][L]   dO·(H̄ q)
  float* abar;       // [H][L]   Ā_t
  float* qsq;        // [H][nb][d] pooled q² (PWT) or null
  float* dwt;        // [H][nb][nb] dw̃ (PWT)
  float* dsig2;      // [H][nb][d]
  float* dqsq;       // [H][nb][d] ½ Σ_j dw̃_{i,j} σ²_j (PWT)
  float* dkbar_part; // [H][nchunk][nbp][d]
  float* dvbar_part; // [H][nchunk][nbp][d]
  float* dh_part;    // [H][nhch][d][d]
  float* dh;         // [H][d][d]
  int* csr_off;      // [H][nb + 1]
  int* csr_list;     // [H][nb * K_sel]
  // Operand tiles of the dQ sweep in the input type (written by bwd_pack_kernel), 64 x d or
  // d x 64 row-major, zeros past the valid rows: [H][nb] block tiles, [H][nbp/64] groups
  char* kt;          // Kᵀ of each key block
  char* kbr;         // k̄ rows of each centroid group
  char* kbt;         // k̄ᵀ of each centroid group
  char* vbr;         // v̄ = ΣV / n rows of each centroid group
  char* qt;          // Qᵀ of each query tile
  char* gt;          // dOᵀ of each query tile
  float* vbias;      // [H][nb][nbp] log2-domain bias of each virtual token (-inf: excluded)
  float* vdphi;      // [H][nb][nbp] φ'(w̃) of each virtual token (0: excluded or gated)
  float* vinvn;      // [nbp] 1 / n_j (0 past nb)
  int H, L, d, nb, nbp, K_sel, nw, nchunk, nhch;
  int w_linear, gate;
  int delta_final;   // Δ in delta is final (taken over every term of the row): the exact dQ
                     // sweep given O uses it as is, with no ε correction and no write-back
};

struct BwdLayout {
  size_t delta, gu, abar, qsq, dwt, dsig2, dqsq, dkp, dvp, dhp, dh, off, list;
  size_t kt, kbr, kbt, vbr, qt, gt, vbias, vdphi, vinvn, total;
  int nchunk, nhch;
};

inline BwdLayout bwd_layout(size_t elem, int H, int L, int d, int K_sel) {
  BwdLayout w;
  const int nb = L / kB, nbp = (nb + kB - 1) / kB * kB, ngrp = nbp / kB;
  long long c = (1024 + static_cast<long long>(H) * ngrp - 1) / (static_cast<long long>(H) * ngrp);
  w.nchunk = static_cast<int>(c < 1 ? 1 : (c > nb ? nb : c));
  long long e = (512 + H - 1) / H;
  w.nhch = static_cast<int>(e < 1 ? 1 : (e > nb ? nb : e));
  const size_t f = sizeof(float), Hs = size_t(H);
  size_t o = 0;
  w.delta = o; o = align256(o + Hs * L * f);
  w.gu = o;    o = align256(o + Hs * L * f);
  w.abar = o;  o = align256(o + Hs * L * f);
  w.qsq = o;   o = align256(o + Hs * nb * d * f);
  w.dwt = o;   o = align256(o + Hs * nb * nb * f);
  w.dsig2 = o; o = align256(o + Hs * nb * d * f);
  w.dqsq = o;  o = align256(o + Hs * nb * d * f);
  w.dkp = o;   o = align256(o + Hs * w.nchunk * nbp * d * f);
  w.dvp = o;   o = align256(o + Hs * w.nchunk * nbp * d * f);
  w.dhp = o;   o = align256(o + Hs * w.nhch * d * d * f);
  w.dh = o;    o = align256(o + Hs * d * d * f);
  w.off = o;   o = align256(o + Hs * (nb + 1) * sizeof(int));
  w.list = o;  o = align256(o + Hs * nb * size_t(K_sel > 0 ? K_sel : 1) * sizeof(int));
  const size_t tiles = Hs * nb * kB * d * elem, groups = Hs * (nbp / kB) * kB * d * elem;
  w.kt = o;    o = align256(o + tiles);
  w.kbr = o;   o = align256(o + groups);
  w.kbt = o;   o = align256(o + groups);
  w.vbr = o;   o = align256(o + groups);
  w.qt = o;    o = align256(o + tiles);
  w.gt = o;    o = align256(o + tiles);
  w.vbias = o; o = align256(o + Hs * nb * nbp * f);
  w.vdphi = o; o = align256(o + Hs * nb * nbp * f);
  w.vinvn = o; o = align256(o + size_t(nbp) * f);
  w.total = o;
  return w;
}

hipError_t launch_block_stats(int bf16, const StatsArgs& a, unsigned flags, hipStream_t s);
hipError_t launch_layout(bool to_blocks, const void* src, void* dst, const int32_t* perm, int H, int L_nat,
                         int L_pad, int row_bytes, hipStream_t s);
hipError_t launch_attention_bwd(int bf16, int mode, const BwdArgs& a, hipStream_t s);
// bf16 LITERAL backward: Δ, dQ and dK / dV sweeps over every (query tile, key block) pair
// (attention_bwd_literal.hip); reads Q, K, V, dO, lse, mask, block_len; writes delta, dQ,
// dK, dV.
hipError_t launch_literal_bwd(const BwdArgs& a, hipStream_t s);
// bf16 PWT_ROW backward (attention_bwd_literal.hip), and the pieces of attention_bwd.hip it
// shares: gu = dO·(H̄ q) per row; dH̄ from Ā, then the statistics' gradients onto the tokens.
hipError_t launch_rowdiag_bwd(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_rows(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_stats_tail(const BwdArgs& a, hipStream_t s);
// The PWT backward's exact sweeps (DROP instances, bf16) with a.delta final and a.lse the
// row normaliser: dQ of the selected keys, then the key-block lists and dK, dV of the
// selected keys.
hipError_t launch_bwd_exact_sweeps(const BwdArgs& a, hipStream_t s);
hipError_t launch_select(int bf16, const SelectArgs& a, hipStream_t s);
hipError_t launch_select_large(const SelectArgs& a, hipStream_t s);
hipError_t launch_pooled_w(const SelectArgs& a, hipStream_t s);
// bf16 LITERAL, second pass: the unselected blocks in block-wise form, merged into the
// O / lse of a DROP pass over the selected blocks (attention_literal.hip).
hipError_t launch_literal_rest(const AttnArgs& a, hipStream_t s);
hipError_t launch_tile_rows(const float* src, float* dst, int H, int nb, int d, hipStream_t s);
hipError_t launch_attention(int bf16, int mode, const AttnArgs& a, hipStream_t s);

}  // namespace pisa
