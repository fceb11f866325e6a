// C ABI: argument validation, workspace sizing and dispatch onto the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "internal.hpp"
#include "pisa.h"

// Fixed scratch of pisa_block_stats_noalloc: the H̄ partials. Every GPU the library runs
// on holds its own copy for the life of the process; host code uses the per-device
// address from hipGetSymbolAddress (stats_scratch below), never the array's name.
static __device__ __align__(256) char scratch[PISA_STATS_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

pisa_status fail(pisa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pisa_status fail(pisa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

pisa_status ok() {
  g_err.clear();
  return PISA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(pisa_dtype dt) { return dt == PISA_BF16 ? 2 : 4; }

// Shape checks common to every call. Returns PISA_OK or an error with the message set.
pisa_status check_shape(int H, int L, int d, int B) {
  if (H < 1) return fail(PISA_ERR_INVALID_ARG, "H must be >= 1 (got %d)", H);
  if (L < 1) return fail(PISA_ERR_INVALID_ARG, "L must be >= 1 (got %d)", L);
  if (B != pisa::kB) return fail(PISA_ERR_UNSUPPORTED, "only B == 64 is supported (got %d)", B);
  if (L % B) return fail(PISA_ERR_INVALID_ARG, "L (%d) must be a multiple of B (%d)", L, B);
  if (d != 64 && d != 128) return fail(PISA_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  if (L / B > 32768) return fail(PISA_ERR_UNSUPPORTED, "at most 32768 blocks are supported (got %d)", L / B);
  if (static_cast<long long>(H) * (L / B) >= (1LL << 31))
    return fail(PISA_ERR_UNSUPPORTED, "H * nb must fit a 31-bit grid");
  return PISA_OK;
}

pisa_status check_dtype(pisa_dtype dt) {
  if (dt != PISA_F32 && dt != PISA_BF16) return fail(PISA_ERR_UNSUPPORTED, "unknown dtype %d", int(dt));
  return PISA_OK;
}

pisa_status check_ptr(const void* p, const char* name, bool need_align = true) {
  if (!p) return fail(PISA_ERR_INVALID_ARG, "%s must not be NULL", name);
  if (need_align && !aligned16(p)) return fail(PISA_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  return PISA_OK;
}

pisa_status hip_fail(hipError_t e, const char* what) {
  return fail(PISA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define PISA_TRY(x)                  \
  do {                               \
    pisa_status _s = (x);            \
    if (_s != PISA_OK) return _s;    \
  } while (0)

pisa_status select_impl(pisa_dtype dt, const void* Q, const void* Q_pre, const void* K_pre,
                        const float* pos, const pisa_rope* rope, const pisa_stats* st, int H,
                        int L, int d, int B, const int32_t* block_len, int K_sel,
                        unsigned route, float eps, int32_t* idx, uint32_t* mask,
                        float* wt, void* workspace, size_t workspace_bytes, void* stream) {
  PISA_TRY(check_dtype(dt));
  PISA_TRY(check_shape(H, L, d, B));
  if (!rope || wt) PISA_TRY(check_ptr(Q, "Q"));
  PISA_TRY(check_ptr(st, "st", false));
  if (route > PISA_ROUTE_ERROR) return fail(PISA_ERR_INVALID_ARG, "unknown route %u", route);
  if (!rope) PISA_TRY(check_ptr(st->kbar, "st->kbar"));
  // The predicted-error route reads σ² for w̃ whether or not w̃ is written out.
  if (wt || route == PISA_ROUTE_ERROR) PISA_TRY(check_ptr(st->ksig2, "st->ksig2"));
  if (rope) {
    PISA_TRY(check_ptr(Q_pre, "Q_pre"));
    PISA_TRY(check_ptr(K_pre, "K_pre"));
    PISA_TRY(check_ptr(pos, "pos", false));
    if (rope->n_axes < 1 || rope->n_axes > 3)
      return fail(PISA_ERR_INVALID_ARG, "rope->n_axes must be 1, 2 or 3 (got %d)", rope->n_axes);
    int sum = 0;
    for (int x = 0; x < rope->n_axes; ++x) {
      if (rope->width[x] < 2 || rope->width[x] % 2)
        return fail(PISA_ERR_INVALID_ARG, "rope->width[%d] must be even and >= 2 (got %d)", x, rope->width[x]);
      sum += rope->width[x];
    }
    if (sum != d) return fail(PISA_ERR_INVALID_ARG, "rope widths must sum to d = %d (got %d)", d, sum);
    if (!(rope->base > 0.f) || rope->base > 3.0e38f)
      return fail(PISA_ERR_INVALID_ARG, "rope->base must be finite and > 0");
    if (rope->pairs != PISA_ROPE_ADJACENT && rope->pairs != PISA_ROPE_HALF)
      return fail(PISA_ERR_INVALID_ARG, "unknown rope->pairs %d", rope->pairs);
  }
  if (route != PISA_ROUTE_MEAN) {
    PISA_TRY(check_ptr(st->hnorm, "st->hnorm", false));
    if (!(eps > 0.f) || eps > 3.0e38f) return fail(PISA_ERR_INVALID_ARG, "eps must be finite and > 0 (got %g)", double(eps));
  }
  const int nb = L / B;
  if (K_sel < 0 || K_sel > nb) return fail(PISA_ERR_INVALID_ARG, "K_sel must be in [0, %d] (got %d)", nb, K_sel);
  if (K_sel > 0) PISA_TRY(check_ptr(idx, "idx", false));
  const size_t need = pisa_select_workspace_bytes(H, L, d, B);
  if (!workspace || workspace_bytes < need)
    return fail(PISA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(PISA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  pisa::SelectArgs a{};
  a.Q = Q;
  a.kbar = st->kbar;
  a.ksig2 = st->ksig2;
  a.hnorm = route != PISA_ROUTE_MEAN ? st->hnorm : nullptr;
  a.route_eps = eps;
  a.route = int(route);
  if (rope) {
    a.Q_pre = Q_pre;
    a.K_pre = K_pre;
    a.pos = pos;
    a.rope_axes = rope->n_axes;
    a.rope_pairs = rope->pairs;
    for (int x = 0; x < 3; ++x) a.rope_width[x] = x < rope->n_axes ? rope->width[x] : 0;
    a.rope_base = rope->base;
  }
  a.block_len = block_len;
  const pisa::SelectLayout wl = pisa::select_layout(H, nb, d);
  char* ws = static_cast<char*>(workspace);
  a.qbar = reinterpret_cast<float*>(ws + wl.qbar);
  a.qsq = reinterpret_cast<float*>(ws + wl.qsq);
  a.krot = reinterpret_cast<float*>(ws + wl.krot);
  a.wt = wt;
  a.idx = idx;
  a.mask = mask;
  a.stile = reinterpret_cast<float*>(ws + wl.stile);
  if (nb <= pisa::kSmallNb) {
    a.scores = reinterpret_cast<float*>(ws + wl.scores);
  } else {
    a.khl = reinterpret_cast<uint4*>(ws + wl.khl);
    a.shl = reinterpret_cast<uint4*>(ws + wl.shl);
    a.lhist = reinterpret_cast<uint32_t*>(ws + wl.lhist);
    a.lstate = reinterpret_cast<int4*>(ws + wl.lstate);
    a.lcoff = reinterpret_cast<int*>(ws + wl.lcoff);
    a.lcnt = reinterpret_cast<int*>(ws + wl.lcnt);
    a.lcand = reinterpret_cast<uint32_t*>(ws + wl.lcand);
    a.lparam = reinterpret_cast<float4*>(ws + wl.lparam);
    a.lkpart = reinterpret_cast<float4*>(ws + wl.lkpart);
    a.lover = reinterpret_cast<int*>(ws + wl.lover);
    a.lks = wl.lks;
    a.lnkp = wl.lnkp;
    if (!a.mask) a.mask = reinterpret_cast<uint32_t*>(ws + wl.lmask);
  }
  a.H = H;
  a.L = L;
  a.d = d;
  a.nb = nb;
  a.K_sel = K_sel;
  a.nw = (nb + 31) / 32;
  hipError_t e = pisa::launch_select(dt == PISA_BF16, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pisa_select_topk launch");
  return ok();
}

// Checks shared by both statistics entry points.
pisa_status stats_checks(pisa_dtype dt, const void* K, const void* V, int H, int L, int d, int B,
                         unsigned flags, const pisa_stats* out) {
  PISA_TRY(check_dtype(dt));
  PISA_TRY(check_shape(H, L, d, B));
  PISA_TRY(check_ptr(K, "K"));
  PISA_TRY(check_ptr(V, "V"));
  PISA_TRY(check_ptr(out, "out", false));
  if (flags & ~7u) return fail(PISA_ERR_INVALID_ARG, "unknown stats flags 0x%x", flags);
  PISA_TRY(check_ptr(out->kbar, "out->kbar"));
  PISA_TRY(check_ptr(out->vsum, "out->vsum"));
  PISA_TRY(check_ptr(out->ksig2, "out->ksig2"));
  PISA_TRY(check_ptr(out->hbarT, "out->hbarT"));
  PISA_TRY(check_ptr(out->packed, "out->packed"));
  if (flags & PISA_STATS_BLOCK_H) PISA_TRY(check_ptr(out->hblk, "out->hblk"));
  if (flags & PISA_STATS_BLOCK_C) PISA_TRY(check_ptr(out->cblk, "out->cblk"));
  if (flags & PISA_STATS_HNORM) PISA_TRY(check_ptr(out->hnorm, "out->hnorm", false));
  return PISA_OK;
}

pisa_status stats_launch(pisa_dtype dt, const void* K, const void* V, int H, int L, int d,
                         const int32_t* block_len, unsigned flags, const pisa_stats* out,
                         float* part, int G, void* stream) {
  pisa::StatsArgs a{};
  a.K = K;
  a.V = V;
  a.block_len = block_len;
  a.kbar = out->kbar;
  a.vsum = out->vsum;
  a.ksig2 = out->ksig2;
  a.hbarT = out->hbarT;
  a.hblk = out->hblk;
  a.cblk = out->cblk;
  a.hnorm = out->hnorm;
  a.packed = static_cast<char*>(out->packed);
  a.part = part;
  a.H = H;
  a.L = L;
  a.d = d;
  a.pl = pisa::packed_layout(elem_size(dt), H, L, d);
  a.nb = a.pl.nb;
  a.nbp = a.pl.nbp;
  a.G = G;
  a.ngroups = (a.nb + a.G - 1) / a.G;
  hipError_t e = pisa::launch_block_stats(dt == PISA_BF16, a, flags, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pisa_block_stats launch");
  return ok();
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, looked up once per device with that device current.
pisa_status stats_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PISA_ERR_UNSUPPORTED, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<float*>(g_scratch_ptr[dev]);
  return PISA_OK;
}

}  // namespace

extern "C" {

size_t pisa_packed_bytes(pisa_dtype dt, int H, int L, int d, int B) {
  if (check_dtype(dt) != PISA_OK || check_shape(H, L, d, B) != PISA_OK) return 0;
  return pisa::packed_layout(elem_size(dt), H, L, d).total;
}

size_t pisa_block_stats_workspace_bytes(int H, int L, int d, int B) {
  if (check_shape(H, L, d, B) != PISA_OK) return 0;
  const int nb = L / B;
  const int G = pisa::stats_group(H, nb);
  const int ng = (nb + G - 1) / G;
  return size_t(H) * ng * d * d * sizeof(float);
}

pisa_status pisa_block_stats(pisa_dtype dt, const void* K, const void* V, int H, int L, int d,
                             int B, const int32_t* block_len, unsigned flags,
                             const pisa_stats* out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  PISA_TRY(stats_checks(dt, K, V, H, L, d, B, flags, out));
  const size_t need = pisa_block_stats_workspace_bytes(H, L, d, B);
  if (!workspace || workspace_bytes < need)
    return fail(PISA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(PISA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return stats_launch(dt, K, V, H, L, d, block_len, flags, out, static_cast<float*>(workspace),
                      pisa::stats_group(H, L / B), stream);
}

pisa_status pisa_block_stats_noalloc(pisa_dtype dt, const void* K, const void* V, int H, int L,
                                     int d, int B, const int32_t* block_len, unsigned flags,
                                     const pisa_stats* out, void* stream) {
  PISA_TRY(stats_checks(dt, K, V, H, L, d, B, flags, out));
  // One d x d fp32 partial of H̄ per (head, group of G blocks). The default grouping is
  // kept when its partials fit the scratch; otherwise G grows until they do.
  const size_t per = size_t(d) * d * sizeof(float);
  const size_t fit = PISA_STATS_SCRATCH_BYTES / (per * size_t(H));    // groups per head that fit
  if (fit < 1)
    return fail(PISA_ERR_WORKSPACE, "pisa_block_stats_noalloc: H = %d heads of d = %d need %zu scratch bytes "
                "(the fixed scratch holds %zu)", H, d, per * size_t(H), size_t(PISA_STATS_SCRATCH_BYTES));
  const int nb = L / B;
  int G = pisa::stats_group(H, nb);
  if (size_t((nb + G - 1) / G) > fit) G = int((size_t(nb) + fit - 1) / fit);
  float* part = nullptr;
  PISA_TRY(stats_scratch(&part));
  return stats_launch(dt, K, V, H, L, d, block_len, flags, out, part, G, stream);
}

size_t pisa_select_workspace_bytes(int H, int L, int d, int B) {
  if (check_shape(H, L, d, B) != PISA_OK) return 0;
  return pisa::select_layout(H, L / B, d).total;
}

pisa_status pisa_select_topk_routed(pisa_dtype dt, const void* Q, const pisa_stats* st, int H,
                                    int L, int d, int B, const int32_t* block_len, int K_sel,
                                    unsigned route, float eps, int32_t* idx, uint32_t* mask,
                                    float* wt, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return select_impl(dt, Q, nullptr, nullptr, nullptr, nullptr, st, H, L, d, B, block_len, K_sel,
                     route, eps, idx, mask, wt, workspace, workspace_bytes, stream);
}

pisa_status pisa_select_topk_rope(pisa_dtype dt, const void* Q, const void* Q_pre, const void* K_pre,
                                  const float* pos, const pisa_rope* rope, const pisa_stats* st,
                                  int H, int L, int d, int B, const int32_t* block_len, int K_sel,
                                  int32_t* idx, uint32_t* mask, float* wt, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  PISA_TRY(check_ptr(rope, "rope", false));
  return select_impl(dt, Q, Q_pre, K_pre, pos, rope, st, H, L, d, B, block_len, K_sel,
                     PISA_ROUTE_MEAN, 1.f, idx, mask, wt, workspace, workspace_bytes, stream);
}

pisa_status pisa_select_topk(pisa_dtype dt, const void* Q, const pisa_stats* st, int H, int L,
                             int d, int B, const int32_t* block_len, int K_sel, int32_t* idx,
                             uint32_t* mask, float* wt, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return pisa_select_topk_routed(dt, Q, st, H, L, d, B, block_len, K_sel, PISA_ROUTE_MEAN, 1.f, idx,
                                 mask, wt, workspace, workspace_bytes, stream);
}

pisa_status pisa_attention_fwd(pisa_dtype dt, const void* Q, const void* K, const void* V,
                               const pisa_stats* st, const int32_t* idx, const uint32_t* mask,
                               const float* wt, int H, int L, int d, int B,
                               const int32_t* block_len, int K_sel, unsigned mode, void* O,
                               float* lse, void* stream) {
  PISA_TRY(check_dtype(dt));
  PISA_TRY(check_shape(H, L, d, B));
  PISA_TRY(check_ptr(Q, "Q"));
  PISA_TRY(check_ptr(K, "K"));
  PISA_TRY(check_ptr(V, "V"));
  PISA_TRY(check_ptr(O, "O"));
  PISA_TRY(check_ptr(st, "st", false));
  PISA_TRY(check_ptr(st->packed, "st->packed"));
  const int nb = L / B;
  if (K_sel < 0 || K_sel > nb) return fail(PISA_ERR_INVALID_ARG, "K_sel must be in [0, %d] (got %d)", nb, K_sel);
  if (K_sel > 0) PISA_TRY(check_ptr(idx, "idx", false));
  const unsigned base = mode & 15u;
  if (base > PISA_MODE_PWT_ROW) return fail(PISA_ERR_INVALID_ARG, "unknown mode %u", base);
  if (mode & ~(15u | PISA_W_LINEAR | PISA_W_EXP | PISA_W_NOGATE))
    return fail(PISA_ERR_INVALID_ARG, "unknown mode bits 0x%x", mode);
  if ((mode & PISA_W_LINEAR) && (mode & PISA_W_EXP))
    return fail(PISA_ERR_INVALID_ARG, "PISA_W_LINEAR and PISA_W_EXP are exclusive");
  if (base != PISA_MODE_DROP) PISA_TRY(check_ptr(mask, "mask", false));
  if (base == PISA_MODE_PWT) PISA_TRY(check_ptr(wt, "wt", false));
  if (base == PISA_MODE_PWT_ROW) PISA_TRY(check_ptr(st->ksig2, "st->ksig2", false));

  pisa::AttnArgs a{};
  a.Q = Q;
  a.K = K;
  a.packed = static_cast<const char*>(st->packed);
  a.block_len = block_len;
  a.idx = idx;
  a.mask = mask;
  a.wt = wt;
  a.ksig2 = st->ksig2;
  a.O = O;
  a.lse = lse;
  a.H = H;
  a.L = L;
  a.d = d;
  a.pl = pisa::packed_layout(elem_size(dt), H, L, d);
  a.nb = a.pl.nb;
  a.nbp = a.pl.nbp;
  a.K_sel = K_sel;
  a.nw = (nb + 31) / 32;
  a.w_linear = base == PISA_MODE_LITERAL ? !(mode & PISA_W_EXP) : !!(mode & PISA_W_LINEAR);
  a.gate = !(mode & PISA_W_NOGATE);
  (void)V;  // V enters through its per-block transpose in st->packed
  hipError_t e = pisa::launch_attention(dt == PISA_BF16, int(base), a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pisa_attention_fwd launch");
  return ok();
}

size_t pisa_attention_bwd_workspace_bytes(pisa_dtype dt, int H, int L, int d, int B, int K_sel) {
  if (check_dtype(dt) != PISA_OK || check_shape(H, L, d, B) != PISA_OK || K_sel < 0 || K_sel > L / B) return 0;
  return pisa::bwd_layout(elem_size(dt), H, L, d, K_sel).total;
}

pisa_status pisa_attention_bwd(pisa_dtype dt, const void* Q, const void* K, const void* V,
                               const pisa_stats* st, const int32_t* idx, const uint32_t* mask,
                               const float* wt, int H, int L, int d, int B,
                               const int32_t* block_len, int K_sel, unsigned mode, const float* lse,
                               const void* O, const void* dO, float* dQ, float* dK, float* dV,
                               void* workspace, size_t workspace_bytes, void* stream) {
  PISA_TRY(check_dtype(dt));
  PISA_TRY(check_shape(H, L, d, B));
  PISA_TRY(check_ptr(Q, "Q"));
  PISA_TRY(check_ptr(K, "K"));
  PISA_TRY(check_ptr(V, "V"));
  PISA_TRY(check_ptr(dO, "dO"));
  if (O) PISA_TRY(check_ptr(O, "O"));
  PISA_TRY(check_ptr(lse, "lse", false));
  PISA_TRY(check_ptr(dQ, "dQ"));
  PISA_TRY(check_ptr(dK, "dK"));
  PISA_TRY(check_ptr(dV, "dV"));
  PISA_TRY(check_ptr(st, "st", false));
  PISA_TRY(check_ptr(st->kbar, "st->kbar"));
  PISA_TRY(check_ptr(st->vsum, "st->vsum"));
  PISA_TRY(check_ptr(st->ksig2, "st->ksig2"));
  PISA_TRY(check_ptr(st->hbarT, "st->hbarT"));
  PISA_TRY(check_ptr(mask, "mask", false));
  const int nb = L / B;
  if (K_sel < 0 || K_sel > nb) return fail(PISA_ERR_INVALID_ARG, "K_sel must be in [0, %d] (got %d)", nb, K_sel);
  if (K_sel > 0) PISA_TRY(check_ptr(idx, "idx", false));
  const unsigned base = mode & 15u;
  if (base > PISA_MODE_PWT_ROW) return fail(PISA_ERR_INVALID_ARG, "unknown mode %u", base);
  if ((base == PISA_MODE_LITERAL || base == PISA_MODE_PWT_ROW) && dt != PISA_BF16)
    return fail(PISA_ERR_UNSUPPORTED, "the LITERAL and PWT_ROW backward takes bf16 inputs");
  if (mode & ~(15u | PISA_W_LINEAR | PISA_W_EXP | PISA_W_NOGATE))
    return fail(PISA_ERR_INVALID_ARG, "unknown mode bits 0x%x", mode);
  if ((mode & PISA_W_LINEAR) && (mode & PISA_W_EXP))
    return fail(PISA_ERR_INVALID_ARG, "PISA_W_LINEAR and PISA_W_EXP are exclusive");
  if (base == PISA_MODE_PWT) PISA_TRY(check_ptr(wt, "wt", false));
  const pisa::BwdLayout w = pisa::bwd_layout(elem_size(dt), H, L, d, K_sel);
  if (!workspace || workspace_bytes < w.total)
    return fail(PISA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", w.total, workspace_bytes);
  if (!aligned16(workspace)) return fail(PISA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  char* ws = static_cast<char*>(workspace);
  pisa::BwdArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.dO = dO;
  a.O = O;
  a.lse = lse;
  a.block_len = block_len;
  a.idx = idx;
  a.mask = mask;
  a.wt = wt;
  a.kbar = st->kbar;
  a.vsum = st->vsum;
  a.ksig2 = st->ksig2;
  a.hbarT = st->hbarT;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.delta = reinterpret_cast<float*>(ws + w.delta);
  a.gu = reinterpret_cast<float*>(ws + w.gu);
  a.abar = reinterpret_cast<float*>(ws + w.abar);
  a.qsq = base == PISA_MODE_PWT ? reinterpret_cast<float*>(ws + w.qsq) : nullptr;
  // LITERAL / PWT_ROW take the pooled-q² region (H nb d >= H L floats) for the renormalised lse
  a.lse2 = base == PISA_MODE_LITERAL || base == PISA_MODE_PWT_ROW ? reinterpret_cast<float*>(ws + w.qsq) : nullptr;
  a.dwt = reinterpret_cast<float*>(ws + w.dwt);
  a.dsig2 = reinterpret_cast<float*>(ws + w.dsig2);
  a.dqsq = reinterpret_cast<float*>(ws + w.dqsq);
  a.dkbar_part = reinterpret_cast<float*>(ws + w.dkp);
  a.dvbar_part = reinterpret_cast<float*>(ws + w.dvp);
  a.dh_part = reinterpret_cast<float*>(ws + w.dhp);
  a.dh = reinterpret_cast<float*>(ws + w.dh);
  a.csr_off = reinterpret_cast<int*>(ws + w.off);
  a.csr_list = reinterpret_cast<int*>(ws + w.list);
  a.kt = ws + w.kt;
  a.kbr = ws + w.kbr;
  a.kbt = ws + w.kbt;
  a.vbr = ws + w.vbr;
  a.qt = ws + w.qt;
  a.gt = ws + w.gt;
  a.vbias = reinterpret_cast<float*>(ws + w.vbias);
  a.vdphi = reinterpret_cast<float*>(ws + w.vdphi);
  a.vinvn = reinterpret_cast<float*>(ws + w.vinvn);
  a.H = H;
  a.L = L;
  a.d = d;
  a.nb = nb;
  a.nbp = (nb + B - 1) / B * B;
  a.K_sel = K_sel;
  a.nw = (nb + 31) / 32;
  a.nchunk = w.nchunk;
  a.nhch = w.nhch;
  a.w_linear = base == PISA_MODE_LITERAL ? !(mode & PISA_W_EXP) : !!(mode & PISA_W_LINEAR);
  a.gate = !(mode & PISA_W_NOGATE);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = base == PISA_MODE_LITERAL   ? pisa::launch_literal_bwd(a, hs)
                 : base == PISA_MODE_PWT_ROW ? pisa::launch_rowdiag_bwd(a, hs)
                                             : pisa::launch_attention_bwd(dt == PISA_BF16, int(base), a, hs);
  if (e != hipSuccess) return hip_fail(e, "pisa_attention_bwd launch");
  return ok();
}

pisa_status pisa_cube_layout(int T, int Hh, int W, int ct, int ch, int cw, int32_t* perm,
                             int32_t* block_len, size_t capacity, int* nb_out) {
  if (T < 1 || Hh < 1 || W < 1 || ct < 1 || ch < 1 || cw < 1)
    return fail(PISA_ERR_INVALID_ARG, "grid and cube sizes must be >= 1");
  if (ct * ch * cw != pisa::kB) return fail(PISA_ERR_UNSUPPORTED, "cube must hold B = 64 tokens (got %d)", ct * ch * cw);
  if (!perm || !block_len || !nb_out) return fail(PISA_ERR_INVALID_ARG, "perm, block_len and nb_out must not be NULL");
  const long long nt = (T + ct - 1) / ct, nh = (Hh + ch - 1) / ch, nw = (W + cw - 1) / cw;
  const long long nb = nt * nh * nw;
  if (static_cast<long long>(T) * Hh * W >= (1LL << 31) || nb > 32768)
    return fail(PISA_ERR_UNSUPPORTED, "grid too large (%lld blocks)", nb);
  if (static_cast<size_t>(nb) * pisa::kB > capacity)
    return fail(PISA_ERR_INVALID_ARG, "perm needs %lld entries (capacity %zu)", nb * pisa::kB, capacity);
  long long j = 0;
  for (long long a = 0; a < nt; ++a)
    for (long long b = 0; b < nh; ++b)
      for (long long c = 0; c < nw; ++c, ++j) {
        int n = 0;
        int32_t* slot = perm + j * pisa::kB;
        for (int dt = 0; dt < ct; ++dt)
          for (int dh = 0; dh < ch; ++dh)
            for (int dw = 0; dw < cw; ++dw) {
              const long long t = a * ct + dt, h = b * ch + dh, w = c * cw + dw;
              if (t < T && h < Hh && w < W) slot[n++] = static_cast<int32_t>((t * Hh + h) * W + w);
            }
        block_len[j] = n;
        for (int k = n; k < pisa::kB; ++k) slot[k] = -1;
      }
  *nb_out = static_cast<int>(nb);
  return ok();
}

static pisa_status layout_call(bool to_blocks, pisa_dtype dt, const void* src, int H, int L_nat, int L_pad,
                               int d, const int32_t* perm, void* dst, void* stream) {
  PISA_TRY(check_dtype(dt));
  if (H < 1 || L_nat < 1 || L_pad < 1 || d < 1) return fail(PISA_ERR_INVALID_ARG, "H, L_nat, L_pad and d must be >= 1");
  const int row_bytes = d * static_cast<int>(elem_size(dt));
  if (row_bytes % 16) return fail(PISA_ERR_UNSUPPORTED, "a row must be a multiple of 16 bytes (d = %d)", d);
  if (static_cast<long long>(H) * L_pad >= (1LL << 31) || static_cast<long long>(L_pad) * (row_bytes / 16) >= (1LL << 40))
    return fail(PISA_ERR_UNSUPPORTED, "sizes too large");
  PISA_TRY(check_ptr(src, "src"));
  PISA_TRY(check_ptr(dst, "dst"));
  PISA_TRY(check_ptr(perm, "perm", false));
  hipError_t e = pisa::launch_layout(to_blocks, src, dst, perm, H, L_nat, L_pad, row_bytes,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "layout launch");
  return ok();
}

pisa_status pisa_layout_to_blocks(pisa_dtype dt, const void* src, int H, int L_nat, int L_pad, int d,
                                  const int32_t* perm, void* dst, void* stream) {
  return layout_call(true, dt, src, H, L_nat, L_pad, d, perm, dst, stream);
}

pisa_status pisa_layout_from_blocks(pisa_dtype dt, const void* src, int H, int L_nat, int L_pad,
                                    int d, const int32_t* perm, void* dst, void* stream) {
  return layout_call(false, dt, src, H, L_nat, L_pad, d, perm, dst, stream);
}

const char* pisa_last_error(void) { return g_err.c_str(); }

const char* pisa_version(void) { return "pisa-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
