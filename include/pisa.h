/*
 * pisa.h — C ABI of the piecewise (exact-or-approximate) block-sparse attention
 * library for AMD Instinct MI355X (gfx950).
 *
 * The method (PISA paper "PISA: Piecewise Sparse Attention Is Wiser for Efficient
 * Diffusion Transformers", §3.2 Formulation Eq. (3.2), §3.3 Hybrid Approximation,
 * §3.4 Hardware-aware Kernel Implementation and Fig. 3; blog "Sparse Linear Attention",
 * sections "Sparse Linear Attention" and "Going Further: Adding the Second-Order Term
 * (PWT)"): keys are cut into blocks of B tokens; each query tile of B rows attends
 * exactly to its K_sel best-scoring key blocks, and every other block enters the same
 * softmax as one Taylor "virtual token" built from the block's statistics.
 *
 * Three stream-ordered calls make one forward pass:
 *   pisa_block_stats    prepare phase: per-block statistics of K and V
 *   pisa_select_topk    prepare phase: pooled-query scores, second-order matrix, top-K
 *   pisa_attention_fwd  fused kernel: exact phase, virtual-token phase, first-order phase
 *
 * Conventions shared by every call
 *   Layout     Q, K, V, O are contiguous row-major [H][L][d] (d fastest); a batch is
 *              folded into H. L is the padded length, a multiple of B. Q, K, V share one
 *              block partition (non-causal self-attention; the PISA paper's appendix on
 *              sparse attention for DiTs covers the bidirectional case only).
 *   Scale      Q already carries the 1/sqrt(d) factor (the pages absorb it into q).
 *   Blocks     block_len is a DEVICE int32[nb] (nb = L / B), shared by all heads, or NULL
 *              when every block is full. Block j's n_j valid tokens occupy its first n_j
 *              slots; values are clamped to [1, B] by the kernels. Padded slots may hold
 *              any finite values: they are masked. Padded query rows produce O = 0 and
 *              lse = -inf.
 *   Supported  B == 64, d in {64, 128}, 1 <= nb <= 32768, dtype PISA_F32 or PISA_BF16
 *              (bfloat16 storage; fp32 accumulation everywhere). Every tensor pointer
 *              must be 16-byte aligned.
 *   Ownership  The caller allocates every buffer (device memory), including the
 *              workspaces, and keeps them alive until the stream work completes. The
 *              library allocates nothing and keeps no state besides the thread-local
 *              error string.
 *   Streams    `stream` is a hipStream_t passed as void* (NULL = default stream). Every
 *              call only enqueues work and returns.
 *   Errors     Argument errors return synchronously, with a message from
 *              pisa_last_error() and nothing enqueued. Unsupported shapes or dtypes give
 *              PISA_ERR_UNSUPPORTED, a short workspace PISA_ERR_WORKSPACE, a failed launch
 *              PISA_ERR_HIP (with hipGetErrorString). Faults inside kernels surface at the
 *              caller's next synchronisation. Inputs are not scanned for NaN/Inf.
 *              Nothing throws or aborts across the ABI.
 */
#ifndef PISA_H
#define PISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PISA_OK = 0,
  PISA_ERR_INVALID_ARG = 1,
  PISA_ERR_UNSUPPORTED = 2,
  PISA_ERR_WORKSPACE = 3,
  PISA_ERR_HIP = 4
} pisa_status;

typedef enum { PISA_F32 = 0, PISA_BF16 = 1 } pisa_dtype;

/* Attention modes (low 4 bits of `mode`). */
enum {
  /* Keep-or-drop block-sparse attention: only the selected blocks (Phase 1).
     With K_sel = nb this is dense attention. */
  PISA_MODE_DROP = 0,
  /* PISA hybrid order: block-wise zeroth-order virtual tokens + global first order
     (A_t H̄ q_t), PISA paper §3.3 and §3.4. */
  PISA_MODE_PISA = 1,
  /* PWT: PISA plus the diagonal, query-pooled, gated second-order mass term
     w̃_{i,j} = ½ Σ_c mean_tile(q_c²) σ²_{j,c} on the virtual-token logit
     (blog, PWT section). */
  PISA_MODE_PWT = 2,
  /* Block-wise first order H_j q_t and per-row w = ½ q_tᵀ C_j q_t with weight 1 + w,
     computed from the raw unselected blocks (blog, PWT derivation; PISA paper Eq. (3.2)
     exact first-order variant). Costs about as much as dense attention. */
  PISA_MODE_LITERAL = 3,
  /* PWT with the per-row diagonal w_{t,j} = ½ Σ_c q_{t,c}² σ²_{j,c} in place of the
     tile-pooled w̃ (blog, PWT section: the ablation of the pooling; each virtual token
     costs a second d-long product per row). Reads st->ksig2; wt is not used. */
  PISA_MODE_PWT_ROW = 4
};

/* Modifier bits of `mode`. */
enum {
  PISA_W_LINEAR = 1u << 4,  /* φ(w) = ln(1 + w) (the 1 + w form); default for LITERAL */
  PISA_W_NOGATE = 1u << 5,  /* disable the validity gate (w > ln n_j => w = 0) */
  PISA_W_EXP = 1u << 6      /* φ(w) = w (the e^w form); default for PWT, needed only to
                               switch LITERAL to it */
};

/* Flags of pisa_block_stats. */
enum {
  PISA_STATS_BLOCK_H = 1u << 0, /* also write every H_j to pisa_stats.hblk */
  PISA_STATS_BLOCK_C = 1u << 1, /* also write every C_j to pisa_stats.cblk */
  PISA_STATS_HNORM = 1u << 2    /* also write M_j = ||H_j - H̄||_F to pisa_stats.hnorm
                                   (a second pass over K and V) */
};

/* Selection rules of pisa_select_topk_routed. */
enum {
  PISA_ROUTE_MEAN = 0,        /* s_{i,j} = q̄_i·k̄_j (block-mean scoring) */
  PISA_ROUTE_COVARIANCE = 1,  /* s_{i,j} = q̄_i·k̄_j + ln(M_j + eps) (covariance-aware) */
  PISA_ROUTE_ERROR = 2        /* s_{i,j} = q̄_i·k̄_j + w̃_{i,j} + ln n_j + ln(M_j + eps)
                                 (predicted truncation error: mass times heterogeneity) */
};

/*
 * Block statistics (device buffers, caller-allocated, row-major). For block j of head h
 * with valid tokens I_j, n_j = |I_j| (blog, notation and PWT sections; PISA paper
 * Fig. 3 prepare phase):
 *   kbar  [H][nb][d]   k̄_j = (1/n_j) Σ_{I_j} k_i
 *   vsum  [H][nb][d]   ΣV_j = Σ_{I_j} v_i
 *   ksig2 [H][nb][d]   σ²_{j,c} = (1/n_j) Σ_{I_j} (k_{i,c} - k̄_{j,c})²
 *   hbarT [H][d][d]    H̄ᵀ[c][e] with H̄ = (1/nb) Σ_j H_j, H_j = Σ_{I_j} v_i (k_i - k̄_j)ᵀ
 *   hblk  [H][nb][d][d] H_j[e][c]              (NULL unless PISA_STATS_BLOCK_H)
 *   cblk  [H][nb][d][d] C_j = (1/n_j) Σ (k_i - k̄_j)(k_i - k̄_j)ᵀ (NULL unless PISA_STATS_BLOCK_C)
 *   hnorm [H][nb]      M_j = ||H_j - H̄||_F, the block's heterogeneity against the global
 *                      first-order statistic (PISA paper §3.3, Error Analysis and
 *                      Covariance-Aware Block Selection; NULL unless PISA_STATS_HNORM)
 *   packed             pisa_packed_bytes() bytes: the same statistics re-laid for the
 *                      attention kernel's operands (plus Vᵀ per block) and the order in
 *                      which it visits query tiles; opaque, written by pisa_block_stats
 *                      and read by pisa_attention_fwd.
 */
typedef struct {
  float* kbar;
  float* vsum;
  float* ksig2;
  float* hbarT;
  float* hblk;
  float* cblk;
  void* packed;
  float* hnorm;
} pisa_stats;

/* Bytes of pisa_stats.packed for these sizes (0 if unsupported). */
size_t pisa_packed_bytes(pisa_dtype dt, int H, int L, int d, int B);

/* Workspace bytes of pisa_block_stats (fp32 partial sums of H̄; 0 if unsupported). */
size_t pisa_block_stats_workspace_bytes(int H, int L, int d, int B);

/*
 * Prepare phase, part 1 (PISA paper §3.4 "Prepare Phase": block centroids, value sums
 * and the global statistic H̄ in a single pass; blog, PWT section: σ²_j).
 * K, V: [H][L][d] device tensors of dtype `dt`. Writes every field of *out (hblk / cblk /
 * hnorm only when flagged). `out` is a host pointer to a struct of device pointers.
 * Repeated calls on the same inputs give bit-identical results.
 */
pisa_status pisa_block_stats(pisa_dtype dt, const void* K, const void* V, int H, int L, int d,
                             int B, const int32_t* block_len, unsigned flags,
                             const pisa_stats* out, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Size of the fixed device scratch of pisa_block_stats_noalloc (64 MiB per GPU). */
#define PISA_STATS_SCRATCH_BYTES (64u << 20)

/*
 * pisa_block_stats for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments, results
 * and errors as pisa_block_stats without the workspace: the fp32 partial sums of H̄ live
 * in a fixed PISA_STATS_SCRATCH_BYTES array in device memory that every GPU the library
 * runs on holds until the process ends. The call allocates nothing. When the default
 * grouping of blocks would need more partials than fit, blocks are grouped more coarsely
 * (H̄ may then differ from pisa_block_stats in the last bits); more than
 * PISA_STATS_SCRATCH_BYTES / (4 d²) heads (1024 at d = 128) give PISA_ERR_WORKSPACE.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller.
 */
pisa_status pisa_block_stats_noalloc(pisa_dtype dt, const void* K, const void* V, int H, int L,
                                     int d, int B, const int32_t* block_len, unsigned flags,
                                     const pisa_stats* out, void* stream);

/* Workspace bytes of pisa_select_topk, pisa_select_topk_routed and pisa_select_topk_rope
 * (pooled queries, rotated key centroids and the fp32 score matrix). */
size_t pisa_select_workspace_bytes(int H, int L, int d, int B);

/*
 * Prepare phase, part 2 (PISA paper Fig. 3 and §3.4: block-wise top-K selection;
 * blog, Sparse Attention section: MoBA block-mean scoring; blog, PWT section: the
 * [query block x key block] matrix w̃).
 * For query tile i: q̄_i = mean of its valid Q rows, \overline{q²}_i = mean of their
 * squares; s_{i,j} = q̄_i·k̄_j in fp32; S_i = the K_sel largest s_{i,j}, ties to the lower
 * block index.
 *   Q      [H][L][d] dtype `dt`
 *   st     reads st->kbar and st->ksig2 (from pisa_block_stats)
 *   idx    [H][nb][K_sel] int32 out: S_i in ascending block order
 *   mask   [H][nb][ceil(nb/32)] uint32 out or NULL: bit j set iff j in S_i
 *   wt     [H][nb][nb] float out or NULL: w̃_{i,j} = ½ Σ_c \overline{q²}_{i,c} σ²_{j,c}
 *          before the gate (needed by PISA_MODE_PWT)
 * 0 <= K_sel <= nb.
 */
pisa_status pisa_select_topk(pisa_dtype dt, const void* Q, const pisa_stats* st, int H, int L,
                             int d, int B, const int32_t* block_len, int K_sel, int32_t* idx,
                             uint32_t* mask, float* wt, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * pisa_select_topk with a choice of block score (PISA paper §3.3, Covariance-Aware Block
 * Selection, Eq. (7)). PISA_ROUTE_COVARIANCE ranks key block j for query tile i by
 * q̄_i·k̄_j + ln(M_j + eps), with M_j read from st->hnorm (pisa_block_stats with
 * PISA_STATS_HNORM on the same K, V). Eq. (7) normalises this score with a softmax over
 * the blocks, which leaves the order within a row, and so the top-K set, unchanged; the
 * pooled q̄_i stands for the query as in block-mean scoring. PISA_ROUTE_ERROR ranks by
 * the log of the predicted truncation error, virtual-token mass n_j e^{q̄_i·k̄_j + w̃_{i,j}}
 * times heterogeneity M_j + eps (blog, PWT section), with w̃ before the gate and n_j from
 * block_len. eps must be finite and > 0. wt is w̃ as in pisa_select_topk (the routing
 * terms do not enter it). PISA_ROUTE_MEAN gives exactly pisa_select_topk.
 */
pisa_status pisa_select_topk_routed(pisa_dtype dt, const void* Q, const pisa_stats* st, int H,
                                    int L, int d, int B, const int32_t* block_len, int K_sel,
                                    unsigned route, float eps, int32_t* idx, uint32_t* mask,
                                    float* wt, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Pairing of dims inside each rotary slice of pisa_rope. */
enum {
  PISA_ROPE_ADJACENT = 0, /* pair f of a slice is dims (2f, 2f + 1) */
  PISA_ROPE_HALF = 1      /* pair f of a slice of width w is dims (f, f + w/2) */
};

/* Rotary position embedding as the caller applied it to Q and K: the head dimension is cut
 * into n_axes consecutive slices of width[a] dims (axis a of the token position, e.g.
 * t, h, w); pair f of slice a turns by the angle pos_a · base^(-2f/width[a]). */
typedef struct {
  int n_axes;     /* 1..3 */
  int width[3];   /* even, >= 2, summing to d (entries past n_axes ignored) */
  float base;     /* finite, > 0 */
  int pairs;      /* PISA_ROPE_ADJACENT or PISA_ROPE_HALF */
} pisa_rope;

/*
 * pisa_select_topk with RoPE-aware centroids (blog "Sparse Linear Attention (2)", section
 * Selection Error): block means of rotated keys mix B different rotations and lose the
 * relative-position form of the score; instead the block is averaged before the rotation
 * and the mean is turned at the block centre c_j. Queries are pooled per tile the same
 * way, so s_{i,j} = (R_{c_i} q̄_i)·(R_{c_j} k̄_j), which depends on c_j - c_i only.
 *   Q_pre, K_pre  [H][L][d] dtype `dt`: Q (with 1/sqrt(d)) and K before the rotation
 *   pos           DEVICE float [L][rope->n_axes]: position of every slot in block order;
 *                 c_j = mean position of block j's valid tokens (padded slots ignored)
 *   Q             the rotated Q of the attention call; read only for wt (may be NULL when
 *                 wt is NULL); st->ksig2 is read for wt, st->kbar is not read
 * Selection, idx, mask and wt as in pisa_select_topk. The attention call itself takes the
 * rotated Q, K, V and the statistics of the rotated K as usual.
 */
pisa_status pisa_select_topk_rope(pisa_dtype dt, const void* Q, const void* Q_pre,
                                  const void* K_pre, const float* pos, const pisa_rope* rope,
                                  const pisa_stats* st, int H, int L, int d, int B,
                                  const int32_t* block_len, int K_sel, int32_t* idx,
                                  uint32_t* mask, float* wt, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Fused kernel (PISA paper §3.4 phases 1-3; Eq. (3.2); blog, PWT section).
 * For valid query t of tile i, o_t = N_t / D_t with one running max and denominator:
 *   D_t = Σ_{j∈S_i} Σ_{n<n_j} e^{q_t·k_{j,n}} + Σ_{j∉S_i} n_j e^{q_t·k̄_j + φ_{t,j}}
 *   N_t = Σ_{j∈S_i} Σ_{n<n_j} e^{q_t·k_{j,n}} v_{j,n} + Σ_{j∉S_i} e^{q_t·k̄_j + φ_{t,j}} ΣV_j
 *         + first order: (Σ_{j∉S_i} e^{q_t·k̄_j + φ_{t,j}}) H̄ q_t      (PISA, PWT)
 *                        Σ_{j∉S_i} e^{q_t·k̄_j + φ_{t,j}} H_j q_t        (LITERAL)
 *   φ = 0 (PISA); φ = w̃_{i,j} (PWT); φ = ½ Σ_c q_{t,c}² σ²_{j,c} (PWT_ROW); per-row
 *   w = ½ q_tᵀC_j q_t mapped to ln(1 + w) (LITERAL); w is zeroed when w > ln n_j unless
 *   PISA_W_NOGATE. DROP keeps S_i only.
 * Inputs: Q, K, V [H][L][d] dtype `dt`; st->packed from pisa_block_stats on the same K, V
 * and the same block_len (the packed tile order holds each query tile's row count from
 * that call); idx from pisa_select_topk with the same K_sel; mask (required unless DROP); wt
 * (required for PWT). Outputs: O [H][L][d] dtype `dt`; lse [H][L] float or NULL
 * (natural-log log-sum-exp of every row's logits, -inf for padded rows and rows with no
 * support). Out-of-range entries of idx are treated as empty blocks.
 * PWT_ROW, and LITERAL for PISA_BF16, with lse given run in two passes that use lse as
 * the hand-over: the selected blocks as DROP (O and lse written), then the virtual tokens
 * (PWT_ROW) or the unselected blocks in their literal form (LITERAL), merged into O and
 * lse; with lse NULL (or fp32 LITERAL) they run in a single (slower) pass. Both give the
 * same result up to rounding.
 */
pisa_status pisa_attention_fwd(pisa_dtype dt, const void* Q, const void* K, const void* V,
                               const pisa_stats* st, const int32_t* idx, const uint32_t* mask,
                               const float* wt, int H, int L, int d, int B,
                               const int32_t* block_len, int K_sel, unsigned mode, void* O,
                               float* lse, void* stream);

/* Workspace bytes of pisa_attention_bwd (0 if unsupported). */
size_t pisa_attention_bwd_workspace_bytes(pisa_dtype dt, int H, int L, int d, int B, int K_sel);

/*
 * Backward of pisa_attention_fwd for PISA_MODE_DROP, PISA_MODE_PISA, PISA_MODE_PWT and (bf16)
 * PISA_MODE_LITERAL and PISA_MODE_PWT_ROW (with the same modifier bits), for sparse fine-tuning (blog, PWT
 * section: gradients flow through the block statistics k̄_j, H̄ and σ²_j; routing is
 * detached). The selection and the gate's decisions are held fixed; the loss is
 * sum(dO * O).
 *   Inputs   Q, K, V, st, idx, mask, wt, block_len, K_sel, mode: as given to the forward
 *            call (mask is required for every mode and must match idx; st needs kbar, vsum,
 *            ksig2 and hbarT); lse: that call's output; dO [H][L][d] dtype `dt`.
 *            O [H][L][d] dtype `dt`: that call's output, or NULL (see Δ below).
 *   Outputs  dQ, dK, dV [H][L][d] float32, overwritten (zeros on padded slots).
 *   Workspace pisa_attention_bwd_workspace_bytes(dt, H, L, d, B, K_sel) bytes.
 * With P = e^{logit - lse} for every exact key and virtual token, u_t = H̄ q_t,
 * Ā_t = Σ_j P_{t,j} / n_j and Δ_t = dO_t·o_t. With O given, Δ_O = dO·O in fp32, and dS =
 * P(dP - Δ_O) and P enter the dQ products in the input type (two products per tile); the
 * fp32 sum ε = Σ dS = Δ - Δ_O then removes O's rounding (dq -= ε Σ P k, Δ = Δ_O + ε). With O NULL,
 * Δ is formed in fp32 as Σ P·dP over every exact key and virtual token (dP = dO·v, or
 * dO·v̄_j + dO·u_t / n_j, which is dO·o exactly) in the same sweep, and dQ as
 * Σ P dP k - Δ Σ P k with hi + lo operand pairs (four products per tile; no rounding of O):
 *   dq_t  = Σ P(dO·v - Δ) k (exact) + Σ P(dO·v̄_j + dO·u_t / n_j - Δ) k̄_j + Ā_t H̄ᵀ dO_t
 *           + (2/m_i) q_t ∘ ½ Σ_j dw̃_{i,j} σ²_j                         (PWT)
 *   dk, dv of exact keys from the same terms; dk̄_j, dv̄_j, dH̄ = Σ_t Ā_t dO_t q_tᵀ and
 *   dσ²_j = ½ Σ_i dw̃_{i,j} \overline{q²}_i reach the tokens of block j through
 *   k̄_j, v̄_j = ΣV_j / n_j, H̄ = (1/nb) Σ_j Σ_i v_i (k_i - k̄_j)ᵀ and σ²_j.
 * PISA_MODE_LITERAL (bf16 inputs; the PISA paper's Eq. (3.2) block-wise first order with the
 * blog's per-row w = ½ qᵀC_j q, PWT section): every unselected block j enters as
 * E (1 + y_n) v_n over its valid keys n, with x_n = q·k_n, s̄ = mean x, y_n = x_n - s̄,
 * w = ½ mean y², φ(w) as in the forward, E = e^{s̄ + φ - lse}; then
 *   dx_n = E dO·v_n + dw y_n / n_j - mean_m(...) + dℓ / n_j,  dℓ = E (Σ_n (1 + y_n) dO·v_n - n_j Δ),
 *   dw = φ'(w) dℓ, and dq = Σ dx k, dk = Σ dx q, dv = Σ (P or E (1 + y)) dO over every
 *   (query tile, key block) pair. Δ is formed in fp32 by a first sweep over all pairs (O is
 *   not read), so this backward costs about three dense score sweeps.
 * PISA_MODE_PWT_ROW (bf16 inputs; w_{t,j} = ½ Σ_c q_{t,c}² σ²_{j,c} per row): as PWT with
 *   dw_{t,j} = φ'(w_{t,j}) dℓ_{t,j} per row, so dq_t gains q_t ∘ Σ_j dw σ²_j and
 *   dσ²_j = ½ Σ_t dw q_t² (in place of the pooled terms); the selected blocks' exact terms,
 *   Δ and Ā as above.
 * For LITERAL and PWT_ROW the Δ sweep also sums P and the later sweeps use lse + ln Σ P (the
 * forward normalised with sums of its bf16 P; the common mean of the keys would amplify
 * the 2^-9 offset in dq). fp32 inputs give PISA_ERR_UNSUPPORTED for these two modes.
 * Sums are taken in a fixed order (repeated calls are bit-identical).
 */
pisa_status pisa_attention_bwd(pisa_dtype dt, const void* Q, const void* K, const void* V,
                               const pisa_stats* st, const int32_t* idx, const uint32_t* mask,
                               const float* wt, int H, int L, int d, int B,
                               const int32_t* block_len, int K_sel, unsigned mode, const float* lse,
                               const void* O, const void* dO, float* dQ, float* dK, float* dV,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Layout step (blog "Sparse Linear Attention", notation: tokens are cut into blocks of B;
 * video latents are grouped into 3D cubes). Block order is the layout every other call
 * takes.
 *
 * pisa_cube_layout (host only, no GPU work): the block order of a T x Hh x W latent grid
 * (natural order row-major over (t, h, w)) cut into ct x ch x cw cubes of B = ct*ch*cw
 * tokens: cubes row-major over their (t, h, w) indices, tokens inside a cube row-major,
 * a cube cut by the grid's edge keeps its valid tokens first and is padded to B slots.
 *   perm       HOST int32 [nb * B] out: natural index of the token in each slot, -1 = padding
 *   block_len  HOST int32 [nb] out: valid tokens per block (n_j)
 *   capacity   entries of perm available; nb * B must fit (nb = product of ceil(grid/cube))
 * Returns PISA_OK and writes *nb_out, or an error (sizes, capacity).
 *
 * pisa_layout_to_blocks: dst[h][s] = perm[s] >= 0 ? src[h][perm[s]] : 0
 *   src [H][L_nat][d], dst [H][L_pad][d] dtype `dt`; perm DEVICE int32 [L_pad].
 * pisa_layout_from_blocks: dst[h][perm[s]] = src[h][s] for the slots with perm[s] >= 0
 *   src [H][L_pad][d], dst [H][L_nat][d]; perm must map the valid slots one-to-one onto
 *   [0, L_nat) (pisa_cube_layout's does); entries outside [0, L_nat) are skipped.
 * Both are stream-ordered copies (HBM-bound); src and dst must not overlap.
 */
pisa_status pisa_cube_layout(int T, int Hh, int W, int ct, int ch, int cw, int32_t* perm,
                             int32_t* block_len, size_t capacity, int* nb_out);
pisa_status pisa_layout_to_blocks(pisa_dtype dt, const void* src, int H, int L_nat, int L_pad, int d,
                                  const int32_t* perm, void* dst, void* stream);
pisa_status pisa_layout_from_blocks(pisa_dtype dt, const void* src, int H, int L_nat, int L_pad,
                                    int d, const int32_t* perm, void* dst, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* pisa_last_error(void);

/* Library version string. */
const char* pisa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PISA_H */
