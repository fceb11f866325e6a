"""CPU oracle for piecewise (exact-or-approximate) block-sparse attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the bench's CPU
baseline leg may import this module. The product path (the HIP library and its Python
binding) never imports, calls or links anything here, and this module imports nothing
from the product package.

Plain float64 numpy, one head at a time. Each function follows one passage of the
pages and names it. There is no blocking, fusion or reordering beyond what those
definitions state; library primitives (matmul, sort) serve as single steps.

Notation (Sparse Linear Attention blog, notation paragraph; PISA paper §3.2
Formulation): q_t, k_i, v_i are rows in R^d with 1/sqrt(d) already folded into q.
Tokens are cut into blocks B_j of (at most) B tokens; block j holds n_j valid tokens
in its first n_j slots. k̄_j is the key centroid, ΣV_j the value sum,
H_j = sum_i v_i (k_i - k̄_j)^T the key-value cross statistic, C_j the within-block
key covariance, σ²_j its diagonal, H̄ the average of H_j over all blocks.
α_{t,j} = exp(q_t·k̄_j). S_i / U_i are the selected / unselected key blocks of
query tile i (every row of a tile shares them: PISA paper §3.2).

Readings taken where the pages are silent or garbled (each is listed with its
reason in the design notes of the repository):
  * ragged blocks: B is replaced by n_j in the centroid, the virtual-token weight
    n_j·α and the ln n_j gate; H̄ = (1/nb) sum_j H_j over all blocks of the head;
  * C_j uses the population normalisation 1/n_j;
  * the second-order factor multiplies the zeroth-order numerator, the first-order
    weight and the denominator alike (blog, PWT section: all three share the
    corrected logit);
  * the garbled k̄_t in the paper's global first-order formula is read as k̄_j and
    the coefficient as sum_{j in U} α_{t,j} (blog, Sparse Linear Attention section);
  * selection ties go to the lower block index; a row with no key support
    (empty selection and no virtual tokens) outputs 0 with lse = -inf; padded query
    rows output 0 with lse = -inf.

Every function here has at least one pin in tests/test_oracle_*.py against closed
forms, reductions to dense attention, invariants or the paper's error bound.
"""
from __future__ import annotations

import math

import numpy as np

# Mode presets. The GPU exposes DROP, PISA, PWT and LITERAL; PISA0 and the keyword
# overrides below exist for the ablation pins only.
PRESETS = {
    # keep-or-drop block-sparse attention: unselected blocks contribute nothing
    "drop": dict(virtual=False, first="none", w_kind="none"),
    # zeroth-order virtual tokens only (PISA paper Table 8 "Zeroth order")
    "pisa0": dict(virtual=True, first="none", w_kind="none"),
    # PISA hybrid order: block-wise zeroth order + global first order (PISA paper §3.3)
    "pisa": dict(virtual=True, first="global", w_kind="none"),
    # PWT: PISA + diagonal, query-pooled, gated second-order mass term (blog, PWT section)
    "pwt": dict(virtual=True, first="global", w_kind="pooled", w_map="exp", guard="gate",
                pooling="sqmean"),
    # PWT with the per-row diagonal w_{t,j} = ½ Σ_c q_{t,c}² σ²_{j,c} instead of the tile-pooled
    # w̃ (blog, PWT section: the accuracy / speed ablation of the pooling)
    "pwt_row": dict(virtual=True, first="global", w_kind="rowdiag", w_map="exp", guard="gate"),
    # block-wise first order H_j q and per-row w = ½ qᵀC_j q, with 1+w (blog, PWT derivation)
    "literal": dict(virtual=True, first="block", w_kind="row", w_map="linear", guard="gate"),
}


# ----------------------------------------------------------------------------- blocks
def block_ranges(L_pad: int, B: int, block_len=None):
    """(start, n_j) of every block: tokens cut in order into blocks of size B
    (blog, notation); ragged blocks keep their n_j valid tokens first."""
    nb = L_pad // B
    if L_pad % B:
        raise ValueError("L_pad must be a multiple of B")
    if block_len is None:
        return [(j * B, B) for j in range(nb)]
    bl = np.asarray(block_len)
    if bl.shape != (nb,) or (bl < 1).any() or (bl > B).any():
        raise ValueError("block_len must hold nb values in [1, B]")
    return [(j * B, int(bl[j])) for j in range(nb)]


# ----------------------------------------------------------------------------- layout
def cube_order(grid, cube=(4, 4, 4)):
    """Block order of a (T, H, W) latent grid cut into cubes (blog, notation: tokens are cut
    into blocks of B; video tokens are grouped into 3D cubes): cubes in row-major order over
    (cube t, cube h, cube w), tokens inside a cube row-major over (dt, dh, dw); a cube cut by
    the grid's edge keeps its valid tokens first and pads to B slots. Returns (perm, n) with
    perm[s] = natural row-major index of the token in slot s (-1 for padding) and n[j] the
    valid tokens of block j."""
    T, Hh, W = grid
    ct, ch, cw = cube
    B = ct * ch * cw
    perm, n = [], []
    for a in range((T + ct - 1) // ct):
        for b in range((Hh + ch - 1) // ch):
            for c in range((W + cw - 1) // cw):
                toks = [(t * Hh + h) * W + w
                        for t in range(a * ct, min(T, a * ct + ct))
                        for h in range(b * ch, min(Hh, b * ch + ch))
                        for w in range(c * cw, min(W, c * cw + cw))]
                n.append(len(toks))
                perm.extend(toks + [-1] * (B - len(toks)))
    return np.array(perm, dtype=np.int64), np.array(n, dtype=np.int64)


def to_blocks(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Natural order [..., L, d] -> block order [..., L_pad, d]: slot s holds token perm[s],
    padding slots hold 0."""
    perm = np.asarray(perm)
    out = np.zeros(x.shape[:-2] + (perm.size, x.shape[-1]), dtype=x.dtype)
    ok = perm >= 0
    out[..., ok, :] = x[..., perm[ok], :]
    return out


def from_blocks(x: np.ndarray, perm: np.ndarray, L: int) -> np.ndarray:
    """Block order [..., L_pad, d] -> natural order [..., L, d] (padding slots dropped)."""
    perm = np.asarray(perm)
    out = np.zeros(x.shape[:-2] + (L, x.shape[-1]), dtype=x.dtype)
    ok = perm >= 0
    out[..., perm[ok], :] = x[..., ok, :]
    return out


# ----------------------------------------------------------------------------- statistics
def block_stats(K: np.ndarray, V: np.ndarray, B: int, block_len=None, per_block: bool = True) -> dict:
    """Per-block statistics of one head.

    k̄_j = (1/n_j) sum_i k_i                       (blog, notation; MoBA centroid)
    ΣV_j = sum_i v_i                                (PISA paper §3.2 "Practical Challenge"; Fig. 3 V̂)
    H_j = sum_i v_i (k_i - k̄_j)^T, stored [e, c]    (blog, Sparse Linear Attention section)
    C_j = (1/n_j) sum_i (k_i - k̄_j)(k_i - k̄_j)^T   (blog, PWT section: within-block key covariance)
    σ²_j = diag C_j                                 (blog, PWT section: diagonal approximation)
    H̄ = (1/nb) sum_j H_j                            (blog: H̄ = (B/L) sum_j H_j with L = nb·B)

    per_block=False keeps only H̄ and σ² (H and C are None): the same sums, without
    storing the nb d x d matrices of long sequences.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L_pad, d = K.shape
    rng = block_ranges(L_pad, B, block_len)
    nb = len(rng)
    kbar = np.zeros((nb, d))
    vsum = np.zeros((nb, d))
    sig2 = np.zeros((nb, d))
    Hj = np.zeros((nb, d, d)) if per_block else None
    Cj = np.zeros((nb, d, d)) if per_block else None
    hsum = np.zeros((d, d))
    n = np.zeros(nb)
    for j, (s, nj) in enumerate(rng):
        k = K[s:s + nj]
        v = V[s:s + nj]
        kbar[j] = k.mean(axis=0)
        vsum[j] = v.sum(axis=0)
        dev = k - kbar[j]
        h = v.T @ dev
        hsum += h
        sig2[j] = (dev ** 2).mean(axis=0)
        if per_block:
            Hj[j] = h
            Cj[j] = dev.T @ dev / nj
        n[j] = nj
    hbar = hsum / nb
    return dict(kbar=kbar, vsum=vsum, H=Hj, C=Cj, sig2=sig2, hbar=hbar, n=n)


def pool_queries(Q: np.ndarray, B: int, block_len=None) -> dict:
    """Per query tile: q̄_i (mean of the valid rows; PISA paper Fig. 3 Q̄) and
    mean of squares  \\overline{q²}_i (blog, PWT section: square first, then average),
    plus the square of the mean q̄_i² kept only for the pooling ablation."""
    Q = np.asarray(Q, dtype=np.float64)
    rng = block_ranges(Q.shape[0], B, block_len)
    d = Q.shape[1]
    qbar = np.zeros((len(rng), d))
    qsq = np.zeros((len(rng), d))
    for i, (s, ni) in enumerate(rng):
        qbar[i] = Q[s:s + ni].mean(axis=0)
        qsq[i] = (Q[s:s + ni] ** 2).mean(axis=0)
    return dict(qbar=qbar, qsq=qsq, qbar_sq=qbar ** 2)


# ----------------------------------------------------------------------------- selection
def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """s_{i,j} = q̄_i · k̄_j: MoBA-style block-mean scoring with the pooled query of
    each tile (blog, Sparse Attention section; PISA paper Fig. 3 prepare phase)."""
    return np.asarray(qbar, dtype=np.float64) @ np.asarray(kbar, dtype=np.float64).T


# Offset inside log(M_j + ε) of the covariance-aware score. The paper leaves ε unstated;
# it only keeps the log finite when a block matches the global statistic exactly.
ROUTE_EPS = 1e-6


def block_heterogeneity(st: dict) -> np.ndarray:
    """M_j = ||H_j - H̄||_F per block: the heterogeneity whose norm bounds the error of
    replacing H_j by the global H̄ (PISA paper §3.3 Error Analysis, Theorem 3.1 with
    M_t = max_j ||H_j - H̄||_2, and Covariance-Aware Block Selection). The Frobenius norm
    is the computable choice; it bounds the spectral norm from above. Needs the per-block
    H_j (block_stats with per_block=True)."""
    H = st["H"]
    if H is None:
        raise ValueError("block_heterogeneity needs per-block H_j")
    return np.sqrt(((H - st["hbar"][None, :, :]) ** 2).sum(axis=(1, 2)))


def routed_scores(qbar: np.ndarray, kbar: np.ndarray, hnorm: np.ndarray, eps: float = ROUTE_EPS) -> np.ndarray:
    """Covariance-aware selection score (PISA paper §3.3 Eq. (7)):
    q̄_i·k̄_j + log(M_j + ε). The softmax of Eq. (7) is monotone along each row, so the
    top-K is taken on its argument; the pooled q̄_i stands for q_t, as in block-mean
    scoring, and 1/sqrt(d) is already folded into Q."""
    return block_scores(qbar, kbar) + np.log(np.asarray(hnorm, dtype=np.float64) + eps)[None, :]


def error_routed_scores(qbar: np.ndarray, kbar: np.ndarray, w: np.ndarray, n: np.ndarray,
                        hnorm: np.ndarray, eps: float = ROUTE_EPS) -> np.ndarray:
    """Routing by predicted truncation error (blog, PWT section: a block's truncation error
    is roughly its mass times its within-block heterogeneity, so the log of the block's
    virtual-token mass n_j e^{q·k̄_j + w} plus the log of its heterogeneity ranks the
    blocks; the PISA paper's covariance-aware selection is this view of routing).
    Score: q̄_i·k̄_j + w̃_{i,j} + ln n_j + ln(M_j + ε), with the pooled q̄_i and w̃_{i,j}
    of the tile (before the gate: a block whose expansion fails is the one to keep
    exact), n_j the valid count (B for a full block) and M_j = ||H_j - H̄||_F as in
    Eq. (7) of the PISA paper."""
    n = np.asarray(n, dtype=np.float64)
    return (block_scores(qbar, kbar) + np.asarray(w, dtype=np.float64) + np.log(n)[None, :]
            + np.log(np.asarray(hnorm, dtype=np.float64) + eps)[None, :])


def rope_rotate(x: np.ndarray, pos: np.ndarray, widths, base: float, pairs: str = "adjacent") -> np.ndarray:
    """Rotary position embedding R_p x of rows x [n, d] at positions pos [n, n_axes]
    (Sparse Linear Attention (2) blog, Selection Error: a position-dependent rotation R_i
    with R_mᵀR_n = R_{n-m}). The head dimension is cut into consecutive slices of
    widths[a] dims, one per position axis a; inside slice a, pair f (dims 2f, 2f+1 for
    "adjacent", f, f + widths[a]/2 for "half") turns by the angle pos_a · base^(-2f/widths[a])."""
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64).reshape(x.shape[0], -1)
    out = x.copy()
    off = 0
    for a, wdt in enumerate(widths):
        f = np.arange(wdt // 2, dtype=np.float64)
        ang = np.outer(pos[:, a], base ** (-2.0 * f / wdt))
        c, s = np.cos(ang), np.sin(ang)
        if pairs == "adjacent":
            i0 = off + 2 * np.arange(wdt // 2)
            i1 = i0 + 1
        elif pairs == "half":
            i0 = off + np.arange(wdt // 2)
            i1 = i0 + wdt // 2
        else:
            raise ValueError(pairs)
        out[:, i0] = x[:, i0] * c - x[:, i1] * s
        out[:, i1] = x[:, i0] * s + x[:, i1] * c
        off += wdt
    if off != x.shape[1]:
        raise ValueError("rotary widths must cover the head dimension")
    return out


def rope_block_scores(Q_pre: np.ndarray, K_pre: np.ndarray, pos: np.ndarray, B: int, block_len,
                      widths, base: float, pairs: str = "adjacent") -> np.ndarray:
    """Block scores with RoPE-aware centroids (Sparse Linear Attention (2) blog, Selection
    Error): average the rows before the rotary embedding, then rotate the average at the
    block centre c_j, so that the score is an inner product that depends on the relative
    position only. Every tile does the same on the query side: q̄_i is the mean of its
    valid pre-rotation rows, turned at its own centre c_i; c is the mean position of the
    valid tokens (tiles and blocks share one partition).
    s_{i,j} = (R_{c_i} q̄_i)·(R_{c_j} k̄_j). pos: [L_pad, n_axes] in block order."""
    pos = np.asarray(pos, dtype=np.float64)
    pos = pos.reshape(pos.shape[0], -1)
    rng = block_ranges(np.asarray(K_pre).shape[0], B, block_len)
    qbar = pool_queries(Q_pre, B, block_len)["qbar"]
    kbar = np.stack([np.asarray(K_pre, dtype=np.float64)[s:s + n].mean(axis=0) for s, n in rng])
    centre = np.stack([pos[s:s + n].mean(axis=0) for s, n in rng])
    return block_scores(rope_rotate(qbar, centre, widths, base, pairs),
                        rope_rotate(kbar, centre, widths, base, pairs))


def select_topk(scores: np.ndarray, K_sel: int) -> np.ndarray:
    """S_i = the K_sel largest scores of row i, ties to the lower block index; returned
    in ascending block order, shape [nq, K_sel] int64."""
    scores = np.asarray(scores)
    nq, nb = scores.shape
    if not 0 <= K_sel <= nb:
        raise ValueError("K_sel out of range")
    out = np.zeros((nq, K_sel), dtype=np.int64)
    j = np.arange(nb)
    for i in range(nq):
        order = np.lexsort((j, -scores[i]))        # primary: score desc, secondary: index asc
        out[i] = np.sort(order[:K_sel])
    return out


# ----------------------------------------------------------------------------- second order
def _guard_and_map(w: np.ndarray, n: np.ndarray, guard: str, w_map: str) -> np.ndarray:
    """Validity gate of the second-order term and its placement in the logit (blog, PWT
    section): w > ln n_j is zeroed (gate) or held at ln n_j (clamp, the rejected first
    attempt); then φ = w (the implementation's e^w) or φ = ln(1 + w) (the 1 + w form)."""
    lim = np.log(n)
    if guard == "gate":
        w = np.where(w > lim, 0.0, w)
    elif guard == "clamp":
        w = np.minimum(w, lim)
    elif guard != "none":
        raise ValueError(guard)
    if w_map == "exp":
        return w
    if w_map == "linear":
        return np.log1p(w)
    raise ValueError(w_map)


# ----------------------------------------------------------------------------- attention
def attention_head(Q, K, V, B: int, block_len=None, K_sel: int = 0, mode: str = "pwt",
                   idx=None, tiles=None, stats=None, **overrides) -> dict:
    """Piecewise sparse attention of one head (non-causal self-attention, Q/K/V share
    the block partition).

    o_t = N_t / D_t with, for query t in tile i (PISA paper §3.2 Eq. (3.2); blog,
    Sparse Linear Attention and PWT sections):
      D_t = sum_{j in S_i} sum_n exp(q_t·k_{j,n}) + sum_{j in U_i} n_j exp(q_t·k̄_j + φ_{t,j})
      N_t = sum_{j in S_i} sum_n exp(q_t·k_{j,n}) v_{j,n}
            + sum_{j in U_i} exp(q_t·k̄_j + φ_{t,j}) ΣV_j                  (zeroth order)
            + first-order term:
                global: (sum_{j in U_i} exp(q_t·k̄_j + φ_{t,j})) H̄ q_t    (PISA paper §3.3)
                block:  sum_{j in U_i} exp(q_t·k̄_j + φ_{t,j}) H_j q_t      (blog; paper Eq. (3.2))
    φ comes from w: pooled w̃_{i,j} = ½ sum_c \\overline{q²}_{i,c} σ²_{j,c} (PWT's diagonal
    + pooled form), or per row ½ q_tᵀ C_j q_t, then gated and mapped (see _guard_and_map).

    The sums are evaluated with one shift c_t = max over every logit of the row
    (exact and virtual, including ln n_j), which leaves N/D unchanged.

    Returns dict(O [L_pad, d], lse [L_pad], idx [nb, K_sel], D_log (= lse)).
    ``idx`` overrides the selection; ``tiles`` restricts the computed query tiles
    (other rows stay 0 / -inf); ``stats`` reuses block_stats output.
    """
    opts = dict(PRESETS[mode])
    opts.update(overrides)
    virtual = opts.get("virtual", True)
    first = opts.get("first", "none")
    w_kind = opts.get("w_kind", "none")
    w_map = opts.get("w_map", "exp")
    guard = opts.get("guard", "gate")
    pooling = opts.get("pooling", "sqmean")
    numerator_w = opts.get("numerator_w", True)

    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L_pad, d = Q.shape
    rng = block_ranges(L_pad, B, block_len)
    nb = len(rng)
    st = stats if stats is not None else block_stats(
        K, V, B, block_len, per_block=(first == "block" or w_kind == "row"))
    pq = pool_queries(Q, B, block_len)
    tile_list = list(range(nb)) if tiles is None else list(tiles)
    if idx is None:
        # selection rows of the evaluated tiles only (other rows stay -1)
        idx = np.full((nb, K_sel), -1, dtype=np.int64)
        idx[tile_list] = select_topk(block_scores(pq["qbar"][tile_list], st["kbar"]), K_sel)
    idx = np.asarray(idx, dtype=np.int64).reshape(nb, -1)
    n = st["n"]

    O = np.zeros((L_pad, d))
    lse = np.full(L_pad, -np.inf)
    for i in tile_list:
        s0, ni = rng[i]
        q = Q[s0:s0 + ni]                                     # [m, d]
        sel = np.zeros(nb, dtype=bool)
        sel[idx[i]] = True
        S = np.flatnonzero(sel)
        U = np.flatnonzero(~sel) if virtual else np.zeros(0, dtype=np.int64)

        # exact branch over the valid tokens of the selected blocks
        ks = np.concatenate([K[rng[j][0]:rng[j][0] + rng[j][1]] for j in S]) if S.size else np.zeros((0, d))
        vs = np.concatenate([V[rng[j][0]:rng[j][0] + rng[j][1]] for j in S]) if S.size else np.zeros((0, d))
        x = q @ ks.T                                          # [m, |tokens|]

        # virtual tokens of the unselected blocks
        s = q @ st["kbar"][U].T                               # q_t·k̄_j, [m, |U|]
        if w_kind == "none":
            w = np.zeros_like(s)
        elif w_kind == "pooled":
            pool = pq["qsq"][i] if pooling == "sqmean" else pq["qbar_sq"][i]
            w = np.broadcast_to(pooled_w(pool[None, :], st["sig2"][U])[0], s.shape)
        elif w_kind == "rowdiag":
            w = 0.5 * (q ** 2) @ st["sig2"][U].T
        elif w_kind == "row":
            w = 0.5 * np.einsum("tc,jce,te->tj", q, st["C"][U], q)
        else:
            raise ValueError(w_kind)
        phi = _guard_and_map(np.asarray(w, dtype=np.float64), n[U][None, :], guard, w_map)
        ell = s + phi + np.log(n[U])[None, :]                 # log of the weight n_j e^{s+φ}

        allmax = np.full(ni, -np.inf)
        if x.shape[1]:
            allmax = np.maximum(allmax, x.max(axis=1))
        if ell.shape[1]:
            allmax = np.maximum(allmax, ell.max(axis=1))
        empty = ~np.isfinite(allmax)
        c = np.where(empty, 0.0, allmax)[:, None]

        ex = np.exp(x - c)
        ev = np.exp(ell - c)
        D = ex.sum(axis=1) + ev.sum(axis=1)
        a = np.exp(s + phi - c) if numerator_w else np.exp(s - c)   # coefficient of ΣV_j and H_j q
        N = ex @ vs + a @ st["vsum"][U]
        if first == "global":
            N = N + a.sum(axis=1)[:, None] * (q @ st["hbar"].T)
        elif first == "block":
            N = N + np.einsum("tj,jec,tc->te", a, st["H"][U], q)
        elif first != "none":
            raise ValueError(first)
        with np.errstate(invalid="ignore", divide="ignore"):
            o = np.where(empty[:, None], 0.0, N / np.where(D > 0, D, 1.0)[:, None])
            l = np.where(empty, -np.inf, c[:, 0] + np.log(np.where(D > 0, D, 1.0)))
        O[s0:s0 + ni] = o
        lse[s0:s0 + ni] = l
    return dict(O=O, lse=lse, idx=idx)


def dense_attention_head(Q, K, V, B: int, block_len=None) -> dict:
    """Dense softmax attention o_t = sum_i e^{q_t·k_i} v_i / sum_i e^{q_t·k_i} over the
    valid keys (PISA paper §3.1), one max shift per row; padded query rows output 0."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L_pad, d = Q.shape
    rng = block_ranges(L_pad, B, block_len)
    valid = np.zeros(L_pad, dtype=bool)
    for s0, nj in rng:
        valid[s0:s0 + nj] = True
    x = Q[valid] @ K[valid].T
    c = x.max(axis=1, keepdims=True)
    e = np.exp(x - c)
    D = e.sum(axis=1)
    O = np.zeros((L_pad, d))
    lse = np.full(L_pad, -np.inf)
    O[valid] = (e @ V[valid]) / D[:, None]
    lse[valid] = c[:, 0] + np.log(D)
    return dict(O=O, lse=lse)


# ----------------------------------------------------------------------------- backward
def attention_head_backward(Q, K, V, dO, B: int, block_len=None, K_sel: int = 0, mode: str = "pwt",
                            idx=None, **overrides) -> dict:
    """Gradients of one head's attention_head output O with respect to Q, K and V for an
    upstream gradient dO (the loss sum(dO * O)), with the top-K selection and the gate's
    decisions held fixed (blog, PWT section: sparse fine-tuning backpropagates through the
    block statistics k̄_j, H̄ and σ²_j while routing stays detached). Modes DROP, PISA and
    PWT (tile-pooled w̃, global first order), PWT_ROW and LITERAL (below).

    With P_{t,k} = e^{x_{t,k} - lse_t} for the exact keys, P_{t,j} = e^{ℓ_{t,j} - lse_t} for
    the virtual tokens (ℓ = q·k̄_j + φ_{i,j} + ln n_j), Δ_t = dO_t·O_t, v̄_j = ΣV_j / n_j,
    u_t = H̄ q_t and Ā_t = Σ_j P_{t,j} / n_j, the output is
        o_t = Σ_k P_{t,k} v_k + Σ_j P_{t,j} v̄_j + Ā_t u_t
    and the softmax rule gives dx_{t,k} = P_{t,k}(dO_t·v_k - Δ_t),
    dℓ_{t,j} = P_{t,j}(dO_t·v̄_j + dO_t·u_t / n_j - Δ_t). Then
        dq_t  = Σ_k dx k_k + Σ_j dℓ k̄_j + Ā_t H̄ᵀ dO_t (+ the pooled-q² term below)
        dk_k, dv_k (exact keys) = Σ_t dx_{t,k} q_t, Σ_t P_{t,k} dO_t
        dk̄_j = Σ_t dℓ_{t,j} q_t,  dv̄_j = Σ_t P_{t,j} dO_t,  dH̄ = Σ_t Ā_t dO_t q_tᵀ
        dw̃_{i,j} = φ'(w̃_{i,j}) Σ_{t in tile i} dℓ_{t,j}   (0 where the gate fired)
        d\\overline{q²}_i = ½ Σ_j dw̃_{i,j} σ²_j,  dσ²_j = ½ Σ_i dw̃_{i,j} \\overline{q²}_i
    and the statistics pass their gradients to the tokens of block j (valid tokens only):
        dk_i += dk̄_j / n_j + (2/n_j)(k_i - k̄_j)∘dσ²_j + (1/nb) dH̄ᵀ (v_i - v̄_j)
        dv_i += dv̄_j / n_j + (1/nb) dH̄ (k_i - k̄_j)
        dq_t += (2/m_i) q_t ∘ d\\overline{q²}_i                (m_i valid rows of tile i)

    PWT with the per-row diagonal w_{t,j} = ½ Σ_c q_{t,c}² σ²_{j,c} (PWT_ROW) differs only in
    w: dw_{t,j} = φ'(w_{t,j}) dℓ_{t,j} per row, so dq_t += q_t ∘ Σ_j dw_{t,j} σ²_j and
    dσ²_j = ½ Σ_t dw_{t,j} q_t² replace the pooled terms.

    LITERAL (block-wise first order and per-row w_{t,j} = ½ q_tᵀ C_j q_t, PISA paper Eq.
    (3.2) with the blog's PWT weight): the unselected block j adds â_{t,j}(ΣV_j + H_j q_t) to
    o_t and n_j â_{t,j} to the denominator, â = e^{q·k̄_j + φ_{t,j} - lse_t}. Then
        dℓ_{t,j} = â (dO_t·ΣV_j + dO_t·H_j q_t) - n_j â Δ_t      (log-weight s + φ)
        dq_t += dℓ k̄_j + φ' dℓ C_j q_t + â H_jᵀ dO_t
        dk̄_j = Σ_t dℓ q_t,  dΣV_j = Σ_t â dO_t,  dH_j = Σ_t â dO_t q_tᵀ,
        dC_j = ½ Σ_t φ' dℓ q_t q_tᵀ
    and block j's tokens receive, besides dk̄_j / n_j and dΣV_j,
        dk_i += dH_jᵀ (v_i - v̄_j) + (1/n_j)(dC_j + dC_jᵀ)(k_i - k̄_j),  dv_i += dH_j (k_i - k̄_j).
    Returns dict(dQ, dK, dV) [L_pad, d] (zeros on padded slots), O, lse, idx."""
    opts = dict(PRESETS[mode])
    opts.update(overrides)
    virtual = opts.get("virtual", True)
    first = opts.get("first", "none")
    w_kind = opts.get("w_kind", "none")
    w_map = opts.get("w_map", "exp")
    guard = opts.get("guard", "gate")
    literal = first == "block" and w_kind == "row"
    if not (literal or (first in ("none", "global") and w_kind in ("none", "pooled", "rowdiag"))) or \
            opts.get("pooling", "sqmean") != "sqmean" or not opts.get("numerator_w", True):
        raise ValueError("backward covers DROP, PISA, PWT, PWT_ROW and LITERAL")
    if guard not in ("gate", "none"):
        raise ValueError("backward takes the gate or no guard")
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    L_pad, d = Q.shape
    rng = block_ranges(L_pad, B, block_len)
    nb = len(rng)
    st = block_stats(K, V, B, block_len, per_block=literal)
    fwd = attention_head(Q, K, V, B, block_len, K_sel, mode, idx=idx, stats=st, **overrides)
    O, lse, idx = fwd["O"], fwd["lse"], fwd["idx"]
    pq = pool_queries(Q, B, block_len)
    n = st["n"]
    vbar = st["vsum"] / n[:, None]
    hbar = st["hbar"]                                          # H̄[e, c]

    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    dkbar = np.zeros((nb, d))
    dvbar = np.zeros((nb, d))
    dsig2 = np.zeros((nb, d))
    dqsq = np.zeros((nb, d))
    dH = np.zeros((d, d))
    dHb = np.zeros((nb, d, d)) if literal else None            # dH_j[e, c]
    dCb = np.zeros((nb, d, d)) if literal else None
    for i in range(nb):
        s0, m = rng[i]
        l_t = lse[s0:s0 + m]
        live = np.isfinite(l_t)
        if not live.any():
            continue
        q, g, o = Q[s0:s0 + m], dO[s0:s0 + m], O[s0:s0 + m]
        g = np.where(live[:, None], g, 0.0)
        lt = np.where(live, l_t, 0.0)[:, None]
        delta = (g * o).sum(axis=1)
        sel = np.zeros(nb, dtype=bool)
        sel[idx[i][(idx[i] >= 0) & (idx[i] < nb)]] = True
        S = np.flatnonzero(sel)
        dq = np.zeros((m, d))
        if S.size:
            tok = np.concatenate([np.arange(rng[j][0], rng[j][0] + rng[j][1]) for j in S])
            ks, vs = K[tok], V[tok]
            P = np.exp(q @ ks.T - lt)
            dx = P * (g @ vs.T - delta[:, None])
            dq += dx @ ks
            np.add.at(dK, tok, dx.T @ q)
            np.add.at(dV, tok, P.T @ g)
        U = np.flatnonzero(~sel) if virtual else np.zeros(0, dtype=np.int64)
        if U.size:
            s = q @ st["kbar"][U].T
            lnn = np.log(n[U])[None, :]
            if w_kind == "none":
                w = np.zeros_like(s)
            elif w_kind == "pooled":
                w = np.broadcast_to(0.5 * (st["sig2"][U] @ pq["qsq"][i]), s.shape)
            elif w_kind == "rowdiag":
                w = 0.5 * (q ** 2) @ st["sig2"][U].T
            else:                                              # row: ½ q_tᵀ C_j q_t
                w = 0.5 * np.einsum("tc,jce,te->tj", q, st["C"][U], q)
            if w_kind == "none":
                phi = dphi = np.zeros_like(s)
            else:
                fired = (w > lnn) if guard == "gate" else np.zeros(s.shape, dtype=bool)
                w0 = np.where(fired, 0.0, w)
                phi = w0 if w_map == "exp" else np.log1p(w0)
                dphi = np.where(fired, 0.0, 1.0 if w_map == "exp" else 1.0 / (1.0 + w0))
            Pv = np.exp(s + phi + lnn - lt)
            if literal:                                        # H_j q_t per block, [m, |U|, d]
                hq = np.einsum("jec,tc->tje", st["H"][U], q)
                gh = np.einsum("te,tje->tj", g, hq)
                dl = Pv * (g @ vbar[U].T + gh / n[U][None, :] - delta[:, None])
            else:
                u = q @ hbar.T                                 # u_t = H̄ q_t
                gu = (g * u).sum(axis=1) if first == "global" else np.zeros(m)
                dl = Pv * (g @ vbar[U].T + gu[:, None] / n[U][None, :] - delta[:, None])
            dq += dl @ st["kbar"][U]
            dkbar[U] += dl.T @ q
            dvbar[U] += Pv.T @ g
            if literal:
                ahat = Pv / n[U][None, :]                      # e^{s + φ - lse}
                dw = dphi * dl
                dq += np.einsum("tj,jce,te->tc", dw, st["C"][U], q)
                dq += np.einsum("tj,jec,te->tc", ahat, st["H"][U], g)
                dHb[U] += np.einsum("tj,te,tc->jec", ahat, g, q)
                dCb[U] += 0.5 * np.einsum("tj,tc,te->jce", dw, q, q)
            if w_kind == "rowdiag":
                dw = dphi * dl
                dq += q * (dw @ st["sig2"][U])
                dsig2[U] += 0.5 * dw.T @ (q ** 2)
            if first == "global":
                abar = (Pv / n[U][None, :]).sum(axis=1)
                dq += abar[:, None] * (g @ hbar)
                dH += (abar[:, None] * g).T @ q
            if w_kind == "pooled":
                dw = (dphi * dl).sum(axis=0)                   # one value per block, pooled over rows
                dqsq[i] += 0.5 * (dw @ st["sig2"][U])
                dsig2[U] += 0.5 * dw[:, None] * pq["qsq"][i][None, :]
        dQ[s0:s0 + m] += dq

    for i, (s0, m) in enumerate(rng):
        dQ[s0:s0 + m] += (2.0 / m) * Q[s0:s0 + m] * dqsq[i][None, :]
    for j, (s0, nj) in enumerate(rng):
        kd = K[s0:s0 + nj] - st["kbar"][j]
        vd = V[s0:s0 + nj] - vbar[j]
        dK[s0:s0 + nj] += dkbar[j] / nj + (2.0 / nj) * kd * dsig2[j] + vd @ dH / nb
        dV[s0:s0 + nj] += dvbar[j] / nj + kd @ dH.T / nb
        if literal:
            dK[s0:s0 + nj] += vd @ dHb[j] + kd @ (dCb[j] + dCb[j].T) / nj
            dV[s0:s0 + nj] += kd @ dHb[j].T
    return dict(dQ=dQ, dK=dK, dV=dV, O=O, lse=lse, idx=idx)


# ----------------------------------------------------------------------------- second-order matrix
def pooled_w(qsq: np.ndarray, sig2: np.ndarray) -> np.ndarray:
    """w̃_{i,j} = ½ sum_c \\overline{q²}_{i,c} σ²_{j,c}, the [query tile x key block] matrix
    of the diagonal + pooled second-order term (blog, PWT section), before the gate."""
    return 0.5 * np.asarray(qsq, dtype=np.float64) @ np.asarray(sig2, dtype=np.float64).T
