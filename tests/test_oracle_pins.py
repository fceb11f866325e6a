"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage it follows. None of them compares the oracle with itself:
they use closed forms, reductions to a library routine (torch's scaled-dot-product
attention in float64 on the CPU), invariants, the PISA paper's error bound and brute
force on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

from oracle import pisa_oracle as orc

MODES = ["drop", "pisa0", "pisa", "pwt", "literal"]


def sdpa_dense(Q, K, V):
    """Library dense attention (torch, float64, CPU, scale 1: q already carries 1/sqrt(d))."""
    q = torch.from_numpy(np.ascontiguousarray(Q))[None]
    k = torch.from_numpy(np.ascontiguousarray(K))[None]
    v = torch.from_numpy(np.ascontiguousarray(V))[None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=1.0)[0].numpy()


def rand_head(seed, L, d, scale_q=None):
    r = np.random.default_rng(seed)
    sq = 1.0 / math.sqrt(d) if scale_q is None else scale_q
    return r.standard_normal((L, d)) * sq, r.standard_normal((L, d)), r.standard_normal((L, d))


def valid_mask(L_pad, B, block_len):
    m = np.zeros(L_pad, dtype=bool)
    for s, n in orc.block_ranges(L_pad, B, block_len):
        m[s:s + n] = True
    return m


# --------------------------------------------------------------------------- reductions to dense
def test_dense_oracle_matches_library():
    """PISA paper §3.1: O = softmax(QKᵀ)V (scale folded into Q)."""
    Q, K, V = rand_head(1, 96, 16)
    ref = sdpa_dense(Q, K, V)
    got = orc.dense_attention_head(Q, K, V, 8)["O"]
    assert np.abs(got - ref).max() < 1e-13


@pytest.mark.parametrize("mode", MODES)
def test_all_blocks_selected_is_dense(mode):
    """Eq. (3.2) with U_i empty (K_sel = nb) is dense softmax attention, in every mode."""
    B, nb, d = 8, 12, 16
    Q, K, V = rand_head(2, B * nb, d)
    out = orc.attention_head(Q, K, V, B, None, nb, mode)["O"]
    assert np.abs(out - sdpa_dense(Q, K, V)).max() < 1e-12


@pytest.mark.parametrize("mode", ["pisa", "pwt", "literal", "pisa0"])
@pytest.mark.parametrize("K_sel", [0, 3, 7])
def test_block_size_one_is_dense(mode, K_sel):
    """With B = 1 every centroid is its token, H_j = 0 and C_j = 0, so each virtual
    token is exact (blog, Sparse Linear Attention section) for any selection."""
    Q, K, V = rand_head(3, 24, 8)
    out = orc.attention_head(Q, K, V, 1, None, K_sel, mode)["O"]
    assert np.abs(out - sdpa_dense(Q, K, V)).max() < 1e-12


def test_drop_is_not_dense():
    """Keep-or-drop discards the unselected blocks (PISA paper §2, Block Sparse Attention)."""
    Q, K, V = rand_head(3, 24, 8)
    out = orc.attention_head(Q, K, V, 1, None, 3, "drop")["O"]
    assert np.abs(out - sdpa_dense(Q, K, V)).max() > 1e-2


@pytest.mark.parametrize("mode", ["pisa", "pwt", "literal", "pisa0"])
def test_identical_tokens_make_virtual_tokens_exact(mode):
    """If every valid key and value of a block is the same token, the block's mass is
    exactly n_j e^{q·k̄_j} and its numerator n_j e^{q·k̄_j} v (H_j = 0, C_j = 0): the
    virtual token reproduces dense attention. Ragged n_j pin the n_j weighting."""
    r = np.random.default_rng(4)
    B, nb, d = 8, 10, 6
    bl = np.array([8, 3, 8, 1, 5, 8, 2, 8, 7, 4])
    L_pad = B * nb
    Q = r.standard_normal((L_pad, d)) * 0.5
    K = np.zeros((L_pad, d))
    V = np.zeros((L_pad, d))
    for j, (s, n) in enumerate(orc.block_ranges(L_pad, B, bl)):
        K[s:s + n] = r.standard_normal(d)
        V[s:s + n] = r.standard_normal(d)
        K[s + n:s + B] = 99.0      # padding must be ignored
        V[s + n:s + B] = -99.0
    m = valid_mask(L_pad, B, bl)
    ref = sdpa_dense(Q[m], K[m], V[m])
    out = orc.attention_head(Q, K, V, B, bl, 3, mode)["O"][m]
    assert np.abs(out - ref).max() < 1e-12


# --------------------------------------------------------------------------- closed forms
def _two_block_case(seed, d=5, delta_axis=None):
    """Two blocks of B = 2: block 0 = (k0, k1) with values (v0, v1); block 1 = (c+δ, c-δ)
    with values (v2, v3). Query tiles are the same 2-row blocks."""
    r = np.random.default_rng(seed)
    k0, k1, c = r.standard_normal((3, d)) * 0.7
    if delta_axis is None:
        delta = r.standard_normal(d) * 0.4
    else:
        delta = np.zeros(d)
        delta[delta_axis] = 0.6
    v0, v1, v2, v3 = r.standard_normal((4, d))
    q = r.standard_normal((4, d)) * 0.5
    K = np.stack([k0, k1, c + delta, c - delta])
    V = np.stack([v0, v1, v2, v3])
    return q, K, V, dict(k0=k0, k1=k1, c=c, delta=delta, v=(v0, v1, v2, v3))


@pytest.mark.parametrize("mode", ["pisa0", "pisa", "pwt", "literal"])
def test_two_token_block_closed_form(mode):
    """Block 0 exact, block 1 virtual. By hand, for row q (blog, Sparse Linear Attention
    and PWT sections; PISA paper Eq. (3.2)):
      exact part  e^{q·k0} v0 + e^{q·k1} v1,  mass e^{q·k0} + e^{q·k1}
      block 1     s = q·c, y = q·δ, ΣV = v2 + v3, H_1 q = (v2 - v3) y
      H̄ q = ½ (H_0 q + H_1 q),  H_0 q = ½ (v0 - v1) (q·(k0 - k1))
      second order: pooled w̃ = ½ mean_tile(q_a²) δ_a² (δ on one axis a), row w = ½ y²."""
    axis = 2
    Q, K, V, p = _two_block_case(5, delta_axis=axis if mode == "pwt" else None)
    v0, v1, v2, v3 = p["v"]
    idx = np.array([[0], [0]])
    out = orc.attention_head(Q, K, V, 2, None, 1, mode, idx=idx)["O"]
    for t in range(4):
        q = Q[t]
        ex0, ex1 = math.exp(q @ p["k0"]), math.exp(q @ p["k1"])
        s, y = q @ p["c"], q @ p["delta"]
        H0q = 0.5 * (v0 - v1) * (q @ (p["k0"] - p["k1"]))
        H1q = (v2 - v3) * y
        if mode == "pisa0":
            num_v, mass_v = math.exp(s) * (v2 + v3), 2 * math.exp(s)
        elif mode == "pisa":
            num_v = math.exp(s) * (v2 + v3 + 0.5 * (H0q + H1q))
            mass_v = 2 * math.exp(s)
        elif mode == "pwt":
            tile = Q[(t // 2) * 2:(t // 2) * 2 + 2]
            w = 0.5 * np.mean(tile[:, axis] ** 2) * p["delta"][axis] ** 2
            assert w < math.log(2)
            num_v = math.exp(s + w) * (v2 + v3 + 0.5 * (H0q + H1q))
            mass_v = 2 * math.exp(s + w)
        else:
            w = 0.5 * y * y
            if w > math.log(2):
                w = 0.0
            num_v = math.exp(s) * (1 + w) * (v2 + v3 + H1q)
            mass_v = 2 * math.exp(s) * (1 + w)
        ref = (ex0 * v0 + ex1 * v1 + num_v) / (ex0 + ex1 + mass_v)
        assert np.abs(out[t] - ref).max() < 1e-13, (mode, t)


def test_single_virtual_block_is_first_order_tanh():
    """Only one 2-token block, nothing selected: exact o = v̄ + ½(v1 - v2) tanh(q·δ);
    PISA gives its first-order Taylor form v̄ + ½(v1 - v2)(q·δ) (blog, Sparse Linear
    Attention section: zeroth + first order)."""
    r = np.random.default_rng(6)
    d = 7
    c, delta = r.standard_normal(d), r.standard_normal(d) * 0.3
    v1, v2 = r.standard_normal((2, d))
    Q = r.standard_normal((2, d))
    K = np.stack([c + delta, c - delta])
    V = np.stack([v1, v2])
    out = orc.attention_head(Q, K, V, 2, None, 0, "pisa")["O"]
    for t in range(2):
        y = Q[t] @ delta
        assert np.abs(out[t] - (0.5 * (v1 + v2) + 0.5 * (v1 - v2) * y)).max() < 1e-13
    dense = sdpa_dense(Q, K, V)
    y = Q @ delta
    assert np.abs(dense - (0.5 * (v1 + v2) + 0.5 * (v1 - v2) * np.tanh(y)[:, None])).max() < 1e-13


def test_second_order_mass_is_cosh_expansion():
    """Exact mass of block k̄ ± δ is 2e^{s}cosh(y); the zeroth order 2e^{s} misses it at
    O(y²), PWT's 2e^{s + y²/2} and 1 + w both match through O(y²) (blog, PWT section).
    Measured through the oracle's lse of a lone virtual block against the closed form."""
    d = 4
    c = np.array([0.3, -0.2, 0.1, 0.4])
    for y_target in [0.05, 0.1, 0.2]:
        delta = np.array([1.0, 0.0, 0.0, 0.0]) * y_target
        Q = np.array([[1.0, 0.5, -0.5, 0.25], [1.0, 0.5, -0.5, 0.25]])
        K = np.stack([c + delta, c - delta])
        V = np.ones((2, d))
        s, y = Q[0] @ c, Q[0] @ delta
        l_pisa = orc.attention_head(Q, K, V, 2, None, 0, "pisa")["lse"][0]
        l_pwt = orc.attention_head(Q, K, V, 2, None, 0, "pwt")["lse"][0]
        l_lit = orc.attention_head(Q, K, V, 2, None, 0, "literal")["lse"][0]
        assert abs(l_pisa - (math.log(2) + s)) < 1e-14
        assert abs(l_pwt - (math.log(2) + s + 0.5 * y * y)) < 1e-14
        assert abs(l_lit - (math.log(2) + s + math.log1p(0.5 * y * y))) < 1e-14
        exact = math.log(2) + s + math.log(math.cosh(y))
        assert abs(l_pwt - exact) < 0.1 * y ** 4 and abs(l_lit - exact) < 0.2 * y ** 4
        assert abs(l_pisa - exact) > 0.4 * y ** 2


def test_pooling_is_square_then_mean():
    """Two query rows q and -q: q̄ = 0, so q̄² = 0, while mean(q²) = q² (blog, PWT section:
    pool q² by squaring first). Pin: w̃ = ½ Σ_c q_c² σ²_c enters the virtual logit."""
    d = 3
    q = np.array([0.4, -0.3, 0.2])
    Q = np.stack([q, -q])
    c = np.array([0.1, 0.2, -0.3])
    delta = np.array([0.5, 0.3, -0.2])
    K = np.stack([c + delta, c - delta])
    V = np.ones((2, d))
    lse = orc.attention_head(Q, K, V, 2, None, 0, "pwt")["lse"]
    w = 0.5 * np.sum(q ** 2 * delta ** 2)
    assert abs(lse[0] - (math.log(2) + q @ c + w)) < 1e-14
    assert abs(lse[1] - (math.log(2) - q @ c + w)) < 1e-14
    lse_bad = orc.attention_head(Q, K, V, 2, None, 0, "pwt", pooling="meansq")["lse"]
    assert abs(lse_bad[0] - (math.log(2) + q @ c)) < 1e-14


def test_pooled_w_hand_computed():
    """w̃ for one tile of rows a = (1, 2), b = (3, -2) and one block of keys k̄ ± δ with
    δ = (1, 3), worked by hand (blog, PWT section: ½ Σ_c mean_tile(q_c²) σ²_{j,c}).
    mean(q²) = ((1 + 9)/2, (4 + 4)/2) = (5, 4); σ² = δ² = (1, 9); w̃ = ½ (5·1 + 4·9) = 20.5.
    Pooling q̄² instead would give ½ (4·1 + 0·9) = 2, a dropped ½ gives 41."""
    Q = np.array([[1.0, 2.0], [3.0, -2.0]])
    kbar, delta = np.array([0.25, -0.5]), np.array([1.0, 3.0])
    K = np.stack([kbar + delta, kbar - delta])
    st = orc.block_stats(K, np.zeros((2, 2)), 2)
    pq = orc.pool_queries(Q, 2)
    w = orc.pooled_w(pq["qsq"], st["sig2"])
    assert w.shape == (1, 1)
    assert w[0, 0] == 20.5
    # the PWT logit of that block, seen by row a: q·k̄ + ln 2 + w̃ (gate off: 20.5 > ln 2)
    lse = orc.attention_head(Q, K, np.ones((2, 2)), 2, None, 0, "pwt", guard="none")["lse"]
    assert abs(lse[0] - (Q[0] @ kbar + math.log(2) + 20.5)) < 1e-12


def test_pooled_w_brute_force_loops():
    """Rectangular case (3 tiles, 5 blocks, ragged) against plain loops over the
    definition: w̃_{i,j} = ½ Σ_c [(1/m_i) Σ_t q_{t,c}²] [(1/n_j) Σ_k (k_{k,c} - k̄_{j,c})²]."""
    r = np.random.default_rng(17)
    B, d = 4, 3
    bl = np.array([4, 2, 3, 4, 1])
    Q = r.standard_normal((B * 5, d))
    K = r.standard_normal((B * 5, d))
    st = orc.block_stats(K, np.zeros_like(K), B, bl)
    pq = orc.pool_queries(Q, B, bl)
    tiles = [0, 2, 3]
    w = orc.pooled_w(pq["qsq"][tiles], st["sig2"])
    assert w.shape == (3, 5)
    for a, i in enumerate(tiles):
        for j in range(5):
            tot = 0.0
            for c in range(d):
                msq = sum(Q[i * B + t, c] ** 2 for t in range(bl[i])) / bl[i]
                mean = sum(K[j * B + k, c] for k in range(bl[j])) / bl[j]
                var = sum((K[j * B + k, c] - mean) ** 2 for k in range(bl[j])) / bl[j]
                tot += msq * var
            assert abs(w[a, j] - 0.5 * tot) < 1e-12


@pytest.mark.parametrize("mode", MODES)
def test_constant_values_give_constant_output(mode):
    """Softmax output is a weighted mean: V ≡ u gives o = u exactly, which requires the
    second-order factor on numerator and denominator alike (blog, PWT section) and
    H_j = 0 for constant V."""
    r = np.random.default_rng(7)
    B, nb, d = 8, 9, 6
    bl = np.array([8, 8, 5, 8, 2, 8, 8, 7, 8])
    L_pad = B * nb
    Q = r.standard_normal((L_pad, d))
    K = r.standard_normal((L_pad, d))
    u = r.standard_normal(d)
    V = np.tile(u, (L_pad, 1))
    out = orc.attention_head(Q, K, V, B, bl, 3, mode)["O"]
    m = valid_mask(L_pad, B, bl)
    assert np.abs(out[m] - u).max() < 1e-12
    assert np.all(out[~m] == 0)


def test_literal_numerator_without_second_order_breaks_constant_values():
    """The counter-case of the previous pin: keeping 1+w only in the denominator turns
    o = u into u / (1 + w)-weighted mixtures, so it is not the reading the pages take."""
    r = np.random.default_rng(7)
    B, nb, d = 8, 6, 6
    Q = r.standard_normal((B * nb, d))
    K = r.standard_normal((B * nb, d))
    u = r.standard_normal(d)
    V = np.tile(u, (B * nb, 1))
    out = orc.attention_head(Q, K, V, B, None, 2, "literal", numerator_w=False)["O"]
    assert np.abs(out - u).max() > 1e-3


# --------------------------------------------------------------------------- invariants / bound
def test_zeroth_order_underestimates_mass():
    """Jensen: n_j e^{q·k̄_j} <= Σ_n e^{q·k_{j,n}} (blog, PWT section; PISA paper App. C),
    so D̂ <= D* and 0 <= ζ < 1 for the zeroth-order and drop denominators."""
    B, nb, d = 8, 16, 8
    Q, K, V = rand_head(8, B * nb, d, scale_q=0.6)
    dense = orc.dense_attention_head(Q, K, V, B)["lse"]
    for mode in ["pisa", "pisa0", "drop"]:
        lse = orc.attention_head(Q, K, V, B, None, 4, mode)["lse"]
        zeta = 1 - np.exp(lse - dense)
        assert np.all(zeta >= -1e-12) and np.all(zeta < 1)


def test_second_order_term_is_nonnegative():
    """w = ½ qᵀC_j q >= 0 (C_j is a covariance), and its pooled diagonal form too."""
    r = np.random.default_rng(9)
    K = r.standard_normal((64, 5))
    V = r.standard_normal((64, 5))
    st = orc.block_stats(K, V, 8)
    Q = r.standard_normal((64, 5))
    pq = orc.pool_queries(Q, 8)
    assert np.all(orc.pooled_w(pq["qsq"], st["sig2"]) >= 0)
    for j in range(8):
        assert np.all(np.linalg.eigvalsh(st["C"][j]) > -1e-12)


def test_block_statistics_definitions():
    """k̄_j is the mean, the deviations sum to zero (so the first-order denominator term
    vanishes: blog, Sparse Linear Attention section), and H̄ equals the average over blocks
    of Σ_i v_i(k_i - k̄_j)ᵀ, i.e. (KᵀV - Σ_j n_j k̄_j v̄_jᵀ)ᵀ / nb for full blocks."""
    r = np.random.default_rng(10)
    B, nb, d = 8, 5, 4
    K = r.standard_normal((B * nb, d))
    V = r.standard_normal((B * nb, d))
    st = orc.block_stats(K, V, B)
    for j in range(nb):
        dev = K[j * B:(j + 1) * B] - st["kbar"][j]
        assert np.abs(dev.sum(axis=0)).max() < 1e-13
    alt = (V.T @ K - sum(np.outer(st["vsum"][j], st["kbar"][j]) for j in range(nb))) / nb
    assert np.abs(alt - st["hbar"]).max() < 1e-13
    # covariance against numpy's population covariance
    for j in range(nb):
        assert np.abs(np.cov(K[j * B:(j + 1) * B].T, bias=True) - st["C"][j]).max() < 1e-13
        assert np.abs(np.var(K[j * B:(j + 1) * B], axis=0) - st["sig2"][j]).max() < 1e-13
    lean = orc.block_stats(K, V, B, per_block=False)
    assert lean["H"] is None and np.abs(lean["hbar"] - st["hbar"]).max() < 1e-13


def test_theorem_error_bound():
    """PISA paper Theorem 3.1 / App. C: with α = e^{q·k̄_j}, δ = q·(k - k̄_j),
    ‖ô - o*‖ <= (C_v e^{η} S₂ + ‖R q‖) / D̂,  S₂ = Σ_U α Σ_n δ², η = max |δ|,
    R = Σ_U α (H_j - H̄), for the PISA output ô (global first order, no w)."""
    B, nb, d = 8, 12, 8
    K_sel = 3
    for seed in range(3):
        Q, K, V = rand_head(20 + seed, B * nb, d, scale_q=0.5)
        st = orc.block_stats(K, V, B)
        res = orc.attention_head(Q, K, V, B, None, K_sel, "pisa", stats=st)
        dense = orc.dense_attention_head(Q, K, V, B)["O"]
        Cv = np.linalg.norm(V, axis=1).max()
        for i in range(nb):
            U = [j for j in range(nb) if j not in set(res["idx"][i])]
            for t in range(i * B, (i + 1) * B):
                q = Q[t]
                D_hat = math.exp(res["lse"][t])
                S2, eta, R = 0.0, 0.0, np.zeros((d, d))
                for j in U:
                    alpha = math.exp(q @ st["kbar"][j])
                    delta = (K[j * B:(j + 1) * B] - st["kbar"][j]) @ q
                    S2 += alpha * np.sum(delta ** 2)
                    eta = max(eta, np.abs(delta).max())
                    R += alpha * (st["H"][j] - st["hbar"])
                bound = (Cv * math.exp(eta) * S2 + np.linalg.norm(R @ q)) / D_hat
                err = np.linalg.norm(res["O"][t] - dense[t])
                assert err <= bound * (1 + 1e-12), (seed, t, err, bound)


def test_taylor_error_vanishes_with_block_spread():
    """Keys k = c_j + εξ: the Taylor branch error goes to 0 as ε → 0, at order ε for the
    global-first-order forms (H̄ replaces H_j = O(ε)) and ε² for the block-wise form
    (remainder O(δ²)); dropping blocks keeps an O(1) error (PISA paper §3.3 error
    analysis; blog, PWT section)."""
    r = np.random.default_rng(11)
    B, nb, d = 8, 8, 6
    L = B * nb
    Q = r.standard_normal((L, d)) * 0.8
    V = r.standard_normal((L, d))
    centres = np.repeat(r.standard_normal((nb, d)), B, axis=0)
    xi = r.standard_normal((L, d))
    idx = np.array([[i, (i + 3) % nb] for i in range(nb)])
    idx.sort(axis=1)
    eps = np.array([1 / 8, 1 / 16, 1 / 32, 1 / 64])
    errs = {m: [] for m in ["drop", "pisa", "pwt", "literal"]}
    for e in eps:
        K = centres + e * xi
        dense = orc.dense_attention_head(Q, K, V, B)["O"]
        for m in errs:
            o = orc.attention_head(Q, K, V, B, None, 2, m, idx=idx)["O"]
            errs[m].append(np.linalg.norm(o - dense) / np.linalg.norm(dense))
    slope = {m: np.polyfit(np.log(eps), np.log(errs[m]), 1)[0] for m in errs if m != "drop"}
    assert 0.8 < slope["pisa"] < 1.3 and 0.8 < slope["pwt"] < 1.3
    assert 1.7 < slope["literal"] < 2.4
    assert min(errs["drop"]) > 0.05


# --------------------------------------------------------------------------- gate / outliers
def test_gate_falls_back_to_zeroth_order_on_outliers():
    """Outlier dimensions of magnitude ~10³ in q/k blow w = ½ q²σ² up (blog, PWT section);
    the ln n_j gate zeroes w so PWT equals PISA there, and the output stays finite.
    Clamping instead hands those blocks the uniform e^{ln n_j} = n_j boost."""
    B, nb, d = 8, 8, 8
    Q, K, V = rand_head(12, B * nb, d)
    Q[:, [1, 5]] *= 1e3 / 8
    K[:, [1, 5]] *= 1e3 / 8
    pwt = orc.attention_head(Q, K, V, B, None, 2, "pwt")
    pisa = orc.attention_head(Q, K, V, B, None, 2, "pisa")
    assert np.all(np.isfinite(pwt["O"]))
    st = orc.block_stats(K, V, B)
    w = orc.pooled_w(orc.pool_queries(Q, B)["qsq"], st["sig2"])
    assert np.all(w > math.log(B))          # every block gated
    assert np.abs(pwt["O"] - pisa["O"]).max() < 1e-12
    nogate = orc.attention_head(Q, K, V, B, None, 2, "pwt", guard="none")
    # no guard: w of order 1e4..1e8 nats swamps the exact branch entirely
    assert np.all(nogate["lse"] - pisa["lse"] > 100)


def test_clamp_gives_uniform_block_boost():
    """The rejected clamp holds w at ln n_j, so a block whose w exceeds the limit gets
    weight n_j e^{s + ln n_j}: n_j times PISA's, where the gate gives PISA's own
    (blog, PWT section). One lone 2-token virtual block with w = 5 > ln 2."""
    Q = np.array([[1.0, 0.0], [1.0, 0.0]])
    K = np.array([[math.sqrt(10.0), 0.0], [-math.sqrt(10.0), 0.0]])
    V = np.ones((2, 2))
    s = 0.0
    gate = orc.attention_head(Q, K, V, 2, None, 0, "pwt")["lse"][0]
    clamp = orc.attention_head(Q, K, V, 2, None, 0, "pwt", guard="clamp")["lse"][0]
    assert abs(gate - (math.log(2) + s)) < 1e-14
    assert abs(clamp - (2 * math.log(2) + s)) < 1e-14


def test_gate_threshold_is_strict_and_per_block():
    """w is kept while w <= ln n_j and zeroed once it exceeds it (blog, PWT section)."""
    d = 2
    for target, kept in [(math.log(2) * 0.999, True), (math.log(2) * 1.001, False)]:
        # tile rows q = (1, 0) and (1, 0); σ² on axis 0 set so w = target
        Q = np.array([[1.0, 0.0], [1.0, 0.0]])
        half = math.sqrt(2 * target)
        K = np.array([[half, 0.0], [-half, 0.0]])
        V = np.ones((2, d))
        lse = orc.attention_head(Q, K, V, 2, None, 0, "pwt")["lse"][0]
        expect = math.log(2) + (target if kept else 0.0)
        assert abs(lse - expect) < 1e-12


# --------------------------------------------------------------------------- selection
def test_selection_matches_counting_definition():
    """Block j is selected iff fewer than K_sel blocks beat it, where j' beats j when
    s_{j'} > s_j or (s_{j'} = s_j and j' < j). Scores rounded to force many ties."""
    r = np.random.default_rng(13)
    for K_sel in [0, 1, 5, 17, 31, 32]:
        s = np.round(r.standard_normal((9, 32)), 1)
        got = orc.select_topk(s, K_sel)
        for i in range(9):
            want = [j for j in range(32)
                    if sum(1 for jj in range(32)
                           if s[i, jj] > s[i, j] or (s[i, jj] == s[i, j] and jj < j)) < K_sel]
            assert list(got[i]) == want


def test_duplicated_blocks_tie_to_lower_index():
    """Two blocks with identical keys score identically; the lower index wins."""
    r = np.random.default_rng(14)
    B, nb, d = 4, 6, 5
    K = r.standard_normal((B * nb, d))
    K[4 * B:5 * B] = K[1 * B:2 * B]
    Q = np.tile(K[1 * B:2 * B].mean(axis=0) * 3, (B * nb, 1))   # q̄ aligned with block 1 = 4
    st = orc.block_stats(K, K, B)
    s = orc.block_scores(orc.pool_queries(Q, B)["qbar"], st["kbar"])
    assert s[0, 1] == s[0, 4] and np.argmax(s[0]) in (1, 4)
    idx = orc.select_topk(s, 1)
    assert np.all(idx[:, 0] == 1)


def test_heterogeneity_two_token_closed_form():
    """For a block of two tokens H_j = ½ (v_1 - v_2)(k_1 - k_2)ᵀ, a rank-one matrix, so
    with two blocks H̄ = ½ (H_1 + H_2) and M_1 = M_2 = ½ ||H_1 - H_2||_F; with identical
    blocks M_j = 0 (PISA paper §3.3 Theorem 3.1, M = ||H_j - H̄||)."""
    r = np.random.default_rng(21)
    d = 3
    K = r.standard_normal((4, d))
    V = r.standard_normal((4, d))
    st = orc.block_stats(K, V, 2)
    H1 = 0.5 * np.outer(V[0] - V[1], K[0] - K[1])
    H2 = 0.5 * np.outer(V[2] - V[3], K[2] - K[3])
    m = orc.block_heterogeneity(st)
    want = 0.5 * math.sqrt(float(((H1 - H2) ** 2).sum()))
    assert abs(m[0] - want) < 1e-12 and abs(m[1] - want) < 1e-12
    same = orc.block_stats(np.tile(K[:2], (3, 1)), np.tile(V[:2], (3, 1)), 2)
    assert np.all(orc.block_heterogeneity(same) < 1e-14)


def test_covariance_routing_prefers_heterogeneous_blocks():
    """With equal centroid scores the covariance-aware score (PISA paper Eq. (7)) picks
    the block whose H_j is farthest from H̄; with every M_j equal it selects exactly what
    plain block-mean scoring selects."""
    r = np.random.default_rng(22)
    B, nb, d = 4, 5, 6
    K = np.zeros((B * nb, d))
    V = np.zeros((B * nb, d))
    base = r.standard_normal((B, d))
    for j in range(nb):                       # same centroid everywhere, spread grows with j
        K[j * B:(j + 1) * B] = 1.0 + (j + 1) * 0.1 * (base - base.mean(axis=0))
        V[j * B:(j + 1) * B] = r.standard_normal((B, d))
    V[3 * B:4 * B] *= 10.0                    # block 3: by far the largest H_j
    st = orc.block_stats(K, V, B)
    pq = orc.pool_queries(r.standard_normal((B * nb, d)), B)
    plain = orc.block_scores(pq["qbar"], st["kbar"])
    assert np.allclose(plain, plain[:, :1])   # all blocks tie on the centroid score
    m = orc.block_heterogeneity(st)
    routed = orc.routed_scores(pq["qbar"], st["kbar"], m)
    assert int(np.argmax(m)) == 3
    assert np.all(orc.select_topk(routed, 1)[:, 0] == 3)
    pq2 = orc.pool_queries(r.standard_normal((B * nb, d)), B)
    st2 = orc.block_stats(r.standard_normal((B * nb, d)), V, B)
    a = orc.select_topk(orc.routed_scores(pq2["qbar"], st2["kbar"], np.full(nb, 2.0)), 2)
    b = orc.select_topk(orc.block_scores(pq2["qbar"], st2["kbar"]), 2)
    assert np.array_equal(a, b)


def test_pooled_query_is_valid_row_mean():
    """q̄_i averages only the n_i valid rows of a ragged tile (PISA paper Fig. 3 Q̄)."""
    Q = np.arange(16, dtype=np.float64).reshape(8, 2)
    pq = orc.pool_queries(Q, 4, np.array([3, 4]))
    assert np.allclose(pq["qbar"][0], Q[:3].mean(axis=0))
    assert np.allclose(pq["qsq"][1], (Q[4:8] ** 2).mean(axis=0))


# --------------------------------------------------------------------------- padding / edges
@pytest.mark.parametrize("mode", MODES)
def test_padding_content_is_ignored(mode):
    """Padded slots hold no tokens: any values there leave every valid output unchanged."""
    r = np.random.default_rng(15)
    B, nb, d = 8, 7, 5
    bl = np.array([8, 3, 8, 6, 1, 8, 4])
    L_pad = B * nb
    Q, K, V = (r.standard_normal((L_pad, d)) for _ in range(3))
    m = valid_mask(L_pad, B, bl)
    a = orc.attention_head(Q, K, V, B, bl, 2, mode)
    for X in (Q, K, V):
        X[~m] = r.standard_normal(X[~m].shape) * 50
    b = orc.attention_head(Q, K, V, B, bl, 2, mode)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.abs(a["O"] - b["O"]).max() < 1e-12
    assert np.all(b["O"][~m] == 0) and np.all(np.isneginf(b["lse"][~m]))


def test_empty_support_outputs_zero():
    """DROP with K_sel = 0 leaves a row with no keys: output 0, lse = -inf (our reading)."""
    Q, K, V = rand_head(16, 32, 4)
    r = orc.attention_head(Q, K, V, 8, None, 0, "drop")
    assert np.all(r["O"] == 0) and np.all(np.isneginf(r["lse"]))


def test_ksel_zero_is_pure_virtual_attention():
    """K_sel = 0: every block is a virtual token; with B = 1 that is dense attention."""
    Q, K, V = rand_head(17, 16, 4)
    out = orc.attention_head(Q, K, V, 1, None, 0, "pisa")["O"]
    assert np.abs(out - sdpa_dense(Q, K, V)).max() < 1e-12


# --------------------------------------------------------------------------- relative quality
def _tiny_errors():
    from block_sparse_attention_43_amd import synth
    inp = synth.make("tiny")
    Q, K, V = inp.f64("Q", 0), inp.f64("K", 0), inp.f64("V", 0)
    dense = orc.dense_attention_head(Q, K, V, 64)["O"]
    err = {}
    for m in ["drop", "pisa0", "pisa", "pwt", "literal"]:
        o = orc.attention_head(Q, K, V, 64, None, inp.K_sel, m)["O"]
        err[m] = np.linalg.norm(o - dense) / np.linalg.norm(dense)
    o = orc.attention_head(Q, K, V, 64, None, inp.K_sel, "pwt", pooling="meansq")["O"]
    err["pwt_meansq"] = np.linalg.norm(o - dense) / np.linalg.norm(dense)
    return err


def test_error_ordering_on_gaussian_inputs():
    """Qualitative claims (numbers unpinned): zeroth order beats dropping, the global first
    order improves on it, the block-wise form improves further (PISA paper Table 8
    ordering); PWT beats PISA on random Gaussian inputs and pooled mean-of-squares
    beats square-of-mean (blog, PWT section)."""
    e = _tiny_errors()
    assert e["drop"] > e["pisa0"] > e["pisa"] > e["literal"]
    assert e["pwt"] < e["pisa"]
    assert e["pwt"] < e["pwt_meansq"]


def test_error_routing_mass_term_prefers_larger_blocks():
    """Blocks of one repeated token (k0, v0) but different valid counts: centroids,
    w̃ = 0 and M_j = 0 all tie, so routing by predicted truncation error (blog, PWT
    section) ranks the blocks by their mass n_j alone, ties to the lower index, while
    block-mean scores agree up to rounding."""
    r = np.random.default_rng(23)
    B, d = 8, 5
    bl = np.array([2, 8, 3, 8, 1, 5])
    nb = len(bl)
    k0, v0 = r.standard_normal(d), r.standard_normal(d)
    K = np.tile(k0, (B * nb, 1))
    V = np.tile(v0, (B * nb, 1))
    st = orc.block_stats(K, V, B, bl)
    m = orc.block_heterogeneity(st)
    assert np.all(m < 1e-12)
    pq = orc.pool_queries(r.standard_normal((B * nb, d)), B, bl)
    w = orc.pooled_w(pq["qsq"], st["sig2"])
    assert np.all(np.abs(w) < 1e-12)
    s = orc.error_routed_scores(pq["qbar"], st["kbar"], w, bl, m)
    assert np.all(orc.select_topk(s, 1)[:, 0] == 1)
    assert np.all(orc.select_topk(s, 3) == [1, 3, 5])
    plain = orc.block_scores(pq["qbar"], st["kbar"])
    assert np.allclose(plain, plain[:, :1], rtol=1e-12, atol=1e-12)


def test_error_routing_second_order_term_prefers_wider_blocks():
    """V = 0 makes every H_j and M_j zero; keys share one centroid with a spread growing
    with j, so the second-order mass w̃_{i,j} = ½ Σ_c mean(q_c²) σ²_{j,c} grows with j and
    alone decides the routing: the widest blocks win, in every tile."""
    r = np.random.default_rng(24)
    B, nb, d = 4, 6, 5
    c = r.standard_normal(d)
    u = r.standard_normal((B, d))
    u -= u.mean(axis=0)
    K = np.concatenate([c + 0.2 * (j + 1) * u for j in range(nb)])
    V = np.zeros((B * nb, d))
    st = orc.block_stats(K, V, B)
    m = orc.block_heterogeneity(st)
    assert np.all(m == 0.0)
    pq = orc.pool_queries(r.standard_normal((B * nb, d)), B)
    w = orc.pooled_w(pq["qsq"], st["sig2"])
    assert np.all(np.diff(w, axis=1) > 0)
    s = orc.error_routed_scores(pq["qbar"], st["kbar"], w, np.full(nb, B), m)
    assert np.all(orc.select_topk(s, 2) == [nb - 2, nb - 1])
    # the same blocks under Eq. (7)'s score tie (equal centroids, equal M_j): lowest indices
    assert np.all(orc.select_topk(orc.routed_scores(pq["qbar"], st["kbar"], m), 2) == [0, 1])


def _grid_positions(grid):
    t, h, w = np.meshgrid(*[np.arange(n) for n in grid], indexing="ij")
    return np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1).astype(np.float64)


def test_rope_scores_with_one_token_blocks_are_rotated_dot_products():
    """B = 1: every block is one token at its own position, so the RoPE-aware score must be
    the dot product of the rotated query and key, here rotated by the input generator's own
    3D rotary embedding (written apart from the oracle)."""
    from block_sparse_attention_43_amd import synth
    r = np.random.default_rng(25)
    grid, d = (2, 3, 4), 16
    widths = (4, 6, 6)
    pos = _grid_positions(grid)
    q, k = r.standard_normal((24, d)), r.standard_normal((24, d))
    qr, kr = synth._rope_3d(q, grid, widths), synth._rope_3d(k, grid, widths)
    s = orc.rope_block_scores(q, k, pos, 1, None, widths, synth.ROPE_BASE)
    assert np.allclose(s, qr @ kr.T, rtol=1e-12, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    """Shifting every position by one vector leaves all scores unchanged (R_aᵀR_b = R_{b-a});
    with every position at 0 the scores are plain block-mean scores of the pre-rotation
    rows; the half-split pairing is the adjacent pairing of permuted dims."""
    r = np.random.default_rng(26)
    B, nb, d = 8, 5, 12
    widths = (4, 4, 4)
    bl = np.array([8, 3, 8, 5, 8])
    pos = r.uniform(0, 20, size=(B * nb, 3))
    Q, K = r.standard_normal((B * nb, d)), r.standard_normal((B * nb, d))
    s = orc.rope_block_scores(Q, K, pos, B, bl, widths, 100.0)
    s2 = orc.rope_block_scores(Q, K, pos + np.array([7.0, -3.5, 11.25]), B, bl, widths, 100.0)
    assert np.allclose(s, s2, rtol=1e-11, atol=1e-11)
    z = orc.rope_block_scores(Q, K, np.zeros_like(pos), B, bl, widths, 100.0)
    pq = orc.pool_queries(Q, B, bl)
    kb = orc.block_stats(K, np.zeros_like(K), B, bl, per_block=False)["kbar"]
    assert np.allclose(z, orc.block_scores(pq["qbar"], kb), rtol=1e-12, atol=1e-12)
    perm = np.concatenate([o + np.concatenate([np.arange(0, w, 2), np.arange(1, w, 2)])
                           for o, w in zip((0, 4, 8), widths)])
    h = orc.rope_block_scores(Q[:, perm], K[:, perm], pos, B, bl, widths, 100.0, pairs="half")
    assert np.allclose(h, s, rtol=1e-12, atol=1e-12)


def test_rope_centroid_undoes_the_rotation_mixture():
    """Keys that are one vector before the rotary embedding: the RoPE-aware score is
    q̄·R_{c_j - c_i} k exactly, while the mean of the rotated keys (a mixture of rotations)
    gives a different value: the distortion the rotation-aware centroid removes."""
    r = np.random.default_rng(27)
    B, nb, d = 8, 3, 8
    widths = (8,)
    pos = np.arange(B * nb, dtype=np.float64)[:, None]
    k = r.standard_normal(d)
    K = np.tile(k, (B * nb, 1))
    Q = np.tile(r.standard_normal(d), (B * nb, 1))
    s = orc.rope_block_scores(Q, K, pos, B, None, widths, 10.0)
    c = pos.reshape(nb, B).mean(axis=1)
    for i in range(nb):
        for j in range(nb):
            want = Q[0] @ orc.rope_rotate(k[None, :], np.array([[c[j] - c[i]]]), widths, 10.0)[0]
            assert abs(s[i, j] - want) < 1e-12
    post = orc.block_scores(orc.rope_rotate(Q, pos, widths, 10.0).reshape(nb, B, d).mean(axis=1),
                            orc.rope_rotate(K, pos, widths, 10.0).reshape(nb, B, d).mean(axis=1))
    assert np.abs(post - s).max() > 1e-3


def test_per_row_diagonal_w_reduces_to_pooled_and_to_full_quadratic_form():
    """Per-row diagonal w_{t,j} = ½ Σ_c q_{t,c}² σ²_{j,c} (blog, PWT section ablation):
    (1) tiles whose rows are ±q share q² row by row, so it equals the tile-pooled w̃ (PWT);
    (2) blocks whose keys deviate along one coordinate only have a diagonal C_j, so it
    equals the full per-row form ½ q_tᵀ C_j q_t (used with the same global first order)."""
    r = np.random.default_rng(28)
    B, nb, d = 4, 6, 6
    q = r.standard_normal((nb, d))
    Q = np.concatenate([np.stack([q[i], -q[i], q[i], -q[i]]) for i in range(nb)]) * 0.7
    K = r.standard_normal((B * nb, d))
    V = r.standard_normal((B * nb, d))
    a = orc.attention_head(Q, K, V, B, None, 2, "pwt_row")
    b = orc.attention_head(Q, K, V, B, None, 2, "pwt")
    assert np.allclose(a["O"], b["O"], rtol=1e-12, atol=1e-12)
    Kd = np.repeat(r.standard_normal((nb, d)), B, axis=0)
    for j in range(nb):                               # block j varies along coordinate j % d
        Kd[j * B:(j + 1) * B, j % d] += r.standard_normal(B) * 0.8
    Q2 = r.standard_normal((B * nb, d)) * 0.7
    c = orc.attention_head(Q2, Kd, V, B, None, 2, "pwt_row")
    e = orc.attention_head(Q2, Kd, V, B, None, 2, "pwt", w_kind="row")
    assert np.allclose(c["O"], e["O"], rtol=1e-12, atol=1e-12)
    f = orc.attention_head(Q2, Kd, V, B, None, 2, "pwt")          # pooled differs here
    assert np.abs(f["O"] - c["O"]).max() > 1e-6


def _fd_grads(Q, K, V, dO, B, bl, K_sel, mode, idx, eps=1e-6, **kw):
    def loss(q, k, v):
        return float((dO * orc.attention_head(q, k, v, B, bl, K_sel, mode, idx=idx, **kw)["O"]).sum())
    out = []
    for which in range(3):
        X = (Q, K, V)[which]
        fd = np.zeros_like(X)
        for t in range(X.shape[0]):
            for c in range(X.shape[1]):
                args_p = [Q, K, V]
                args_m = [Q, K, V]
                Xp, Xm = X.copy(), X.copy()
                Xp[t, c] += eps
                Xm[t, c] -= eps
                args_p[which], args_m[which] = Xp, Xm
                fd[t, c] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        out.append(fd)
    return out


@pytest.mark.parametrize("mode,kw", [("drop", {}), ("pisa", {}), ("pwt", {}), ("pwt", dict(w_map="linear")),
                                     ("pwt", dict(guard="none")), ("pwt_row", {}), ("pwt_row", dict(w_map="linear")),
                                     ("pwt_row", dict(guard="none")), ("literal", {}), ("literal", dict(w_map="exp")),
                                     ("literal", dict(guard="none"))])
def test_backward_matches_finite_differences(mode, kw):
    """The analytic gradients (selection and gate decisions held fixed) against central
    differences of the forward definition itself, ragged blocks included; one block's keys
    are spread so widely that its w exceeds ln n_j for some rows or tiles (the gate fires
    there) while other pairs stay below it."""
    r = np.random.default_rng(29)
    B, nb, d = 4, 5, 3
    bl = np.array([4, 2, 4, 3, 1])
    Q = r.standard_normal((B * nb, d)) * 0.8
    K = r.standard_normal((B * nb, d))
    K[8:12] *= 4.0                                   # block 2: large σ², gated in PWT
    V = r.standard_normal((B * nb, d))
    dO = r.standard_normal((B * nb, d))
    g = orc.attention_head_backward(Q, K, V, dO, B, bl, 2, mode, **kw)
    if mode != "drop" and mode != "pisa" and kw.get("guard", "gate") == "gate":
        st = orc.block_stats(K, V, B, bl, per_block=True)
        if mode == "pwt":
            w = orc.pooled_w(orc.pool_queries(Q, B, bl)["qsq"], st["sig2"])
        elif mode == "pwt_row":
            w = 0.5 * (Q ** 2) @ st["sig2"].T
        else:
            w = 0.5 * np.einsum("tc,jce,te->tj", Q, st["C"], Q)
        assert (w > np.log(st["n"])[None, :]).any() and (w < np.log(st["n"])[None, :]).any()
    fd = _fd_grads(Q, K, V, dO, B, bl, 2, mode, g["idx"], **kw)
    for name, a, b in zip(("dQ", "dK", "dV"), (g["dQ"], g["dK"], g["dV"]), fd):
        assert np.abs(a - b).max() <= 1e-7 * (np.abs(b).max() + 1.0), name


def test_backward_with_every_block_selected_is_dense_attention_gradient():
    """K_sel = nb: every mode is dense softmax attention, whose gradients torch's autograd
    gives in float64 (a library routine); padded keys and rows excluded."""
    import torch
    r = np.random.default_rng(30)
    B, nb, d = 4, 4, 5
    bl = np.array([4, 3, 4, 2])
    ok = (np.arange(B)[None, :] < bl[:, None]).reshape(-1)
    Q, K, V, dO = (r.standard_normal((B * nb, d)) for _ in range(4))
    q, k, v = (torch.tensor(x[ok], requires_grad=True) for x in (Q, K, V))
    o = torch.softmax(q @ k.T, dim=-1) @ v
    o.backward(torch.tensor(dO[ok]))
    for mode in ("drop", "pisa", "pwt", "pwt_row", "literal"):
        g = orc.attention_head_backward(Q, K, V, dO, B, bl, nb, mode)
        for a, t in ((g["dQ"], q), (g["dK"], k), (g["dV"], v)):
            assert np.allclose(a[ok], t.grad.numpy(), rtol=1e-10, atol=1e-12)
            assert np.all(a[~ok] == 0.0)


@pytest.mark.parametrize("grid", [(5, 6, 7), (8, 8, 8), (1, 3, 9), (21, 30, 52)])
def test_cube_order_is_a_padded_bijection(grid):
    """Every token appears in exactly one slot, each block holds the tokens of one 4x4x4 cube
    (coordinates within one cube's box), valid tokens come first, and block lengths count
    them; to_blocks / from_blocks round-trip."""
    perm, n = orc.cube_order(grid)
    T, Hh, W = grid
    L = T * Hh * W
    assert perm.size == n.size * 64 and n.sum() == L
    assert np.array_equal(np.sort(perm[perm >= 0]), np.arange(L))
    for j in range(n.size):
        blk = perm[j * 64:(j + 1) * 64]
        assert np.all(blk[:n[j]] >= 0) and np.all(blk[n[j]:] == -1)
        t, r = np.divmod(blk[:n[j]], Hh * W)
        h, w = np.divmod(r, W)
        for c in (t, h, w):
            assert c.max() // 4 == c.min() // 4
    x = np.random.default_rng(31).standard_normal((2, L, 3))
    y = orc.to_blocks(x, perm)
    assert np.all(y[:, perm < 0] == 0)
    assert np.array_equal(orc.from_blocks(y, perm, L), x)
