"""Helpers shared by the GPU parity tests: moving canonical inputs to the device, running
the three library calls, and comparing with the oracle."""
from __future__ import annotations

import numpy as np
import torch

from block_sparse_attention_43_amd import synth

MODE_NAMES = ["drop", "pisa", "pwt", "literal", "pwt_row"]


def to_device(inp: synth.Inputs):
    """Canonical host arrays -> CUDA tensors (bf16 bits reinterpreted, no rounding)."""
    def conv(x):
        t = torch.from_numpy(np.ascontiguousarray(x))
        if inp.cfg.dtype == "bf16":
            t = t.view(torch.bfloat16)
        return t.cuda()
    Q, K, V = conv(inp.Q), conv(inp.K), conv(inp.V)
    bl = inp.layout.block_len
    blt = None if (bl == synth.B_DEFAULT).all() else torch.from_numpy(bl.astype(np.int32)).cuda()
    return Q, K, V, blt


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def gpu_run(pisa, inp: synth.Inputs, mode: str, K_sel: int, flags: int = 0, mode_bits: int = 0,
            tensors=None, route: str = "mean"):
    Q, K, V, blt = tensors if tensors is not None else to_device(inp)
    base = pisa.MODES[mode]
    if route != "mean":
        flags |= pisa.STATS_HNORM
    st = pisa.block_stats(K, V, blt, flags=flags)
    idx, mask, wt = pisa.select_topk(Q, st, K_sel, blt, want_wt=True, route=route)
    O, lse = pisa.attention_fwd(Q, K, V, st, idx, mask, wt if base == pisa.MODE_PWT else None, K_sel,
                                base | mode_bits, blt)
    torch.cuda.synchronize()
    return dict(O=to_f64(O), lse=to_f64(lse), idx=idx.cpu().numpy().astype(np.int64),
                mask=mask.cpu().numpy().view(np.uint32), wt=to_f64(wt),
                kbar=to_f64(st.kbar), vsum=to_f64(st.vsum), ksig2=to_f64(st.ksig2),
                hbarT=to_f64(st.hbarT),
                hblk=None if st.hblk is None else to_f64(st.hblk),
                cblk=None if st.cblk is None else to_f64(st.cblk),
                hnorm=None if st.hnorm is None else to_f64(st.hnorm))


def oracle_scores(inp: synth.Inputs, h: int, route: str = "mean"):
    """The oracle's block scores of head h (block-mean, covariance-aware or predicted
    error, with its own M_j) and its PWT weights, from the seeded inputs only."""
    from oracle import pisa_oracle as orc
    bl = inp.layout.block_len
    st = orc.block_stats(inp.f64("K", h), inp.f64("V", h), 64, bl, per_block=(route != "mean"))
    pq = orc.pool_queries(inp.f64("Q", h), 64, bl)
    w = orc.pooled_w(pq["qsq"], st["sig2"])
    if route == "covariance":
        s = orc.routed_scores(pq["qbar"], st["kbar"], orc.block_heterogeneity(st))
    elif route == "error":
        s = orc.error_routed_scores(pq["qbar"], st["kbar"], w, bl, orc.block_heterogeneity(st))
    else:
        s = orc.block_scores(pq["qbar"], st["kbar"])
    return s, w


def oracle_selection(inp: synth.Inputs, K_sel: int, route: str = "mean"):
    """The oracle's own selection and PWT weights for every head, from the seeded inputs
    only: idx [H, nb, K_sel] (ascending) and w [H, nb, nb] (before the gate)."""
    from oracle import pisa_oracle as orc
    idx = np.zeros((inp.H, inp.nb, K_sel), dtype=np.int64)
    w = np.zeros((inp.H, inp.nb, inp.nb))
    for h in range(inp.H):
        s, w[h] = oracle_scores(inp, h, route)
        idx[h] = orc.select_topk(s, K_sel)
    return idx, w


def selection_to_device(idx: np.ndarray, w: np.ndarray, nb: int):
    """Host selection -> the device tensors the attention call takes: idx int32, the
    membership bitmask [H, nb, ceil(nb / 32)] and fp32 weights."""
    H, nq, K_sel = idx.shape
    nw = (nb + 31) // 32
    member = np.zeros((H, nq, nw * 32), dtype=bool)
    hh, ii, kk = np.nonzero((idx >= 0) & (idx < nb))
    member[hh, ii, idx[hh, ii, kk]] = True
    mask = np.packbits(member, axis=-1, bitorder="little").view(np.uint32).reshape(H, nq, nw)
    di = torch.zeros(H, nq, max(K_sel, 1), dtype=torch.int32)
    di[:, :, :K_sel] = torch.from_numpy(idx.astype(np.int32))
    return (di.cuda()[:, :, :K_sel],
            torch.from_numpy(mask.view(np.int32)).cuda(),
            torch.from_numpy(w.astype(np.float32)).cuda())


def gpu_attention_on(pisa, inp: synth.Inputs, K_sel: int, mode: str, idx: np.ndarray, w: np.ndarray,
                     mode_bits: int = 0, tensors=None, flags: int = 0):
    """GPU statistics and attention on a given (oracle) selection."""
    Q, K, V, blt = tensors if tensors is not None else to_device(inp)
    base = pisa.MODES[mode]
    st = pisa.block_stats(K, V, blt, flags=flags)
    di, dm, dw = selection_to_device(idx, w, inp.nb)
    O, lse = pisa.attention_fwd(Q, K, V, st, di, dm, dw if base == pisa.MODE_PWT else None, K_sel,
                                base | mode_bits, blt)
    torch.cuda.synchronize()
    return dict(O=to_f64(O), lse=to_f64(lse))


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def valid_rows(inp: synth.Inputs) -> np.ndarray:
    bl = inp.layout.block_len
    return (np.arange(synth.B_DEFAULT)[None, :] < bl[:, None]).reshape(-1)


def mask_to_sets(mask: np.ndarray, nb: int):
    bits = np.unpackbits(mask.view(np.uint8), bitorder="little")
    return bits.reshape(mask.shape[:-1] + (-1,))[..., :nb].astype(bool)


def check_selection(gpu_idx: np.ndarray, scores: np.ndarray, K_sel: int, rtol: float = 2e-6, rows=None):
    """GPU selection (fp32 scores) against fp64 oracle scores (``scores`` row r belongs
    to tile rows[r]). Where the gap between the
    K_sel-th and the next score exceeds the fp32 rounding bound the sets must be equal;
    inside the bound any choice among the near-tied blocks is valid (and counted), except
    at an exact tie of the fp64 scores (gap 0), where the lower-index rule decides and
    the sets must be equal. Returns (n_exact_tiles, n_near_tie_tiles, min_gap)."""
    nq, nb = scores.shape
    rows = range(nq) if rows is None else rows
    exact = near = 0
    min_gap = np.inf
    for r, i in enumerate(rows):
        s = scores[r]
        got = set(int(x) for x in gpu_idx[i])
        assert len(got) == K_sel and list(gpu_idx[i]) == sorted(got), "indices must be ascending and unique"
        if K_sel in (0, nb):
            assert got == set(range(nb)) if K_sel == nb else not got
            exact += 1
            continue
        order = np.lexsort((np.arange(nb), -s))
        want = set(int(x) for x in order[:K_sel])
        kth, nxt = s[order[K_sel - 1]], s[order[K_sel]]
        tol = rtol * (np.abs(s).max() + 1e-30)
        gap = kth - nxt
        min_gap = min(min_gap, gap)
        if gap > tol or gap == 0.0:
            assert got == want, f"tile {i}: selection differs with gap {gap:.3e} (tol {tol:.3e})"
            exact += 1
        else:
            lo = nxt - tol
            assert all(s[j] >= lo for j in got), f"tile {i}: selected a block below the near-tie band"
            assert all(j in got for j in range(nb) if s[j] > kth + tol), f"tile {i}: missed a clear winner"
            near += 1
    return exact, near, min_gap


def small_case(name):
    """Seeded parity case by name: (inputs, K_sel). Several tiles, ragged blocks, both
    dtypes and head sizes, a partial centroid group (nb = 70, 130)."""
    if name == "tiny":
        return synth.make("tiny"), 4
    if name == "bf16_d128_ragged":
        bl = [64, 64, 17, 64, 1, 64, 40, 64, 64, 33]
        return synth.random_blocks(101, H=2, nb=10, d=128, dtype="bf16", block_len=bl, smooth=2.0), 3
    if name == "bf16_d64":
        return synth.random_blocks(102, H=3, nb=7, d=64, dtype="bf16", smooth=2.0), 2
    if name == "f32_d128_ragged":
        bl = [64, 8, 64, 64, 50, 64, 64, 2, 64]
        return synth.random_blocks(103, H=2, nb=9, d=128, dtype="f32", block_len=bl, smooth=2.0), 4
    if name == "bf16_nb70":
        return synth.random_blocks(104, H=1, nb=70, d=128, dtype="bf16", smooth=2.0), 9
    if name == "f32_d64_ragged_nb130":
        bl = np.full(130, 64)
        bl[[3, 64, 129]] = [5, 63, 1]
        return synth.random_blocks(105, H=1, nb=130, d=64, dtype="f32", block_len=bl, smooth=1.0), 13
    raise KeyError(name)


CASES = ["tiny", "bf16_d128_ragged", "bf16_d64", "f32_d128_ragged", "bf16_nb70", "f32_d64_ragged_nb130"]
