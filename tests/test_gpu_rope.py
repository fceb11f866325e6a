"""GPU parity of RoPE-aware centroids (Sparse Linear Attention (2) blog, Selection Error):
selection scored on pre-rotation block means turned at the block centres, against the
oracle, on small rotary workloads (both dim pairings, both head sizes) and on the full
HunyuanVideo-like workload (sampled tiles), plus attention on the resulting selection.

Bars: selection bit-exact wherever the score gap exceeds the band of fp32 sums and an
fp32 rotation (relative 1e-5 of the row's largest score); near ties are validated and
counted. w̃ (from the rotated Q) within rel-L2 1e-5. Outputs on the routed selection as
for block-mean scoring (bf16 2e-2 end to end, 1e-2 on the oracle's selection).
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_43_amd import synth
from oracle import pisa_oracle as orc
from helpers import check_selection, mask_to_sets, rel_l2, selection_to_device, to_device, valid_rows

pytestmark = pytest.mark.gpu

RTOL = 1e-5

SMALL = {
    "d64": synth.Config("rope_d64", H=2, d=64, dtype="bf16", kind="video", seed=141, grid=(6, 10, 12),
                        keep=0.2, n_modes=8, noise_var=0.5, rope=True, rope_split=(16, 24, 24)),
    "d128": synth.Config("rope_d128", H=2, d=128, dtype="bf16", kind="video", seed=142, grid=(5, 9, 13),
                         keep=0.15, n_modes=8, noise_var=0.5, rope=True),
}


def _device_rope(inp):
    conv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).view(torch.bfloat16).cuda()
    return conv(inp.extra["Q_pre"]), conv(inp.extra["K_pre"]), torch.from_numpy(inp.extra["pos"]).cuda()


def _oracle_rope_scores(inp, h, pairs, rows=None):
    widths = synth.rope_split_for(inp.cfg)
    s = orc.rope_block_scores(synth.to_float64(inp.extra["Q_pre"][h], "bf16"),
                              synth.to_float64(inp.extra["K_pre"][h], "bf16"), inp.extra["pos"], 64,
                              inp.layout.block_len, widths, synth.ROPE_BASE, pairs)
    return s if rows is None else s[rows]


def _gpu_rope_select(pisa, inp, tensors, pairs, want_wt=True):
    Q, K, V, blt = tensors
    Qp, Kp, pos = _device_rope(inp)
    st = pisa.block_stats(K, V, blt)
    idx, mask, wt = pisa.select_topk_rope(Q if want_wt else None, Qp, Kp, pos, synth.rope_split_for(inp.cfg),
                                          synth.ROPE_BASE, st, inp.K_sel, blt, pairs=pairs, want_wt=want_wt)
    torch.cuda.synchronize()
    return st, idx, mask, wt


@pytest.mark.parametrize("pairs", ["adjacent", "half"])
@pytest.mark.parametrize("case", list(SMALL))
def test_rope_selection_parity(gpu_lib, case, pairs):
    inp = synth.make(SMALL[case], keep_pre_rope=True)
    tensors = to_device(inp)
    st, idx, mask, wt = _gpu_rope_select(gpu_lib, inp, tensors, pairs)
    idx_h, sets = idx.cpu().numpy(), mask_to_sets(mask.cpu().numpy().view(np.uint32), inp.nb)
    bl = inp.layout.block_len
    changed = 0
    for h in range(inp.H):
        s = _oracle_rope_scores(inp, h, pairs)
        exact, near, gap = check_selection(idx_h[h], s, inp.K_sel, rtol=RTOL)
        print(f"{case} {pairs} h{h}: {exact} tiles bit-exact, {near} near ties, min gap {gap:.3e}")
        for i in range(inp.nb):
            assert set(np.flatnonzero(sets[h, i])) == set(idx_h[h, i])
        ost = orc.block_stats(inp.f64("K", h), inp.f64("V", h), 64, bl, per_block=False)
        pq = orc.pool_queries(inp.f64("Q", h), 64, bl)
        assert rel_l2(wt[h].cpu().numpy(), orc.pooled_w(pq["qsq"], ost["sig2"])) < 1e-5
        plain = orc.select_topk(orc.block_scores(pq["qbar"], ost["kbar"]), inp.K_sel)
        changed += int(np.any(plain != orc.select_topk(s, inp.K_sel), axis=1).sum())
    print(f"{case} {pairs}: tiles whose selection the rotation-aware centroids change: {changed}")


def test_rope_selection_without_wt_skips_q(gpu_lib):
    """Q may be absent when w̃ is not requested; the selection is the same."""
    inp = synth.make(SMALL["d128"], keep_pre_rope=True)
    tensors = to_device(inp)
    _, idx_a, mask_a, _ = _gpu_rope_select(gpu_lib, inp, tensors, "adjacent", want_wt=True)
    _, idx_b, mask_b, wt_b = _gpu_rope_select(gpu_lib, inp, tensors, "adjacent", want_wt=False)
    assert wt_b is None
    assert torch.equal(idx_a, idx_b) and torch.equal(mask_a, mask_b)


@pytest.mark.parametrize("mode", ["pisa", "pwt"])
def test_rope_attention_parity(gpu_lib, mode):
    inp = synth.make(SMALL["d128"], keep_pre_rope=True)
    tensors = to_device(inp)
    Q, K, V, blt = tensors
    st, idx, mask, wt = _gpu_rope_select(gpu_lib, inp, tensors, "adjacent")
    O, _ = gpu_lib.attention_fwd(Q, K, V, st, idx, mask, wt if mode == "pwt" else None, inp.K_sel, mode, blt)
    bl = inp.layout.block_len
    sel = np.stack([orc.select_topk(_oracle_rope_scores(inp, h, "adjacent"), inp.K_sel) for h in range(inp.H)])
    w = np.stack([orc.pooled_w(orc.pool_queries(inp.f64("Q", h), 64, bl)["qsq"],
                               orc.block_stats(inp.f64("K", h), inp.f64("V", h), 64, bl, per_block=False)["sig2"])
                  for h in range(inp.H)])
    di, dm, dw = selection_to_device(sel, w, inp.nb)
    O2, _ = gpu_lib.attention_fwd(Q, K, V, st, di, dm, dw if mode == "pwt" else None, inp.K_sel, mode, blt)
    torch.cuda.synchronize()
    ok = valid_rows(inp)
    for h in range(inp.H):
        ref = orc.attention_head(inp.f64("Q", h), inp.f64("K", h), inp.f64("V", h), 64, bl, inp.K_sel, mode,
                                 idx=sel[h])
        e_own = rel_l2(O[h].float().cpu().numpy()[ok], ref["O"][ok])
        e_same = rel_l2(O2[h].float().cpu().numpy()[ok], ref["O"][ok])
        print(f"{mode} h{h}: rel-L2 end to end {e_own:.2e}, on the oracle's selection {e_same:.2e}")
        assert e_own <= 2e-2 and e_same <= 1e-2


@pytest.mark.timeout(900)
def test_rope_selection_full_hunyuan(gpu_lib):
    """The HunyuanVideo-like workload at full size (24 heads, 1920 blocks), in the call
    sequence the bench times with RoPE-aware selection; 512 sampled tiles of heads 0 and 23
    against the oracle's scores from the full pre-rotation means."""
    inp = synth.make("hunyuan", keep_pre_rope=True)
    tensors = to_device(inp)
    st, idx, mask, wt = _gpu_rope_select(gpu_lib, inp, tensors, "adjacent")
    idx_h = idx.cpu().numpy()
    rng = np.random.default_rng(143)
    rows = sorted(rng.choice(inp.nb, size=512, replace=False).tolist())
    for h in (0, 23):
        s = _oracle_rope_scores(inp, h, "adjacent", rows)
        exact, near, gap = check_selection(idx_h[h], s, inp.K_sel, rtol=RTOL, rows=rows)
        print(f"hunyuan h{h}: {exact} tiles bit-exact, {near} near ties, min gap {gap:.3e}")
        assert exact >= 0.9 * len(rows)
