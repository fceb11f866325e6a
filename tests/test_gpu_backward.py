"""GPU parity of the backward call (DROP, PISA, PWT) against the oracle's gradients, which
are pinned to central differences of the forward definition.

Both sides take the oracle's selection and PWT weights (the GPU forward runs on them too,
so lse comes from the GPU), and the same seeded dO. Bars: rel-L2 of dQ, dK, dV over valid
slots <= 1e-4 for fp32 inputs and <= 2e-2 for bf16 inputs (P enters dV in bf16 as in the
forward pass, and so does dS into dK; dS enters dQ as a hi + lo bf16 pair when the forward
output is not passed, in bf16 when it is); padded slots exactly 0. `with_o` passes the forward
output O, so the dQ sweep starts from Δ_O = dO·O and corrects O's bf16 rounding with the
fp32 sum of dS (without that correction bf16 dQ misses the bar: rel-L2 ~2.4e-2 on
bf16_d128_ragged, from Δ_O's error times the keys' common mean).
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_43_amd import synth
from oracle import pisa_oracle as orc
from helpers import oracle_selection, rel_l2, selection_to_device, small_case, to_device, valid_rows

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
MODES = ["drop", "pisa", "pwt"]


def _dO(inp, seed):
    r = np.random.default_rng(seed)
    g = r.standard_normal((inp.H, inp.layout.L_pad, inp.d)).astype(np.float32)
    return synth.f32_to_bf16_bits(g) if inp.cfg.dtype == "bf16" else g


def _gpu_backward(pisa, inp, K_sel, mode, sel, w, dO_host, mode_bits=0, tensors=None, with_o=False):
    Q, K, V, blt = tensors if tensors is not None else to_device(inp)
    st = pisa.block_stats(K, V, blt)
    di, dm, dw = selection_to_device(sel, w, inp.nb)
    base = pisa.MODES[mode]
    wt = dw if base == pisa.MODE_PWT else None
    O, lse = pisa.attention_fwd(Q, K, V, st, di, dm, wt, K_sel, base | mode_bits, blt)
    t = torch.from_numpy(np.ascontiguousarray(dO_host))
    dO = (t.view(torch.bfloat16) if inp.cfg.dtype == "bf16" else t).cuda()
    dQ, dK, dV = pisa.attention_bwd(Q, K, V, st, di, dm, wt, K_sel, lse, dO, base | mode_bits, blt,
                                    O=O if with_o else None)
    torch.cuda.synchronize()
    return [x.cpu().numpy().astype(np.float64) for x in (dQ, dK, dV)]


def _check(inp, K_sel, mode, sel, got, dO_host, heads=None, **kw):
    ok = valid_rows(inp)
    dO64 = synth.to_float64(dO_host, inp.cfg.dtype)
    worst = 0.0
    for h in (range(inp.H) if heads is None else heads):
        ref = orc.attention_head_backward(inp.f64("Q", h), inp.f64("K", h), inp.f64("V", h), dO64[h], 64,
                                          inp.layout.block_len, K_sel, mode, idx=sel[h], **kw)
        for name, g, r in zip(("dQ", "dK", "dV"), got, (ref["dQ"], ref["dK"], ref["dV"])):
            e = rel_l2(g[h][ok], r[ok])
            worst = max(worst, e)
            assert np.all(g[h][~ok] == 0), name
            assert e <= TOL[inp.cfg.dtype], (name, h, e)
    return worst


@pytest.mark.parametrize("with_o", [False, True])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", ["tiny", "bf16_d128_ragged", "bf16_d64", "f32_d128_ragged", "bf16_nb70",
                                  "f32_d64_ragged_nb130"])
def test_backward_parity(gpu_lib, case, mode, with_o):
    inp, K_sel = small_case(case)
    sel, w = oracle_selection(inp, K_sel)
    dO = _dO(inp, 151)
    got = _gpu_backward(gpu_lib, inp, K_sel, mode, sel, w, dO, with_o=with_o)
    worst = _check(inp, K_sel, mode, sel, got, dO)
    print(f"{case} {mode} O={with_o}: worst rel-L2 of dQ, dK, dV {worst:.2e}")


@pytest.mark.parametrize("bits,kw", [("W_LINEAR", dict(w_map="linear")), ("W_NOGATE", dict(guard="none"))])
def test_backward_mode_bits(gpu_lib, bits, kw):
    inp, K_sel = small_case("bf16_d128_ragged")
    sel, w = oracle_selection(inp, K_sel)
    dO = _dO(inp, 152)
    got = _gpu_backward(gpu_lib, inp, K_sel, "pwt", sel, w, dO, mode_bits=getattr(gpu_lib, bits))
    _check(inp, K_sel, "pwt", sel, got, dO, **kw)


@pytest.mark.parametrize("with_o", [False, True])
def test_backward_gate_fires(gpu_lib, with_o):
    """Blocks with widely spread keys: their w̃ exceeds ln n_j, the gate zeroes it and its
    gradient."""
    inp = synth.random_blocks(153, H=1, nb=8, d=128, dtype="bf16", block_len=[64, 64, 40, 64, 64, 64, 17, 64])
    k = synth.bf16_bits_to_f32(inp.K)
    k[0, 2 * 64:3 * 64] *= 6.0
    k[0, 5 * 64:6 * 64] *= 6.0
    k[:, ~valid_rows(inp), :] = 0.0
    inp.K[...] = synth.f32_to_bf16_bits(k)
    sel, w = oracle_selection(inp, 3)
    st = orc.block_stats(inp.f64("K", 0), inp.f64("V", 0), 64, inp.layout.block_len, per_block=False)
    assert (w[0] > np.log(st["n"])[None, :]).any()
    dO = _dO(inp, 154)
    got = _gpu_backward(gpu_lib, inp, 3, "pwt", sel, w, dO, with_o=with_o)
    _check(inp, 3, "pwt", sel, got, dO)


@pytest.mark.parametrize("with_o", [False, True])
@pytest.mark.parametrize("which", ["zero", "all"])
def test_backward_selection_extremes(gpu_lib, which, with_o):
    """K_sel = 0 (PWT: virtual tokens only) and K_sel = nb (dense attention's gradient)."""
    inp, _ = small_case("bf16_d128_ragged")
    K_sel = 0 if which == "zero" else inp.nb
    sel, w = oracle_selection(inp, K_sel)
    dO = _dO(inp, 155)
    got = _gpu_backward(gpu_lib, inp, K_sel, "pwt", sel, w, dO, with_o=with_o)
    _check(inp, K_sel, "pwt", sel, got, dO)


@pytest.mark.parametrize("with_o", [False, True])
def test_backward_deterministic(gpu_lib, with_o):
    inp, K_sel = small_case("bf16_nb70")
    sel, w = oracle_selection(inp, K_sel)
    dO = _dO(inp, 156)
    tensors = to_device(inp)
    a = _gpu_backward(gpu_lib, inp, K_sel, "pwt", sel, w, dO, tensors=tensors, with_o=with_o)
    b = _gpu_backward(gpu_lib, inp, K_sel, "pwt", sel, w, dO, tensors=tensors, with_o=with_o)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("with_o", [False, True])
def test_backward_full_wan(gpu_lib, with_o):
    """The Wan-like workload at full size (40 heads, 624 blocks, K_sel = 63), PWT, forward
    and backward on the oracle's selection and weights for every head; head 0 against the
    oracle's gradients."""
    inp = synth.make("wan")
    K_sel = inp.K_sel
    sel, w = oracle_selection(inp, K_sel)
    dO = _dO(inp, 157)
    got = _gpu_backward(gpu_lib, inp, K_sel, "pwt", sel, w, dO, with_o=with_o)
    worst = _check(inp, K_sel, "pwt", sel, got, dO, heads=[0])
    print(f"wan pwt head 0 O={with_o}: worst rel-L2 of dQ, dK, dV {worst:.2e}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("with_o", [False, True])
def test_backward_long_tile_lists(gpu_lib, with_o):
    """More than 512 tiles on every list (K_sel = 515 of nb = 520): the query sweep's and the
    key sweep's tile descriptors are staged 256 at a time, so both refill mid-loop."""
    inp = synth.random_blocks(107, H=1, nb=520, d=64, dtype="bf16", smooth=2.0)
    K_sel = 515
    sel, w = oracle_selection(inp, K_sel)
    dO = _dO(inp, 153)
    got = _gpu_backward(gpu_lib, inp, K_sel, "pwt", sel, w, dO, with_o=with_o)
    worst = _check(inp, K_sel, "pwt", sel, got, dO)
    print(f"nb=520 K_sel=515 pwt O={with_o}: worst rel-L2 of dQ, dK, dV {worst:.2e}")
