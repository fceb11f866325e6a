"""Benchmark of the piecewise sparse attention forward pass on one MI355X.

A step is one pass of the whole path over one batch of resident synthetic input:
pisa_block_stats -> pisa_select_topk -> pisa_attention_fwd (PWT mode by default).
Default workload: the Wan2.1-like video config (40 heads, latent grid 21x30x52 =
32,760 tokens in 4x4x4 cubes, d = 128, bf16, keep 10% of key blocks per query cube).

Prints ONE JSON line with the effective throughput (exact + compensation FLOPs over
valid tokens only, divided by the measured step time), the per-call split, the dense
baselines, the attention kernel's roofline and the CPU oracle's time on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms/call + effective TFLOP/s (% bf16 MFMA peak), Wan2.1-like L=32760 H=40 d=128"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA peaks
PEAK_HBM_GBS = 8000.0


def flop_counts(idx: np.ndarray, block_len: np.ndarray, d: int, mode: str) -> dict:
    """Algorithmic FLOPs of one step over valid tokens only.

    exact    4d per (valid query, valid key of a selected block)      (QKᵀ and PV)
    virtual  4d per (valid query, unselected block)                   (PISA/PWT)
             6d per (valid query, unselected block)                   (PWT_ROW: + 2d for w)
             4d per (valid query, valid key of an unselected block)   (LITERAL)
    first    2d² per valid query                                      (A_t H̄ q_t, PISA/PWT)
    prepare  2d² per valid key (H̄ cross term) + 2d·nb² per head for the block scores,
             and another 2d·nb² per head for w̃ (PWT)
    """
    H, nb, K_sel = idx.shape
    bl = block_len.astype(np.int64)
    sel_tokens = bl[idx].sum(axis=-1) if K_sel else np.zeros((H, nb), dtype=np.int64)   # [H, nb]
    rows = bl[None, :]
    exact = int((4 * d * rows * sel_tokens).sum())
    unsel_blocks = nb - K_sel
    virtual = first = 0
    if mode in ("pisa", "pwt", "pwt_row"):
        virtual = int((6 if mode == "pwt_row" else 4) * d * rows.sum() * unsel_blocks * H)
        first = int(2 * d * d * rows.sum() * H)
    elif mode == "literal":
        virtual = int((4 * d * rows * (bl.sum() - sel_tokens)).sum())
    prepare = int(2 * d * d * bl.sum() * H + 2 * d * nb * nb * H * (2 if mode == "pwt" else 1))
    return dict(exact=exact, virtual=virtual, first=first, prepare=prepare,
                attention=exact + virtual + first, total=exact + virtual + first + prepare)


def kernel_source_hash(dtype: str = "bf16") -> str:
    """Hash of the sources of the measured attention kernel: the register-streamed kernel
    for bf16 inputs, the LDS-staged one (attention_split_kernel) for fp32."""
    h = hashlib.sha256()
    main = "attention_frag.hip" if dtype == "bf16" else "attention_fwd.hip"
    for name in (main, "common.hpp", "attention.hpp"):
        with open(os.path.join(ROOT, "block_sparse_attention_43_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _large_splits(H: int, nb: int) -> int:
    """Key splits of the selection over rows of more than 2048 blocks (as the library
    picks them: enough workgroups of 128 rows to fill the GPU, at most 16)."""
    nrg, tiles, ks = (nb + 127) // 128, (nb + 31) // 32, 1
    while ks < 16 and nrg * H * ks < 2048 and tiles // (2 * ks) >= 4:
        ks *= 2
    return ks


def load_traffic(workload: str, dtype: str):
    """HBM bytes per attention launch measured with rocprofv3 counters, if they were taken
    on the current kernel source (profiles/attention_fwd_<workload>_traffic.json)."""
    p = os.path.join(ROOT, "profiles", f"attention_fwd_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("kernel_sha256_16") != kernel_source_hash(dtype):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, mode: str, heads: int) -> dict:
    """The oracle as it stands, timed on the first ``heads`` heads of the same workload
    (every query tile, per-head statistics included)."""
    from oracle import pisa_oracle as orc
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = 1
    host = {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}
    bl = inp.layout.block_len
    if inp.nb > 4096:
        # one head, 64 sampled query tiles (statistics of the whole head included), the
        # attention part extrapolated linearly to every tile
        rng = np.random.default_rng(0)
        tiles = sorted(rng.choice(inp.nb, size=64, replace=False).tolist())
        Q, K, V = inp.f64("Q", 0), inp.f64("K", 0), inp.f64("V", 0)
        t0 = time.perf_counter()
        st = orc.block_stats(K, V, 64, bl, per_block=False)
        t1 = time.perf_counter()
        res = orc.attention_head(Q, K, V, 64, bl, inp.K_sel, mode, tiles=tiles, stats=st)
        t2 = time.perf_counter()
        scale = inp.nb / len(tiles)
        dt = (t1 - t0) + (t2 - t1) * scale
        # FLOPs of the sampled tiles (same counting as flop_counts), scaled like the time
        d, b = inp.d, bl.astype(np.int64)
        rows = b[tiles]
        sel_tok = b[res["idx"][tiles]].sum(axis=1)
        attn = 4 * d * rows * sel_tok
        if mode in ("pisa", "pwt"):
            attn = attn + 4 * d * rows * (inp.nb - inp.K_sel) + 2 * d * d * rows
        elif mode == "literal":
            attn = attn + 4 * d * rows * (b.sum() - sel_tok)
        prep = 2 * d * d * b.sum() + 2 * d * inp.nb * inp.nb * (2 if mode == "pwt" else 1)
        total = float(attn.sum()) * scale + float(prep)
        return {"value": total / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
                "sample": f"head 0 of {inp.H}: statistics of the whole head ({t1 - t0:.1f} s) plus 64 of "
                          f"{inp.nb} query tiles ({t2 - t1:.1f} s), extrapolated linearly to all tiles; "
                          f"{mode}, float64 numpy", **host}
    hs = list(range(min(heads, inp.H)))
    sel = []
    dt = 0.0
    for h in hs:
        Q, K, V = inp.f64("Q", h), inp.f64("K", h), inp.f64("V", h)
        t0 = time.perf_counter()
        res = orc.attention_head(Q, K, V, 64, bl, inp.K_sel, mode)
        dt += time.perf_counter() - t0
        sel.append(res["idx"])
        if dt > 20.0:       # bounded sample: stop after about 20 s of oracle time
            break
    hs = hs[:len(sel)]
    fc = flop_counts(np.stack(sel), bl, inp.d, mode)
    return {"value": fc["total"] / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(hs)} of {inp.H} heads, all {inp.nb} query tiles each, {mode}, float64 numpy "
                      f"(per-head statistics and selection included): {dt:.1f} s", **host}


def progress(what: str):
    """One line per finished leg on stderr (the JSON record alone goes to stdout)."""
    print(f"[bench] {what}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="wan", help="tiny | flux | wan | hunyuan | long")
    ap.add_argument("--mode", default="pwt", help="drop | pisa | pwt | literal")
    ap.add_argument("--route", default="mean", help="mean | covariance | error (block selection score)")
    ap.add_argument("--rope-select", action="store_true",
                    help="rotary workloads: select with RoPE-aware centroids in the timed step")
    ap.add_argument("--cpu-heads", type=int, default=12, help="heads in the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--traffic-driver", action="store_true",
                    help="counter-collection driver: a 512 MiB device copy (calibration) x3, then "
                         "statistics + selection once and three attention launches; prints one line")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this build runs on exactly one GPU: every workload fits one "
                                   "MI355X and the path has no multi-GPU mode; run with --gpus 1"}))
        sys.exit(2)

    import torch
    from block_sparse_attention_43_amd import pisa, synth

    torch.cuda.set_device(0)
    pisa.load()
    inp = synth.make(args.config, keep_pre_rope=True)
    cfg = inp.cfg
    K_sel = inp.K_sel
    mode = args.mode
    base = pisa.MODES[mode]

    def dev(x):
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.view(torch.bfloat16) if cfg.dtype == "bf16" else t).cuda()

    Q, K, V = dev(inp.Q), dev(inp.K), dev(inp.V)
    bl = inp.layout.block_len
    blt = None if (bl == 64).all() else torch.from_numpy(bl.astype(np.int32)).cuda()
    H, L, d = Q.shape
    nb = L // 64

    if args.traffic_driver:
        src = torch.ones(512 * 2**20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        st = pisa.block_stats(K, V, blt)
        idx, mask, wt = pisa.select_topk(Q, st, K_sel, blt, want_wt=(base == pisa.MODE_PWT))
        O = torch.empty_like(Q)
        for _ in range(3):
            pisa.attention_fwd(Q, K, V, st, idx, mask, wt, K_sel, mode, blt, out=O)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_driver": cfg.name, "mode": mode, "copy_bytes": 512 * 2**20,
                          "kernel_sha256_16": kernel_source_hash(cfg.dtype)}))
        return

    # every buffer allocated once, outside the timed region
    route = args.route
    rope_select = args.rope_select
    if rope_select and (not cfg.rope or route != "mean"):
        print(json.dumps({"error": "--rope-select needs a rotary workload (hunyuan) and the mean route"}))
        sys.exit(2)
    if cfg.rope:
        Qp, Kp = dev(inp.extra["Q_pre"]), dev(inp.extra["K_pre"])
        pos = torch.from_numpy(inp.extra["pos"]).cuda()
        widths = synth.rope_split_for(cfg)
    sflags = pisa.STATS_HNORM if route != "mean" else 0
    st = pisa.alloc_stats(K, sflags)
    ws_stats = torch.empty(max(pisa.load().pisa_block_stats_workspace_bytes(H, L, d, 64), 16),
                           dtype=torch.uint8, device="cuda")
    ws_sel = torch.empty(pisa.load().pisa_select_workspace_bytes(H, L, d, 64), dtype=torch.uint8, device="cuda")
    idx = torch.empty(H, nb, max(K_sel, 1), dtype=torch.int32, device="cuda")[:, :, :K_sel]
    mask = torch.empty(H, nb, (nb + 31) // 32, dtype=torch.int32, device="cuda")
    wt = torch.empty(H, nb, nb, dtype=torch.float32, device="cuda") if base == pisa.MODE_PWT else None
    O = torch.empty_like(Q)
    lse = torch.empty(H, L, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        pisa.block_stats(K, V, blt, flags=sflags, out=st, workspace=ws_stats)
        if ev is not None:
            ev[1].record(stream)
        if rope_select:
            pisa.select_topk_rope(Q, Qp, Kp, pos, widths, synth.ROPE_BASE, st, K_sel, blt,
                                  out=(idx, mask, wt), workspace=ws_sel)
        else:
            pisa.select_topk(Q, st, K_sel, blt, out=(idx, mask, wt), workspace=ws_sel, route=route)
        if ev is not None:
            ev[2].record(stream)
        pisa.attention_fwd(Q, K, V, st, idx, mask, wt, K_sel, mode, blt, out=O, lse=lse)
        if ev is not None:
            ev[3].record(stream)

    progress("inputs on the device")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        step(evs[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    ms_stats = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    ms_sel = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_attn = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))

    fc = flop_counts(idx.cpu().numpy(), bl, d, mode)
    value = fc["total"] / (ms_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg.dtype]
    attn_tflops = fc["attention"] / (ms_attn * 1e-3) / 1e12
    # the two prepare calls are HBM-bound: bytes they move by design per call
    es = 2 if cfg.dtype == "bf16" else 4
    nbp = (nb + 63) // 64 * 64
    stats_bytes = (2 * H * L * d * es                        # read K, V
                   + (2 if es == 2 else 1) * H * L * d * es  # write Vᵀ (+ operand-order K for bf16)
                   + 3 * H * nb * d * 4 + 2 * H * nbp * d * es + H * d * d * (4 + es))
    nw = (nb + 31) // 32
    sel_bytes = (H * L * d * es + 2 * H * nb * d * 4 * 2     # read Q; write q̄, mean(q²), read them back
                 + 2 * H * nb * d * 4                        # read k̄, σ²
                 + H * nb * (K_sel + nw) * 4                 # idx, mask
                 + (H * nb * nb * 4 if wt is not None else 0))   # w̃
    if nb <= 2048:
        sel_bytes += 2 * H * nb * nb * 4                     # score rows written and read back
    else:
        # recomputed scores: per row the bin counts of every key split (written, read) and
        # the mask words written twice and read once
        sel_bytes += H * nb * (2 * 512 * _large_splits(H, nb) + 2 * nw * 4)
    prepare = {k: {"bytes": int(b), "gbs": round(b / (ms * 1e-3) / 1e9, 1),
                   "frac_of_hbm": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
               for k, b, ms in (("pisa_block_stats", stats_bytes, ms_stats), ("pisa_select_topk", sel_bytes, ms_sel))}
    traffic = load_traffic(args.config, cfg.dtype)

    # exact branch alone: DROP on the same selection (phase 1 only)
    def timed(fn, n=5):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    progress("timed steps done")
    # the same step captured once in a HIP graph and replayed: the library issues no
    # memset or allocation, so the graph holds every kernel of the step (launch overhead
    # removed; what matters for the launch-bound small workload)
    graph = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g_step = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step):
            step()
        torch.cuda.synchronize()
        g_step.replay()
        torch.cuda.synchronize()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ga.record(stream)
        for _ in range(args.steps):
            g_step.replay()
        gb.record(stream)
        torch.cuda.synchronize()
        graph = {"ms_per_step": round(ga.elapsed_time(gb) / args.steps, 4)}
        del g_step
    except Exception as e:  # pragma: no cover - capture support depends on the runtime
        graph = {"error": str(e)[:200]}
    ms_exact = timed(lambda: pisa.attention_fwd(Q, K, V, st, idx, mask, None, K_sel, "drop", blt, out=O))
    exact_tflops = fc["exact"] / (ms_exact * 1e-3) / 1e12

    progress("exact branch done")
    # covariance-aware routing, the optional selection rule: its prepare-phase cost (second
    # statistics pass for M_j + routed scores) and how many tiles change their selection
    routing = None
    rules = {("rope" if rope_select else route): (idx.clone(), mask.clone())}
    if route == "mean":
        st_r = pisa.alloc_stats(K, pisa.STATS_HNORM)
        idx_r, mask_r = torch.empty_like(idx), torch.empty_like(mask)
        wt_r = None if wt is None else torch.empty_like(wt)

        def prep_routed():
            pisa.block_stats(K, V, blt, flags=pisa.STATS_HNORM, out=st_r, workspace=ws_stats)
            pisa.select_topk(Q, st_r, K_sel, blt, out=(idx_r, mask_r, wt_r), workspace=ws_sel,
                             route="covariance")

        ms_prep_r = timed(prep_routed)
        changed = float((idx_r != idx).any(dim=-1).float().mean().item()) if K_sel else 0.0
        routing = {"ms_prepare_covariance": round(ms_prep_r, 4),
                   "ms_prepare_mean": round(ms_stats + ms_sel, 4),
                   "tiles_with_changed_selection": round(changed, 4)}
        rules["covariance"] = (idx_r.clone(), mask_r.clone())
        pisa.select_topk(Q, st_r, K_sel, blt, out=(idx_r, mask_r, wt_r), workspace=ws_sel, route="error")
        rules["error"] = (idx_r.clone(), mask_r.clone())
        del st_r, idx_r, mask_r, wt_r

    progress("routing leg done")
    # RoPE-aware centroids on rotary workloads: selection cost and how many tiles change
    rope_leg = None
    if cfg.rope and not rope_select:
        idx_p, mask_p = torch.empty_like(idx), torch.empty_like(mask)
        wt_p = None if wt is None else torch.empty_like(wt)
        ms_sel_rope = timed(lambda: pisa.select_topk_rope(Q, Qp, Kp, pos, widths, synth.ROPE_BASE, st, K_sel,
                                                          blt, out=(idx_p, mask_p, wt_p), workspace=ws_sel))
        changed = float((idx_p != idx).any(dim=-1).float().mean().item()) if K_sel else 0.0
        rope_leg = {"ms_select_rope": round(ms_sel_rope, 4), "ms_select_mean": round(ms_sel, 4),
                    "tiles_with_changed_selection": round(changed, 4)}
        rules["rope"] = (idx_p.clone(), mask_p.clone())
        del idx_p, mask_p, wt_p

    progress("rope leg done")
    # cold cache: a 512 MiB fill between runs evicts L2 and the Infinity Cache
    flush = torch.empty(512 * 2**20, dtype=torch.uint8, device="cuda")
    cold_step, cold_attn = [], []
    for _ in range(5):
        flush.zero_()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        step(ev)
        torch.cuda.synchronize()
        cold_step.append(ev[0].elapsed_time(ev[3]))
        cold_attn.append(ev[2].elapsed_time(ev[3]))
    del flush

    progress("cold-cache runs done")
    # step a0, not part of the three calls: natural (t, h, w) order -> padded cube order
    perm = torch.from_numpy(inp.layout.perm.astype(np.int32)).cuda()
    nat = torch.zeros(H, inp.layout.L, d, dtype=Q.dtype, device="cuda")
    cube = torch.empty_like(Q)
    ms_perm = timed(lambda: pisa.layout_to_blocks(nat, perm, out=cube))
    del nat, cube

    progress("permutation done")
    # backward of the timed mode (DROP / PISA / PWT) on the same selection: dQ, dK, dV from dO
    backward = None
    if mode in ("drop", "pisa", "pwt"):
        dO = torch.randn(Q.shape, dtype=torch.float32, device="cuda", generator=torch.Generator(device="cuda").manual_seed(7)).to(Q.dtype)
        gbuf = tuple(torch.empty(H, L, d, dtype=torch.float32, device="cuda") for _ in range(3))
        ws_bwd = torch.empty(max(pisa.load().pisa_attention_bwd_workspace_bytes(1 if cfg.dtype == "bf16" else 0, H, L, d,
                                                                                64, K_sel), 16),
                             dtype=torch.uint8, device="cuda")
        pisa.attention_fwd(Q, K, V, st, idx, mask, wt, K_sel, mode, blt, out=O, lse=lse)
        # with the forward output (Δ = dO·O read), as a training step has it; and without
        ms_bwd = timed(lambda: pisa.attention_bwd(Q, K, V, st, idx, mask, wt, K_sel, lse, dO, mode, blt,
                                                  out=gbuf, workspace=ws_bwd, O=O), 3)
        ms_bwd_no_o = timed(lambda: pisa.attention_bwd(Q, K, V, st, idx, mask, wt, K_sel, lse, dO, mode, blt,
                                                       out=gbuf, workspace=ws_bwd), 3)
        fb = flop_counts(idx.cpu().numpy(), bl, d, mode)
        bflops = int(2.5 * (fb["exact"] + fb["virtual"]) + 2 * fb["first"] + 4 * d * d * int(bl.sum()) * H)
        backward = {"ms": round(ms_bwd, 4), "ms_without_o": round(ms_bwd_no_o, 4), "algorithmic_flops": bflops,
                    "tflops": round(bflops / (ms_bwd * 1e-3) / 1e12, 2),
                    "ratio_to_forward_attention": round(ms_bwd / ms_attn, 2)}
        del gbuf, ws_bwd, dO

    progress("backward done")
    def row_backward_ms(name):
        """One backward call of LITERAL or PWT_ROW (bf16) on the step's selection, after its
        forward call; one warm-up call and one timed call."""
        g = torch.randn(Q.shape, dtype=torch.float32, device="cuda",
                        generator=torch.Generator(device="cuda").manual_seed(7)).to(Q.dtype)
        bufs = tuple(torch.empty(H, L, d, dtype=torch.float32, device="cuda") for _ in range(3))
        ws_r = torch.empty(pisa.load().pisa_attention_bwd_workspace_bytes(1, H, L, d, 64, K_sel),
                           dtype=torch.uint8, device="cuda")
        pisa.attention_fwd(Q, K, V, st, idx, mask, None, K_sel, name, blt, out=O, lse=lse)
        ms_r = timed(lambda: pisa.attention_bwd(Q, K, V, st, idx, mask, None, K_sel, lse, g, name, blt,
                                                out=bufs, workspace=ws_r), 1)
        del g, bufs, ws_r
        return ms_r

    # PWT with the per-row diagonal w (the pooling ablation), on the same selection
    pwt_row = None
    if mode != "pwt_row":
        fr = flop_counts(idx.cpu().numpy(), bl, d, "pwt_row")
        ms_row = timed(lambda: pisa.attention_fwd(Q, K, V, st, idx, mask, None, K_sel, "pwt_row", blt, out=O), 3)
        pwt_row = {"ms_attention": round(ms_row, 4), "attention_flops": fr["attention"],
                   "tflops": round(fr["attention"] / (ms_row * 1e-3) / 1e12, 2)}
        if cfg.dtype == "bf16" and nb <= 2048:
            pwt_row["backward_ms"] = round(row_backward_ms("pwt_row"), 4)

    progress("per-row w done")
    # LITERAL, reported but not held to the dense target
    literal = None
    if mode != "literal":
        fl = flop_counts(idx.cpu().numpy(), bl, d, "literal")
        ms_lit = timed(lambda: pisa.attention_fwd(Q, K, V, st, idx, mask, None, K_sel, "literal", blt, out=O), 3)
        literal = {"ms_attention": round(ms_lit, 4), "attention_flops": fl["attention"],
                   "tflops": round(fl["attention"] / (ms_lit * 1e-3) / 1e12, 2)}
        # its backward sweeps every (query tile, key block) pair three times: timed where that
        # stays within seconds
        if cfg.dtype == "bf16" and nb * nb * H <= 2 * 10 ** 7:
            literal["backward_ms"] = round(row_backward_ms("literal"), 4)

    progress("LITERAL done")
    dense = {}
    if not args.no_dense:
        idx_all = torch.arange(nb, dtype=torch.int32, device="cuda").expand(H, nb, nb).contiguous()
        ms_drop_all = timed(lambda: pisa.attention_fwd(Q, K, V, st, idx_all, None, None, nb, "drop", blt, out=O), 3)
        # selection quality: the share of each row's dense softmax mass that the selected
        # blocks hold, exp(lse over the selected keys - lse over all keys), mean over valid rows
        lse_all = torch.empty(H, L, dtype=torch.float32, device="cuda")
        lse_sel = torch.empty_like(lse_all)
        pisa.attention_fwd(Q, K, V, st, idx_all, None, None, nb, "drop", blt, out=O, lse=lse_all)
        valid = torch.from_numpy((np.arange(64)[None, :] < bl[:, None]).reshape(-1)).cuda()
        recall = {}
        for name_r, (idx_x, mask_x) in rules.items():
            pisa.attention_fwd(Q, K, V, st, idx_x, mask_x, None, K_sel, "drop", blt, out=O, lse=lse_sel)
            recall[name_r] = round(float(torch.exp(lse_sel - lse_all)[:, valid].mean().item()), 5)
        dense["selection_mass_recall"] = recall
        if backward is not None:
            # dense backward baseline: DROP with every block selected (the same kernels as the
            # sparse backward), forward output given; forward + backward against the step's
            mask_all = torch.zeros(H, nb, (nb + 31) // 32 * 32, dtype=torch.bool)
            mask_all[:, :, :nb] = True
            mask_all = torch.from_numpy(np.packbits(mask_all.numpy(), axis=-1, bitorder="little")
                                        .view(np.int32).reshape(H, nb, -1).copy()).cuda()
            dO = torch.randn(Q.shape, dtype=torch.float32, device="cuda",
                             generator=torch.Generator(device="cuda").manual_seed(7)).to(Q.dtype)
            gbuf = tuple(torch.empty(H, L, d, dtype=torch.float32, device="cuda") for _ in range(3))
            ws_bd = torch.empty(max(pisa.load().pisa_attention_bwd_workspace_bytes(
                1 if cfg.dtype == "bf16" else 0, H, L, d, 64, nb), 16), dtype=torch.uint8, device="cuda")
            pisa.attention_fwd(Q, K, V, st, idx_all, mask_all, None, nb, "drop", blt, out=O, lse=lse_all)
            ms_bwd_dense = timed(lambda: pisa.attention_bwd(Q, K, V, st, idx_all, mask_all, None, nb, lse_all, dO,
                                                            "drop", blt, out=gbuf, workspace=ws_bd, O=O), 1)
            dense["dense_backward_ms"] = round(ms_bwd_dense, 4)
            del gbuf, ws_bd, dO, mask_all
        del idx_all, lse_all, lse_sel
        ok = torch.from_numpy(inp.layout.perm >= 0).cuda()
        q = Q[:, ok].unsqueeze(0).contiguous()
        k = K[:, ok].unsqueeze(0).contiguous()
        v = V[:, ok].unsqueeze(0).contiguous()
        try:
            ms_sdpa = timed(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=1.0), 3)
        except Exception as e:  # pragma: no cover - backend dependent
            ms_sdpa = None
            dense["sdpa_error"] = str(e)[:200]
        del q, k, v
        best = min(x for x in (ms_drop_all, ms_sdpa) if x is not None)
        dense.update(dense_ours_ms=round(ms_drop_all, 4),
                     dense_sdpa_ms=None if ms_sdpa is None else round(ms_sdpa, 4),
                     dense_best_ms=round(best, 4), speedup_vs_dense=round(best / ms_step, 3))
        if graph and "ms_per_step" in graph:
            graph["speedup_vs_dense"] = round(best / graph["ms_per_step"], 3)
        if "dense_backward_ms" in dense:
            # forward + backward: the dense pair against the sparse step and its backward
            dense["fwd_bwd_speedup_vs_dense"] = round((best + dense["dense_backward_ms"])
                                                      / (ms_step + backward["ms"]), 3)

    # yardstick for the matrix-core fraction: the vendor library's bf16 GEMM on this card
    calibration = None
    if cfg.dtype == "bf16" and not args.no_dense:
        ga = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
        gb = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
        gc = torch.empty_like(ga)
        ms_gemm = timed(lambda: torch.matmul(ga, gb, out=gc), n=20)
        g_tflops = 2 * 8192 ** 3 / (ms_gemm * 1e-3) / 1e12
        calibration = {"gemm": "torch.matmul bf16 8192x8192x8192 (vendor library)", "ms": round(ms_gemm, 4),
                       "tflops": round(g_tflops, 2), "frac": round(g_tflops / peak, 4),
                       "exact_branch_vs_gemm": round(exact_tflops / g_tflops, 4)}
        del ga, gb, gc

    cpu = None
    progress("dense and selection recall done")
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, mode, args.cpu_heads)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded smooth 3D field + noise, cube layout; no model activations)",
        "config": {"workload": f"{cfg.name}: H={H} L={inp.layout.L} (padded {L}) d={d} B=64 "
                               f"K_sel={K_sel}/{nb} mode={mode}" + (f" route={route}" if route != "mean" else "")
                               + (" rope-aware selection" if rope_select else ""),
                   "heads": H, "seq_len": inp.layout.L, "head_dim": d, "block": 64,
                   "k_sel": K_sel, "n_blocks": nb, "mode": mode, "route": route, "rope_select": rope_select},
        "ms_stats": round(ms_stats, 4),
        "ms_select": round(ms_sel, 4),
        "ms_attention": round(ms_attn, 4),
        "frac_of_peak_total": round(value / peak, 4),
        "prepare_hbm": prepare,
        "exact_branch": {"ms": round(ms_exact, 4), "tflops": round(exact_tflops, 2),
                         "frac": round(exact_tflops / peak, 4)},
        "cold_cache": {"ms_per_step": round(float(np.median(cold_step)), 4),
                       "ms_attention": round(float(np.median(cold_attn)), 4),
                       "runs": len(cold_step), "flush_bytes": 512 * 2**20},
        "graph": graph,
        "layout_permutation_ms": round(ms_perm, 4),
        "literal": literal,
        "pwt_row": pwt_row,
        "backward": backward,
        "covariance_routing": routing,
        "rope_selection": rope_leg,
        "flops": fc,
        **dense,
        "gemm_calibration": calibration,
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4), "traffic": traffic,
                     "kernel": ("pisa_attention_fwd: attention_frag_kernel, one launch for query "
                                "tiles of more than 32 rows and one for the rest" if cfg.dtype == "bf16" else
                                "pisa_attention_fwd: attention_split_kernel (fp32 inputs), one launch"),
                     "algorithmic_flops_per_launch": fc["attention"]},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
