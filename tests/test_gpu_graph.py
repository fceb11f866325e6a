"""The three calls of one step (statistics, selection, attention) captured in a HIP graph
(torch.cuda.CUDAGraph on the stream the binding launches on) and replayed. The library
issues no memset and no allocation, so the captured kernels are the whole step. Every
replay, with eager work (fills of the outputs) and synchronisations between replays,
must reproduce the eager step bit for bit: the kernels have no floating-point atomics
and fixed summation orders.
"""
import pytest
import torch

from helpers import small_case, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case,mode", [("tiny", "pwt"), ("bf16_d128_ragged", "pwt"), ("bf16_nb70", "drop"),
                                       ("bf16_d64", "literal")])
def test_graph_replay_matches_eager(gpu_lib, case, mode):
    pisa = gpu_lib
    lib = pisa.load()
    inp, K_sel = small_case(case)
    Q, K, V, blt = to_device(inp)
    H, L, d = Q.shape
    nb = L // 64
    st = pisa.alloc_stats(K, 0)
    ws_stats = torch.empty(max(lib.pisa_block_stats_workspace_bytes(H, L, d, 64), 16), dtype=torch.uint8,
                           device="cuda")
    ws_sel = torch.empty(lib.pisa_select_workspace_bytes(H, L, d, 64), dtype=torch.uint8, device="cuda")
    idx = torch.empty(H, nb, K_sel, dtype=torch.int32, device="cuda")
    mask = torch.empty(H, nb, (nb + 31) // 32, dtype=torch.int32, device="cuda")
    wt = torch.empty(H, nb, nb, dtype=torch.float32, device="cuda") if mode == "pwt" else None
    O = torch.empty_like(Q)
    lse = torch.empty(H, L, dtype=torch.float32, device="cuda")

    def step():
        pisa.block_stats(K, V, blt, out=st, workspace=ws_stats)
        pisa.select_topk(Q, st, K_sel, blt, out=(idx, mask, wt), workspace=ws_sel)
        pisa.attention_fwd(Q, K, V, st, idx, mask, wt, K_sel, mode, blt, out=O, lse=lse)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (O, lse, idx, mask)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    print(f"graph case {case} {mode}", flush=True)
    for rep in range(3):
        O.fill_(0)
        lse.fill_(0)
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("O", "lse", "idx", "mask"), (O, lse, idx, mask), ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager step"
