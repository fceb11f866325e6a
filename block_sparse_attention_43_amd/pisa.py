"""Python binding of the C ABI in include/pisa.h (argument marshalling only).

PyTorch provides device memory and the current HIP stream; every step of the forward
pass runs in the library's HIP kernels. Loading fails loudly if ``libpisa.so`` is
missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpisa.so")

PISA_F32, PISA_BF16 = 0, 1
MODE_DROP, MODE_PISA, MODE_PWT, MODE_LITERAL, MODE_PWT_ROW = 0, 1, 2, 3, 4
W_LINEAR, W_NOGATE, W_EXP = 1 << 4, 1 << 5, 1 << 6
STATS_BLOCK_H, STATS_BLOCK_C, STATS_HNORM = 1 << 0, 1 << 1, 1 << 2
ROUTE_MEAN, ROUTE_COVARIANCE, ROUTE_ERROR = 0, 1, 2
ROUTES = {"mean": ROUTE_MEAN, "covariance": ROUTE_COVARIANCE, "error": ROUTE_ERROR}
ROUTE_EPS = 1e-6          # ε of ln(M_j + ε) in covariance-aware scores
MODES = {"drop": MODE_DROP, "pisa": MODE_PISA, "pwt": MODE_PWT, "literal": MODE_LITERAL,
         "pwt_row": MODE_PWT_ROW}
B = 64

# Every symbol include/pisa.h declares.
EXPORTS = ("pisa_packed_bytes", "pisa_block_stats_workspace_bytes", "pisa_block_stats",
           "pisa_block_stats_noalloc",
           "pisa_select_workspace_bytes", "pisa_select_topk", "pisa_select_topk_routed",
           "pisa_select_topk_rope",
           "pisa_attention_fwd", "pisa_attention_bwd_workspace_bytes", "pisa_attention_bwd",
           "pisa_cube_layout", "pisa_layout_to_blocks", "pisa_layout_from_blocks",
           "pisa_last_error", "pisa_version")


class PisaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"pisa status {status}: {msg}")
        self.status = status


class _Stats(ctypes.Structure):
    _fields_ = [("kbar", ctypes.c_void_p), ("vsum", ctypes.c_void_p), ("ksig2", ctypes.c_void_p),
                ("hbarT", ctypes.c_void_p), ("hblk", ctypes.c_void_p), ("cblk", ctypes.c_void_p),
                ("packed", ctypes.c_void_p), ("hnorm", ctypes.c_void_p)]


ROPE_PAIRS = {"adjacent": 0, "half": 1}


class _Rope(ctypes.Structure):
    _fields_ = [("n_axes", ctypes.c_int), ("width", ctypes.c_int * 3), ("base", ctypes.c_float),
                ("pairs", ctypes.c_int)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m block_sparse_attention_43_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint
    sp = ctypes.POINTER(_Stats)
    lib.pisa_packed_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.pisa_packed_bytes.restype = sz
    lib.pisa_block_stats_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.pisa_block_stats_workspace_bytes.restype = sz
    lib.pisa_select_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.pisa_select_workspace_bytes.restype = sz
    lib.pisa_block_stats.argtypes = [i32, vp, vp, i32, i32, i32, i32, vp, u32, sp, vp, sz, vp]
    lib.pisa_block_stats.restype = i32
    lib.pisa_block_stats_noalloc.argtypes = [i32, vp, vp, i32, i32, i32, i32, vp, u32, sp, vp]
    lib.pisa_block_stats_noalloc.restype = i32
    lib.pisa_select_topk.argtypes = [i32, vp, sp, i32, i32, i32, i32, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.pisa_select_topk.restype = i32
    lib.pisa_select_topk_routed.argtypes = [i32, vp, sp, i32, i32, i32, i32, vp, i32, u32, ctypes.c_float,
                                            vp, vp, vp, vp, sz, vp]
    lib.pisa_select_topk_routed.restype = i32
    lib.pisa_select_topk_rope.argtypes = [i32, vp, vp, vp, vp, ctypes.POINTER(_Rope), sp, i32, i32, i32, i32,
                                          vp, i32, vp, vp, vp, vp, sz, vp]
    lib.pisa_select_topk_rope.restype = i32
    lib.pisa_attention_fwd.argtypes = [i32, vp, vp, vp, sp, vp, vp, vp, i32, i32, i32, i32, vp, i32,
                                       u32, vp, vp, vp]
    lib.pisa_attention_fwd.restype = i32
    lib.pisa_attention_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.pisa_attention_bwd_workspace_bytes.restype = sz
    lib.pisa_attention_bwd.argtypes = [i32, vp, vp, vp, sp, vp, vp, vp, i32, i32, i32, i32, vp, i32, u32,
                                       vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.pisa_attention_bwd.restype = i32
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.pisa_cube_layout.argtypes = [i32, i32, i32, i32, i32, i32, ip, ip, sz, ctypes.POINTER(ctypes.c_int)]
    lib.pisa_cube_layout.restype = i32
    for fn in (lib.pisa_layout_to_blocks, lib.pisa_layout_from_blocks):
        fn.argtypes = [i32, vp, i32, i32, i32, i32, vp, vp, vp]
        fn.restype = i32
    lib.pisa_last_error.argtypes = []
    lib.pisa_last_error.restype = ctypes.c_char_p
    lib.pisa_version.argtypes = []
    lib.pisa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise PisaError(status, load().pisa_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PISA_F32
    if t.dtype == torch.bfloat16:
        return PISA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _keep(stream, *tensors):
    """Buffers the binding allocated on the current stream but hands to work on another
    stream: tell the caching allocator not to reuse them before that stream is done."""
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _shape(Q: torch.Tensor):
    if Q.dim() != 3 or not Q.is_contiguous():
        raise ValueError("tensors must be contiguous [H, L, d]")
    H, L, d = Q.shape
    return H, L, d


@dataclass
class Stats:
    """Device buffers of pisa_stats (see include/pisa.h)."""
    kbar: torch.Tensor
    vsum: torch.Tensor
    ksig2: torch.Tensor
    hbarT: torch.Tensor
    packed: torch.Tensor
    hblk: torch.Tensor | None = None
    cblk: torch.Tensor | None = None
    hnorm: torch.Tensor | None = None

    def struct(self) -> _Stats:
        return _Stats(self.kbar.data_ptr(), self.vsum.data_ptr(), self.ksig2.data_ptr(),
                      self.hbarT.data_ptr(), _ptr(self.hblk), _ptr(self.cblk), self.packed.data_ptr(),
                      _ptr(self.hnorm))


def packed_bytes(dtype: torch.dtype, H: int, L: int, d: int) -> int:
    code = PISA_BF16 if dtype == torch.bfloat16 else PISA_F32
    return load().pisa_packed_bytes(code, H, L, d, B)


def alloc_stats(K: torch.Tensor, flags: int = 0) -> Stats:
    H, L, d = _shape(K)
    nb = L // B
    dev = K.device
    f = dict(dtype=torch.float32, device=dev)
    return Stats(kbar=torch.empty(H, nb, d, **f), vsum=torch.empty(H, nb, d, **f),
                 ksig2=torch.empty(H, nb, d, **f), hbarT=torch.empty(H, d, d, **f),
                 packed=torch.empty(packed_bytes(K.dtype, H, L, d), dtype=torch.uint8, device=dev),
                 hblk=torch.empty(H, nb, d, d, **f) if flags & STATS_BLOCK_H else None,
                 cblk=torch.empty(H, nb, d, d, **f) if flags & STATS_BLOCK_C else None,
                 hnorm=torch.empty(H, nb, **f) if flags & STATS_HNORM else None)


def block_stats(K, V, block_len=None, flags: int = 0, out: Stats | None = None, workspace=None,
                stream=None) -> Stats:
    lib = load()
    H, L, d = _shape(K)
    st = out if out is not None else alloc_stats(K, flags)
    need = lib.pisa_block_stats_workspace_bytes(H, L, d, B)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=K.device)
        _keep(stream, workspace)
    if out is None:
        _keep(stream, st.kbar, st.vsum, st.ksig2, st.hbarT, st.packed, st.hblk, st.cblk, st.hnorm)
    s = st.struct()
    _check(lib.pisa_block_stats(_dtype_code(K), _ptr(K), _ptr(V), H, L, d, B, _ptr(block_len), flags,
                                ctypes.byref(s), _ptr(workspace), workspace.numel(), _stream(stream)))
    return st


STATS_SCRATCH_BYTES = 64 << 20     # PISA_STATS_SCRATCH_BYTES


def block_stats_noalloc(K, V, block_len, out: Stats, flags: int = 0, stream=None) -> Stats:
    """pisa_block_stats_noalloc: the statistics into caller-allocated ``out``, with the
    H̄ partials in the library's fixed device scratch (no allocation in the call)."""
    lib = load()
    H, L, d = _shape(K)
    s = out.struct()
    _check(lib.pisa_block_stats_noalloc(_dtype_code(K), _ptr(K), _ptr(V), H, L, d, B, _ptr(block_len), flags,
                                        ctypes.byref(s), _stream(stream)))
    return out


def select_topk(Q, st: Stats, K_sel: int, block_len=None, want_wt: bool = True, want_mask: bool = True,
                out=None, workspace=None, stream=None, route="mean", eps: float = ROUTE_EPS):
    """Returns (idx [H, nb, K_sel] int32, mask [H, nb, nw] int32 bit pattern or None,
    wt [H, nb, nb] float32 or None). route="covariance" or "error" needs st.hnorm
    (block_stats with STATS_HNORM)."""
    lib = load()
    H, L, d = _shape(Q)
    nb = L // B
    nw = (nb + 31) // 32
    if out is None:
        idx = torch.empty(H, nb, max(K_sel, 1), dtype=torch.int32, device=Q.device)[:, :, :K_sel]
        mask = torch.empty(H, nb, nw, dtype=torch.int32, device=Q.device) if want_mask else None
        wt = torch.empty(H, nb, nb, dtype=torch.float32, device=Q.device) if want_wt else None
        _keep(stream, idx, mask, wt)
    else:
        idx, mask, wt = out
    need = lib.pisa_select_workspace_bytes(H, L, d, B)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
        _keep(stream, workspace)
    r = ROUTES[route] if isinstance(route, str) else int(route)
    s = st.struct()
    _check(lib.pisa_select_topk_routed(_dtype_code(Q), _ptr(Q), ctypes.byref(s), H, L, d, B,
                                       _ptr(block_len), K_sel, r, eps, _ptr(idx), _ptr(mask), _ptr(wt),
                                       _ptr(workspace), workspace.numel(), _stream(stream)))
    return idx, mask, wt


def select_topk_rope(Q, Q_pre, K_pre, pos, widths, base: float, st: Stats, K_sel: int, block_len=None,
                     pairs: str = "adjacent", want_wt: bool = True, want_mask: bool = True, out=None,
                     workspace=None, stream=None):
    """pisa_select_topk with RoPE-aware centroids. Q_pre, K_pre: [H, L, d] before the rotary
    embedding; pos: [L, n_axes] float32 device positions in block order; widths: dims per
    axis. Q (rotated) is read only for wt and may be None when want_wt is False."""
    lib = load()
    H, L, d = _shape(Q_pre)
    nb = L // B
    nw = (nb + 31) // 32
    if out is None:
        idx = torch.empty(H, nb, max(K_sel, 1), dtype=torch.int32, device=Q_pre.device)[:, :, :K_sel]
        mask = torch.empty(H, nb, nw, dtype=torch.int32, device=Q_pre.device) if want_mask else None
        wt = torch.empty(H, nb, nb, dtype=torch.float32, device=Q_pre.device) if want_wt else None
        _keep(stream, idx, mask, wt)
    else:
        idx, mask, wt = out
    if pos.dtype != torch.float32 or not pos.is_contiguous() or pos.shape[0] != L:
        raise ValueError("pos must be a contiguous float32 [L, n_axes] tensor")
    w = list(widths) + [0] * (3 - len(widths))
    rope = _Rope(len(widths), (ctypes.c_int * 3)(*w), base, ROPE_PAIRS[pairs])
    if workspace is None:
        workspace = torch.empty(lib.pisa_select_workspace_bytes(H, L, d, B), dtype=torch.uint8,
                                device=Q_pre.device)
        _keep(stream, workspace)
    s = st.struct()
    _check(lib.pisa_select_topk_rope(_dtype_code(Q_pre), _ptr(Q), _ptr(Q_pre), _ptr(K_pre), _ptr(pos),
                                     ctypes.byref(rope), ctypes.byref(s), H, L, d, B, _ptr(block_len), K_sel,
                                     _ptr(idx), _ptr(mask), _ptr(wt), _ptr(workspace), workspace.numel(),
                                     _stream(stream)))
    return idx, mask, wt


def attention_fwd(Q, K, V, st: Stats, idx, mask, wt, K_sel: int, mode="pwt", block_len=None,
                  out=None, lse=None, want_lse: bool = True, stream=None):
    lib = load()
    H, L, d = _shape(Q)
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    if out is None:
        out = torch.empty_like(Q)
        _keep(stream, out)
    if lse is None and want_lse:
        lse = torch.empty(H, L, dtype=torch.float32, device=Q.device)
        _keep(stream, lse)
    s = st.struct()
    _check(lib.pisa_attention_fwd(_dtype_code(Q), _ptr(Q), _ptr(K), _ptr(V), ctypes.byref(s), _ptr(idx),
                                  _ptr(mask), _ptr(wt), H, L, d, B, _ptr(block_len), K_sel, m, _ptr(out),
                                  _ptr(lse), _stream(stream)))
    return out, lse


def attention_bwd(Q, K, V, st: Stats, idx, mask, wt, K_sel: int, lse, dO, mode="pwt", block_len=None,
                  out=None, workspace=None, stream=None, O=None):
    """Gradients (dQ, dK, dV) float32 [H, L, d] of sum(dO * O) for the forward call that
    produced lse with the same arguments (DROP, PISA, PWT, or LITERAL for bf16 inputs).
    Passing that call's output O lets Δ = dO·O be read instead of formed in the dQ sweep
    (half its products); LITERAL always forms Δ itself."""
    lib = load()
    H, L, d = _shape(Q)
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    if out is None:
        out = tuple(torch.empty(H, L, d, dtype=torch.float32, device=Q.device) for _ in range(3))
        _keep(stream, *out)
    dQ, dK, dV = out
    if workspace is None:
        need = lib.pisa_attention_bwd_workspace_bytes(_dtype_code(Q), H, L, d, B, K_sel)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=Q.device)
        _keep(stream, workspace)
    s = st.struct()
    _check(lib.pisa_attention_bwd(_dtype_code(Q), _ptr(Q), _ptr(K), _ptr(V), ctypes.byref(s), _ptr(idx),
                                  _ptr(mask), _ptr(wt), H, L, d, B, _ptr(block_len), K_sel, m, _ptr(lse),
                                  _ptr(O), _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(workspace), workspace.numel(),
                                  _stream(stream)))
    return dQ, dK, dV


def cube_layout(grid, cube=(4, 4, 4)):
    """Host-side block order of a (T, H, W) grid cut into cubes: (perm int32 [nb*64], -1 for
    padding slots; block_len int32 [nb]) as numpy arrays."""
    import numpy as np
    lib = load()
    T, Hh, W = grid
    nb = -(-T // cube[0]) * -(-Hh // cube[1]) * -(-W // cube[2])
    perm = np.empty(nb * B, dtype=np.int32)
    bl = np.empty(nb, dtype=np.int32)
    out = ctypes.c_int(0)
    ip = ctypes.POINTER(ctypes.c_int32)
    _check(lib.pisa_cube_layout(T, Hh, W, *cube, perm.ctypes.data_as(ip), bl.ctypes.data_as(ip), perm.size,
                                ctypes.byref(out)))
    return perm, bl


def layout_to_blocks(x, perm, L_pad: int | None = None, out=None, stream=None):
    """[H, L_nat, d] natural order -> [H, L_pad, d] block order (perm: device int32 [L_pad])."""
    lib = load()
    if x.dim() != 3 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [H, L, d] tensor")
    H, Ln, d = x.shape
    Lp = perm.numel() if L_pad is None else L_pad
    if out is None:
        out = torch.empty(H, Lp, d, dtype=x.dtype, device=x.device)
        _keep(stream, out)
    _check(lib.pisa_layout_to_blocks(_dtype_code(x), _ptr(x), H, Ln, Lp, d, _ptr(perm), _ptr(out), _stream(stream)))
    return out


def layout_from_blocks(x, perm, L_nat: int, out=None, stream=None):
    """[H, L_pad, d] block order -> [H, L_nat, d] natural order (padding slots dropped)."""
    lib = load()
    if x.dim() != 3 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [H, L, d] tensor")
    H, Lp, d = x.shape
    if out is None:
        out = torch.empty(H, L_nat, d, dtype=x.dtype, device=x.device)
        _keep(stream, out)
    _check(lib.pisa_layout_from_blocks(_dtype_code(x), _ptr(x), H, L_nat, Lp, d, _ptr(perm), _ptr(out),
                                       _stream(stream)))
    return out


def forward(Q, K, V, K_sel: int, mode="pwt", block_len=None, flags: int = 0, stream=None, route="mean"):
    """One full pass: statistics, selection, fused attention. Returns (O, lse, idx, stats)."""
    base = (MODES[mode] if isinstance(mode, str) else int(mode)) & 15
    r = ROUTES[route] if isinstance(route, str) else int(route)
    st = block_stats(K, V, block_len, flags=flags | (STATS_HNORM if r != ROUTE_MEAN else 0),
                     stream=stream)
    idx, mask, wt = select_topk(Q, st, K_sel, block_len, want_wt=(base == MODE_PWT), stream=stream,
                                route=r)
    O, lse = attention_fwd(Q, K, V, st, idx, mask, wt, K_sel, mode, block_len, stream=stream)
    return O, lse, idx, st


def version() -> str:
    return load().pisa_version().decode()
