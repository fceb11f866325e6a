"""Seeded synthetic inputs for piecewise sparse attention (shared by tests, bench and smoke).

This module draws random numbers and lays tokens out in blocks. It holds none of
the attention method's arithmetic: no block statistics, no scores, no softmax.
Both the CPU oracle and the HIP path receive the arrays it returns, bit for bit.

Workloads (the pages measure on real diffusion-transformer activations, which are
not available here; these seeded fields stand in for them):

* ``tiny``    1 head, L=1024, d=64, fp32, Q/K/V i.i.d. N(0,1), 16 blocks of 64, K_sel=4.
* ``flux``    24 heads, 512 text + 64x64 image tokens, d=128, bf16, keep 25% of blocks.
              N(0,1) noise on every token plus one smooth 2D field (8 Fourier modes,
              per-coordinate RMS 1) added to Q, K and V of every head on image tokens.
* ``wan``     40 heads, latent grid 21x30x52 (L=32760), d=128, bf16, 4x4x4 cubes, keep 10%.
              Per head one smooth 3D field (16 Fourier modes, RMS 1) shared by that
              head's Q, K, V, plus N(0, 0.5) noise (variance 0.5).
* ``hunyuan`` 24 heads, grid 30x48x80 (L=115200), same generator as ``wan``, keep 5%,
              then 3D rotary position embedding applied to Q and K.
* ``long``    1 head, grid 80x128x128 (L=1,310,720), same generator as ``wan``, keep 5%.

Token layout (the pages cut tokens into blocks of B; video tokens are grouped into
3D cubes, Sparse Linear Attention blog, notation and "Sparse Attention" sections):
configs without a grid use contiguous 64-token blocks in sequence order; grid configs
permute natural (t, h, w) order into 4x4x4 cubes (cube index row-major over
(ct, ch, cw), in-cube (dt, dh, dw) row-major over the valid tokens), pad ragged edge
cubes to 64 slots with zeros and report the valid count per block in ``block_len``.

Q carries the 1/sqrt(d) factor (the pages absorb it into q). Generation is numpy
``Generator(PCG64(seed))`` in float64, then rounded to the config dtype
(round-to-nearest-even); the rounded tensors are the canonical inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

B_DEFAULT = 64


@dataclass(frozen=True)
class Config:
    name: str
    H: int
    d: int
    dtype: str                 # "f32" or "bf16"
    kind: str                  # "iid" | "flux" | "video"
    seed: int
    L: int = 0                 # natural sequence length (iid / flux)
    text: int = 0              # flux: text tokens before the image
    img: tuple = ()            # flux: image (rows, cols)
    grid: tuple = ()           # video: (T, Hh, W)
    keep: float = 0.0          # fraction of key blocks kept per query tile
    keep_blocks: int = 0       # explicit K_sel (tiny)
    rope: bool = False
    rope_split: tuple = ()     # dims per (t, h, w) axis; () = ROPE_SPLIT
    cube: tuple = (4, 4, 4)
    n_modes: int = 0
    noise_var: float = 1.0


CONFIGS = {
    "tiny": Config("tiny", H=1, d=64, dtype="f32", kind="iid", seed=0, L=1024, keep_blocks=4),
    "flux": Config("flux", H=24, d=128, dtype="bf16", kind="flux", seed=1, text=512, img=(64, 64),
                   keep=0.25, n_modes=8, noise_var=1.0),
    "wan": Config("wan", H=40, d=128, dtype="bf16", kind="video", seed=2, grid=(21, 30, 52),
                  keep=0.10, n_modes=16, noise_var=0.5),
    "hunyuan": Config("hunyuan", H=24, d=128, dtype="bf16", kind="video", seed=3, grid=(30, 48, 80),
                      keep=0.05, n_modes=16, noise_var=0.5, rope=True),
    "long": Config("long", H=1, d=128, dtype="bf16", kind="video", seed=4, grid=(80, 128, 128),
                   keep=0.05, n_modes=16, noise_var=0.5),
}

# Axis split of the rotary embedding for the hunyuan-like config (t, h, w dims; sum = d).
ROPE_SPLIT = (32, 48, 48)
ROPE_BASE = 10000.0


# ----------------------------------------------------------------------------- dtype helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 (or float64 via float32) to bfloat16 with round-to-nearest-even; uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Canonical tensor (float32 or bf16 bits) -> exact float64 copy."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- layout
@dataclass
class Layout:
    L: int                     # natural length
    L_pad: int                 # padded length (multiple of B)
    B: int
    perm: np.ndarray           # [L_pad] natural index of each padded slot, -1 = padding
    block_len: np.ndarray      # [nb] int32 valid tokens per block (first n_j slots)

    @property
    def nb(self) -> int:
        return self.L_pad // self.B

    @property
    def ragged(self) -> bool:
        return bool((self.block_len < self.B).any())


def contiguous_layout(L: int, B: int = B_DEFAULT) -> Layout:
    nb = -(-L // B)
    L_pad = nb * B
    perm = np.arange(L_pad, dtype=np.int64)
    perm[perm >= L] = -1
    block_len = np.full(nb, B, dtype=np.int32)
    if L % B:
        block_len[-1] = L % B
    return Layout(L, L_pad, B, perm, block_len)


def cube_layout(grid: tuple, cube: tuple = (4, 4, 4)) -> Layout:
    """Natural (t,h,w) row-major order -> 4x4x4 cube order, ragged cubes padded at their end."""
    T, Hh, W = grid
    ct, ch, cw = cube
    nt, nh, nw = -(-T // ct), -(-Hh // ch), -(-W // cw)
    B = ct * ch * cw
    nb = nt * nh * nw
    perm = np.full(nb * B, -1, dtype=np.int64)
    block_len = np.zeros(nb, dtype=np.int32)
    # in-cube offsets, row-major over (dt, dh, dw)
    dt, dh, dw = np.meshgrid(np.arange(ct), np.arange(ch), np.arange(cw), indexing="ij")
    dt, dh, dw = dt.ravel(), dh.ravel(), dw.ravel()
    j = 0
    for a in range(nt):
        for b in range(nh):
            for c in range(nw):
                t = a * ct + dt
                h = b * ch + dh
                w = c * cw + dw
                ok = (t < T) & (h < Hh) & (w < W)
                nat = (t[ok] * Hh + h[ok]) * W + w[ok]
                n = nat.size
                perm[j * B:j * B + n] = nat
                block_len[j] = n
                j += 1
    return Layout(T * Hh * W, nb * B, B, perm, block_len)


def layout_for(cfg: Config) -> Layout:
    if cfg.kind == "iid":
        return contiguous_layout(cfg.L)
    if cfg.kind == "flux":
        return contiguous_layout(cfg.text + cfg.img[0] * cfg.img[1])
    return cube_layout(cfg.grid, cfg.cube)


def k_sel_for(cfg: Config, nb: int) -> int:
    """Selected blocks per query tile: an explicit count, else ceil(keep * nb)."""
    if cfg.keep_blocks:
        return cfg.keep_blocks
    return min(nb, int(math.ceil(cfg.keep * nb - 1e-9)))


def to_blocks(x_nat: np.ndarray, layout: Layout) -> np.ndarray:
    """[..., L, d] natural order -> [..., L_pad, d] block order with zero padding."""
    out = np.zeros(x_nat.shape[:-2] + (layout.L_pad, x_nat.shape[-1]), dtype=x_nat.dtype)
    ok = layout.perm >= 0
    out[..., ok, :] = x_nat[..., layout.perm[ok], :]
    return out


def from_blocks(x_blk: np.ndarray, layout: Layout) -> np.ndarray:
    """[..., L_pad, d] block order -> [..., L, d] natural order (padding dropped)."""
    out = np.empty(x_blk.shape[:-2] + (layout.L, x_blk.shape[-1]), dtype=x_blk.dtype)
    ok = layout.perm >= 0
    out[..., layout.perm[ok], :] = x_blk[..., ok, :]
    return out


# ----------------------------------------------------------------------------- fields
def _fourier_field(rng: np.random.Generator, coords: list, extents: tuple, n_modes: int, d: int) -> np.ndarray:
    """sum_m a_m cos(2*pi*sum_axis f_{m,axis} x_axis / extent_axis + phi_m); a_m ~ N(0, 2/n_modes)."""
    ax = len(extents)
    f = rng.uniform(-2.0, 2.0, size=(n_modes, ax))
    phi = rng.uniform(0.0, 2.0 * np.pi, size=n_modes)
    a = rng.normal(0.0, math.sqrt(2.0 / n_modes), size=(n_modes, d))
    phase = np.zeros((coords[0].size, n_modes))
    for k in range(ax):
        phase += np.outer(coords[k] / extents[k], f[:, k])
    cosm = np.cos(2.0 * np.pi * phase + phi[None, :])
    return cosm @ a                                          # [n_points, d]


def _grid_coords(grid: tuple) -> list:
    T, Hh, W = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(Hh), np.arange(W), indexing="ij")
    return [t.ravel().astype(np.float64), h.ravel().astype(np.float64), w.ravel().astype(np.float64)]


def _rope_3d(x: np.ndarray, grid: tuple, split: tuple = ROPE_SPLIT, base: float = ROPE_BASE) -> np.ndarray:
    """Rotary embedding over (t, h, w): dims split ``split``, adjacent pairs rotated."""
    coords = _grid_coords(grid)
    out = x.copy()
    off = 0
    for axis, width in enumerate(split):
        k = np.arange(width // 2, dtype=np.float64)
        theta = base ** (-2.0 * k / width)
        ang = np.outer(coords[axis], theta)                 # [L, width/2]
        c, s = np.cos(ang), np.sin(ang)
        x0 = x[:, off:off + width:2]
        x1 = x[:, off + 1:off + width:2]
        out[:, off:off + width:2] = x0 * c - x1 * s
        out[:, off + 1:off + width:2] = x0 * s + x1 * c
        off += width
    return out


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x.astype(np.float32))
    return x.astype(np.float32)


# ----------------------------------------------------------------------------- public API
@dataclass
class Inputs:
    cfg: Config
    layout: Layout
    Q: np.ndarray              # [H, L_pad, d] float32, or uint16 bf16 bits
    K: np.ndarray
    V: np.ndarray
    K_sel: int
    extra: dict = field(default_factory=dict)

    @property
    def H(self) -> int:
        return self.cfg.H

    @property
    def d(self) -> int:
        return self.cfg.d

    @property
    def nb(self) -> int:
        return self.layout.nb

    def f64(self, name: str, h: int | None = None) -> np.ndarray:
        x = getattr(self, name)
        if h is not None:
            x = x[h]
        return to_float64(x, self.cfg.dtype)


def rope_split_for(cfg: Config) -> tuple:
    return cfg.rope_split or ROPE_SPLIT


def positions(cfg: Config, layout: Layout) -> np.ndarray:
    """[L_pad, 3] float32 (t, h, w) grid position of every slot in block order (0 for padding):
    the positions the rotary embedding of a rope config used."""
    coords = np.stack(_grid_coords(cfg.grid), axis=1)
    return to_blocks(coords, layout).astype(np.float32)


def make_head(cfg: Config, h: int, rng: np.random.Generator, layout: Layout, pre: dict | None = None):
    """Natural-order float64 (q, k, v) for one head, consuming rng in the documented order.
    For a rope config, ``pre`` (if given) receives q and k before the rotation."""
    d = cfg.d
    if cfg.kind == "iid":
        raise ValueError("iid draws whole tensors, not heads")
    if cfg.kind == "flux":
        raise ValueError("flux draws its shared field first")
    coords = _grid_coords(cfg.grid)
    F = _fourier_field(rng, coords, cfg.grid, cfg.n_modes, d)
    sd = math.sqrt(cfg.noise_var)
    L = layout.L
    q = F + sd * rng.standard_normal((L, d))
    k = F + sd * rng.standard_normal((L, d))
    v = F + sd * rng.standard_normal((L, d))
    q *= 1.0 / math.sqrt(d)
    if cfg.rope:
        if pre is not None:
            pre["q"], pre["k"] = q, k
        q = _rope_3d(q, cfg.grid, rope_split_for(cfg))
        k = _rope_3d(k, cfg.grid, rope_split_for(cfg))
    return q, k, v


def make(name: str | Config, heads: int | None = None, keep_pre_rope: bool = False) -> Inputs:
    """Canonical inputs of a named workload, in block layout. ``heads`` truncates H (tests).
    keep_pre_rope (rope configs): also return Q and K before the rotary embedding, each
    rounded to the dtype on its own (as a model holds them), and the token positions, in
    ``extra`` under "Q_pre", "K_pre" and "pos"."""
    cfg = CONFIGS[name] if isinstance(name, str) else name
    layout = layout_for(cfg)
    H = cfg.H if heads is None else min(heads, cfg.H)
    d = cfg.d
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    store = np.uint16 if cfg.dtype == "bf16" else np.float32
    Q = np.zeros((H, layout.L_pad, d), dtype=store)
    K = np.zeros_like(Q)
    V = np.zeros_like(Q)
    if cfg.kind == "iid":
        L = layout.L
        q = rng.standard_normal((cfg.H, L, d))[:H] / math.sqrt(d)
        k = rng.standard_normal((cfg.H, L, d))[:H]
        v = rng.standard_normal((cfg.H, L, d))[:H]
        Q[:] = to_blocks(_round(q, cfg.dtype), layout)
        K[:] = to_blocks(_round(k, cfg.dtype), layout)
        V[:] = to_blocks(_round(v, cfg.dtype), layout)
    elif cfg.kind == "flux":
        rows, cols = cfg.img
        y, x = np.meshgrid(np.arange(rows), np.arange(cols), indexing="ij")
        F = _fourier_field(rng, [y.ravel().astype(np.float64), x.ravel().astype(np.float64)],
                           (rows, cols), cfg.n_modes, d)
        L = layout.L
        for h in range(H):
            parts = []
            for _ in range(3):
                t = rng.standard_normal((L, d))
                t[cfg.text:] += F
                parts.append(t)
            q, k, v = parts
            q *= 1.0 / math.sqrt(d)
            Q[h] = to_blocks(_round(q, cfg.dtype), layout)
            K[h] = to_blocks(_round(k, cfg.dtype), layout)
            V[h] = to_blocks(_round(v, cfg.dtype), layout)
    else:
        keep = keep_pre_rope and cfg.rope
        if keep:
            extra = dict(Q_pre=np.zeros_like(Q), K_pre=np.zeros_like(K), pos=positions(cfg, layout))
        for h in range(H):
            pre = {} if keep else None
            q, k, v = make_head(cfg, h, rng, layout, pre)
            Q[h] = to_blocks(_round(q, cfg.dtype), layout)
            K[h] = to_blocks(_round(k, cfg.dtype), layout)
            V[h] = to_blocks(_round(v, cfg.dtype), layout)
            if keep:
                extra["Q_pre"][h] = to_blocks(_round(pre["q"], cfg.dtype), layout)
                extra["K_pre"][h] = to_blocks(_round(pre["k"], cfg.dtype), layout)
        if keep:
            return Inputs(cfg, layout, Q, K, V, k_sel_for(cfg, layout.nb), extra)
    return Inputs(cfg, layout, Q, K, V, k_sel_for(cfg, layout.nb))


def random_blocks(seed: int, H: int, nb: int, d: int, B: int = 64, dtype: str = "bf16",
                  block_len=None, scale_q: float | None = None, smooth: float = 0.0) -> Inputs:
    """Small seeded case for parity tests: i.i.d. normal (optionally plus a per-head 1D smooth
    field of strength ``smooth`` so that selection is peaked), ragged lengths if given."""
    rng = np.random.Generator(np.random.PCG64(seed))
    L_pad = nb * B
    if block_len is None:
        block_len = np.full(nb, B, dtype=np.int32)
    block_len = np.asarray(block_len, dtype=np.int32)
    valid = (np.arange(B)[None, :] < block_len[:, None]).reshape(-1)
    sq = 1.0 / math.sqrt(d) if scale_q is None else scale_q
    store = np.uint16 if dtype == "bf16" else np.float32
    out = []
    fieldv = None
    if smooth:
        pos = np.arange(L_pad, dtype=np.float64) / L_pad
        fieldv = np.zeros((H, L_pad, d))
        for h in range(H):
            f = rng.uniform(-4, 4, size=8)
            ph = rng.uniform(0, 2 * np.pi, size=8)
            a = rng.normal(0, math.sqrt(2.0 / 8), size=(8, d))
            fieldv[h] = np.cos(2 * np.pi * np.outer(pos, f) + ph) @ a
    for which in range(3):
        x = rng.standard_normal((H, L_pad, d))
        if fieldv is not None:
            x = x + smooth * fieldv
        if which == 0:
            x = x * sq
        x[:, ~valid, :] = 0.0
        out.append(_round(x, dtype).astype(store))
    cfg = Config("random", H=H, d=d, dtype=dtype, kind="iid", seed=seed, L=int(block_len.sum()))
    layout = Layout(int(block_len.sum()), L_pad, B,
                    np.where(valid, np.cumsum(valid) - 1, -1).astype(np.int64), block_len)
    return Inputs(cfg, layout, out[0], out[1], out[2], 0)
