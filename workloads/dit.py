"""Seeded synthetic DiT-shaped attention inputs.

This module only draws random inputs and describes workload shapes. It holds
none of the attention method's arithmetic, so both the fp64 oracle (through
the tests) and the HIP path (through the binding) can consume its tensors.

Token geometry follows the video / image diffusion transformers evaluated in
"PISA: Piecewise Sparse Attention Is Wiser for Efficient Diffusion
Transformers", section 4 (Wan2.1, HunyuanVideo, FLUX.1, SD3.5): tokens of a
(t, y, x) latent grid in raster order, x fastest, optionally followed by text
tokens. Trained weights are not available, so queries and keys are built
from random Fourier features of the normalised grid coordinates (spatially
smooth, like real DiT keys) plus white noise, and values are unit normal.

Recipe (all draws from numpy's PCG64 ``default_rng``):
  * shared stream ``default_rng(seed)``: omega ~ N(0, freq_std^2), shape
    (n_feat, 3) (one frequency per grid axis), then phi ~ U[0, 2*pi), shape
    (n_feat,).
  * coordinates c_a = i_a / n_a on each axis; features f_m(c) = cos(omega_m . c
    + phi_m), m = 1..n_feat, shared by all heads.
  * per (b, h) stream ``default_rng([seed, b, h])``, drawn in this order:
    W_q (n_feat x d), W_k (n_feat x d), noise_q (L_img x d), noise_k
    (L_img x d), V (L x d), then for text tokens q_text, k_text (L_text x d),
    all standard normal.
  * image tokens: Q = f W_q / sqrt(n_feat) + 0.5 noise_q, K likewise.
  * text tokens (appended after the image tokens): Q, K, V iid N(0, 1).
  * values are computed in float32 and rounded to the storage dtype with
    round-to-nearest-even (torch's conversion).
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch

N_FEAT = 32
NOISE_STD = 0.5


@dataclass(frozen=True)
class Workload:
    """One synthetic attention problem.

    ``keep_permille`` gives the kept fraction of kv-blocks per query block in
    units of 1/1000; ``keep_k`` overrides it with an explicit count.
    """

    name: str
    dtype: str              # "bf16" or "fp32"
    B: int
    H: int
    d: int
    grid: tuple             # (t, y, x) image/video latent grid
    text_tokens: int = 0
    block: int = 64
    keep_permille: int | None = None
    keep_k: int | None = None
    lam: float = 0.1
    seed: int = 0
    freq_std: float = 3.0
    note: str = ""

    @property
    def L(self) -> int:
        t, y, x = self.grid
        return t * y * x + self.text_tokens

    @property
    def T(self) -> int:
        return -(-self.L // self.block)

    @property
    def k(self) -> int:
        """Exact kv-blocks per query block: an explicit count, else ceil(keep * T)."""
        if self.keep_k is not None:
            return int(self.keep_k)
        return -(-self.keep_permille * self.T // 1000)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)

    def describe(self) -> dict:
        return {
            "workload": self.name, "dtype": self.dtype, "B": self.B, "H": self.H,
            "L": self.L, "d": self.d, "grid_txy": list(self.grid),
            "text_tokens": self.text_tokens, "block": self.block, "T": self.T,
            "keep_k": self.k, "lambda": self.lam, "seed": self.seed,
        }


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", "fp32", 1, 2, 64, (4, 16, 16), 0, 64,
                          keep_k=4, lam=0.1, seed=0,
                          note="1024 tokens on a 4x16x16 grid, fp32 check case"),
    "image_4608": Workload("image_4608", "bf16", 1, 24, 128, (1, 64, 64), 512, 64,
                           keep_permille=250, lam=0.1, seed=1,
                           note="image DiT: 64x64 latent + 512 text tokens"),
    "video480p_32760": Workload("video480p_32760", "bf16", 1, 12, 128, (21, 30, 52), 0, 64,
                                keep_permille=125, lam=0.1, seed=2,
                                note="480p video DiT: 21x30x52 latent grid"),
    "video720p_75600": Workload("video720p_75600", "bf16", 1, 40, 128, (21, 45, 80), 0, 64,
                                keep_permille=125, lam=0.1, seed=3,
                                note="720p video DiT: 21x45x80 latent grid"),
    "video_long_118800": Workload("video_long_118800", "bf16", 1, 24, 128, (33, 45, 80), 0, 64,
                                  keep_permille=100, lam=0.1, seed=4,
                                  note="long video DiT: 33x45x80 latent grid"),
}
# Dense-attention control of the long-video shape: every kv-block exact.
WORKLOADS["video_long_118800_dense"] = WORKLOADS["video_long_118800"].with_(
    name="video_long_118800_dense", keep_permille=1000)


def _features(w: Workload) -> np.ndarray:
    """Random Fourier features of the normalised (t, y, x) coordinates, [L_img, N_FEAT]."""
    rng = np.random.default_rng(w.seed)
    omega = rng.normal(0.0, w.freq_std, size=(N_FEAT, 3))
    phi = rng.uniform(0.0, 2.0 * np.pi, size=(N_FEAT,))
    nt, ny, nx = w.grid
    ct = np.arange(nt) / nt
    cy = np.arange(ny) / ny
    cx = np.arange(nx) / nx
    # raster order, x fastest
    T_, Y_, X_ = np.meshgrid(ct, cy, cx, indexing="ij")
    coords = np.stack([T_.ravel(), Y_.ravel(), X_.ravel()], axis=1)   # [L_img, 3]
    return np.cos(coords @ omega.T + phi[None, :])                     # [L_img, N_FEAT]


def _one_head(w: Workload, feats32: np.ndarray, b: int, h: int):
    """Draw (q, k, v) float32 arrays [L, d] for batch b, head h."""
    rng = np.random.default_rng([w.seed, b, h])
    d = w.d
    l_img = feats32.shape[0]
    f32 = np.float32
    wq = rng.standard_normal((N_FEAT, d), dtype=f32)
    wk = rng.standard_normal((N_FEAT, d), dtype=f32)
    nq = rng.standard_normal((l_img, d), dtype=f32)
    nk = rng.standard_normal((l_img, d), dtype=f32)
    v = rng.standard_normal((w.L, d), dtype=f32)
    inv = f32(1.0 / math.sqrt(N_FEAT))
    q = feats32 @ wq * inv + f32(NOISE_STD) * nq
    k = feats32 @ wk * inv + f32(NOISE_STD) * nk
    if w.text_tokens:
        qt = rng.standard_normal((w.text_tokens, d), dtype=f32)
        kt = rng.standard_normal((w.text_tokens, d), dtype=f32)
        q = np.concatenate([q, qt], axis=0)
        k = np.concatenate([k, kt], axis=0)
    return q, k, v


def make_inputs(w: Workload | str, heads=None, threads: int | None = None):
    """Return CPU tensors (q, k, v), each [B, H', L, d] in the workload dtype.

    ``heads`` selects a subset of head indices; each head has its own random
    stream, so a subset reproduces exactly those heads of the full tensor.
    By default all H heads are drawn.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    heads = list(range(w.H)) if heads is None else list(heads)
    feats32 = _features(w).astype(np.float32)
    shape = (w.B, len(heads), w.L, w.d)
    dt = w.torch_dtype
    q = torch.empty(shape, dtype=dt)
    k = torch.empty(shape, dtype=dt)
    v = torch.empty(shape, dtype=dt)
    jobs = [(b, hi, h) for b in range(w.B) for hi, h in enumerate(heads)]

    def run(job):
        b, hi, h = job
        qa, ka, va = _one_head(w, feats32, b, h)
        q[b, hi].copy_(torch.from_numpy(qa).to(dt))
        k[b, hi].copy_(torch.from_numpy(ka).to(dt))
        v[b, hi].copy_(torch.from_numpy(va).to(dt))

    nthreads = threads or min(16, os.cpu_count() or 1, max(1, len(jobs)))
    if nthreads <= 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(run, jobs))
    return q, k, v


def random_uniform_inputs(B, H, L, d, dtype=torch.float32, seed=0, scale=1.0):
    """Plain iid N(0, scale^2) q, k, v (for edge-case shapes not tied to a grid)."""
    g = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        a = g.standard_normal((B, H, L, d)).astype(np.float32) * np.float32(scale)
        out.append(torch.from_numpy(a).to(dtype))
    return tuple(out)


def varying_need_inputs(B, H, L, d, dtype=torch.bfloat16, seed=17):
    """Inputs whose query blocks need very different numbers of exact blocks
    (a stand-in for DiT attention in which some outputs attend sharply and
    others broadly, the situation the ALLOT review's per-output budgets are
    for). Recipe, numpy ``default_rng(seed)``:
      * base q, k, v iid N(0, 0.8^2), shape [B, H, L, d];
      * every key of block j is offset by mu_j ~ N(0, 3^2 I) (drawn per
        (b, h, j)), so block centroids are far apart and the centroid logits
        vary across blocks;
      * a unit direction u (drawn per (b, h)) scaled to norm 3; the queries of
        block i are 0.1 q + f_i u with f_i = 0.2, 1, 5 repeating over the
        blocks, so blocks with a small f spread their attention over many
        blocks and blocks with a large f concentrate it on a few.
    v is left as drawn. Values are rounded to ``dtype`` at the end."""
    g = np.random.default_rng(seed)
    f32 = np.float32
    T = -(-L // 64)
    q = g.standard_normal((B, H, L, d), dtype=f32) * f32(0.8)
    k = g.standard_normal((B, H, L, d), dtype=f32) * f32(0.8)
    v = g.standard_normal((B, H, L, d), dtype=f32) * f32(0.8)
    mu = g.standard_normal((B, H, T, d), dtype=f32) * f32(3.0)
    k += np.repeat(mu, 64, axis=2)[:, :, :L]
    u = g.standard_normal((B, H, 1, d), dtype=f32)
    u *= f32(3.0) / np.linalg.norm(u, axis=-1, keepdims=True)
    f = np.tile(np.repeat(np.array([0.2, 1.0, 5.0], dtype=f32), 64), -(-L // 192))[:L]
    q = f32(0.1) * q + f[None, None, :, None] * u
    return tuple(torch.from_numpy(np.ascontiguousarray(x)).to(dtype) for x in (q, k, v))
