"""Seeded synthetic workloads with the shapes of the WaveAlign evaluation.

The WaveAlign page ("WaveAlign: Cache-Aware Query-Row Scheduling for Sparse
Attention in Long-Video Generation", §VI-A) measures real Q/K/V captured from
Wan2.1 and LTX2.3 with masks from four sparse-attention methods.  Neither the
weights nor the prompts are available here, so every tensor below is drawn from
a fixed seed with the same shapes: video token grids (t, y, x) flattened to one
sequence, head dimension 128, block size 128, and block masks whose density and
row-length spread resemble dynamic sparse attention.

Seven workloads are defined (``CONFIGS``):

``tiny``         1 head, d=64, grid 4x16x16 (L=1,024), block 64.  Q/K/V are
                 fp32 N(0,1) rounded to bf16.  Mask: diagonal plus Bernoulli(0.5),
                 with query block 7 fully masked.
``layer16k``     12 heads, d=128, grid 16x32x32 (L=16,384), block 128.  Smooth
                 field plus noise.  Mask: blocks within Chebyshev distance 2 on
                 the (frame, row-band) block grid plus a lognormal number of far
                 blocks (about 20% density).
``wan75k``       40 heads, d=128, grid 21x45x80 (L=75,600, padded to 75,648),
                 block 128.  Smooth field plus noise.  Mask: per-head Top-k of
                 pooled block scores with k drawn from 5%..25% of the blocks, plus
                 the diagonal.
``hunyuan119k``  24 heads, d=128, grid 33x45x80 (L=118,800), block 128, tokens
                 along a generalized Hilbert curve over (t, y, x).  Mask: per-row Top-p
                 (0.9) over the softmax of pooled block scores.
``gsrs75k``      The ``wan75k`` tensors with an all-ones mask (the first, dense
                 search pass of the GSRS pipeline).
``random20``     The Wan shape with structureless masks: every block Bernoulli(0.2)
                 plus the diagonal, the random-mask locality floor of WaveAlign
                 Table I.
``wan364k``      The ``wan75k`` recipe at the length WaveAlign profiles its locality
                 and stage ablation on (§VI-D Fig. 11, §VI-E Fig. 12: 401 frames at
                 720x1280): grid 101x45x80 (L=363,600, 2,841 blocks per side), 40
                 heads.

Any field can be overridden (``make_workload("wan75k", grid=(9, 45, 80),
heads=16, density=0.1)``): ``density`` fixes the Top-k budget of every head,
which the skip-calibration sweep uses.

Smooth field: per head, 8 sinusoids sin(2*pi*f.p + phase) over normalised grid
coordinates p = (t/(T-1), y/(Y-1), x/(X-1)), f ~ U(-3, 3)^3, phase ~ U[0, 2*pi),
shared by Q, K and V of that head; each tensor projects the 8 channels to d
with its own N(0,1) 8 x d matrix and adds N(0, 0.5^2) noise.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

from .hilbert import video_hilbert_order

BASE_SEED = 20260928

_PURPOSES = {
    "field": 1, "proj_q": 2, "proj_k": 3, "proj_v": 4,
    "noise_q": 5, "noise_k": 6, "noise_v": 7, "mask": 8, "x0": 9,
    "topk": 10, "qkv": 11,
}


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    index: int
    heads: int
    head_dim: int
    grid: tuple  # (frames, height, width)
    block: int
    qkv: str     # "gaussian" | "smooth"
    mask: str    # "bernoulli" | "neighbour" | "topk" | "topp" | "dense" | "random"
    hilbert: bool = False
    density: float | None = None  # "topk": a fixed k = round(density * NB) for every head

    @property
    def seq_len(self) -> int:
        t, y, x = self.grid
        return t * y * x

    @property
    def num_blocks(self) -> int:
        return -(-self.seq_len // self.block)

    @property
    def padded_len(self) -> int:
        return self.num_blocks * self.block


CONFIGS = {
    "tiny": WorkloadConfig("tiny", 0, 1, 64, (4, 16, 16), 64, "gaussian", "bernoulli"),
    "layer16k": WorkloadConfig("layer16k", 1, 12, 128, (16, 32, 32), 128, "smooth", "neighbour"),
    "wan75k": WorkloadConfig("wan75k", 2, 40, 128, (21, 45, 80), 128, "smooth", "topk"),
    "hunyuan119k": WorkloadConfig("hunyuan119k", 3, 24, 128, (33, 45, 80), 128, "smooth", "topp",
                                  hilbert=True),
    "gsrs75k": WorkloadConfig("gsrs75k", 4, 40, 128, (21, 45, 80), 128, "smooth", "dense"),
    "random20": WorkloadConfig("random20", 5, 40, 128, (21, 45, 80), 128, "smooth", "random",
                               density=0.2),
    "wan364k": WorkloadConfig("wan364k", 6, 40, 128, (101, 45, 80), 128, "smooth", "topk"),
}


def get_config(name: str, **overrides) -> WorkloadConfig:
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


@dataclass
class Workload:
    cfg: WorkloadConfig
    q: torch.Tensor      # [H, L_pad, d] bf16, rows >= L are zero
    k: torch.Tensor
    v: torch.Tensor
    mask: torch.Tensor   # [H, MB, NB] uint8
    x0: torch.Tensor     # [H, MB, 2] float32, U[-1, 1): start block of the subspace iteration
    seq_len: int
    block: int

    @property
    def heads(self) -> int:
        return self.q.shape[0]

    @property
    def head_dim(self) -> int:
        return self.q.shape[2]

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def _seed(*parts: int) -> int:
    """Deterministic 63-bit seed from integer parts (a multiply-xorshift mix)."""
    h = 0x9E3779B97F4A7C15
    for p in parts:
        h ^= (p + 0x632BE59BD9B4E019) & 0xFFFFFFFFFFFFFFFF
        h = (h * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 29
    return h & 0x7FFFFFFFFFFFFFFF


def _gen(device, cfg_index: int, purpose: str, head: int, seed: int = BASE_SEED) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, cfg_index, _PURPOSES[purpose], head))
    return g


def _grid_coords(cfg: WorkloadConfig, device) -> torch.Tensor:
    t, y, x = cfg.grid
    tt = torch.arange(t, device=device, dtype=torch.float32) / max(t - 1, 1)
    yy = torch.arange(y, device=device, dtype=torch.float32) / max(y - 1, 1)
    xx = torch.arange(x, device=device, dtype=torch.float32) / max(x - 1, 1)
    g = torch.stack(torch.meshgrid(tt, yy, xx, indexing="ij"), dim=-1)
    return g.reshape(-1, 3)  # row-major (t, y, x)


def _smooth_qkv(cfg: WorkloadConfig, device, seed: int):
    H, d, L, Lp = cfg.heads, cfg.head_dim, cfg.seq_len, cfg.padded_len
    coords = _grid_coords(cfg, device)
    order = None
    if cfg.hilbert:
        order = torch.from_numpy(video_hilbert_order(*cfg.grid)).to(device)
    out = [torch.zeros(H, Lp, d, dtype=torch.bfloat16, device=device) for _ in range(3)]
    for h in range(H):
        g = _gen(device, cfg.index, "field", h, seed)
        freq = torch.rand(8, 3, generator=g, device=device) * 6.0 - 3.0
        phase = torch.rand(8, generator=g, device=device) * (2.0 * math.pi)
        field = torch.sin(2.0 * math.pi * (coords @ freq.T) + phase)  # [L, 8]
        if order is not None:
            field = field[order]
        for i, name in enumerate("qkv"):
            proj = torch.randn(8, d, generator=_gen(device, cfg.index, "proj_" + name, h, seed),
                               device=device)
            noise = torch.randn(L, d, generator=_gen(device, cfg.index, "noise_" + name, h, seed),
                                device=device)
            out[i][h, :L] = (field @ proj + 0.5 * noise).to(torch.bfloat16)
    return out


def _gaussian_qkv(cfg: WorkloadConfig, device, seed: int):
    H, d, L, Lp = cfg.heads, cfg.head_dim, cfg.seq_len, cfg.padded_len
    out = [torch.zeros(H, Lp, d, dtype=torch.bfloat16, device=device) for _ in range(3)]
    for h in range(H):
        g = _gen(device, cfg.index, "qkv", h, seed)
        for i in range(3):
            # fp32 N(0, 1), rounded to bf16 (round-to-nearest-even) for upload.
            out[i][h, :L] = torch.randn(L, d, generator=g, device=device).to(torch.bfloat16)
    return out


def _pooled_scores(q: torch.Tensor, k: torch.Tensor, L: int, block: int) -> torch.Tensor:
    """Unscaled mean(Q_blk) . mean(K_blk) over valid tokens, [H, MB, NB] fp32."""
    H, Lp, d = q.shape
    nb = Lp // block
    counts = torch.full((nb,), float(block), device=q.device)
    counts[-1] = float(L - (nb - 1) * block)
    qp = q.float().reshape(H, nb, block, d).sum(2) / counts[None, :, None]
    kp = k.float().reshape(H, nb, block, d).sum(2) / counts[None, :, None]
    return qp @ kp.transpose(1, 2)


def _order_desc(scores: torch.Tensor) -> torch.Tensor:
    """Column order per row by descending score, ties to the lower column."""
    nb = scores.shape[-1]
    # Stable sort of -score keeps equal scores in ascending column order.
    return torch.sort(-scores, dim=-1, stable=True).indices[..., :nb]


def _mask_bernoulli(cfg: WorkloadConfig, device, seed: int) -> torch.Tensor:
    H, nb = cfg.heads, cfg.num_blocks
    m = torch.zeros(H, nb, nb, dtype=torch.uint8, device=device)
    for h in range(H):
        g = _gen(device, cfg.index, "mask", h, seed)
        m[h] = (torch.rand(nb, nb, generator=g, device=device) < 0.5).to(torch.uint8)
        m[h].fill_diagonal_(1)
        if nb > 7:
            m[h, 7, :] = 0  # one fully masked query block
    return m


def _mask_random(cfg: WorkloadConfig, device, seed: int) -> torch.Tensor:
    """Every block Bernoulli(density) plus the diagonal (no structure to exploit)."""
    H, nb = cfg.heads, cfg.num_blocks
    m = torch.zeros(H, nb, nb, dtype=torch.uint8, device=device)
    for h in range(H):
        g = _gen(device, cfg.index, "mask", h, seed)
        m[h] = (torch.rand(nb, nb, generator=g, device=device) < cfg.density).to(torch.uint8)
        m[h].fill_diagonal_(1)
    return m


def _mask_neighbour(cfg: WorkloadConfig, device, seed: int) -> torch.Tensor:
    """Chebyshev-2 neighbours on the (frame, row band) block grid + lognormal far blocks."""
    H, nb = cfg.heads, cfg.num_blocks
    t_, y_, x_ = cfg.grid
    rows_per_block = cfg.block // x_
    assert rows_per_block * x_ == cfg.block and y_ % rows_per_block == 0
    bands = y_ // rows_per_block
    bt = torch.arange(nb, device=device) // bands
    by = torch.arange(nb, device=device) % bands
    near = ((bt[:, None] - bt[None, :]).abs() <= 2) & ((by[:, None] - by[None, :]).abs() <= 2)
    m = torch.zeros(H, nb, nb, dtype=torch.uint8, device=device)
    mu, sigma = math.log(6.0) - 0.32, 0.8  # lognormal with mean 6
    for h in range(H):
        g = _gen(device, cfg.index, "mask", h, seed)
        kfar = torch.exp(mu + sigma * torch.randn(nb, generator=g, device=device)).round().long()
        keys = torch.rand(nb, nb, generator=g, device=device)
        keys = keys.masked_fill(near, 2.0)  # neighbours are never drawn as far blocks
        rank = torch.argsort(torch.argsort(keys, dim=1), dim=1)
        avail = (~near).sum(1)
        kfar = torch.minimum(kfar, avail)
        far = rank < kfar[:, None]
        m[h] = (near | far).to(torch.uint8)
    return m


def _mask_topk(cfg: WorkloadConfig, q, k, device, seed: int) -> torch.Tensor:
    H, nb = q.shape[0], cfg.num_blocks
    scores = _pooled_scores(q, k, cfg.seq_len, cfg.block)
    lo, hi = math.ceil(0.05 * nb), math.floor(0.25 * nb)
    m = torch.zeros(H, nb, nb, dtype=torch.uint8, device=device)
    ar = torch.arange(nb, device=device)
    for h in range(H):
        g = _gen(device, cfg.index, "topk", h, seed)
        kk = int(torch.randint(lo, hi + 1, (1,), generator=g, device=device).item())
        if cfg.density is not None:
            kk = max(1, min(nb, round(cfg.density * nb)))
        idx = _order_desc(scores[h])[:, :kk]
        m[h].scatter_(1, idx, 1)
        m[h, ar, ar] = 1
    return m


def _mask_topp(cfg: WorkloadConfig, q, k, device, p: float = 0.9) -> torch.Tensor:
    H, nb = q.shape[0], cfg.num_blocks
    scores = _pooled_scores(q, k, cfg.seq_len, cfg.block).double()
    probs = torch.softmax(scores, dim=-1)
    m = torch.zeros(H, nb, nb, dtype=torch.uint8, device=device)
    for h in range(H):
        idx = _order_desc(probs[h])
        sp = torch.gather(probs[h], 1, idx)
        before = torch.cumsum(sp, dim=1) - sp
        keep = before < p  # smallest prefix whose mass reaches p
        m[h].scatter_(1, idx, keep.to(torch.uint8))
    return m


def make_workload(name_or_cfg, device="cpu", seed: int = BASE_SEED, **overrides) -> Workload:
    """Build one workload.  ``overrides`` replace config fields (e.g. ``heads=2``)."""
    cfg = name_or_cfg if isinstance(name_or_cfg, WorkloadConfig) else get_config(name_or_cfg)
    if overrides:
        cfg = replace(cfg, **overrides)
    device = torch.device(device)
    if cfg.qkv == "gaussian":
        q, k, v = _gaussian_qkv(cfg, device, seed)
    else:
        q, k, v = _smooth_qkv(cfg, device, seed)
    if cfg.mask == "bernoulli":
        mask = _mask_bernoulli(cfg, device, seed)
    elif cfg.mask == "neighbour":
        mask = _mask_neighbour(cfg, device, seed)
    elif cfg.mask == "topk":
        mask = _mask_topk(cfg, q, k, device, seed)
    elif cfg.mask == "topp":
        mask = _mask_topp(cfg, q, k, device)
    elif cfg.mask == "dense":
        mask = torch.ones(cfg.heads, cfg.num_blocks, cfg.num_blocks, dtype=torch.uint8, device=device)
    elif cfg.mask == "random":
        mask = _mask_random(cfg, device, seed)
    else:
        raise ValueError(cfg.mask)
    x0 = torch.empty(cfg.heads, cfg.num_blocks, 2, dtype=torch.float32, device=device)
    for h in range(cfg.heads):
        g = _gen(device, cfg.index, "x0", h, seed)
        x0[h] = torch.rand(cfg.num_blocks, 2, generator=g, device=device) * 2.0 - 1.0
    return Workload(cfg, q, k, v, mask, x0, cfg.seq_len, cfg.block)


def random_tiny_case(seed: int, heads: int = 2, seq_len: int = 300, head_dim: int = 64,
                     block: int = 64, density: float = 0.5, diagonal: bool = True,
                     empty_rows: tuple = (), device="cpu") -> Workload:
    """Small random case for property tests: N(0,1) Q/K/V, Bernoulli block mask."""
    nb = -(-seq_len // block)
    lp = nb * block
    g = torch.Generator(device=device)
    g.manual_seed(_seed(BASE_SEED, 1000 + seed))
    q, k, v = (torch.zeros(heads, lp, head_dim, dtype=torch.bfloat16, device=device) for _ in range(3))
    for t in (q, k, v):
        t[:, :seq_len] = torch.randn(heads, seq_len, head_dim, generator=g, device=device).to(torch.bfloat16)
    mask = (torch.rand(heads, nb, nb, generator=g, device=device) < density).to(torch.uint8)
    if diagonal:
        idx = torch.arange(nb, device=device)
        mask[:, idx, idx] = 1
    for r in empty_rows:
        if r < nb:
            mask[:, r, :] = 0
    x0 = torch.rand(heads, nb, 2, generator=g, device=device) * 2.0 - 1.0
    cfg = WorkloadConfig(f"random{seed}", 100 + seed, heads, head_dim, (1, 1, seq_len), block,
                         "gaussian", "bernoulli")
    return Workload(cfg, q, k, v, mask, x0, seq_len, block)


def wide_range_case(seed: int, heads: int = 2, seq_len: int = 1000, head_dim: int = 128,
                    block: int = 128, density: float = 0.6, device="cpu") -> Workload:
    """random_tiny_case with scores spread over hundreds of log2 units: Q is scaled by
    8 and each K block by a factor drawn from {0, 1, 8} (powers of two, exact in
    bf16).  Along a query block's list the block maxima then rise by far more than
    any lazy reference bound, blocks lie far below the row maximum (a zero block has
    all scores 0) and the kept probabilities span the whole fp32 range."""
    w = random_tiny_case(seed, heads=heads, seq_len=seq_len, head_dim=head_dim, block=block,
                         density=density, device=device)
    nb = w.mask.shape[1]
    g = torch.Generator(device=device)
    g.manual_seed(_seed(BASE_SEED, 2000 + seed))
    choice = torch.randint(0, 3, (heads, nb), generator=g, device=device)
    factor = torch.tensor([0.0, 1.0, 8.0], device=device)[choice]
    k = (w.k.float().view(heads, nb, block, head_dim) * factor[:, :, None, None])
    w.k = k.view(heads, nb * block, head_dim).to(torch.bfloat16)
    w.q = (w.q.float() * 8.0).to(torch.bfloat16)
    return w


def drift_states(w: Workload, n_states: int, sigma: float = 0.3, seed: int = BASE_SEED):
    """Q, K, V that drift across denoising steps: state s (0 <= s < n_states) is
    x + (s / (n_states - 1)) * delta_x for x in Q, K, V, with delta_x ~ N(0, sigma^2)
    drawn once per tensor from the seed (rows past L stay zero).  Returns a list of
    (q, k, v) in bf16 on the workload's device."""
    cfg = w.cfg
    dev = w.q.device
    deltas = []
    for name, x in (("noise_q", w.q), ("noise_k", w.k), ("noise_v", w.v)):
        g = _gen(dev, cfg.index + 1000, name, 0, seed)
        d = torch.randn(x.shape, generator=g, device=dev, dtype=torch.float32) * sigma
        d[:, w.seq_len:, :] = 0.0
        deltas.append(d)
    states = []
    for s in range(n_states):
        a = s / max(n_states - 1, 1)
        states.append(tuple((x.float() + a * d).to(torch.bfloat16)
                            for x, d in zip((w.q, w.k, w.v), deltas)))
    return states


def minhash_params(n_hash: int = 2, seed: int = BASE_SEED):
    """Coefficients of n_hash linear hash functions v -> (a v + b) mod (2^31 - 1) for the
    MinHash comparator order: a in [1, 2^31 - 2], b in [0, 2^31 - 2], drawn from the
    seed.  Returns two lists of Python ints."""
    g = torch.Generator(device="cpu")
    g.manual_seed(_seed(seed, 7919, n_hash))
    p = (1 << 31) - 1
    a = torch.randint(1, p, (n_hash,), generator=g, dtype=torch.int64).tolist()
    b = torch.randint(0, p, (n_hash,), generator=g, dtype=torch.int64).tolist()
    return a, b
