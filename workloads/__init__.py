"""Seeded synthetic inputs for the five decode-step workloads.

This module only draws random inputs: sequence lengths, activity, absolute
positions, block-table assignments, bf16 activations and history FP8 codes.
It holds none of the attention, quantisation or layout arithmetic of the
method; both the HIP path and the CPU oracle receive what it produces.

History codes are torch's own float8_e4m3fn casts of N(0,1)/scale draws, i.e.
the cache holds what a quantised N(0,1) history looks like.  Referenced blocks
get codes in every byte; unreferenced blocks are filled with 0x7F (an FP8 NaN)
so that any read outside the tables shows up.
"""
from dataclasses import dataclass, field
import math

import numpy as np
import torch

POISON = 0x7F


@dataclass(frozen=True)
class Config:
    name: str
    kinds: tuple            # per layer: "swa" or "full"; layer i uses buffer i // 2
    batch: int
    hq: int
    hkv: int
    head_dim: int
    block: int
    ctx: tuple              # ("fixed", L) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    seed: int
    window: int = 128
    n_inactive: int = 0
    pos_offset_max: int = 0  # absolute positions = U{0..max} + token index
    k_scale: float = 1.0 / 8
    v_scale: float = 1.0 / 16
    nb_policy: tuple = ("slack", 1.25)   # ("fixed", nb) | ("slack", f) | ("hbm_frac", f)
    max_ctx: int = 0        # table width = ceil(max_ctx / block)

    @property
    def layers(self):
        return len(self.kinds)

    @property
    def n_buffers(self):
        return (self.layers + 1) // 2

    @property
    def table_width(self):
        return -(-self.max_ctx // self.block)


CONFIGS = {
    "cfg1": Config("cfg1_full_b1_h8x1_bk16_L256", ("full",), 1, 8, 1, 64, 16,
                   ("fixed", 256), seed=0, k_scale=1.0 / 8, v_scale=1.0 / 8,
                   nb_policy=("fixed", 64), max_ctx=256),
    "cfg2": Config("cfg2_pair_b8_h64x8_bk32_L1k-4k", ("swa", "full"), 8, 64, 8, 64, 32,
                   ("uniform", 1024, 4096), seed=1, max_ctx=4096),
    "cfg3": Config("cfg3_36L_b64_h64x8_bk32_L8192", ("swa", "full") * 18, 64, 64, 8, 64, 32,
                   ("fixed", 8192), seed=2, max_ctx=8192),
    "cfg4": Config("cfg4_full_b128_h64x8_bk32_L128-32k", ("full",), 128, 64, 8, 64, 32,
                   ("loguniform", 128, 32768), seed=3, nb_policy=("hbm_frac", 0.30),
                   max_ctx=32768),
    "cfg5": Config("cfg5_pair_b256_64off_h64x8_bk16_L100-600", ("swa", "full"), 256, 64, 8,
                   64, 16, ("uniform", 100, 600), seed=4, n_inactive=64,
                   pos_offset_max=100000, max_ctx=600),
}


def block_bytes(cfg: Config) -> int:
    """Bytes one block id occupies across both halves of a buffer."""
    return 2 * cfg.hkv * cfg.block * cfg.head_dim


def _draw_lengths(cfg: Config, rng) -> np.ndarray:
    kind = cfg.ctx[0]
    if kind == "fixed":
        return np.full(cfg.batch, cfg.ctx[1], dtype=np.int32)
    if kind == "uniform":
        return rng.integers(cfg.ctx[1], cfg.ctx[2] + 1, size=cfg.batch).astype(np.int32)
    if kind == "loguniform":
        u = rng.uniform(math.log(cfg.ctx[1]), math.log(cfg.ctx[2]), size=cfg.batch)
        return np.clip(np.round(np.exp(u)), cfg.ctx[1], cfg.ctx[2]).astype(np.int32)
    raise ValueError(kind)


def _bf16(x_f32: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)


@dataclass
class Workload:
    cfg: Config
    nb: int
    seq_lens: np.ndarray        # int32 [B], tokens including the new one
    active: np.ndarray          # uint8 [B]
    positions: np.ndarray       # int64 [B], absolute position of the new token
    bt_full: np.ndarray         # int32 [B, width], -1 where unallocated
    bt_swa: np.ndarray          # int32 [B, width], -1 where unallocated
    q: torch.Tensor             # bf16 [layers, B, Hq, D] (host)
    k_new: torch.Tensor         # bf16 [layers, B, Hkv, D] (host)
    v_new: torch.Tensor         # bf16 [layers, B, Hkv, D] (host)
    k_scale: list = field(default_factory=list)
    v_scale: list = field(default_factory=list)
    referenced: np.ndarray = None   # int64 sorted block ids present in any table

    @property
    def half_bytes(self):
        c = self.cfg
        return self.nb * c.hkv * c.block * c.head_dim


def make_workload(cfg: Config, hbm_bytes: int = None, swa_keep_blocks: int = None) -> Workload:
    """Draw everything except the cache bytes.

    Block ids come from one random permutation of [0, nb): all full-table
    blocks first, then the sliding-window blocks, so the two sets are
    disjoint.  The sliding-window table, like a scheduler that frees blocks
    behind the window, only holds blocks for the last logical blocks of each
    sequence (enough to cover ``window + block`` recent tokens); elsewhere -1.
    """
    rng = np.random.default_rng(cfg.seed)
    B, Bk = cfg.batch, cfg.block
    L = _draw_lengths(cfg, rng)
    active = np.ones(B, dtype=np.uint8)
    if cfg.n_inactive:
        active[rng.choice(B, size=cfg.n_inactive, replace=False)] = 0
    positions = (L.astype(np.int64) - 1)
    if cfg.pos_offset_max:
        positions = positions + rng.integers(0, cfg.pos_offset_max + 1, size=B)
    n_full = -(-L // Bk)
    has_swa = "swa" in cfg.kinds
    if has_swa:
        keep = swa_keep_blocks or (-(-(cfg.window + Bk) // Bk))
        swa_first = np.maximum(0, n_full - keep)
        n_swa = n_full - swa_first
    else:
        swa_first = n_full
        n_swa = np.zeros(B, dtype=np.int64)
    needed = int(n_full.sum() + n_swa.sum())
    pol = cfg.nb_policy
    if pol[0] == "fixed":
        nb = int(pol[1])
    elif pol[0] == "slack":
        nb = int(math.ceil(pol[1] * needed))
    elif pol[0] == "hbm_frac":
        if hbm_bytes is None:
            raise ValueError("hbm_frac sizing needs the device's HBM size")
        nb = int(pol[1] * hbm_bytes) // block_bytes(cfg)
    else:
        raise ValueError(pol)
    if nb < needed:
        raise ValueError(f"pool of {nb} blocks cannot hold {needed}")
    if nb > np.iinfo(np.int32).max:
        raise ValueError("block ids must fit int32")
    if pol[0] == "hbm_frac":
        # a full permutation of millions of ids is wasteful: draw distinct ids
        perm = rng.choice(nb, size=needed, replace=False)
    else:
        perm = rng.permutation(nb)
    W = cfg.table_width
    bt_full = np.full((B, W), -1, dtype=np.int32)
    bt_swa = np.full((B, W), -1, dtype=np.int32)
    at = 0
    for b in range(B):
        bt_full[b, :n_full[b]] = perm[at:at + n_full[b]]
        at += int(n_full[b])
    for b in range(B):
        bt_swa[b, swa_first[b]:n_full[b]] = perm[at:at + n_swa[b]]
        at += int(n_swa[b])
    referenced = np.sort(np.asarray(perm[:at], dtype=np.int64))
    nl = cfg.layers
    q = _bf16(rng.standard_normal((nl, B, cfg.hq, cfg.head_dim), dtype=np.float32))
    k_new = _bf16(rng.standard_normal((nl, B, cfg.hkv, cfg.head_dim), dtype=np.float32))
    v_new = _bf16(rng.standard_normal((nl, B, cfg.hkv, cfg.head_dim), dtype=np.float32))
    return Workload(cfg, nb, L, active, positions, bt_full, bt_swa, q, k_new, v_new,
                    [cfg.k_scale] * nl, [cfg.v_scale] * nl, referenced)


def rope_tables(wl: Workload, base: float = 10000.0):
    """Per-sequence rotary cosines and sines for this step, float32 [B, D/2].

    The pages carry cos/sin in the attention control but give no frequency
    schedule; this draws them from the geometric schedule of the original
    rotary-embedding paper (frequency i = base^(-2i/D)) at each sequence's
    absolute position, angles in float64, then rounded to float32.  Large
    absolute positions (the offset workload) give angles far from zero, so
    every quadrant and both signs of cos/sin occur.
    """
    D = wl.cfg.head_dim
    inv = base ** (-2.0 * np.arange(D // 2, dtype=np.float64) / D)
    ang = wl.positions.astype(np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _codes_like_normal(n: int, scale: float, gen: torch.Generator, device) -> torch.Tensor:
    x = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
    return x.div_(scale).to(torch.float8_e4m3fn).view(torch.uint8)


def fill_buffer(buf: torch.Tensor, wl: Workload, buffer_index: int,
                chunk_blocks: int = 8192) -> None:
    """Fill one shared buffer (uint8 [2 * half_bytes], any device) in place:
    history codes in referenced blocks, 0x7F elsewhere.  Deterministic in
    (seed, buffer_index) for a given device type."""
    cfg = wl.cfg
    per_blk = cfg.hkv * cfg.block * cfg.head_dim
    halves = buf.view(2, wl.nb, per_blk)
    halves.fill_(POISON)
    gen = torch.Generator(device=buf.device)
    gen.manual_seed(1_000_003 * (cfg.seed + 1) + 7919 * buffer_index)
    ids = torch.from_numpy(wl.referenced).to(buf.device)
    for half, scale in ((0, cfg.k_scale), (1, cfg.v_scale)):
        for s in range(0, ids.numel(), chunk_blocks):
            sel = ids[s:s + chunk_blocks]
            codes = _codes_like_normal(sel.numel() * per_blk, scale, gen, buf.device)
            halves[half].index_copy_(0, sel, codes.view(sel.numel(), per_blk))


def make_buffers(wl: Workload, device="cpu"):
    """All shared buffers of a workload, filled."""
    bufs = []
    for j in range(wl.cfg.n_buffers):
        t = torch.empty(2 * wl.half_bytes, dtype=torch.uint8, device=device)
        fill_buffer(t, wl, j)
        bufs.append(t)
    return bufs
