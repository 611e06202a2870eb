"""Seeded synthetic workloads for the folded split-KV MLA decode.

This module only draws inputs: lengths, block tables, FP8 query rows and a paged FP8
latent cache.  It holds none of the decode's arithmetic, and both the HIP path and the
CPU oracle are fed from it.

Recipe (one ``numpy.random.default_rng(seed)`` stream, drawn in this order):
  1. KV lengths per request;
  2. one permutation of the page pool; requests take their pages from it in order,
     so every block table is shuffled; unused table entries are -1 (never read);
  3. the query, x_q of shape [R, k*H, 576], row i = t*H + h (token-major, then head);
  4. the latent cache pool, x_kv of shape [pool, 64, 576] (512 latent then 64 rope).
FP8 codes follow the usual per-tensor convention code = e4m3(x / scale), x_hat =
code * scale, with x clipped to +-448 * scale first (torch turns out-of-range values
into NaN rather than saturating).  Cache slots past a request's length in its last page,
and whole unused pages, are filled with the E4M3 NaN code 0x7F, so that any read of
them shows up in the results.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

PAGE = 64
KDIM = 576
VDIM = 512
NAN_CODE = 0x7F
E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    R: int
    k: int
    H: int
    lengths: str          # "fixed:<L0>,<L1>,..." | "uniform:<L>" | "loguniform:<lo>,<hi>"
    pool_pages: int = 0   # 0: exactly the pages the requests use
    value_std: float = 1.0
    scale: float = 0.0    # 0: per-tensor amax / 448
    description: str = ""

    @property
    def M(self) -> int:
        return self.k * self.H


CONFIGS = {
    "c1": Config("c1", 2, 4, 8, "fixed:200,317", pool_pages=16, value_std=0.5, scale=1.0 / 64,
                 description="R=2 k=4 H=8, lengths 200 and 317, 16-page pool"),
    "c2": Config("c2", 64, 4, 8, "uniform:8192",
                 description="R=64 k=4 H=8 (32 rows), every length 8192"),
    "c3": Config("c3", 128, 7, 8, "loguniform:512,65536",
                 description="R=128 k=7 H=8 (56 rows), lengths log-uniform in [512, 65536]"),
    "c4": Config("c4", 32, 4, 64, "uniform:32768",
                 description="R=32 k=4 H=64 (256 rows), every length 32768"),
    "c5": Config("c5", 16, 7, 64, "fixed:131072" + ",1024" * 15,
                 description="R=16 k=7 H=64 (448 rows), one length 131072 and fifteen 1024"),
}

SM_SCALE = 1.0 / math.sqrt(192.0)   # qk_nope 128 + rope 64


@dataclasses.dataclass
class Workload:
    cfg: Config
    lengths: np.ndarray       # int32 [R]
    block_table: np.ndarray   # int32 [R, cols]
    q8: np.ndarray            # uint8 [R, M, 576]
    kv8: np.ndarray           # uint8 [pool, 64, 576]
    q_scale: float
    k_scale: float
    sm_scale: float = SM_SCALE

    @property
    def R(self) -> int:
        return self.q8.shape[0]

    @property
    def M(self) -> int:
        return self.q8.shape[1]

    @property
    def kv_bytes(self) -> int:
        """Bytes of KV each request reads once: sum_r L_r * 576."""
        return int(self.lengths.astype(np.int64).sum()) * KDIM


def draw_lengths(spec: str, R: int, rng: np.random.Generator) -> np.ndarray:
    kind, _, arg = spec.partition(":")
    if kind == "fixed":
        vals = [int(v) for v in arg.split(",")]
        assert len(vals) == R, (spec, R)
        return np.array(vals, dtype=np.int32)
    if kind == "uniform":
        return np.full(R, int(arg), dtype=np.int32)
    if kind == "loguniform":
        lo, hi = (int(v) for v in arg.split(","))
        x = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), R)))
        return np.clip(x, lo, hi).astype(np.int32)
    raise ValueError(spec)


def encode_e4m3(x: np.ndarray, scale: float) -> np.ndarray:
    """float32 values -> E4M3FN codes of x / scale, saturated to +-448 (torch cast)."""
    y = np.clip(x / np.float32(scale), -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _codes(x: np.ndarray, scale: float, chunk: int = 1 << 26) -> np.ndarray:
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for s in range(0, flat.size, chunk):
        out[s:s + chunk] = encode_e4m3(flat[s:s + chunk], scale)
    return out.reshape(x.shape)


def build_tables(lengths: np.ndarray, pool: int, rng: np.random.Generator, cols: int = 0):
    pages = (lengths.astype(np.int64) + PAGE - 1) // PAGE
    used = int(pages.sum())
    assert used <= pool, (used, pool)
    perm = rng.permutation(pool).astype(np.int32)
    cols = max(cols, int(pages.max()) if len(pages) else 1, 1)
    bt = np.full((len(lengths), cols), -1, dtype=np.int32)
    pos = 0
    for r, p in enumerate(pages):
        bt[r, :p] = perm[pos:pos + p]
        pos += p
    return bt, perm[:used]


def _draw_values(cfg: Config, lengths, bt, used, pool: int, rng: np.random.Generator,
                 poison: bool = True):
    """Query rows, then the cache pool, of one layer; NaN codes in unused pages and past
    each request's length (steps 3 and 4 of the recipe)."""
    R = lengths.shape[0]
    pages = (lengths.astype(np.int64) + PAGE - 1) // PAGE
    xq = rng.standard_normal((R, cfg.M, KDIM), dtype=np.float32) * np.float32(cfg.value_std)
    q_scale = cfg.scale or float(np.abs(xq).max()) / E4M3_MAX
    q8 = _codes(xq, q_scale)
    del xq

    xkv = rng.standard_normal((pool, PAGE, KDIM), dtype=np.float32)
    if cfg.value_std != 1.0:
        xkv *= np.float32(cfg.value_std)
    k_scale = cfg.scale or float(np.abs(xkv).max()) / E4M3_MAX
    kv8 = _codes(xkv, k_scale)
    del xkv

    if poison:
        mask = np.ones(pool, dtype=bool)
        mask[used] = False
        kv8[mask] = NAN_CODE
        for r in range(R):
            tail = int(lengths[r]) % PAGE
            if pages[r] > 0 and tail:
                kv8[bt[r, pages[r] - 1], tail:, :] = NAN_CODE
    return q8, kv8, float(q_scale), float(k_scale)


def generate(cfg: Config | str, seed: int = 0, lengths: np.ndarray | None = None,
             pool_pages: int | None = None, poison: bool = True) -> Workload:
    """Draw one workload.  ``lengths``/``pool_pages`` override the config (for tests)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = draw_lengths(cfg.lengths, cfg.R, rng)
    lengths = np.asarray(lengths, dtype=np.int32)
    R = lengths.shape[0]
    pages = (lengths.astype(np.int64) + PAGE - 1) // PAGE
    pool = pool_pages if pool_pages is not None else (cfg.pool_pages or int(pages.sum()))
    pool = max(pool, int(pages.sum()), 1)
    bt, used = build_tables(lengths, pool, rng)

    q8, kv8, q_scale, k_scale = _draw_values(cfg, lengths, bt, used, pool, rng, poison)
    return Workload(cfg, lengths, bt, q8, kv8, float(q_scale), float(k_scale))


def layers(w: Workload, n: int, seed: int = 0) -> list[Workload]:
    """The caches of n model layers over one batch: every layer shares the requests'
    lengths and block tables (one page id names the same token slot in every layer's
    pool) and has its own query rows and cache pool, drawn from the stream (seed, 3, layer)
    by steps 3 and 4 of the recipe.  Layer 0 is ``w`` itself."""
    pool = w.kv8.shape[0]
    pages = (w.lengths.astype(np.int64) + PAGE - 1) // PAGE
    used = np.concatenate([w.block_table[r, :pages[r]] for r in range(w.R)]) \
        if w.R else np.zeros(0, np.int32)
    out = [w]
    for li in range(1, n):
        rng = np.random.default_rng([seed, 3, li])
        q8, kv8, qs, ks = _draw_values(w.cfg, w.lengths, w.block_table, used, pool, rng)
        out.append(Workload(w.cfg, w.lengths, w.block_table, q8, kv8, qs, ks, w.sm_scale))
    return out


def small(R: int, k: int, H: int, lengths, seed: int = 0, extra_pages: int = 3,
          value_std: float = 1.0) -> Workload:
    """A small ad-hoc workload for tests: given lengths, a few spare (poisoned) pages."""
    cfg = Config("adhoc", R, k, H, "fixed:" + ",".join(str(int(v)) for v in lengths),
                 value_std=value_std)
    pages = sum((int(v) + PAGE - 1) // PAGE for v in lengths)
    return generate(cfg, seed=seed, pool_pages=pages + extra_pages)


UV_DIM = 128   # v_head_dim: the per-head output width of the W_UV up-projection


def uv_weights(H: int, seed: int = 0, std: float | None = None) -> np.ndarray:
    """Synthetic W_UV for H heads as BF16 bits (uint16), latent-contiguous: logical
    [H, 512, 128], stored [H][128][512] (for each head and output dim, the 512 latent
    weights are adjacent).  Values N(0, 1) * std (default 1/sqrt(512), so a projected row
    keeps the scale of the latent), rounded to BF16 by torch's cast.  Drawn from their own
    stream (seed, 1), so adding them leaves every other input unchanged."""
    rng = np.random.default_rng([seed, 1])
    s = np.float32(std if std is not None else 1.0 / math.sqrt(VDIM))
    x = rng.standard_normal((H, UV_DIM, VDIM), dtype=np.float32) * s
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def dcp_shards(w: Workload, world: int, interleave: int, seed: int = 0) -> list[Workload]:
    """Split a workload's KV cache over `world` decode-context-parallel ranks.

    Global position p of a request is stored on rank (p // interleave) % world, at local
    position (p // (interleave * world)) * interleave + p % interleave: blocks of
    `interleave` tokens dealt round-robin over the ranks.  Each rank gets its own paged
    pool (shuffled pages from a seeded permutation, NaN codes past each request's local
    length and in spare pages), block table and local lengths; every rank keeps the whole
    query.  Pure data movement: the rows are copied from the global cache unchanged."""
    rng = np.random.default_rng([seed, 2, world, interleave])
    R = w.R
    out = []
    for d in range(world):
        locs = []
        for r in range(R):
            T = int(w.lengths[r])
            p = np.arange(T, dtype=np.int64)
            mine = p[(p // interleave) % world == d]
            locs.append(mine)
        lengths = np.array([len(m) for m in locs], dtype=np.int32)
        pages = (lengths.astype(np.int64) + PAGE - 1) // PAGE
        pool = int(pages.sum()) + 2
        bt, used = build_tables(lengths, pool, rng)
        kv = np.full((pool, PAGE, KDIM), NAN_CODE, dtype=np.uint8)
        for r in range(R):
            mine = locs[r]
            if len(mine) == 0:
                continue
            src = w.kv8[w.block_table[r, mine // PAGE], mine % PAGE]     # [L_d, 576]
            j = np.arange(len(mine))
            kv[bt[r, j // PAGE], j % PAGE] = src
        out.append(Workload(w.cfg, lengths, bt, w.q8, kv, w.q_scale, w.k_scale, w.sm_scale))
    return out


@dataclasses.dataclass
class QueryBuildInputs:
    q: np.ndarray            # BF16 bits [n, H, 192]: q_nope (128) then q_pe (64) per head
    w_uk: np.ndarray         # BF16 bits [H, 512, 128]: W_UK_T [H, 128, 512] stored c-contiguous
    kv_c: np.ndarray         # BF16 bits [n, 512]: the normalised latent of each new token
    k_pe: np.ndarray         # BF16 bits [n, 64]: its rope key, before the rotation
    positions: np.ndarray    # int64 [n]
    cos_sin: np.ndarray      # float32 [max_pos, 64]: cos of 32 angles, then their sin
    neox: bool
    q_scale: float
    k_scale: float


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def query_build_inputs(n: int, H: int, seed: int = 0, max_pos: int = 1 << 17,
                       neox: bool = False) -> QueryBuildInputs:
    """Synthetic inputs of the step before the decode: the projected query of n new tokens
    and H heads, W_UK_T, the tokens' latent and rope key, their positions and a rotary
    table (angle i of position p: p * 10000^(-i/32)).  Scales are per tensor, amax / 448 of
    values bounded by construction (|ql_nope| <= sum |q_nope| |W|, |rope| <= |x| sqrt 2)."""
    rng = np.random.default_rng([seed, 3])
    q = _bf16_bits(rng.standard_normal((n, H, 192), dtype=np.float32))
    w = _bf16_bits(rng.standard_normal((H, VDIM, 128), dtype=np.float32) / np.float32(math.sqrt(128)))
    kv_c = _bf16_bits(rng.standard_normal((n, VDIM), dtype=np.float32))
    k_pe = _bf16_bits(rng.standard_normal((n, 64), dtype=np.float32))
    positions = rng.integers(0, max_pos, n).astype(np.int64)
    inv = 10000.0 ** (-np.arange(32) / 32.0)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    cos_sin = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    # scales from a bound of the largest value (the query: 6 sigma of a 128-term dot product
    # with unit-variance terms; the cache: the drawn amax, times sqrt 2 for the rotation)
    q_scale = 6.0 * 1.05 / E4M3_MAX
    kvf = torch.from_numpy(kv_c.view(np.int16)).view(torch.bfloat16).float().abs().max().item()
    kpf = torch.from_numpy(k_pe.view(np.int16)).view(torch.bfloat16).float().abs().max().item()
    k_scale = max(kvf, kpf * math.sqrt(2.0)) / E4M3_MAX
    return QueryBuildInputs(q, w, kv_c, k_pe, positions, cos_sin, neox, q_scale, k_scale)
