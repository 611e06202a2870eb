"""CPU oracle of the folded split-KV absorbed-MLA decode.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` are the only users.  The product package never imports this
module, and this module imports nothing from the product package.

The numeric parts (E4M3 decode, FP64 attention, LSE merge, split plan) live in
``oracle.c`` (built by ``oracle/build.py`` into ``liboracle.so``); this wrapper only
marshals numpy arrays.  The host-side fold rules and the value stage (the W_UV
up-projection after the merge: a BF16 decode and one matrix product per head) are small
enough to state here in Python, each with the passage it follows.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

PAGE = 64
KDIM = 576
VDIM = 512
BALANCED, FIXED = 0, 1


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build  # compile the checker on first use

            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        i32p = ctypes.POINTER(ctypes.c_int32)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        f64p = ctypes.POINTER(ctypes.c_double)
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_threads.argtypes = []
        lib.oracle_set_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_table.restype = None
        lib.oracle_e4m3_table.argtypes = [f64p]
        lib.oracle_attend.restype = ctypes.c_int
        lib.oracle_attend.argtypes = [u8p, u8p, ctypes.c_int64, i32p, ctypes.c_int32, i32p,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                      ctypes.c_double, ctypes.c_double, i32p, ctypes.c_int32,
                                      f64p, f64p]
        lib.oracle_merge.restype = None
        lib.oracle_merge.argtypes = [f64p, f64p, ctypes.c_int32, f64p, f64p]
        lib.oracle_plan.restype = ctypes.c_int
        lib.oracle_plan.argtypes = [i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, i32p, i32p,
                                    i32p, ctypes.c_int32]
        lib.oracle_item_range.restype = ctypes.c_int
        lib.oracle_item_range.argtypes = [i32p, ctypes.c_int32, i32p, ctypes.c_int32,
                                          ctypes.c_int32, i32p, i32p, i32p]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def threads() -> int:
    """Host threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> int:
    """Use n host threads from now on; returns the previous count."""
    return int(_load().oracle_set_threads(int(n)))


# --------------------------------------------------------------------------- E4M3FN

def e4m3_value(code: int) -> float:
    """Real value of one float8 E4M3FN code (NaN for 0x7F / 0xFF)."""
    return _load().oracle_e4m3_value(int(code) & 0xFF)


def e4m3_table() -> np.ndarray:
    """All 256 E4M3FN codes decoded to float64."""
    out = np.empty(256, dtype=np.float64)
    _load().oracle_e4m3_table(_ptr(out, ctypes.c_double))
    return out


# ------------------------------------------------------------------------ attention

def attend(q8, kv8, block_table, lengths, tasks, q_scale, k_scale, sm_scale):
    """Exact FP64 attention of folded rows over key ranges.

    q8: uint8 [R, M, 576]; kv8: uint8 [pool, 64, 576]; block_table: int32 [R, cols];
    lengths: int32 [R]; tasks: int32 [n, 4] of (request, row, key_begin, key_end).
    Returns (out float64 [n, 512], lse float64 [n], log2 units).
    """
    q8 = np.ascontiguousarray(q8, dtype=np.uint8)
    kv8 = np.ascontiguousarray(kv8, dtype=np.uint8)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    lengths = np.ascontiguousarray(lengths, dtype=np.int32)
    tasks = np.ascontiguousarray(tasks, dtype=np.int32).reshape(-1, 4)
    R, M = q8.shape[0], q8.shape[1]
    assert q8.shape[2] == KDIM and kv8.shape[1:] == (PAGE, KDIM)
    assert bt.ndim == 2 and bt.shape[0] == R and lengths.shape == (R,)
    n = tasks.shape[0]
    out = np.empty((n, VDIM), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    rc = _load().oracle_attend(_ptr(q8, ctypes.c_uint8), _ptr(kv8, ctypes.c_uint8),
                               kv8.shape[0], _ptr(bt, ctypes.c_int32), bt.shape[1],
                               _ptr(lengths, ctypes.c_int32), R, M, float(q_scale),
                               float(k_scale), float(sm_scale), _ptr(tasks, ctypes.c_int32),
                               n, _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_attend: task, length or page id out of range")
    return out, lse


def decode(q8, kv8, block_table, lengths, q_scale, k_scale, sm_scale, rows=None):
    """Folded decode of every request over its full key set [0, L_r).

    rows: optional iterable of (request, row) pairs to compute (default: all).
    Returns (out float64 [n, 512], lse float64 [n]) in the order of ``rows`` (default:
    request-major, then row).
    """
    R, M = q8.shape[0], q8.shape[1]
    if rows is None:
        rows = [(r, i) for r in range(R) for i in range(M)]
    tasks = np.array([(r, i, 0, int(lengths[r])) for r, i in rows], dtype=np.int32).reshape(-1, 4)
    return attend(q8, kv8, block_table, lengths, tasks, q_scale, k_scale, sm_scale)


# ---------------------------------------------------------------------------- merge

def merge(o, lse):
    """LSE merge of partials o [n, 512], lse [n] (log2) -> (out [512], lse)."""
    o = np.ascontiguousarray(o, dtype=np.float64).reshape(-1, VDIM)
    lse = np.ascontiguousarray(lse, dtype=np.float64).reshape(-1)
    assert o.shape[0] == lse.shape[0]
    out = np.empty(VDIM, dtype=np.float64)
    lo = np.empty(1, dtype=np.float64)
    _load().oracle_merge(_ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double), lse.shape[0],
                         _ptr(out, ctypes.c_double), _ptr(lo, ctypes.c_double))
    return out, float(lo[0])


# ----------------------------------------------------------------------------- plan

def plan(lengths, bt_cols, M, MT, W, min_split_tokens=256, max_splits=256, mode=BALANCED,
         list_len=None, split_cost=0):
    """Split plan: (counts int32 [R], offsets int32 [R+1], work int32 [list_len], items).

    work: items in request order as (request, first page) pairs, then the first item of each
    of the G = max(1, W // ceil(M / MT)) worker groups (G + 1 entries) at 2 * (R + W).
    split_cost: what one split costs a worker beyond its pages, in pages (BALANCED)."""
    lengths = np.ascontiguousarray(lengths, dtype=np.int32)
    R = lengths.shape[0]
    if list_len is None:
        list_len = 2 * (R + 2 * W)
    counts = np.zeros(R, dtype=np.int32)
    offsets = np.zeros(R + 1, dtype=np.int32)
    work = np.zeros(max(list_len, 1), dtype=np.int32)
    n = _load().oracle_plan(_ptr(lengths, ctypes.c_int32), R, bt_cols, M, MT, W,
                            min_split_tokens, max_splits, split_cost, mode,
                            _ptr(counts, ctypes.c_int32),
                            _ptr(offsets, ctypes.c_int32), _ptr(work, ctypes.c_int32), list_len)
    if n == -1:
        raise ValueError("oracle_plan: invalid arguments or lengths")
    if n == -2:
        raise ValueError("oracle_plan: list_len too small")
    return counts, offsets, work[:list_len], n


def item_range(work, n, lengths, i):
    """(request, first token, end token) of item i of a plan's work list of n items."""
    work = np.ascontiguousarray(work, dtype=np.int32)
    lengths = np.ascontiguousarray(lengths, dtype=np.int32)
    r, a, b = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    if _load().oracle_item_range(_ptr(work, ctypes.c_int32), int(n), _ptr(lengths, ctypes.c_int32),
                                 lengths.shape[0], int(i), ctypes.byref(r), ctypes.byref(a),
                                 ctypes.byref(b)) != 0:
        raise ValueError("oracle_item_range: bad item")
    return r.value, a.value, b.value


def group_starts(work, R, W, M, MT):
    """The first item of each worker group (G + 1 entries) from a plan's work list."""
    mt = -(-M // MT)
    G = max(1, W // mt)
    base = 2 * (R + W)
    return np.asarray(work[base:base + G + 1], dtype=np.int64)


# ------------------------------------------------------------------- fold (host rules)

def foldable(causal: bool, num_reqs: int, num_rows: int, num_decode_tokens: int,
             block_table_rows: int, max_query_len: int) -> int:
    """Query tokens per request when a decode batch can be folded, else 0.

    Page "drafter.attention", section foldable.  The rule: a batch folds into k tokens
    per request exactly when it is a non-causal draft block in which every request
    contributes a block of the same k >= 2 query tokens, every row is a decode token, and
    each request has a block-table row.  Uniform blocks are known from the shape alone:
    the rows split evenly over the requests and the longest block is that share.
    """
    k = num_rows // num_reqs if num_reqs > 0 else 0
    uniform_blocks = (num_reqs > 0 and k * num_reqs == num_rows
                      and max_query_len == k and num_rows == num_decode_tokens)
    folds = (not causal) and uniform_blocks and k >= 2 and block_table_rows >= num_reqs
    return k if folds else 0


def fold_plan(k: int, heads: int, need_lse: bool, max_fold_heads: int) -> int:
    """Tokens folded into one decode row.

    Page "drafter.attention", section fold_plan: with no LSE to return all k tokens fold
    into one row; a kernel that returns an LSE takes at most `max_fold_heads` heads per
    row, so the fold is the largest divisor f of k whose f * heads stays within it.
    """
    if not need_lse:
        return k
    f = k
    while f > 1 and (k % f != 0 or f * heads > max_fold_heads):
        f -= 1
    return f


# ------------------------------------------------------------ value stage (W_UV)

UVDIM = 128


def bf16_values(bits) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float64.  A BF16 value is the float32 whose upper 16
    bits are the pattern and whose lower 16 bits are zero."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):      # signalling-NaN patterns stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def uv_project(latent, w_uv_bits, heads: int) -> np.ndarray:
    """Attention output of folded rows: each merged latent row times its head's W_UV.

    Page "drafter.attention", DraftDcp (value stage: the merged BF16 latent rows times
    W_UV, accumulated in FP32 there, exactly here) and latent_major (W_UV [H, 512, 128]
    stored latent-contiguous, [H][128][512] in memory).  Folded row i of a request is
    draft token t = i // H of head h = i % H (page "drafter.attention", folded_decode), so
    its output is the 128 values sum_c latent[r, i, c] * W_UV[h, c, v], which land at
    [r * k + t, h * 128 + v] of the [R * k, H * 128] attention output.

    latent: float64 [R, M, 512]; w_uv_bits: uint16 [H, 128, 512]; returns float64
    [R, M, 128].
    """
    lat = np.asarray(latent, dtype=np.float64)
    assert lat.ndim == 3 and lat.shape[2] == VDIM and lat.shape[1] % heads == 0
    w = bf16_values(w_uv_bits).reshape(heads, UVDIM, VDIM)    # [h][v][c]
    out = np.empty(lat.shape[:2] + (UVDIM,), dtype=np.float64)
    for h in range(heads):
        out[:, h::heads, :] = lat[:, h::heads, :] @ w[h].T     # rows i with i % H == h
    return out


# ------------------------------------------------- decode context parallelism (DCP)

def dcp_owner(p: int, world: int, interleave: int):
    """(rank, local position) of global KV position p under DCP.

    Page "...cutedsl.mla.balanced", BalancedMla.decode: a rank holds a shard of each
    request's KV, described by cp = (world, rank, interleave).  Reading: blocks of
    `interleave` consecutive positions are dealt round-robin over the ranks, and a rank
    keeps its positions in global order."""
    blk = p // interleave
    return blk % world, (blk // world) * interleave + p % interleave


def dcp_local_count(n: int, world: int, rank: int, interleave: int) -> int:
    """How many of the global positions 0 .. n-1 the rank holds (by enumeration)."""
    if n <= 0:
        return 0
    p = np.arange(n, dtype=np.int64)
    return int(np.count_nonzero((p // interleave) % world == rank))


def visible_keys(total: int, k: int, t: int, causal: bool) -> int:
    """Global keys visible to draft token t (0 <= t < k) of a request of `total` keys
    (the block included).  Non-causal (page "drafter.attention", module docstring): the
    whole cache.  Causal (page "...cutedsl.mla.balanced", module docstring and
    BalancedMla.decode, the causal mask in global positions from the global lengths):
    token t sits at position total - k + t and sees positions up to and including it."""
    return total if not causal else max(0, total - k + t + 1)


def decode_causal(q8, kv8, block_table, totals, k, heads, q_scale, k_scale, sm_scale,
                  causal=True, rows=None):
    """Unsharded folded decode with each row's own key range [0, visible_keys)."""
    R, M = q8.shape[0], q8.shape[1]
    if rows is None:
        rows = [(r, i) for r in range(R) for i in range(M)]
    tasks = [(r, i, 0, visible_keys(int(totals[r]), k, i // heads, causal)) for r, i in rows]
    return attend(q8, kv8, block_table, totals, np.array(tasks, np.int32).reshape(-1, 4),
                  q_scale, k_scale, sm_scale)


def decode_dcp_rank(q8, kv8, block_table, local_lengths, totals, k, heads, q_scale, k_scale,
                    sm_scale, world, rank, interleave, causal=True, rows=None):
    """One rank's folded decode over its local shard: row i of request r attends to the
    rank's local keys whose global positions the row may see (a prefix of the shard,
    since the rank keeps its positions in global order).  Returns (out, lse) per row;
    rows that see none of the rank's keys get out 0 and lse -inf."""
    R, M = q8.shape[0], q8.shape[1]
    if rows is None:
        rows = [(r, i) for r in range(R) for i in range(M)]
    tasks = []
    for r, i in rows:
        n = visible_keys(int(totals[r]), k, i // heads, causal)
        lim = dcp_local_count(n, world, rank, interleave)
        assert lim <= int(local_lengths[r])
        tasks.append((r, i, 0, lim))
    return attend(q8, kv8, block_table, local_lengths, np.array(tasks, np.int32).reshape(-1, 4),
                  q_scale, k_scale, sm_scale)


def merge_sources(outs, lses):
    """Rows from several DCP sources merged (page "drafter.attention", DraftDcp: exp2
    weights of lse_s - max over their sum): outs [S, n, 512], lses [S, n] -> (out [n, 512],
    lse [n]); a row every source leaves empty stays out 0, lse -inf."""
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    n = outs.shape[1]
    out = np.zeros((n, VDIM))
    lse = np.full(n, -np.inf)
    for j in range(n):
        if np.all(np.isneginf(lses[:, j])):
            continue
        out[j], lse[j] = merge(outs[:, j], lses[:, j])
    return out, lse


# ------------------------------------------------ query build and cache write

def bf16_round(x) -> np.ndarray:
    """x rounded to the nearest BF16 value (8 significant bits), ties to even; written from
    the format's definition for normal-range values."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                         # x = m 2^e, 1/2 <= |m| < 1
    return np.ldexp(np.round(m * 256.0), e - 8)   # numpy rounds halves to even


def e4m3_encode(y) -> np.ndarray:
    """E4M3FN codes of real values y, rounded to nearest with ties to the even code and
    saturated at +-448 (the cast convention of the inputs: clip, then cast); NaN -> 0x7F.
    Written from the format's definition: the nearest of the decoded code values."""
    y = np.asarray(y, dtype=np.float64)
    table = e4m3_table()
    pos = np.arange(0, 0x7F)                  # codes 0x00 .. 0x7E: 0 .. 448, increasing
    vals = table[pos]
    a = np.minimum(np.abs(y), 448.0)
    j = np.clip(np.searchsorted(vals, a), 1, len(vals) - 1)
    lo, hi = vals[j - 1], vals[j]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & ((pos[j - 1] & 1) == 1))
    code = np.where(pick_hi, pos[j], pos[j - 1]).astype(np.uint8)
    code = np.where(a == 0, 0, code).astype(np.uint8)
    code = np.where(np.signbit(y), code | 0x80, code)      # negative values keep the sign,
    return np.where(np.isnan(y), 0x7F, code).astype(np.uint8)   # zero included


def rope(x, cos, sin, neox: bool):
    """Rotary embedding of the last axis (64 dims) with per-row cos/sin [.., 32].
    Non-NeoX: pairs (2i, 2i+1) turn by angle i; NeoX: pairs (i, i + 32)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    if neox:
        a, b = x[..., :32], x[..., 32:]
        out[..., :32] = a * cos - b * sin
        out[..., 32:] = b * cos + a * sin
    else:
        a, b = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = a * cos - b * sin
        out[..., 1::2] = b * cos + a * sin
    return out


def build_query_and_cache(q_bits, w_uk_bits, kv_c_bits, k_pe_bits, positions, cos_sin, neox):
    """Exact (FP64) values of the absorbed decode query and of the cache rows, before the
    FP8 cast.  Page "drafter.attention", DraftDcp._forward: q [n, H, 192] splits into
    q_nope (128) and q_pe (64); ql_nope = q_nope times W_UK_T per head ([H, 128, 512],
    given here stored [H][512][128]); the query row is ql_nope ++ rope(q_pe) (576) and the
    cache row kv_c_normed ++ rope(k_pe) (576), at each token's position (cos/sin from the
    table row of that position: 32 cos then 32 sin).  Returns (query [n, H, 576], cache
    rows [n, 576])."""
    q = bf16_values(q_bits)                                   # [n, H, 192]
    n, H = q.shape[0], q.shape[1]
    w = bf16_values(w_uk_bits).reshape(H, VDIM, 128)          # [h][l][c]
    kvc = bf16_values(kv_c_bits).reshape(n, VDIM)
    kpe = bf16_values(k_pe_bits).reshape(n, 64)
    cs = np.asarray(cos_sin, dtype=np.float64)[np.asarray(positions)]   # [n, 64]
    cos, sin = cs[:, :32], cs[:, 32:]
    query = np.empty((n, H, KDIM))
    for h in range(H):
        query[:, h, :VDIM] = q[:, h, :128] @ w[h].T
    query[:, :, VDIM:] = rope(q[:, :, 128:], cos[:, None, :], sin[:, None, :], neox)
    rows = np.empty((n, KDIM))
    rows[:, :VDIM] = kvc
    rows[:, VDIM:] = rope(kpe, cos, sin, neox)
    return query, rows


def e4m3_cast_scaled(x, scale: float) -> np.ndarray:
    """E4M3 codes of x / scale with the scaling decided in FP32 as the kernels decide it:
    x (a BF16 value, exact in FP32) times the FP32 reciprocal of the FP32 scale, rounded
    to FP32, then cast.  (An exact division would settle exact ties differently when the
    scale makes x / scale land on one.)"""
    inv = np.float32(1.0) / np.float32(scale)
    y = np.asarray(x, dtype=np.float64).astype(np.float32) * inv
    return e4m3_encode(y.astype(np.float64))


def e4m3_valid_codes(y, rel: float):
    """The E4M3 codes a cast of any value within a relative distance `rel` of y may give:
    (low, high) codes of the interval's ends (the cast is monotone)."""
    y = np.asarray(y, dtype=np.float64)
    lo = e4m3_encode(y - np.abs(y) * rel)
    hi = e4m3_encode(y + np.abs(y) * rel)
    return lo, hi
