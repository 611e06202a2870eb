"""ctypes binding of libamla.so (include/amla.h): argument marshalling only.

Every step of the decode runs in the HIP kernels of csrc/amla.hip.  torch is used for
device memory (``data_ptr()``) and streams (``torch.cuda.current_stream().cuda_stream``)
and nothing else.  There is no CPU fallback: ``load()`` raises when the library is
missing or was not built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libamla.so")

PAGE = 64
KDIM = 576
VDIM = 512
UVDIM = 128
MAX_ROWS = 1024
MAX_REQS = 4096
MAX_SPLITS = 256
MAX_SPLIT_COST = 4096
# pages a split costs its worker beyond its own (query rows, partials), measured on gfx950
SPLIT_COST_ONE_TILE = 8    # splits of one row tile (M <= MT)
SPLIT_COST_MULTI_TILE = 4  # splits of several row tiles


def split_cost_default(mtile, rows_per_req):
    """The library's measured split cost for splits of ``rows_per_req`` rows in tiles of
    ``mtile`` rows."""
    return SPLIT_COST_ONE_TILE if rows_per_req <= mtile else SPLIT_COST_MULTI_TILE

OK = 0
ERR_INVALID = -1
ERR_WORKSPACE = -2
ERR_LIST = -3
ERR_HIP = -4

DEV_BAD_LENGTH = 1
DEV_BAD_PAGE = 2
DEV_BAD_ITEM = 4
DEV_BAD_POSITION = 8

PLAN_BALANCED = 0
PLAN_FIXED = 1
PLAN_SLACK = 2      # a plan may hold num_reqs + PLAN_SLACK * workers splits

EXPORTS = (
    "amla_fold_plan", "amla_bmm_scales", "amla_decode_config", "amla_reducer_bands",
    "amla_workspace_bytes", "amla_plan_splits", "amla_folded_decode", "amla_combine",
    "amla_combine_uv", "amla_folded_decode_dcp", "amla_merge_sources", "amla_build_query_cache",
    "amla_status_string", "amla_folded_decode_noalloc",
)
NOALLOC_SCRATCH_BYTES = 64 << 20
MAX_SOURCES = 64


class PlanParams(ctypes.Structure):
    _fields_ = [
        ("rows_per_req", ctypes.c_int32),
        ("mtile", ctypes.c_int32),
        ("workers", ctypes.c_int32),
        ("min_split_tokens", ctypes.c_int32),
        ("max_splits", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("split_cost_pages", ctypes.c_int32),
    ]

    def __repr__(self):
        return ("PlanParams(rows_per_req=%d, mtile=%d, workers=%d, min_split_tokens=%d, "
                "max_splits=%d, mode=%d, split_cost_pages=%d)"
                % (self.rows_per_req, self.mtile, self.workers, self.min_split_tokens,
                   self.max_splits, self.mode, self.split_cost_pages))


class DcpParams(ctypes.Structure):
    """amla_dcp_params: the KV shard of one decode-context-parallel rank."""
    _fields_ = [
        ("heads", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("world", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("interleave", ctypes.c_int32),
    ]


class AmlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} ({status})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """The HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python absorbed_mla_split_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, f32, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    i32p = ctypes.POINTER(ctypes.c_int32)
    f32p = ctypes.POINTER(ctypes.c_float)
    pp = ctypes.POINTER(PlanParams)
    sig = {
        "amla_fold_plan": (ctypes.c_int, [i32, i32, i32, i32, i32, i32, i32, i32, i32, i32p, i32p]),
        "amla_bmm_scales": (ctypes.c_int, [f32, f32, f32, f32p, f32p]),
        "amla_decode_config": (ctypes.c_int, [i32, i32, i32p, i32p]),
        "amla_reducer_bands": (ctypes.c_int, [i32, i32, i32p]),
        "amla_workspace_bytes": (sz, [i32, i32, i32]),
        "amla_plan_splits": (ctypes.c_int, [vp, i32, i32, pp, vp, vp, vp, i32, vp, sz, vp]),
        "amla_folded_decode": (ctypes.c_int, [vp, vp, i64, vp, i32, vp, i32, pp, f32, f32, vp,
                                              vp, vp, i32, vp, sz, vp]),
        "amla_combine": (ctypes.c_int, [vp, sz, vp, vp, i32, pp, i32, vp, vp, vp]),
        "amla_combine_uv": (ctypes.c_int, [vp, sz, vp, vp, i32, pp, i32, vp, vp, vp, vp, vp]),
        "amla_folded_decode_dcp": (ctypes.c_int, [vp, vp, i64, vp, i32, vp, i32, pp, f32, f32,
                                                  vp, vp, vp, i32, vp, sz,
                                                  ctypes.POINTER(DcpParams), vp, vp]),
        "amla_merge_sources": (ctypes.c_int, [i32, vp, vp, i64, vp, vp, vp]),
        "amla_build_query_cache": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32,
                                                  f32, f32, vp, vp, i64, vp, vp]),
        "amla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "amla_folded_decode_noalloc": (ctypes.c_int, [vp, vp, i64, vp, i32, vp, i32, pp, f32,
                                                      f32, i32, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().amla_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != OK:
        raise AmlaError(fn, status)


# ----------------------------------------------------------------------- host helpers

def fold_plan(causal, num_reqs, num_rows, num_decode_tokens, block_table_rows, max_query_len,
              heads, need_lse, max_fold_heads=MAX_ROWS):
    """(k, fold) of a decode batch: k = 0 when it does not fold."""
    k, f = ctypes.c_int32(), ctypes.c_int32()
    _check("amla_fold_plan", load().amla_fold_plan(int(bool(causal)), num_reqs, num_rows,
                                                   num_decode_tokens, block_table_rows,
                                                   max_query_len, heads, int(bool(need_lse)),
                                                   max_fold_heads, ctypes.byref(k), ctypes.byref(f)))
    return k.value, f.value


def bmm_scales(softmax_scale, q_scale, k_scale):
    b1, b2 = ctypes.c_float(), ctypes.c_float()
    _check("amla_bmm_scales", load().amla_bmm_scales(softmax_scale, q_scale, k_scale,
                                                     ctypes.byref(b1), ctypes.byref(b2)))
    return b1.value, b2.value


def decode_config(compute_units, rows_per_req):
    w, mt = ctypes.c_int32(), ctypes.c_int32()
    _check("amla_decode_config", load().amla_decode_config(compute_units, rows_per_req,
                                                           ctypes.byref(w), ctypes.byref(mt)))
    return w.value, mt.value


def reducer_bands(rows, compute_units):
    b = ctypes.c_int32()
    _check("amla_reducer_bands", load().amla_reducer_bands(rows, compute_units, ctypes.byref(b)))
    return b.value


def workspace_bytes(num_reqs, rows_per_req, workers):
    return int(load().amla_workspace_bytes(num_reqs, rows_per_req, workers))


def make_params(rows_per_req, mtile, workers, min_split_tokens=256, max_splits=MAX_SPLITS,
                mode=PLAN_BALANCED, split_cost_pages=None) -> PlanParams:
    if split_cost_pages is None:
        split_cost_pages = split_cost_default(mtile, rows_per_req)
    return PlanParams(rows_per_req, mtile, workers, min_split_tokens, max_splits, mode,
                      split_cost_pages)


# ----------------------------------------------------------------------- device calls

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def plan_splits(lengths, bt_cols, params: PlanParams, counts, offsets, work, workspace,
                stream=None):
    _check("amla_plan_splits", load().amla_plan_splits(
        _ptr(lengths), lengths.numel(), bt_cols, ctypes.byref(params), _ptr(counts),
        _ptr(offsets), _ptr(work), work.numel(), _ptr(workspace), workspace.numel(),
        _stream(stream)))


def folded_decode(q, kv, block_table, lengths, params: PlanParams, bmm1, bmm2, counts, offsets,
                  work, workspace, stream=None):
    _check("amla_folded_decode", load().amla_folded_decode(
        _ptr(q), _ptr(kv), kv.shape[0], _ptr(block_table), block_table.stride(0),
        _ptr(lengths), lengths.numel(), ctypes.byref(params), bmm1, bmm2, _ptr(counts),
        _ptr(offsets), _ptr(work), work.numel(), _ptr(workspace), workspace.numel(),
        _stream(stream)))


def combine(workspace, counts, offsets, num_reqs, params: PlanParams, compute_units, out, lse,
            stream=None):
    _check("amla_combine", load().amla_combine(
        _ptr(workspace), workspace.numel(), _ptr(counts), _ptr(offsets), num_reqs,
        ctypes.byref(params), compute_units, _ptr(out), _ptr(lse), _stream(stream)))


def folded_decode_dcp(q, kv, block_table, lengths, params: PlanParams, bmm1, bmm2, counts,
                      offsets, work, workspace, dcp: DcpParams, totals=None, stream=None):
    """Decode of one DCP rank's KV shard (``lengths``: local; ``totals``: global lengths,
    needed for the causal mask)."""
    _check("amla_folded_decode_dcp", load().amla_folded_decode_dcp(
        _ptr(q), _ptr(kv), kv.shape[0], _ptr(block_table), block_table.stride(0),
        _ptr(lengths), lengths.numel(), ctypes.byref(params), bmm1, bmm2, _ptr(counts),
        _ptr(offsets), _ptr(work), work.numel(), _ptr(workspace), workspace.numel(),
        ctypes.byref(dcp), _ptr(totals), _stream(stream)))


def folded_decode_noalloc(q, kv, block_table, lengths, params: PlanParams, bmm1, bmm2,
                          compute_units, out, lse, status=None, stream=None):
    """Plan, decode and merge in one call with the library's static device scratch (no
    workspace, nothing allocated): out [R, M, 512] BF16, lse [R, M]; ``status`` (one int32,
    optional) receives the device status word."""
    _check("amla_folded_decode_noalloc", load().amla_folded_decode_noalloc(
        _ptr(q), _ptr(kv), kv.shape[0], _ptr(block_table), block_table.stride(0),
        _ptr(lengths), lengths.numel(), ctypes.byref(params), bmm1, bmm2, compute_units,
        _ptr(out), _ptr(lse), _ptr(status), _stream(stream)))


def merge_sources(rows, lse, out, lse_out, stream=None):
    """Merge BF16 rows [S, n, 512] with log2 LSE [S, n] over the S sources into out
    [n, 512] BF16 and lse_out [n]."""
    n_src = rows.shape[0]
    n_rows = rows[0].numel() // VDIM if n_src else 0
    _check("amla_merge_sources", load().amla_merge_sources(
        n_src, _ptr(rows), _ptr(lse), n_rows, _ptr(out), _ptr(lse_out), _stream(stream)))


def build_query_cache(q, w_uk, kv_c, k_pe, positions, cos_sin, slot_mapping, neox, q_scale,
                      k_scale, q_out, kv_cache, status=None, stream=None):
    """The absorbed decode query q_out [n, H, 576] (E4M3) and the new tokens' cache rows,
    written into kv_cache [pages, 64, 576] at slot_mapping (see amla.h)."""
    n, H = q.shape[0], q.shape[1]
    _check("amla_build_query_cache", load().amla_build_query_cache(
        _ptr(q), _ptr(w_uk), _ptr(kv_c), _ptr(k_pe), _ptr(positions), _ptr(cos_sin),
        cos_sin.shape[0], _ptr(slot_mapping), n, H, int(bool(neox)), q_scale, k_scale,
        _ptr(q_out), _ptr(kv_cache), kv_cache.shape[0], _ptr(status), _stream(stream)))


def combine_uv(workspace, counts, offsets, num_reqs, params: PlanParams, heads, w_uv, attn_out,
               out=None, lse=None, stream=None):
    """Merge fused with the W_UV up-projection: attn_out [R*k, heads*128] BF16 from the
    split partials and W_UV (BF16 bits [heads][128][512], latent-contiguous); the merged
    BF16 latent ``out`` and LSE ``lse`` are written only when given."""
    _check("amla_combine_uv", load().amla_combine_uv(
        _ptr(workspace), workspace.numel(), _ptr(counts), _ptr(offsets), num_reqs,
        ctypes.byref(params), heads, _ptr(w_uv), _ptr(attn_out), _ptr(out), _ptr(lse),
        _stream(stream)))


# ------------------------------------------------------------------------ the decoder

class FoldedDecoder:
    """Plan buffers plus one split-KV workspace for up to ``max_reqs`` requests of
    ``rows_per_req`` folded rows, allocated once (before any graph capture).  ``plan`` runs
    once per decode step; ``decode`` once per layer (page "...cutedsl.mla.balanced",
    BalancedMla)."""

    def __init__(self, max_reqs, rows_per_req, device=None, mode=PLAN_BALANCED,
                 min_split_tokens=256, max_splits=MAX_SPLITS, workers=None, mtile=None,
                 split_cost_pages=None):
        import torch

        load()
        self.device = torch.device(device if device is not None else "cuda")
        props = torch.cuda.get_device_properties(self.device)
        self.compute_units = props.multi_processor_count
        w, mt = decode_config(self.compute_units, rows_per_req)
        self.params = make_params(rows_per_req, mtile or mt, workers or w, min_split_tokens,
                                  max_splits, mode, split_cost_pages)
        self.max_reqs = max_reqs
        i32 = dict(dtype=torch.int32, device=self.device)
        self.counts = torch.zeros(max(max_reqs, 1), **i32)
        self.offsets = torch.zeros(max_reqs + 1, **i32)
        self.work = torch.full((2 * (max_reqs + PLAN_SLACK * self.params.workers),), -1, **i32)
        nbytes = workspace_bytes(max_reqs, rows_per_req, self.params.workers)
        if nbytes == 0:
            raise ValueError("unsupported sizes")
        self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        self.num_reqs = 0

    def plan(self, lengths, bt_cols, stream=None):
        n = lengths.numel()
        if n > self.max_reqs:
            raise ValueError(f"{n} requests > {self.max_reqs}")
        self.num_reqs = n
        plan_splits(lengths, bt_cols, self.params, self.counts[:n], self.offsets[:n + 1],
                    self.work, self.workspace, stream)

    def decode(self, q, kv, block_table, lengths, bmm1, bmm2, out=None, lse=None, stream=None):
        import torch

        R, M = q.shape[0], q.shape[1]
        if R != self.num_reqs or M != self.params.rows_per_req:
            raise ValueError("decode shape does not match the plan")
        if q.dtype != torch.uint8 or kv.dtype != torch.uint8:
            raise TypeError("q and kv are float8_e4m3fn codes viewed as uint8")
        if out is None:
            out = torch.empty((R, M, VDIM), dtype=torch.bfloat16, device=q.device)
        if lse is None:
            lse = torch.empty((R, M), dtype=torch.float32, device=q.device)
        folded_decode(q, kv, block_table, lengths, self.params, bmm1, bmm2, self.counts[:R],
                      self.offsets[:R + 1], self.work, self.workspace, stream)
        combine(self.workspace, self.counts[:R], self.offsets[:R + 1], R, self.params,
                self.compute_units, out, lse, stream)
        return out, lse

    def decode_uv(self, q, kv, block_table, lengths, bmm1, bmm2, heads, w_uv, attn_out=None,
                  out=None, lse=None, stream=None):
        """Decode, then the merge fused with W_UV: returns attn_out [R*k, heads*128] BF16
        (``out``/``lse``, the merged latent and LSE, are filled only when given)."""
        import torch

        R, M = q.shape[0], q.shape[1]
        if R != self.num_reqs or M != self.params.rows_per_req or M % heads:
            raise ValueError("decode shape does not match the plan")
        if w_uv.dtype not in (torch.uint16, torch.int16, torch.bfloat16) or \
                tuple(w_uv.shape) != (heads, UVDIM, VDIM) or not w_uv.is_contiguous():
            raise TypeError("w_uv is BF16 [heads, 128, 512] (latent-contiguous), contiguous")
        if attn_out is None:
            attn_out = torch.empty((R * (M // heads), heads * UVDIM), dtype=torch.bfloat16,
                                   device=q.device)
        folded_decode(q, kv, block_table, lengths, self.params, bmm1, bmm2, self.counts[:R],
                      self.offsets[:R + 1], self.work, self.workspace, stream)
        combine_uv(self.workspace, self.counts[:R], self.offsets[:R + 1], R, self.params, heads,
                   w_uv, attn_out, out, lse, stream)
        return attn_out

    def device_status(self) -> int:
        """The workspace's device status word (synchronises; for checks, not hot loops)."""
        return int(self.workspace[:4].view(dtype=__import__("torch").int32).item())

    def plan_host(self):
        """(counts, offsets, work, items) of the current plan, copied to the host."""
        R = self.num_reqs
        counts = self.counts[:R].cpu().numpy()
        offsets = self.offsets[:R + 1].cpu().numpy()
        work = self.work.cpu().numpy()
        return counts, offsets, work, int(offsets[R]) if R >= 0 else 0
