"""Python binding of the gfx950 k8v4 attention library (``libq8k4v.so``).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  There is no CPU
fallback: importing works without the library, but every call raises if it is
not built or cannot be loaded.

Entry points (same names as the C ABI in ``include/q8k4v.h``):
``kv_quant_append``, ``attn_decode_q8k4v``, ``attn_verify_q8k4v``,
``tune_select``; plus ``workspace_bytes`` and ``PagedKVCache`` (allocates the
four cache pools as torch tensors).
"""

from __future__ import annotations

import ctypes as C
import json
import math
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libq8k4v.so")

Q8K4V_OK = 0
F32, BF16 = 0, 1
PAGE_SIZE = 16
MAX_DRAFT = 16

ERRORS = {-1: "EINVAL", -2: "EUNSUPPORTED", -3: "EWORKSPACE", -4: "EHIP", -5: "ENOMEM"}


class Q8K4VError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {ERRORS.get(code, code)} ({msg})")
        self.code = code


CODEC_SYMMETRIC, CODEC_AFFINE = 0, 1


class CacheDesc(C.Structure):
    _fields_ = [("num_pages", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("page_size", C.c_int32), ("k_codes", C.c_void_p), ("k_scales", C.c_void_p),
                ("v_codes", C.c_void_p), ("v_scales", C.c_void_p), ("codec", C.c_int32),
                ("k_zeros", C.c_void_p), ("v_zeros", C.c_void_p)]


class Config(C.Structure):
    _fields_ = [("wgs_per_cu", C.c_int32), ("split_pages", C.c_int32), ("tile_pages", C.c_int32),
                ("waves_per_wg", C.c_int32), ("fused_combine", C.c_int32), ("qualified", C.c_int32),
                ("variant", C.c_int32), ("stages", C.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class TuneRef(C.Structure):
    _fields_ = [("cache", C.POINTER(CacheDesc)), ("q", C.c_void_p), ("page_table", C.c_void_p),
                ("len", C.c_int32), ("max_pages", C.c_int32), ("out", C.c_void_p), ("sigma", C.c_void_p),
                ("seq_lens", C.c_void_p), ("n_seqs", C.c_int32), ("n_prefix_pages", C.c_int32)]


class TuneRequest(C.Structure):
    _fields_ = [("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("n_draft", C.c_int32), ("ctx_small", C.c_int32), ("ctx_large", C.c_int32),
                ("budget_ms", C.c_int64), ("mem_cap_bytes", C.c_size_t), ("seed", C.c_uint64),
                ("install", C.c_int32), ("max_candidates", C.c_int32), ("n_sessions", C.c_int32),
                ("ref", TuneRef * 6), ("ref_tol", C.c_float),
                ("softmax_scale", C.c_float), ("record_path", C.c_char_p)]


# the terms of the tuner's service cost, in the order of
# q8k4v_tune_request.ref (the last two with n_sessions >= 2 only)
TUNE_TERMS = ("decode_small", "decode_large", "verify_small", "verify_large",
              "multi_session_small", "multi_session_large")


_lib = None


def load_library(path: str = LIB_PATH) -> C.CDLL:
    """Load ``libq8k4v.so`` (raises if it is missing: build it with
    ``python -m decode_attention_quantized_kv_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run python -m decode_attention_quantized_kv_amd.build)")
    # torch first: its bundled HIP runtime then satisfies the library's
    # libamdhip64.so.7 dependency, so the process holds one HIP runtime (the
    # other order loads the system runtime as well and the two do not share
    # devices or memory)
    import torch  # noqa: F401
    lib = C.CDLL(path)
    i32, vp, sz = C.c_int32, C.c_void_p, C.c_size_t
    lib.q8k4v_last_error.restype = C.c_char_p
    lib.q8k4v_version.restype = C.c_char_p
    lib.kv_quant_append.restype = i32
    lib.kv_quant_append.argtypes = [C.POINTER(CacheDesc), vp, vp, i32, vp, vp, vp, i32, i32, i32, vp]
    lib.q8k4v_workspace_bytes.restype = sz
    lib.q8k4v_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, C.POINTER(Config)]
    lib.attn_decode_q8k4v.restype = i32
    lib.attn_decode_q8k4v.argtypes = [C.POINTER(CacheDesc), vp, i32, vp, i32, i32, vp, i32, vp, i32,
                                      C.c_float, C.POINTER(Config), vp, sz, vp]
    lib.attn_decode_prefix_q8k4v.restype = i32
    lib.attn_decode_prefix_q8k4v.argtypes = [C.POINTER(CacheDesc), vp, i32, vp, i32, i32, vp, i32, vp, i32, i32,
                                             C.c_float, C.POINTER(Config), vp, sz, vp]
    lib.q8k4v_prefix_workspace_bytes.restype = sz
    lib.q8k4v_prefix_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, C.POINTER(Config)]
    lib.attn_decode_append_q8k4v.restype = i32
    lib.attn_decode_append_q8k4v.argtypes = [C.POINTER(CacheDesc), vp, vp, i32, vp, i32, vp, i32, i32, vp, i32, vp,
                                             i32, C.c_float, C.POINTER(Config), vp, sz, vp]
    lib.attn_prefill_q8k4v.restype = i32
    lib.attn_prefill_q8k4v.argtypes = [C.POINTER(CacheDesc), vp, i32, vp, i32, i32, i32, vp, i32, vp, i32,
                                       C.c_float, C.POINTER(Config), vp, sz, vp]
    lib.attn_verify_q8k4v.restype = i32
    lib.attn_verify_q8k4v.argtypes = [C.POINTER(CacheDesc), vp, i32, vp, i32, i32, i32, vp, i32, vp, i32,
                                      C.c_float, C.POINTER(Config), vp, sz, vp]
    lib.tune_select.restype = i32
    lib.tune_select.argtypes = [C.POINTER(TuneRequest), C.POINTER(Config), C.c_char_p, sz]
    lib.attn_decode_q8k4v_noalloc.restype = i32
    lib.attn_decode_q8k4v_noalloc.argtypes = [C.POINTER(CacheDesc), vp, i32, vp, i32, i32, vp, i32, vp, i32,
                                              C.c_float, C.POINTER(Config), vp]
    lib.q8k4v_hbm_probe.restype = i32
    lib.q8k4v_hbm_probe.argtypes = [C.POINTER(CacheDesc), i32, vp, i32, vp, i32, i32, i32, i32, vp]
    lib.q8k4v_stream_probe.restype = i32
    lib.q8k4v_stream_probe.argtypes = [vp, sz, i32, i32, vp]
    _lib = lib
    return lib


def version() -> str:
    return load_library().q8k4v_version().decode()


def _check(fn: str, rc: int):
    if rc != Q8K4V_OK:
        raise Q8K4VError(fn, rc, load_library().q8k4v_last_error().decode())


def _torch():
    import torch
    return torch


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _ptr(t, name: str = "tensor", i32: bool = False) -> C.c_void_p:
    """Device pointer of a tensor argument: the library reads it as a dense
    array on the current device, so it must be a contiguous device tensor
    (int32 for lengths, positions and page tables)."""
    if t is None:
        return C.c_void_p(0)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if i32 and t.dtype != _torch().int32:
        raise TypeError(f"{name} must be int32, got {t.dtype}")
    return C.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def make_config(**kw) -> Config:
    c = Config()
    for k, v in kw.items():
        setattr(c, k, int(v))
    return c


class PagedKVCache:
    """The device pools of a paged k8v4 cache (torch tensors), in the
    library's layout:

    ``k_codes [P][H][16][D] int8``, ``k_scales [P][H][16]`` fp16 bits,
    ``v_codes [P][H][D][8] uint8``, ``v_scales [P][H][16][D/32]`` fp16 bits;
    with ``codec="affine"`` also ``k_zeros [P][H][16] int8`` and
    ``v_zeros [P][H][16][D/32] uint8``."""

    def __init__(self, num_pages: int, num_kv_heads: int, head_dim: int, device="cuda", codec: str = "symmetric"):
        torch = _torch()
        if codec not in ("symmetric", "affine"):
            raise ValueError("codec must be 'symmetric' or 'affine'")
        P, H, D = num_pages, num_kv_heads, head_dim
        self.num_pages, self.num_kv_heads, self.head_dim = P, H, D
        self.codec = codec
        self.k_codes = torch.zeros((P, H, PAGE_SIZE, D), dtype=torch.int8, device=device)
        self.k_scales = torch.zeros((P, H, PAGE_SIZE), dtype=torch.int16, device=device)
        self.v_codes = torch.zeros((P, H, D, PAGE_SIZE // 2), dtype=torch.uint8, device=device)
        self.v_scales = torch.zeros((P, H, PAGE_SIZE, D // 32), dtype=torch.int16, device=device)
        self.k_zeros = self.v_zeros = None
        if codec == "affine":
            self.k_zeros = torch.zeros((P, H, PAGE_SIZE), dtype=torch.int8, device=device)
            self.v_zeros = torch.zeros((P, H, PAGE_SIZE, D // 32), dtype=torch.uint8, device=device)
        self._desc = None

    def pools(self):
        extra = (self.k_zeros, self.v_zeros) if self.codec == "affine" else ()
        return (self.k_codes, self.k_scales, self.v_codes, self.v_scales) + extra

    @property
    def desc(self) -> CacheDesc:
        if self._desc is None:
            aff = self.codec == "affine"
            self._desc = CacheDesc(self.num_pages, self.num_kv_heads, self.head_dim, PAGE_SIZE,
                                   self.k_codes.data_ptr(), self.k_scales.data_ptr(),
                                   self.v_codes.data_ptr(), self.v_scales.data_ptr(),
                                   CODEC_AFFINE if aff else CODEC_SYMMETRIC,
                                   self.k_zeros.data_ptr() if aff else None,
                                   self.v_zeros.data_ptr() if aff else None)
        return self._desc

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.pools())


def kv_quant_append(cache: PagedKVCache, k_new, v_new, cu_new, start_pos, page_table,
                    total_new: Optional[int] = None, stream=None) -> None:
    """``k_new``/``v_new``: ``[N][H][D]`` float32 or bfloat16 (device);
    ``cu_new [B+1]``, ``start_pos [B]``, ``page_table [B][max_pages]`` int32
    (device)."""
    lib = load_library()
    if total_new is None:
        total_new = int(k_new.shape[0])
    n_seqs = int(start_pos.shape[0])
    rc = lib.kv_quant_append(C.byref(cache.desc), _ptr(k_new, "k_new"), _ptr(v_new, "v_new"), _dtype_code(k_new), _ptr(cu_new, "cu_new", i32=True),
                             _ptr(start_pos, "start_pos", i32=True), _ptr(page_table, "page_table", i32=True), int(page_table.shape[1]), n_seqs,
                             int(total_new), _stream(stream))
    _check("kv_quant_append", rc)


def workspace_bytes(n_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int, max_seq_len: int,
                    n_draft: int = 0, cfg: Optional[Config] = None) -> int:
    lib = load_library()
    return int(lib.q8k4v_workspace_bytes(n_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, n_draft,
                                         C.byref(cfg) if cfg is not None else None))


def _workspace(nbytes: int, device):
    torch = _torch()
    return torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)


def attn_decode_q8k4v(cache: PagedKVCache, q, seq_lens, max_seq_len: int, page_table,
                      softmax_scale: Optional[float] = None, out=None, cfg: Optional[Config] = None,
                      workspace=None, stream=None):
    """``q [B][Hq][D]`` (float32/bfloat16, device) -> ``out [B][Hq][D]`` float32."""
    torch = _torch()
    lib = load_library()
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = _workspace(workspace_bytes(B, Hq, cache.num_kv_heads, D, max_seq_len, 0, cfg), q.device)
    rc = lib.attn_decode_q8k4v(C.byref(cache.desc), _ptr(q, "q"), _dtype_code(q), _ptr(out, "out"), B, Hq, _ptr(seq_lens, "seq_lens", i32=True),
                               int(max_seq_len), _ptr(page_table, "page_table", i32=True), int(page_table.shape[1]),
                               float(softmax_scale), C.byref(cfg) if cfg is not None else None,
                               _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("attn_decode_q8k4v", rc)
    return out


def attn_decode_q8k4v_noalloc(cache: PagedKVCache, q, seq_lens, max_seq_len: int, page_table,
                              softmax_scale: Optional[float] = None, out=None, cfg: Optional[Config] = None,
                              stream=None):
    """:func:`attn_decode_q8k4v` without a workspace argument: the library's
    static per-GPU scratch array holds the split records (the call
    allocates no device memory; ``out`` should be passed to keep it so)."""
    torch = _torch()
    lib = load_library()
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    rc = lib.attn_decode_q8k4v_noalloc(C.byref(cache.desc), _ptr(q, "q"), _dtype_code(q), _ptr(out, "out"), B, Hq,
                                       _ptr(seq_lens, "seq_lens", i32=True), int(max_seq_len),
                                       _ptr(page_table, "page_table", i32=True), int(page_table.shape[1]),
                                       float(softmax_scale), C.byref(cfg) if cfg is not None else None,
                                       _stream(stream))
    _check("attn_decode_q8k4v_noalloc", rc)
    return out


def prefix_workspace_bytes(n_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int, max_seq_len: int,
                           n_prefix_pages: int, cfg: Optional[Config] = None) -> int:
    lib = load_library()
    return int(lib.q8k4v_prefix_workspace_bytes(n_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                                n_prefix_pages, C.byref(cfg) if cfg is not None else None))


def attn_decode_prefix_q8k4v(cache: PagedKVCache, q, seq_lens, max_seq_len: int, page_table, n_prefix_pages: int,
                             softmax_scale: Optional[float] = None, out=None, cfg: Optional[Config] = None,
                             workspace=None, stream=None):
    """Decode of sessions sharing their first ``n_prefix_pages`` pages (same
    physical ids in every row of ``page_table``): ``q [B][Hq][D]`` ->
    ``out [B][Hq][D]`` float32, as :func:`attn_decode_q8k4v`."""
    torch = _torch()
    lib = load_library()
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = _workspace(prefix_workspace_bytes(B, Hq, cache.num_kv_heads, D, max_seq_len,
                                                      n_prefix_pages, cfg), q.device)
    rc = lib.attn_decode_prefix_q8k4v(C.byref(cache.desc), _ptr(q, "q"), _dtype_code(q), _ptr(out, "out"), B, Hq,
                                      _ptr(seq_lens, "seq_lens", i32=True), int(max_seq_len), _ptr(page_table, "page_table", i32=True), int(page_table.shape[1]),
                                      int(n_prefix_pages), float(softmax_scale),
                                      C.byref(cfg) if cfg is not None else None,
                                      _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("attn_decode_prefix_q8k4v", rc)
    return out


def attn_decode_append_q8k4v(cache: PagedKVCache, k_new, v_new, q, seq_lens, max_seq_len: int, page_table,
                             softmax_scale: Optional[float] = None, out=None, cfg: Optional[Config] = None,
                             workspace=None, stream=None):
    """One decode step: appends ``k_new``/``v_new`` ``[B][H][D]`` (each
    sequence's new token, at position ``seq_lens[b] - 1``) and returns the
    decode of ``q [B][Hq][D]`` over the cache including it."""
    torch = _torch()
    lib = load_library()
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = _workspace(workspace_bytes(B, Hq, cache.num_kv_heads, D, max_seq_len, 0, cfg), q.device)
    rc = lib.attn_decode_append_q8k4v(C.byref(cache.desc), _ptr(k_new, "k_new"), _ptr(v_new, "v_new"), _dtype_code(k_new), _ptr(q, "q"),
                                      _dtype_code(q), _ptr(out, "out"), B, Hq, _ptr(seq_lens, "seq_lens", i32=True), int(max_seq_len),
                                      _ptr(page_table, "page_table", i32=True), int(page_table.shape[1]), float(softmax_scale),
                                      C.byref(cfg) if cfg is not None else None, _ptr(workspace, "workspace"),
                                      workspace.numel() * workspace.element_size(), _stream(stream))
    _check("attn_decode_append_q8k4v", rc)
    return out


def attn_prefill_q8k4v(cache: PagedKVCache, q, seq_lens, max_seq_len: int, page_table,
                       softmax_scale: Optional[float] = None, out=None, cfg: Optional[Config] = None,
                       workspace=None, stream=None):
    """Chunked prefill: ``q [B][n_new][Hq][D]`` -> ``out [B][n_new][Hq][D]``
    float32; new token j of sequence b sees positions
    ``0 .. seq_lens[b] - n_new + j`` (the new tokens are already appended)."""
    torch = _torch()
    lib = load_library()
    B, Wn, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Wn, Hq, D), dtype=torch.float32, device=q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = _workspace(workspace_bytes(B, Hq, cache.num_kv_heads, D, max_seq_len, Wn, cfg), q.device)
    rc = lib.attn_prefill_q8k4v(C.byref(cache.desc), _ptr(q, "q"), _dtype_code(q), _ptr(out, "out"), B, Hq, Wn,
                                _ptr(seq_lens, "seq_lens", i32=True), int(max_seq_len), _ptr(page_table, "page_table", i32=True), int(page_table.shape[1]),
                                float(softmax_scale), C.byref(cfg) if cfg is not None else None,
                                _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("attn_prefill_q8k4v", rc)
    return out


def attn_verify_q8k4v(cache: PagedKVCache, q, seq_lens, max_seq_len: int, page_table,
                      softmax_scale: Optional[float] = None, out=None, cfg: Optional[Config] = None,
                      workspace=None, stream=None):
    """``q [B][W][Hq][D]`` -> ``out [B][W][Hq][D]`` float32; draft j of
    sequence b sees positions ``0 .. seq_lens[b] - W + j``."""
    torch = _torch()
    lib = load_library()
    B, Wd, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Wd, Hq, D), dtype=torch.float32, device=q.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = _workspace(workspace_bytes(B, Hq, cache.num_kv_heads, D, max_seq_len, Wd, cfg), q.device)
    rc = lib.attn_verify_q8k4v(C.byref(cache.desc), _ptr(q, "q"), _dtype_code(q), _ptr(out, "out"), B, Hq, Wd,
                               _ptr(seq_lens, "seq_lens", i32=True), int(max_seq_len), _ptr(page_table, "page_table", i32=True), int(page_table.shape[1]),
                               float(softmax_scale), C.byref(cfg) if cfg is not None else None,
                               _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("attn_verify_q8k4v", rc)
    return out


def tune_select(num_q_heads: int, num_kv_heads: int, head_dim: int, n_draft: int = 8,
                ctx_small: int = 4096, ctx_large: int = 65536, budget_ms: int = 60000,
                mem_cap_bytes: int = 0, seed: int = 0, install: bool = False, max_candidates: int = 0,
                refs=None, ref_tol: float = 0.0, report_cap: int = 1 << 20,
                record_path: Optional[str] = None, n_sessions: int = 0):
    """Runs the on-device tuner.  ``n_sessions`` >= 2 adds the multi-session
    unit (the shared-prefix entry point's suffix pass over that many
    sessions).  ``refs`` (optional): a dict keyed by :data:`TUNE_TERMS`, each a
    dict with ``cache`` (PagedKVCache), ``q`` (device bf16 ``[n][Hq][D]``),
    ``page_table`` (device int32: one sequence's pages, or ``[n_seqs][max_pages]``
    for the multi-session terms), ``length`` (tokens attended; the longest
    session for the multi-session terms), ``out`` (host float32
    ``[n][Hq][D]``, the expected output) and optionally ``sigma`` (host
    ``[Hq][D]``, which normalises the deviation); the multi-session terms also
    take ``seq_lens`` (device int32 ``[n_seqs]``) and ``n_prefix_pages``.
    ``ref_tol`` bounds the normalised deviation.  ``record_path`` (optional):
    file of stored choices, reused for the same device identity and request
    shape.  Returns (decode Config, verify Config, multi-session Config or
    None, report dict)."""
    import numpy as np
    lib = load_library()
    req = TuneRequest()
    req.num_q_heads, req.num_kv_heads, req.head_dim, req.n_draft = num_q_heads, num_kv_heads, head_dim, n_draft
    req.ctx_small, req.ctx_large, req.budget_ms = ctx_small, ctx_large, budget_ms
    req.mem_cap_bytes, req.seed, req.install, req.max_candidates = mem_cap_bytes, seed, int(install), max_candidates
    req.n_sessions = int(n_sessions)
    keep = []
    for k, term in enumerate(TUNE_TERMS):
        r = (refs or {}).get(term)
        if r is None:
            continue
        out = np.ascontiguousarray(r["out"], dtype=np.float32)
        keep.append(out)
        pt = r["page_table"]
        req.ref[k].cache = C.pointer(r["cache"].desc)
        req.ref[k].q = _ptr(r["q"], "q").value
        req.ref[k].page_table = _ptr(pt, "page_table", i32=True).value
        req.ref[k].len = int(r["length"])
        req.ref[k].max_pages = int(pt.shape[-1])
        req.ref[k].out = out.ctypes.data
        if r.get("sigma") is not None:
            sig = np.ascontiguousarray(r["sigma"], dtype=np.float32)
            keep.append(sig)
            req.ref[k].sigma = sig.ctypes.data
        if k >= 4:
            req.ref[k].seq_lens = _ptr(r["seq_lens"], "seq_lens", i32=True).value
            req.ref[k].n_seqs = int(r["seq_lens"].shape[0])
            req.ref[k].n_prefix_pages = int(r["n_prefix_pages"])
    req.ref_tol = float(ref_tol)
    if record_path is not None:
        req.record_path = os.fsencode(record_path)
    table = (Config * 3)()
    buf = C.create_string_buffer(report_cap)
    rc = lib.tune_select(C.byref(req), table, buf, report_cap)
    _check("tune_select", rc)
    text = buf.value.decode()
    try:
        report = json.loads(text) if text else {}
    except json.JSONDecodeError:
        report = {"raw": text}
    return table[0], table[1], (table[2] if n_sessions >= 2 else None), report


def hbm_probe(cache: PagedKVCache, seq_lens, max_seq_len: int, page_table, waves_per_wg: int = 4,
              stages: int = 3, heads_per_wg: int = 1, stream=None) -> None:
    """Streams the page-head blocks a decode launch over ``cache`` reads
    (same split and mapping, HBM -> LDS, no compute): the memory system's
    rate for that access pattern.  ``heads_per_wg`` > 1 streams that many
    kv heads of each page per workgroup."""
    lib = load_library()
    rc = lib.q8k4v_hbm_probe(C.byref(cache.desc), int(seq_lens.shape[0]), _ptr(seq_lens, "seq_lens", i32=True),
                             int(max_seq_len), _ptr(page_table, "page_table", i32=True), int(page_table.shape[1]),
                             int(waves_per_wg), int(stages), int(heads_per_wg), _stream(stream))
    _check("q8k4v_hbm_probe", rc)


def stream_probe(buf, waves_per_wg: int = 4, stages: int = 3, stream=None) -> None:
    """Streams the bytes of the contiguous device tensor ``buf`` into LDS
    (the sequential reference rate)."""
    lib = load_library()
    rc = lib.q8k4v_stream_probe(_ptr(buf, "buf"), buf.numel() * buf.element_size(), int(waves_per_wg), int(stages),
                                _stream(stream))
    _check("q8k4v_stream_probe", rc)


__all__ = ["kv_quant_append", "attn_decode_q8k4v", "attn_decode_prefix_q8k4v", "attn_verify_q8k4v",
           "attn_prefill_q8k4v", "attn_decode_append_q8k4v", "attn_decode_q8k4v_noalloc", "tune_select",
           "hbm_probe", "stream_probe",
           "TUNE_TERMS",
           "workspace_bytes", "prefix_workspace_bytes",
           "PagedKVCache", "Config", "make_config", "load_library", "version", "Q8K4VError", "LIB_PATH"]
