"""Thin ctypes binding of libdsa.so (see include/dsa.h for the contract of each call).

Argument marshalling only: tensors are checked for device, dtype and layout and
their device pointers handed to the C entry points with torch's current HIP
stream. Outputs and the workspace are allocated with torch when the caller does
not pass them. Every computation runs in the library's HIP kernels; when the
library is missing, every call raises.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdsa.so")
_lib = None

FLAG_FORCE_FALLBACK = 1
FLAG_TABLE_IN_MEMORY = 2  # dsa_decode_step_paged only (testing)
DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
STATUS_NAMES = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED",
                3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_HIP"}
EXPORTED = ("dsa_status_string", "dsa_workspace_size", "dsa_index_scores", "dsa_topk_select",
            "dsa_sparse_attn", "dsa_decode_step", "dsa_decode_step_timed", "dsa_decode_step_noalloc",
            "dsa_read_stats", "dsa_index_scores_paged", "dsa_sparse_attn_paged", "dsa_decode_step_paged")
PAGE_SIZE = 256  # positions per page of a paged pool (DSA_PAGE_SIZE)


class DSAError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__("%s: %s" % (what, dsa_status_string(code)))


class RowStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("path", "reason", "selected", "kth_score",
                                              "candidates", "tied_at_kth", "bad_indices",
                                              "reserved")]


def library_path():
    return _LIB_PATH


def build():
    from .buildlib import build as _build
    return _build()


def load_library():
    """Load libdsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise DSAError(4, "libdsa.so is missing at %s; build it with "
                              "__graft_entry__.build()" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        p, i32, i64, u32, sz, f32 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint,
                                     ctypes.c_size_t, ctypes.c_float)
        lib.dsa_status_string.argtypes = [i32]
        lib.dsa_status_string.restype = ctypes.c_char_p
        lib.dsa_workspace_size.argtypes = [i32, i64, i32, i32, i32]
        lib.dsa_workspace_size.restype = sz
        lib.dsa_index_scores.argtypes = [p, p, p, p, i32, i32, i32, i64, p, p]
        lib.dsa_topk_select.argtypes = [p, p, i32, i64, i32, p, p, sz, u32, p]
        lib.dsa_sparse_attn.argtypes = [p, p, p, i32, i32, i32, i32, i64, i32, f32, i32, p, p, sz, p]
        lib.dsa_decode_step.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64, i32,
                                        f32, i32, p, p, p, p, sz, u32, p]
        lib.dsa_decode_step_timed.argtypes = lib.dsa_decode_step.argtypes + [p]
        lib.dsa_decode_step_noalloc.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64, i32,
                                                f32, i32, p, p, p, u32, p]
        lib.dsa_read_stats.argtypes = [p, sz, i32, p, p]
        lib.dsa_index_scores_paged.argtypes = [p, p, p, p, i64, p, i32, i32, i32, i64, p, p]
        lib.dsa_sparse_attn_paged.argtypes = [p, p, p, i64, p, i32, i32, i32, i32, i64, i32, f32, i32, p, p,
                                              sz, p]
        lib.dsa_decode_step_paged.argtypes = [p, p, p, p, p, p, i64, p, i32, i32, i32, i32, i32, i32, i64,
                                              i32, f32, i32, p, p, p, p, sz, u32, p, p]
        for name in EXPORTED[2:]:
            getattr(lib, name).restype = i32
        _lib = lib
    return _lib


def dsa_status_string(code):
    if _lib is None and not os.path.exists(_LIB_PATH):
        return STATUS_NAMES.get(int(code), "unknown")
    return load_library().dsa_status_string(int(code)).decode()


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a tensor on the GPU" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _host_lens(ctx_len, B):
    a = np.ascontiguousarray(np.asarray(ctx_len.cpu() if hasattr(ctx_len, "cpu") else ctx_len,
                                        dtype=np.int32).reshape(-1))
    if a.shape[0] != B:
        raise ValueError("ctx_len must hold B=%d values" % B)
    return a


def _check(rc, what):
    if rc != 0:
        raise DSAError(rc, what)


def _attn_dtype(q, kv):
    """float32 q and kv, bfloat16 q and kv, or bfloat16 q with a float8_e4m3fn kv."""
    torch = _torch()
    if q.dtype == torch.float32 and kv.dtype == torch.float32:
        return DSA_F32
    if q.dtype == torch.bfloat16 and kv.dtype == torch.bfloat16:
        return DSA_BF16
    if q.dtype == torch.bfloat16 and kv.dtype == torch.float8_e4m3fn:
        return DSA_FP8_E4M3
    raise TypeError("q and kv: both float32, both bfloat16, or bfloat16 q with float8_e4m3fn kv; got %s "
                    "and %s" % (q.dtype, kv.dtype))


def dsa_workspace_size(B, N, k, Hq=1, Dv=1):
    return int(load_library().dsa_workspace_size(B, N, k, Hq, Dv))


def new_workspace(B, N, k, Hq=1, Dv=1, device=None):
    """A workspace tensor of dsa_workspace_size() bytes (uint8, 256-byte aligned by torch)."""
    torch = _torch()
    n = dsa_workspace_size(B, N, k, Hq, Dv)
    if n == 0:
        raise DSAError(1, "dsa_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def dsa_index_scores(iq, iw, ik, ctx_len, scores=None, stream=None):
    """iq [B,Hi,Di], iw [B,Hi], ik [N,Di] int8 on the GPU -> scores [B,N] int32."""
    torch = _torch()
    lib = load_library()
    B, Hi, Di = iq.shape
    N = ik.shape[0]
    lens = _host_lens(ctx_len, B)
    if scores is None:
        scores = torch.zeros((B, N), dtype=torch.int32, device=ik.device)
    rc = lib.dsa_index_scores(_dev(iq, "iq", torch.int8), _dev(iw, "iw", torch.int8),
                              _dev(ik, "ik", torch.int8), lens.ctypes.data_as(ctypes.c_void_p),
                              B, Hi, Di, N, _dev(scores, "scores", torch.int32), _stream(stream))
    _check(rc, "dsa_index_scores")
    return scores


def dsa_topk_select(scores, ctx_len, k, idx=None, workspace=None, flags=0, stream=None):
    """scores [B,N] int32 -> idx [B,k] int32 (score desc, position asc; -1 padding)."""
    torch = _torch()
    lib = load_library()
    B, N = scores.shape
    lens = _host_lens(ctx_len, B)
    if idx is None:
        idx = torch.empty((B, k), dtype=torch.int32, device=scores.device)
    if workspace is None:
        workspace = new_workspace(B, N, k, 1, 1, scores.device)
    rc = lib.dsa_topk_select(_dev(scores, "scores", torch.int32), lens.ctypes.data_as(ctypes.c_void_p),
                             B, N, k, _dev(idx, "idx", torch.int32), _dev(workspace, "workspace"),
                             workspace.numel() * workspace.element_size(), flags, _stream(stream))
    _check(rc, "dsa_topk_select")
    return idx


def dsa_sparse_attn(q, kv, idx, Dv, scale, out=None, workspace=None, stream=None):
    """q [B,Hq,Dk], kv [N,Dk] (float32 or bfloat16), idx [B,k] int32 -> out [B,Hq,Dv] float32."""
    torch = _torch()
    lib = load_library()
    B, Hq, Dk = q.shape
    N = kv.shape[0]
    k = idx.shape[1]
    dt = _attn_dtype(q, kv)
    if out is None:
        out = torch.empty((B, Hq, Dv), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = new_workspace(B, N, k, Hq, Dv, q.device)
    rc = lib.dsa_sparse_attn(_dev(q, "q"), _dev(kv, "kv"), _dev(idx, "idx", torch.int32), B, Hq, Dk,
                             Dv, N, k, float(scale), dt, _dev(out, "out", torch.float32),
                             _dev(workspace, "workspace"),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "dsa_sparse_attn")
    return out


def _decode_step_args(iq, iw, ik, q, kv, ctx_len, k, Dv, scale, scores, idx, out, workspace, flags, stream):
    torch = _torch()
    B, Hi, Di = iq.shape
    _, Hq, Dk = q.shape
    N = ik.shape[0]
    if kv.shape[0] != N:
        raise ValueError("ik and kv must cover the same N positions")
    lens = _host_lens(ctx_len, B)
    dt = _attn_dtype(q, kv)
    dev = ik.device
    if scores is None:
        scores = torch.zeros((B, N), dtype=torch.int32, device=dev)
    if idx is None:
        idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((B, Hq, Dv), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = new_workspace(B, N, k, Hq, Dv, dev)
    args = [_dev(iq, "iq", torch.int8), _dev(iw, "iw", torch.int8), _dev(ik, "ik", torch.int8),
            _dev(q, "q"), _dev(kv, "kv"), lens.ctypes.data_as(ctypes.c_void_p), B, Hi, Di, Hq, Dk,
            Dv, N, k, float(scale), dt, _dev(scores, "scores", torch.int32),
            _dev(idx, "idx", torch.int32), _dev(out, "out", torch.float32),
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), flags,
            _stream(stream)]
    return args, lens, scores, idx, out


def dsa_decode_step(iq, iw, ik, q, kv, ctx_len, k, Dv, scale, scores=None, idx=None, out=None,
                    workspace=None, flags=0, stream=None, kernel_events=None):
    """The three stages through one layer; returns (scores, idx, out).

    kernel_events: optional sequence of 6 torch.cuda.Event(enable_timing=True), each
    already recorded once (torch creates the HIP event lazily). Events 2i, 2i+1 take
    the start and end of stage i's kernel (dsa_decode_step_timed)."""
    lib = load_library()
    args, lens, scores, idx, out = _decode_step_args(iq, iw, ik, q, kv, ctx_len, k, Dv, scale, scores, idx,
                                                     out, workspace, flags, stream)
    if kernel_events is None:
        rc = lib.dsa_decode_step(*args)
    else:
        if len(kernel_events) != 6:
            raise ValueError("kernel_events must hold 6 events")
        evs = (ctypes.c_void_p * 6)(*[e.cuda_event for e in kernel_events])
        rc = lib.dsa_decode_step_timed(*args, ctypes.cast(evs, ctypes.c_void_p))
    _check(rc, "dsa_decode_step")
    return scores, idx, out


def prepared_decode_step(iq, iw, ik, q, kv, ctx_len, k, Dv, scale, scores, idx, out, workspace, flags=0,
                         stream=None):
    """dsa_decode_step with its arguments marshalled once: returns a function of no
    arguments that makes the C call again (and raises on a nonzero status). For
    measuring the host's cost of issuing a step; the tensors must stay alive."""
    lib = load_library()
    args, lens, scores, idx, out = _decode_step_args(iq, iw, ik, q, kv, ctx_len, k, Dv, scale, scores, idx,
                                                     out, workspace, flags, stream)
    fn = lib.dsa_decode_step

    def call():
        rc = fn(*args)
        if rc != 0:
            raise DSAError(rc, "dsa_decode_step")
    call.keep = (lens, args)
    return call


def dsa_decode_step_noalloc(iq, iw, ik, q, kv, ctx_len, k, Dv, scale, scores, idx, out, flags=0,
                            stream=None):
    """dsa_decode_step on the library's static per-device scratch (no workspace argument);
    the outputs must be given. Returns (scores, idx, out)."""
    torch = _torch()
    lib = load_library()
    B, Hi, Di = iq.shape
    _, Hq, Dk = q.shape
    N = ik.shape[0]
    if kv.shape[0] != N:
        raise ValueError("ik and kv must cover the same N positions")
    lens = _host_lens(ctx_len, B)
    dt = _attn_dtype(q, kv)
    rc = lib.dsa_decode_step_noalloc(_dev(iq, "iq", torch.int8), _dev(iw, "iw", torch.int8),
                                     _dev(ik, "ik", torch.int8), _dev(q, "q"), _dev(kv, "kv"),
                                     lens.ctypes.data_as(ctypes.c_void_p), B, Hi, Di, Hq, Dk, Dv, N, k,
                                     float(scale), dt, _dev(scores, "scores", torch.int32),
                                     _dev(idx, "idx", torch.int32), _dev(out, "out", torch.float32), flags,
                                     _stream(stream))
    _check(rc, "dsa_decode_step_noalloc")
    return scores, idx, out


def dsa_read_stats(workspace, B, stream=None):
    """Per-row stats of the last selection that used `workspace` (synchronises the stream)."""
    lib = load_library()
    arr = (RowStats * B)()
    rc = lib.dsa_read_stats(_dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                            B, ctypes.cast(arr, ctypes.c_void_p), _stream(stream))
    _check(rc, "dsa_read_stats")
    return [{f: getattr(r, f) for f, _ in RowStats._fields_} for r in arr]


def _paging(page_table, pools, N):
    """Checks a page table (int32 on the GPU) against the pools ([pool_pages * 256, ...] each)
    and the logical length N (default: every page of the table); returns (N, pool_pages)."""
    torch = _torch()
    _dev(page_table, "page_table", torch.int32)
    rows = pools[0].shape[0]
    if rows % PAGE_SIZE != 0 or any(p.shape[0] != rows for p in pools):
        raise ValueError("the pools must hold the same whole number of %d-row pages" % PAGE_SIZE)
    n_tab = page_table.numel()
    N = n_tab * PAGE_SIZE if N is None else int(N)
    if N < 1 or (N + PAGE_SIZE - 1) // PAGE_SIZE > n_tab:
        raise ValueError("page_table must hold ceil(N / %d) entries" % PAGE_SIZE)
    return N, rows // PAGE_SIZE


def dsa_index_scores_paged(iq, iw, ik_pool, page_table, ctx_len, N=None, scores=None, stream=None):
    """dsa_index_scores over an indexer key pool [pool_pages * 256, Di] read through
    page_table [ceil(N / 256)] int32 (pool page of each logical page) -> scores [B,N] int32."""
    torch = _torch()
    lib = load_library()
    B, Hi, Di = iq.shape
    N, pool_pages = _paging(page_table, (ik_pool,), N)
    lens = _host_lens(ctx_len, B)
    if scores is None:
        scores = torch.zeros((B, N), dtype=torch.int32, device=ik_pool.device)
    rc = lib.dsa_index_scores_paged(_dev(iq, "iq", torch.int8), _dev(iw, "iw", torch.int8),
                                    _dev(ik_pool, "ik_pool", torch.int8), _dev(page_table, "page_table"),
                                    pool_pages, lens.ctypes.data_as(ctypes.c_void_p), B, Hi, Di, N,
                                    _dev(scores, "scores", torch.int32), _stream(stream))
    _check(rc, "dsa_index_scores_paged")
    return scores


def dsa_sparse_attn_paged(q, kv_pool, page_table, idx, Dv, scale, N=None, out=None, workspace=None,
                          stream=None):
    """dsa_sparse_attn over a latent pool [pool_pages * 256, Dk] read through page_table;
    idx holds logical positions (< N)."""
    torch = _torch()
    lib = load_library()
    B, Hq, Dk = q.shape
    N, pool_pages = _paging(page_table, (kv_pool,), N)
    k = idx.shape[1]
    dt = _attn_dtype(q, kv_pool)
    if out is None:
        out = torch.empty((B, Hq, Dv), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = new_workspace(B, N, k, Hq, Dv, q.device)
    rc = lib.dsa_sparse_attn_paged(_dev(q, "q"), _dev(kv_pool, "kv_pool"), _dev(page_table, "page_table"),
                                   pool_pages, _dev(idx, "idx", torch.int32), B, Hq, Dk, Dv, N, k,
                                   float(scale), dt, _dev(out, "out", torch.float32), _dev(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "dsa_sparse_attn_paged")
    return out


def dsa_decode_step_paged(iq, iw, ik_pool, q, kv_pool, page_table, ctx_len, k, Dv, scale, N=None,
                          scores=None, idx=None, out=None, workspace=None, flags=0, stream=None,
                          kernel_events=None):
    """dsa_decode_step over paged pools (ik_pool [pool_pages * 256, Di], kv_pool
    [pool_pages * 256, Dk]) read through one page table; returns (scores, idx, out) with
    logical positions, as the contiguous call on the caches the table describes."""
    torch = _torch()
    lib = load_library()
    B, Hi, Di = iq.shape
    _, Hq, Dk = q.shape
    N, pool_pages = _paging(page_table, (ik_pool, kv_pool), N)
    lens = _host_lens(ctx_len, B)
    dt = _attn_dtype(q, kv_pool)
    dev = ik_pool.device
    if scores is None:
        scores = torch.zeros((B, N), dtype=torch.int32, device=dev)
    if idx is None:
        idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((B, Hq, Dv), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = new_workspace(B, N, k, Hq, Dv, dev)
    evs = None
    if kernel_events is not None:
        if len(kernel_events) != 6:
            raise ValueError("kernel_events must hold 6 events")
        evs = ctypes.cast((ctypes.c_void_p * 6)(*[e.cuda_event for e in kernel_events]), ctypes.c_void_p)
    rc = lib.dsa_decode_step_paged(_dev(iq, "iq", torch.int8), _dev(iw, "iw", torch.int8),
                                   _dev(ik_pool, "ik_pool", torch.int8), _dev(q, "q"), _dev(kv_pool, "kv_pool"),
                                   _dev(page_table, "page_table"), pool_pages,
                                   lens.ctypes.data_as(ctypes.c_void_p), B, Hi, Di, Hq, Dk, Dv, N, k,
                                   float(scale), dt, _dev(scores, "scores", torch.int32),
                                   _dev(idx, "idx", torch.int32), _dev(out, "out", torch.float32),
                                   _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                   flags, _stream(stream), evs)
    _check(rc, "dsa_decode_step_paged")
    return scores, idx, out
