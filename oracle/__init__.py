"""Plain CPU oracle for the DSA decode step (indexer scores, exact top-k, attention).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline leg
of the benchmark may import this package; the product path never does. It shares
no code with the HIP library. The arithmetic lives in ``dsa_oracle.cpp`` (plain
C++, int64 scores, std::stable_sort, fp64 softmax); this module compiles it with
g++ and calls it through ctypes on numpy arrays.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle_dsa.so")
_LIB_OMP = os.path.join(_HERE, "liboracle_dsa_omp.so")  # the same source with -fopenmp
_libs = {}

F32, BF16, BF16_Q_E4M3_KV = 0, 1, 2


def build(force=True):
    """Compile dsa_oracle.cpp into liboracle_dsa.so next to it (plain g++, -O2), and the
    same source with -fopenmp into liboracle_dsa_omp.so (the all-core CPU baseline)."""
    for path, extra in ((_LIB, []), (_LIB_OMP, ["-fopenmp"])):
        if not force and os.path.exists(path):
            continue
        tmp = path + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", "-O2", "-std=c++17", *extra, "-shared", "-fPIC", "-o", tmp, _SRC])
        os.replace(tmp, path)
    return _LIB


def _load(omp=False):
    path = _LIB_OMP if omp else _LIB
    if path not in _libs:
        if not os.path.exists(path):
            build(force=False)
        lib = ctypes.CDLL(path)
        p, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.dsa_ref_index_scores.argtypes = [p, p, p, p, i32, i32, i32, i64, p]
        lib.dsa_ref_topk_select.argtypes = [p, p, i32, i64, i32, p]
        lib.dsa_ref_sparse_attn.argtypes = [p, p, p, i32, i32, i32, i32, i64, i32, dbl, i32, p]
        lib.dsa_ref_decode_step.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32,
                                            i64, i32, dbl, i32, p, p, p]
        lib.dsa_ref_gather_pages.argtypes = [p, i64, p, i64, i32, i64, p]
        lib.dsa_ref_gather_pages.restype = ctypes.c_int
        lib.dsa_ref_e4m3_to_f64.argtypes = [p, i64, p]
        lib.dsa_ref_e4m3_to_f64.restype = None
        for f in (lib.dsa_ref_index_scores, lib.dsa_ref_topk_select, lib.dsa_ref_sparse_attn,
                  lib.dsa_ref_decode_step, lib.dsa_ref_threads):
            f.restype = ctypes.c_int
        _libs[path] = lib
    return _libs[path]


def threads(omp=False):
    """Threads the oracle's loops use (1, or OpenMP's count for the omp build)."""
    return int(_load(omp).dsa_ref_threads())


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError("%s failed: oracle code %d (1 = bad argument, 2 = score overflows int32)"
                         % (what, rc))


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def _attn_dtype(q, kv):
    """Attention input formats: fp32 both, bf16 both (uint16 bit patterns), or bf16 queries
    with an FP8 E4M3 latent cache (uint8 codes)."""
    if q.dtype == np.float32 and kv.dtype == np.float32:
        return F32
    if q.dtype == np.uint16 and kv.dtype == np.uint16:
        return BF16
    if q.dtype == np.uint16 and kv.dtype == np.uint8:
        return BF16_Q_E4M3_KV
    raise TypeError("attention inputs: float32 q and kv, bf16 bits (uint16) q and kv, or bf16 q with "
                    "e4m3 codes (uint8) kv; got %s and %s" % (q.dtype, kv.dtype))


def e4m3_to_f64(codes):
    """FP8 E4M3 (e4m3fn) codes (uint8) -> their exact values as float64 (NaN for 0x7F/0xFF)."""
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float64)
    _load().dsa_ref_e4m3_to_f64(_ptr(codes), codes.size, _ptr(out))
    return out


def index_scores(iq, iw, ik, ctx_len, omp=False):
    """iq [B,Hi,Di] int8, iw [B,Hi] int8, ik [N,Di] int8, ctx_len [B] int32 -> scores [B,N] int32.

    Entries at or past ctx_len[b] are left at 0 (the oracle never writes them).
    """
    iq, iw, ik = _c(iq, np.int8), _c(iw, np.int8), _c(ik, np.int8)
    ctx_len = _c(ctx_len, np.int32)
    B, Hi, Di = iq.shape
    N = ik.shape[0]
    assert ik.shape[1] == Di and iw.shape == (B, Hi) and ctx_len.shape == (B,)
    scores = np.zeros((B, N), np.int32)
    _check(_load(omp).dsa_ref_index_scores(_ptr(iq), _ptr(iw), _ptr(ik), _ptr(ctx_len), B, Hi, Di, N,
                                        _ptr(scores)), "index_scores")
    return scores


def topk_select(scores, ctx_len, k, omp=False):
    """scores [B,N] int32, ctx_len [B] int32 -> idx [B,k] int32 ((score desc, pos asc), -1 pad)."""
    scores, ctx_len = _c(scores, np.int32), _c(ctx_len, np.int32)
    B, N = scores.shape
    idx = np.empty((B, k), np.int32)
    _check(_load(omp).dsa_ref_topk_select(_ptr(scores), _ptr(ctx_len), B, N, k, _ptr(idx)),
           "topk_select")
    return idx


def sparse_attn(q, kv, idx, Dv, scale, omp=False):
    """q [B,Hq,Dk], kv [N,Dk] (see _attn_dtype for the formats), idx [B,k] -> out [B,Hq,Dv] float64."""
    dt = _attn_dtype(q, kv)
    q, kv, idx = np.ascontiguousarray(q), np.ascontiguousarray(kv), _c(idx, np.int32)
    B, Hq, Dk = q.shape
    N = kv.shape[0]
    k = idx.shape[1]
    assert kv.shape[1] == Dk and idx.shape[0] == B
    out = np.empty((B, Hq, Dv), np.float64)
    _check(_load(omp).dsa_ref_sparse_attn(_ptr(q), _ptr(kv), _ptr(idx), B, Hq, Dk, Dv, N, k,
                                       float(scale), dt, _ptr(out)), "sparse_attn")
    return out


def decode_step(iq, iw, ik, q, kv, ctx_len, k, Dv, scale, omp=False):
    """All three stages; returns (scores [B,N] int32, idx [B,k] int32, out [B,Hq,Dv] float64)."""
    iq, iw, ik = _c(iq, np.int8), _c(iw, np.int8), _c(ik, np.int8)
    ctx_len = _c(ctx_len, np.int32)
    dt = _attn_dtype(q, kv)
    q, kv = np.ascontiguousarray(q), np.ascontiguousarray(kv)
    B, Hi, Di = iq.shape
    _, Hq, Dk = q.shape
    N = ik.shape[0]
    assert kv.shape == (N, Dk)
    scores = np.zeros((B, N), np.int32)
    idx = np.empty((B, k), np.int32)
    out = np.empty((B, Hq, Dv), np.float64)
    _check(_load(omp).dsa_ref_decode_step(_ptr(iq), _ptr(iw), _ptr(ik), _ptr(q), _ptr(kv), _ptr(ctx_len),
                                       B, Hi, Di, Hq, Dk, Dv, N, k, float(scale), dt,
                                       _ptr(scores), _ptr(idx), _ptr(out)), "decode_step")
    return scores, idx, out


PAGE = 256  # positions per pool page (a 1,048,576-token pool held in 4,096 pages)


def gather_pages(pool, page_table, N, page=PAGE):
    """The contiguous cache [N, ...] that page_table describes in pool [pool_pages * page, ...]:
    row s is pool row page_table[s // page] * page + s % page."""
    pool = np.ascontiguousarray(pool)
    page_table = _c(page_table, np.int32)
    if pool.shape[0] % page != 0:
        raise ValueError("the pool must hold whole pages")
    if page_table.shape[0] * page < N:
        raise ValueError("the table must cover N positions")
    row_bytes = pool[0].nbytes
    out = np.empty((N,) + pool.shape[1:], pool.dtype)
    _check(_load().dsa_ref_gather_pages(_ptr(pool), row_bytes, _ptr(page_table), pool.shape[0] // page,
                                        page, N, _ptr(out)), "gather_pages")
    return out


def decode_step_paged(iq, iw, ik_pool, q, kv_pool, page_table, ctx_len, k, Dv, scale, N):
    """The step over paged pools: the contiguous step on the caches the table describes."""
    ik = gather_pages(ik_pool, page_table, N)
    kv = gather_pages(kv_pool, page_table, N)
    return decode_step(iq, iw, ik, q, kv, ctx_len, k, Dv, scale)
