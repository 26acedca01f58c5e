"""Seeded synthetic inputs for the DSA decode step (shared by the tests, the oracle
checks and the benchmark). This module draws numbers and nothing else: none of the
method's arithmetic lives here.

Workloads (no real GLM-5.3-Flash weights or caches are available, so every array
is synthetic with the shapes of the model's DSA layers):

  tiny_4k           B=1, context 4,096, k=256; indexer 4 heads x 64, query and keys
                    int8 uniform on [-8, 8], head weights uniform on [1, 4]; attention
                    8 heads x 64, one shared fp32 N(0,1) row per position used as key
                    and value; scale 1/8.
  ctx16k            B=1, context 16,384, k=2,048; indexer 64 heads x 128 with one
                    shared 128-dim key per position, int8 uniform on [-16, 16], head
                    weights uniform on [1, 8]; attention 16 heads over a shared latent
                    row of 512 latent + 64 rope values per position, bf16 N(0,1)*0.5;
                    output 512 values per head; scale 1/sqrt(576) = 1/24.
  ctx62k_11layers   ctx16k shapes at context 62,464, eleven independent layers (own
                    seeds) per step.
  ctx300k           ctx16k shapes at context 300,000 with indexer keys on the coarse
                    grid {-2..2}.
  verify8_ctx131k   width-8 verify block: B=8 over a shared 131,072-position cache;
                    row r sees ctx_len = 131,065 + r.
  verify16_ctx131k  the widest verify block: B=16 over the same cache shape, row r
                    sees ctx_len = 131,057 + r (own seed).
  ctx300k_tiepool   ctx300k with every key row drawn from a pool of 512 rows, so that
                    many positions share a score exactly (ties at the threshold).
  ctx16k_zeroquery  ctx16k with an all-zero indexer query: every score is 0.
  ctx16k_fp8kv,     ctx16k and ctx300k (same seeds, so the same indexer inputs and
  ctx300k_fp8kv     the same normal draws) with the latent cache stored as FP8 E4M3
                    codes (round to nearest even from the fp32 draw) and bf16 queries.
  ctx16k_hotstride  ctx16k with the key rows of every 256th block of 32 positions
                    (positions 0-31 and 8,192-8,223) replaced by the indexer query of
                    row 0, head 0: those 64 positions tie at one score that only about
                    120 other positions exceed, so all 64 are in the top 2,048.

Integer ranges are inclusive. Seeds (numpy PCG64 ``default_rng(seed)``): tiny_4k
1000, ctx16k 1001, ctx300k 1003, verify8_ctx131k 1004, verify16_ctx131k 1005, ctx300k_tiepool 1030,
ctx16k_zeroquery 1090, ctx16k_hotstride 1091, and 2000 + l for layer l of ctx62k_11layers; the integer
arrays are drawn from it in the order iq, iw, ik. The normal arrays are drawn in
blocks of 16,384 rows, block j of q from ``default_rng([seed, 1, j])`` and of kv
from ``default_rng([seed, 2, j])`` (so they can be drawn on several threads).

bf16 values are carried as uint16 bit patterns and FP8 E4M3 (e4m3fn) values as uint8
codes, each rounded to nearest even from the fp32 draw.

Paged pools (``paged``): a workload's two caches placed in pools of 256-position
pages, as the shared KV pool of the glm53-tensorfold-spark README holds them
(1,048,576 tokens in 4,096 pages). The sequence's ceil(N / 256) logical pages go to
distinct pool pages in a seeded random order (``default_rng([seed, 3])``
permutation of the pool), so neighbouring pages are scattered over the pool. Every
pool row the sequence does not own, including the tail of its last page, holds
decoy values: indexer keys drawn uniformly from the workload's key range
(``default_rng([seed, 4])``) and latent rows of constant 8.0 (exact in fp32, bf16
and E4M3), large enough to dominate any softmax they were wrongly let into.
"""
import numpy as np

_LAYER = dict(Hi=64, Di=128, Hq=16, Dk=576, Dv=512, dtype="bf16", scale=1.0 / 24.0, qk_range=16,
              w_range=(1, 8), key_range=16, layers=1)

CONFIGS = {
    "tiny_4k": dict(B=1, N=4096, k=256, Hi=4, Di=64, Hq=8, Dk=64, Dv=64, dtype="f32", scale=1.0 / 8.0,
                    qk_range=8, w_range=(1, 4), key_range=8, layers=1, seed=1000),
    "ctx16k": dict(_LAYER, B=1, N=16384, k=2048, seed=1001),
    "ctx62k_11layers": dict(_LAYER, B=1, N=62464, k=2048, layers=11, seed=2000),
    "ctx300k": dict(_LAYER, B=1, N=300000, k=2048, key_range=2, seed=1003),
    "verify8_ctx131k": dict(_LAYER, B=8, N=131072, k=2048, seed=1004, verify_offsets=True),
    "verify16_ctx131k": dict(_LAYER, B=16, N=131072, k=2048, seed=1005, verify_offsets=True),
    "ctx300k_tiepool": dict(_LAYER, B=1, N=300000, k=2048, key_range=2, seed=1030, key_pool=512),
    "ctx16k_zeroquery": dict(_LAYER, B=1, N=16384, k=2048, seed=1090, zero_query=True),
    "ctx16k_hotstride": dict(_LAYER, B=1, N=16384, k=2048, seed=1091, hot_stride=256),
    "ctx16k_fp8kv": dict(_LAYER, B=1, N=16384, k=2048, seed=1001, dtype="fp8"),
    "ctx300k_fp8kv": dict(_LAYER, B=1, N=300000, k=2048, key_range=2, seed=1003, dtype="fp8"),
}


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even) and return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    try:  # torch's multi-threaded conversion, same rounding; plain numpy otherwise
        import torch
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    except ImportError:
        pass
    flat = x.reshape(-1).view(np.uint32)
    out = np.empty(flat.shape, np.uint16)
    step = 1 << 22
    for s in range(0, flat.size, step):  # chunked: keeps temporaries in cache
        u = flat[s:s + step]
        t = u >> np.uint32(16)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)
        t += u
        t >>= np.uint32(16)
        out[s:s + step] = t
    return out.reshape(x.shape)


def f32_to_e4m3_codes(x):
    """Round float32 values to FP8 E4M3 (e4m3fn; nearest, ties to even) and return the
    uint8 codes (torch's conversion)."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bf16_bits_to_f32(b):
    """Widen uint16 bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def ctx_lengths(name):
    c = CONFIGS[name]
    if c.get("verify_offsets"):  # row r of a B-row block sees N - (B - 1) + r positions
        return np.array([c["N"] - c["B"] + 1 + r for r in range(c["B"])], np.int32)
    return np.full(c["B"], c["N"], np.int32)


_BLOCK_ROWS = 16384


def _normal(seed, tag, shape, dtype, mul):
    """N(0,1)*mul of the given shape (rows along axis 0), drawn block by block."""
    shape = tuple(shape)
    x = np.empty(shape, np.float32)
    nblk = (shape[0] + _BLOCK_ROWS - 1) // _BLOCK_ROWS

    def fill(j):
        a, b = j * _BLOCK_ROWS, min(shape[0], (j + 1) * _BLOCK_ROWS)
        r = np.random.default_rng([seed, tag, j])
        x[a:b] = r.standard_normal(size=(b - a,) + shape[1:], dtype=np.float32)
        if mul != 1.0:
            x[a:b] *= np.float32(mul)

    if nblk > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(min(8, nblk)) as ex:
            list(ex.map(fill, range(nblk)))
    else:
        fill(0)
    if dtype == "f32":
        return x
    return f32_to_e4m3_codes(x) if dtype == "e4m3" else f32_to_bf16_bits(x)


def make(name, layer=0):
    """Inputs of one layer of workload ``name`` as a dict of numpy arrays plus its shapes."""
    c = dict(CONFIGS[name])
    if not 0 <= layer < c["layers"]:
        raise ValueError("layer out of range")
    rng = np.random.default_rng(c["seed"] + layer)
    B, N, Hi, Di, Hq, Dk = c["B"], c["N"], c["Hi"], c["Di"], c["Hq"], c["Dk"]
    qr, kr = c["qk_range"], c["key_range"]
    iq = rng.integers(-qr, qr + 1, size=(B, Hi, Di), dtype=np.int8)
    iw = rng.integers(c["w_range"][0], c["w_range"][1] + 1, size=(B, Hi), dtype=np.int8)
    if c.get("key_pool"):
        pool = rng.integers(-kr, kr + 1, size=(c["key_pool"], Di), dtype=np.int8)
        ik = pool[rng.integers(0, c["key_pool"], size=N)]
    else:
        ik = rng.integers(-kr, kr + 1, size=(N, Di), dtype=np.int8)
    if c.get("zero_query"):
        iq[...] = 0
    if c.get("hot_stride"):
        blocks = np.arange(N) // 32
        ik = ik.copy()
        ik[blocks % c["hot_stride"] == 0] = iq[0, 0]
    mul = 1.0 if c["dtype"] == "f32" else 0.5
    seed = c["seed"] + layer
    qd, kvd = {"f32": ("f32", "f32"), "bf16": ("bf16", "bf16"), "fp8": ("bf16", "e4m3")}[c["dtype"]]
    q = _normal(seed, 1, (B, Hq, Dk), qd, mul)
    kv = _normal(seed, 2, (N, Dk), kvd, mul)
    c.update(iq=iq, iw=iw, ik=np.ascontiguousarray(ik), q=q, kv=kv, ctx_len=ctx_lengths(name),
             name=name, layer=layer)
    return c


def random_case(seed, B, N, k, Hi, Di, Hq, Dk, Dv, dtype="bf16", ctx_len=None, qk_range=16,
                key_range=16, w_range=(1, 8), scale=None):
    """A seeded case of arbitrary shape with the same value recipe as the workloads."""
    rng = np.random.default_rng(seed)
    iq = rng.integers(-qk_range, qk_range + 1, size=(B, Hi, Di), dtype=np.int8)
    iw = rng.integers(w_range[0], w_range[1] + 1, size=(B, Hi), dtype=np.int8)
    ik = rng.integers(-key_range, key_range + 1, size=(N, Di), dtype=np.int8)
    mul = 1.0 if dtype == "f32" else 0.5
    qd, kvd = {"f32": ("f32", "f32"), "bf16": ("bf16", "bf16"), "fp8": ("bf16", "e4m3")}[dtype]
    q = _normal(seed, 1, (B, Hq, Dk), qd, mul)
    kv = _normal(seed, 2, (N, Dk), kvd, mul)
    if ctx_len is None:
        ctx_len = np.full(B, N, np.int32)
    return dict(B=B, N=N, k=k, Hi=Hi, Di=Di, Hq=Hq, Dk=Dk, Dv=Dv, dtype=dtype,
                scale=(1.0 / np.sqrt(Dk)) if scale is None else scale, iq=iq, iw=iw, ik=ik, q=q,
                kv=kv, ctx_len=np.asarray(ctx_len, np.int32), layers=1, name="random", layer=0)


PAGE = 256  # positions per pool page


def paged(c, seed=7, pool_pages=None):
    """Pools and page table holding the caches of case ``c``: returns dict(ik_pool, kv_pool,
    page_table, pool_pages). The pool has ``pool_pages`` pages (default: twice the
    sequence's pages, plus three)."""
    N = c["N"]
    n_tab = (N + PAGE - 1) // PAGE
    pool_pages = 2 * n_tab + 3 if pool_pages is None else int(pool_pages)
    if pool_pages < n_tab:
        raise ValueError("the pool must hold the sequence's pages")
    table = np.random.default_rng([seed, 3]).permutation(pool_pages)[:n_tab].astype(np.int32)
    rows = pool_pages * PAGE
    kr = c.get("key_range", 16)
    ik_pool = np.random.default_rng([seed, 4]).integers(-kr, kr + 1, size=(rows, c["Di"]), dtype=np.int8)
    kv = c["kv"]
    eight = np.array([8.0], np.float32)
    decoy = {np.dtype(np.float32): eight, np.dtype(np.uint16): f32_to_bf16_bits(eight),
             np.dtype(np.uint8): f32_to_e4m3_codes(eight)}[kv.dtype][0]
    kv_pool = np.full((rows, kv.shape[1]), decoy, kv.dtype)
    pos = np.arange(N, dtype=np.int64)
    prow = table[pos // PAGE].astype(np.int64) * PAGE + pos % PAGE
    ik_pool[prow] = c["ik"]
    kv_pool[prow] = kv
    return dict(ik_pool=ik_pool, kv_pool=kv_pool, page_table=table, pool_pages=pool_pages)
