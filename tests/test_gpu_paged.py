"""Paged caches on the GPU: the three stages read the indexer keys and the latent rows
from pools of 256-position pages through a page table (the glm53-tensorfold-spark
README's shared KV pool: 1,048,576 tokens in 4,096 pages). A paged call must give
what the contiguous call gives on the caches the table describes, bit for bit, and
so match the oracle (which gathers those caches) as the contiguous path does:
scores and indices exactly, attention within max|gpu - ref| <= 1e-2 and relative
L2 <= 2e-3. The pools scatter the sequence's pages in a seeded random order and
fill every other row with decoys (random indexer keys, latent rows of 8.0), so a
read of a wrong row changes the scores or dominates the softmax."""
import sys

import numpy as np
import pytest

import oracle
from sparse_attention_decode_scores_amd import inputs

pytestmark = pytest.mark.gpu

MAX_ABS, REL_L2 = 1e-2, 2e-3
_cache = {}


def note(*a):
    print("[gpu-paged]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


@pytest.fixture(scope="module")
def dsa(torch):
    from sparse_attention_decode_scores_amd import binding
    binding.load_library()
    return binding


def to_dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if a.dtype == np.uint8:  # FP8 E4M3 codes
        return torch.from_numpy(a).view(torch.float8_e4m3fn).cuda()
    return torch.from_numpy(a).cuda()


def case(name):
    if name not in _cache:
        c = inputs.make(name)
        ref = oracle.decode_step(c["iq"], c["iw"], c["ik"], c["q"], c["kv"], c["ctx_len"], c["k"], c["Dv"],
                                 c["scale"])
        p = inputs.paged(c)
        # the pools hold exactly the caches the oracle ran on
        assert np.array_equal(oracle.gather_pages(p["ik_pool"], p["page_table"], c["N"]), c["ik"])
        assert np.array_equal(oracle.gather_pages(p["kv_pool"], p["page_table"], c["N"]), c["kv"])
        if len(_cache) > 2:
            _cache.clear()
        _cache[name] = (c, ref, p)
    return _cache[name]


def check_attention(out, ref, what):
    out = np.asarray(out, np.float64)
    err = np.abs(out - ref)
    rel = np.linalg.norm(out - ref) / max(np.linalg.norm(ref), 1e-300)
    note("%s: max-abs %.3e rel-l2 %.3e" % (what, err.max(), rel))
    assert err.max() <= MAX_ABS, what
    assert rel <= REL_L2, what


def bits_equal(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


def run(torch, dsa, c, p=None, flags=0, events=None):
    """One decode step on the contiguous caches (p None) or on the pools of p."""
    ws = dsa.new_workspace(c["B"], c["N"], c["k"], c["Hq"], c["Dv"])
    ws[:32 * c["B"]].fill_(0x5A)
    idx = torch.full((c["B"], c["k"]), -7, dtype=torch.int32, device="cuda")
    iq, iw, q = (to_dev(torch, c[key]) for key in ("iq", "iw", "q"))
    if p is None:
        scores, idx, out = dsa.dsa_decode_step(iq, iw, to_dev(torch, c["ik"]), q, to_dev(torch, c["kv"]),
                                               c["ctx_len"], c["k"], c["Dv"], c["scale"], idx=idx, workspace=ws,
                                               flags=flags)
    else:
        scores, idx, out = dsa.dsa_decode_step_paged(iq, iw, to_dev(torch, p["ik_pool"]), q,
                                                     to_dev(torch, p["kv_pool"]), to_dev(torch, p["page_table"]),
                                                     c["ctx_len"], c["k"], c["Dv"], c["scale"], N=c["N"], idx=idx,
                                                     workspace=ws, flags=flags, kernel_events=events)
    torch.cuda.synchronize()
    stats = dsa.dsa_read_stats(ws, c["B"])
    return scores.cpu().numpy(), idx.cpu().numpy(), out.cpu().numpy(), stats


@pytest.mark.parametrize("name", ["tiny_4k", "ctx16k", "ctx16k_fp8kv", "ctx16k_hotstride", "verify8_ctx131k",
                                  "verify16_ctx131k", "ctx300k"])
def test_paged_step_matches_oracle_and_contiguous(torch, dsa, name):
    note("paged decode_step", name)
    c, (rs, ri, ro), p = case(name)
    if c["N"] <= 16384:  # the oracle's own paged step agrees with it on the contiguous caches
        r2 = oracle.decode_step_paged(c["iq"], c["iw"], p["ik_pool"], c["q"], p["kv_pool"], p["page_table"],
                                      c["ctx_len"], c["k"], c["Dv"], c["scale"], N=c["N"])
        assert np.array_equal(r2[1], ri) and np.array_equal(r2[2], ro)
    note("running", name, "B=%d N=%d pool pages %d" % (c["B"], c["N"], p["pool_pages"]))
    s1, i1, o1, st1 = run(torch, dsa, c, p)
    for b, n in enumerate(c["ctx_len"]):
        assert np.array_equal(s1[b, :n], rs[b, :n]), "%s row %d scores" % (name, b)
    assert np.array_equal(i1, ri), name + " indices"
    check_attention(o1, ro, name)
    s0, i0, o0, st0 = run(torch, dsa, c)
    assert bits_equal(o1, o0) and np.array_equal(i1, i0), name + ": paged and contiguous differ"
    assert st1 == st0


@pytest.mark.parametrize("name", ["ctx16k", "verify8_ctx131k"])
def test_paged_forced_fallback_matches_contiguous(torch, dsa, name):
    note("paged forced fallback", name)
    c, (rs, ri, ro), p = case(name)
    s1, i1, o1, st1 = run(torch, dsa, c, p, flags=dsa.FLAG_FORCE_FALLBACK)
    s0, i0, o0, st0 = run(torch, dsa, c, flags=dsa.FLAG_FORCE_FALLBACK)
    assert np.array_equal(i1, ri) and np.array_equal(i1, i0)
    assert bits_equal(o1, o0)
    assert st1 == st0 and all(st["path"] == 1 and st["reason"] == 1 for st in st1)


@pytest.mark.parametrize("name", ["ctx16k", "verify8_ctx131k"])
def test_paged_table_read_from_memory(torch, dsa, name):
    # the selection kernel's path for tables too large for its LDS, forced by a flag
    note("paged table in memory", name)
    c, (rs, ri, ro), p = case(name)
    s1, i1, o1, st1 = run(torch, dsa, c, p, flags=dsa.FLAG_TABLE_IN_MEMORY)
    s0, i0, o0, st0 = run(torch, dsa, c, p)
    assert np.array_equal(i1, ri) and np.array_equal(i1, i0)
    assert bits_equal(o1, o0) and st1 == st0


def test_paged_timed_step_matches_untimed(torch, dsa):
    note("paged timed step")
    c, (rs, ri, ro), p = case("ctx16k")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in evs:
        e.record()
    s1, i1, o1, _ = run(torch, dsa, c, p, events=evs)
    s0, i0, o0, _ = run(torch, dsa, c, p)
    assert np.array_equal(i1, i0) and bits_equal(o1, o0)
    for j in range(3):
        assert evs[2 * j].elapsed_time(evs[2 * j + 1]) > 0


@pytest.mark.parametrize("B,N,ctx", [(1, 5000, [4999]), (3, 5000, [5000, 257, 4100]),
                                     (2, 16284, [16284, 9000])])
def test_paged_ragged_pages_and_rows(torch, dsa, B, N, ctx):
    # the sequence's last page is partly used (its tail holds decoys), rows end anywhere
    note("paged ragged", B, N, ctx)
    c = inputs.random_case(700 + B, B=B, N=N, k=1024, Hi=64, Di=128, Hq=16, Dk=576, Dv=512, ctx_len=ctx)
    p = inputs.paged(c, seed=11)
    rs, ri, ro = oracle.decode_step_paged(c["iq"], c["iw"], p["ik_pool"], c["q"], p["kv_pool"], p["page_table"],
                                          c["ctx_len"], c["k"], c["Dv"], c["scale"], N=N)
    s1, i1, o1, st1 = run(torch, dsa, c, p)
    for b, n in enumerate(ctx):
        assert np.array_equal(s1[b, :n], rs[b, :n])
    assert np.array_equal(i1, ri)
    check_attention(o1, ro, "ragged B=%d" % B)
    s0, i0, o0, _ = run(torch, dsa, c)
    assert bits_equal(o1, o0)


def test_paged_table_may_repeat_and_fill_the_pool(torch, dsa):
    # two logical pages on one pool page (a shared prefix page), and a pool with no
    # spare page: the described cache is whatever the table reads
    note("paged aliasing")
    c = inputs.random_case(801, B=1, N=4096, k=512, Hi=64, Di=128, Hq=16, Dk=576, Dv=512)
    p = inputs.paged(c, seed=12, pool_pages=16)
    p["page_table"][5] = p["page_table"][2]
    ik = oracle.gather_pages(p["ik_pool"], p["page_table"], c["N"])
    kv = oracle.gather_pages(p["kv_pool"], p["page_table"], c["N"])
    assert np.array_equal(ik[5 * 256:6 * 256], ik[2 * 256:3 * 256])
    rs, ri, ro = oracle.decode_step(c["iq"], c["iw"], ik, c["q"], kv, c["ctx_len"], c["k"], c["Dv"], c["scale"])
    s1, i1, o1, _ = run(torch, dsa, c, p)
    assert np.array_equal(s1[0], rs[0]) and np.array_equal(i1, ri)
    check_attention(o1, ro, "aliased table")


@pytest.mark.parametrize("ctx", [[4999], [5000, 300, 4097]])
def test_paged_index_scores_standalone(torch, dsa, ctx):
    # one row (the one-row launch of the pass without candidates) and several
    note("paged index_scores", ctx)
    B = len(ctx)
    c = inputs.random_case(802, B=B, N=5000, k=64, Hi=64, Di=128, Hq=1, Dk=64, Dv=64, ctx_len=ctx)
    p = inputs.paged(c, seed=13)
    ref = oracle.index_scores(c["iq"], c["iw"], c["ik"], c["ctx_len"])
    scores = torch.full((B, 5000), -5, dtype=torch.int32, device="cuda")
    dsa.dsa_index_scores_paged(to_dev(torch, c["iq"]), to_dev(torch, c["iw"]), to_dev(torch, p["ik_pool"]),
                               to_dev(torch, p["page_table"]), c["ctx_len"], N=5000, scores=scores)
    got = scores.cpu().numpy()
    for b, n in enumerate(c["ctx_len"]):
        assert np.array_equal(got[b, :n], ref[b, :n])
        assert (got[b, n:] == -5).all()


@pytest.mark.parametrize("name", ["ctx16k", "ctx16k_fp8kv"])
def test_paged_sparse_attn_standalone(torch, dsa, name):
    note("paged sparse_attn", name)
    c, (rs, ri, ro), p = case(name)
    idx = ri.copy()
    idx[0, 5] = -1
    idx[0, 9] = c["N"] + 3  # outside [0, N): skipped and counted
    q = to_dev(torch, c["q"])
    ws1 = dsa.new_workspace(1, c["N"], c["k"], c["Hq"], c["Dv"])
    o1 = dsa.dsa_sparse_attn_paged(q, to_dev(torch, p["kv_pool"]), to_dev(torch, p["page_table"]),
                                   torch.from_numpy(idx).cuda(), c["Dv"], c["scale"], N=c["N"], workspace=ws1)
    ws0 = dsa.new_workspace(1, c["N"], c["k"], c["Hq"], c["Dv"])
    o0 = dsa.dsa_sparse_attn(q, to_dev(torch, c["kv"]), torch.from_numpy(idx).cuda(), c["Dv"], c["scale"],
                             workspace=ws0)
    torch.cuda.synchronize()
    assert bits_equal(o1.cpu().numpy(), o0.cpu().numpy())
    keep = idx.copy()
    keep[0, 9] = -1
    ref = oracle.sparse_attn(c["q"], c["kv"], keep, c["Dv"], c["scale"])
    check_attention(o1.cpu().numpy(), ref, "paged sparse_attn")
    assert dsa.dsa_read_stats(ws1, 1)[0]["bad_indices"] == 1
