"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Scores and indices must match bit for bit; attention must satisfy
max|gpu - ref| <= 1e-2 and ||gpu - ref||_2 / ||ref||_2 <= 2e-3 (over every output of
the case). Full workload sizes are compared element by element: the oracle
finishes each of them in seconds. Beyond the oracle, the GPU paths must agree with
each other bit for bit: the candidate path and the forced exhaustive path, the
decode step and the stand-alone attention over its own indices, and repeated runs
(the ds4 branch post's long-context paragraph: same positions, same order, same
outputs)."""
import sys
import zlib

import numpy as np
import pytest

import oracle
from sparse_attention_decode_scores_amd import inputs

pytestmark = pytest.mark.gpu

MAX_ABS, REL_L2 = 1e-2, 2e-3
_cache = {}


def note(*a):
    print("[gpu-parity]", *a, flush=True)
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


def dev_inputs(torch, c):
    d = {}
    for key in ("iq", "iw", "ik"):
        d[key] = torch.from_numpy(np.ascontiguousarray(c[key])).cuda()
    for key in ("q", "kv"):
        a = np.ascontiguousarray(c[key])
        if a.dtype == np.uint16:  # bf16 bit patterns
            d[key] = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        elif a.dtype == np.uint8:  # FP8 E4M3 codes
            d[key] = torch.from_numpy(a).view(torch.float8_e4m3fn).cuda()
        else:
            d[key] = torch.from_numpy(a).cuda()
    return d


def case(name, layer=0):
    key = (name, layer)
    if key not in _cache:
        c = inputs.make(name, layer)
        ref = oracle.decode_step(c["iq"], c["iw"], c["ik"], c["q"], c["kv"], c["ctx_len"], c["k"],
                                 c["Dv"], c["scale"])
        if len(_cache) > 3:
            _cache.clear()
        _cache[key] = (c, ref)
    return _cache[key]


def check_attention(out, ref, what):
    out = np.asarray(out, np.float64)
    err = np.abs(out - ref)
    rel = np.linalg.norm(out - ref) / max(np.linalg.norm(ref), 1e-300)
    note("%s: max-abs %.3e rel-l2 %.3e" % (what, err.max(), rel))
    assert err.max() <= MAX_ABS, what
    assert rel <= REL_L2, what


def check_scores(gpu, ref, ctx_len, what):
    for b, n in enumerate(ctx_len):
        assert np.array_equal(gpu[b, :n], ref[b, :n]), "%s row %d scores differ" % (what, b)


def run_step(torch, dsa, c, d, flags=0):
    ws = dsa.new_workspace(c["B"], c["N"], c["k"], c["Hq"], c["Dv"])
    # every index slot and row record must be written by the call: start from values
    # no call leaves (the records are the workspace's first B x 32 bytes)
    ws[:32 * c["B"]].fill_(0x5A)
    idx = torch.full((c["B"], c["k"]), -7, dtype=torch.int32, device="cuda")
    scores, idx, out = dsa.dsa_decode_step(d["iq"], d["iw"], d["ik"], d["q"], d["kv"], c["ctx_len"],
                                           c["k"], c["Dv"], c["scale"], idx=idx, workspace=ws, flags=flags)
    torch.cuda.synchronize()
    stats = dsa.dsa_read_stats(ws, c["B"])
    return scores.cpu().numpy(), idx.cpu().numpy(), out.cpu().numpy(), stats


def expected_ties(ref_scores, ref_idx, ctx_len, k):
    t = []
    for b, n in enumerate(ctx_len):
        m = min(k, n)
        sel = ref_scores[b, ref_idx[b, :m]]
        t.append(int((sel == sel[-1]).sum()))
    return t


@pytest.mark.parametrize("name", ["tiny_4k", "ctx16k", "ctx300k", "verify8_ctx131k", "verify16_ctx131k", "ctx300k_tiepool",
                                  "ctx16k_zeroquery", "ctx16k_hotstride", "ctx16k_fp8kv", "ctx300k_fp8kv"])
def test_decode_step_matches_oracle(torch, dsa, name):
    note("decode_step", name)
    c, (rs, ri, ro) = case(name)
    d = dev_inputs(torch, c)
    note("running", name, "B=%d N=%d k=%d" % (c["B"], c["N"], c["k"]))
    s, i, o, stats = run_step(torch, dsa, c, d)
    check_scores(s, rs, c["ctx_len"], name)
    assert np.array_equal(i, ri), name + " indices differ"
    check_attention(o, ro, name)
    ties = expected_ties(rs, ri, c["ctx_len"], c["k"])
    for b, st in enumerate(stats):
        note(name, "row", b, st)
        assert st["selected"] == min(c["k"], int(c["ctx_len"][b]))
        assert st["kth_score"] == int(rs[b, ri[b, st["selected"] - 1]])
        assert st["tied_at_kth"] == ties[b]
        # One-row chunks are interleaved units (c, c + G, ...; G = 256 here): on a
        # constant row chunk c keeps the row's unit c, so the union holds the 8,192
        # earliest positions and covers the top k. The hot-stride row puts 64 tied
        # best keys into chunk 0, more than its 32 slots: the coverage check fails.
        assert st["path"] == (1 if name == "ctx16k_hotstride" else 0)
        if name == "ctx16k_hotstride":
            assert st["reason"] == 2


def test_ctx62k_eleven_layers(torch, dsa):
    c0 = inputs.make("ctx62k_11layers", 0)
    outs, refs = [], []
    for layer in range(c0["layers"]):
        note("ctx62k_11layers layer", layer)
        c, (rs, ri, ro) = case("ctx62k_11layers", layer)
        d = dev_inputs(torch, c)
        s, i, o, _ = run_step(torch, dsa, c, d)
        check_scores(s, rs, c["ctx_len"], "ctx62k_11layers layer %d" % layer)
        assert np.array_equal(i, ri), "ctx62k_11layers layer %d indices differ" % layer
        outs.append(o)
        refs.append(ro)
    check_attention(np.stack(outs), np.stack(refs), "ctx62k_11layers all layers")


def bits_equal(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


@pytest.mark.parametrize("name", ["ctx16k", "ctx300k", "ctx300k_tiepool", "verify8_ctx131k", "ctx16k_zeroquery",
                                  "ctx16k_hotstride", "ctx300k_fp8kv"])
def test_forced_fallback_matches_fast_path(torch, dsa, name):
    # The exhaustive path selects the same positions in the same order, and attention
    # split s takes the positions of output slots [s*per, (s+1)*per) on either path,
    # so the outputs are equal bit for bit. The exhaustive path's list: the union's
    # keys plus rescans of the few chunks whose best dropped key reaches the
    # threshold (ctx16k ... verify8: few or none; hot stride: the chunk holding the
    # tied best keys); on the zero-query row every chunk reaches it, so the row is
    # streamed whole, the list overflows and the radix selection runs.
    note("forced fallback", name)
    c, (rs, ri, ro) = case(name)
    d = dev_inputs(torch, c)
    s1, i1, o1, st1 = run_step(torch, dsa, c, d)
    s2, i2, o2, st2 = run_step(torch, dsa, c, d, flags=dsa.FLAG_FORCE_FALLBACK)
    check_scores(s2, rs, c["ctx_len"], name + " exhaustive path")
    assert np.array_equal(i2, ri)
    assert np.array_equal(i1, i2)
    check_attention(o2, ro, name + " exhaustive path")
    check_attention(o1, ro, name + " fast path")
    assert bits_equal(o1, o2), name + ": fast path and exhaustive path outputs differ"
    assert all(st["path"] == 1 and st["reason"] == 1 for st in st2)
    assert all(st["path"] == (1 if name == "ctx16k_hotstride" else 0) for st in st1)
    for a, b in zip(st1, st2):
        assert (a["selected"], a["kth_score"], a["tied_at_kth"]) == (b["selected"], b["kth_score"],
                                                                     b["tied_at_kth"])


@pytest.mark.parametrize("name", ["ctx16k", "ctx300k", "verify8_ctx131k", "ctx16k_hotstride", "ctx16k_fp8kv"])
def test_decode_step_matches_attention_over_its_indices(torch, dsa, name):
    # dsa_sparse_attn over the step's own ordered indices splits them the same way
    # (slots [s*per, (s+1)*per) per split), so it returns the step's output bit for bit.
    note("step vs stand-alone attention", name)
    c, _ = case(name)
    d = dev_inputs(torch, c)
    _, i1, o1, _ = run_step(torch, dsa, c, d)
    out = dsa.dsa_sparse_attn(d["q"], d["kv"], torch.from_numpy(i1).cuda(), c["Dv"], c["scale"])
    torch.cuda.synchronize()
    assert bits_equal(out.cpu().numpy(), o1)


@pytest.mark.parametrize("name", ["ctx16k", "ctx300k", "verify8_ctx131k"])
def test_runs_are_bit_identical(torch, dsa, name):
    c, _ = case(name)
    d = dev_inputs(torch, c)
    first = run_step(torch, dsa, c, d)
    for rep in range(9):
        again = run_step(torch, dsa, c, d)
        for a, b in zip(first[:3], again[:3]):
            assert bits_equal(a, b), "%s run %d differs" % (name, rep + 1)


@pytest.mark.parametrize("name", ["ctx16k", "verify8_ctx131k"])
def test_timed_step_matches_untimed(torch, dsa, name):
    """dsa_decode_step_timed gives the same bytes as dsa_decode_step, and its events hold
    positive kernel durations (ctx16k: one query row; verify8_ctx131k: eight)."""
    c, _ = case(name)
    d = dev_inputs(torch, c)
    plain = run_step(torch, dsa, c, d)
    ws = dsa.new_workspace(c["B"], c["N"], c["k"], c["Hq"], c["Dv"])
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    scores, idx, out = dsa.dsa_decode_step(d["iq"], d["iw"], d["ik"], d["q"], d["kv"], c["ctx_len"],
                                           c["k"], c["Dv"], c["scale"], workspace=ws,
                                           kernel_events=evs)
    torch.cuda.synchronize()
    for a, b in zip(plain[:3], (scores.cpu().numpy(), idx.cpu().numpy(), out.cpu().numpy())):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    ms = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(3)]
    note("%s kernel ms: %s" % (name, ms))
    assert all(0.0 < t < 50.0 for t in ms)
    with pytest.raises(ValueError):
        dsa.dsa_decode_step(d["iq"], d["iw"], d["ik"], d["q"], d["kv"], c["ctx_len"], c["k"], c["Dv"],
                            c["scale"], workspace=ws, kernel_events=evs[:4])


# ---------------------------------------------------------------- stand-alone stages

def test_index_scores_standalone(torch, dsa):
    for name in ("ctx16k", "verify8_ctx131k"):
        c, (rs, _, _) = case(name)
        d = dev_inputs(torch, c)
        note("index_scores", name)
        s = dsa.dsa_index_scores(d["iq"], d["iw"], d["ik"], c["ctx_len"])
        torch.cuda.synchronize()
        check_scores(s.cpu().numpy(), rs, c["ctx_len"], name)


def test_scores_past_ctx_len_untouched(torch, dsa):
    c = inputs.random_case(5, B=2, N=700, k=64, Hi=8, Di=64, Hq=1, Dk=64, Dv=64,
                           ctx_len=[700, 333])
    d = dev_inputs(torch, c)
    s = torch.full((2, 700), -12345, dtype=torch.int32, device="cuda")
    dsa.dsa_index_scores(d["iq"], d["iw"], d["ik"], c["ctx_len"], scores=s)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    ref = oracle.index_scores(c["iq"], c["iw"], c["ik"], c["ctx_len"])
    assert np.array_equal(s[0], ref[0]) and np.array_equal(s[1, :333], ref[1, :333])
    assert (s[1, 333:] == -12345).all()


@pytest.mark.parametrize("name", ["ctx16k", "ctx300k_tiepool", "ctx16k_zeroquery", "ctx16k_hotstride"])
@pytest.mark.parametrize("flags", [0, 1])
def test_topk_standalone(torch, dsa, name, flags):
    c, (rs, ri, _) = case(name)
    note("topk_select", name, "flags", flags)
    idx = dsa.dsa_topk_select(torch.from_numpy(rs).cuda(), c["ctx_len"], c["k"], flags=flags)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ri)


def test_topk_heavy_ties_and_short_rows(torch, dsa):
    rng = np.random.default_rng(77)
    for N, k, span, ctx in [(20000, 2048, 3, [20000, 15000, 2000, 1]), (9000, 4096, 50, [9000, 9000]),
                            (300, 256, 1 << 30, [300, 10]), (70000, 1, 5, [70000]),
                            (150000, 4096, 1 << 20, [150000, 149999])]:
        B = len(ctx)
        s = rng.integers(-span, span, size=(B, N)).astype(np.int32)
        ctx = np.array(ctx, np.int32)
        ref = oracle.topk_select(s, ctx, k)
        note("topk random N=%d k=%d span=%d" % (N, k, span))
        for flags in (0, 1):
            idx = dsa.dsa_topk_select(torch.from_numpy(s).cuda(), ctx, k, flags=flags)
            torch.cuda.synchronize()
            assert np.array_equal(idx.cpu().numpy(), ref), (N, k, span, flags)


def test_topk_exhaustive_list_falls_back(torch, dsa):
    """Rows whose narrowed list cannot hold the top k on the exhaustive path, which then
    takes the radix selection over every position: (a) the best keys all in wave 0's
    64-position slices (positions p with p % 512 < 64), more than its list segment
    holds; (b) the best scores exactly at the sampled runs of 64 (run r from
    r * n // 256), so the sampled threshold lies above the k-th best score."""
    rng = np.random.default_rng(91)
    N = 40000
    s = rng.integers(-1000, 1000, size=(1, N)).astype(np.int32)
    hot = (np.arange(N) % 512) < 64
    s[0, hot] = rng.integers(10 ** 6, 2 * 10 ** 6, size=int(hot.sum()))
    N2 = 300000
    s2 = rng.integers(0, 1000, size=(1, N2)).astype(np.int32)
    runs = (np.arange(256)[:, None] * N2 // 256 + np.arange(64)[None, :]).ravel()
    s2[0, runs] = rng.integers(10 ** 6, 2 * 10 ** 6, size=runs.size)
    for scores, k in ((s, 2048), (s2, 2048), (s2, 4096)):
        ctx = np.array([scores.shape[1]], np.int32)
        ref = oracle.topk_select(scores, ctx, k)
        note("topk list fallback N=%d k=%d" % (scores.shape[1], k))
        for flags in (0, 1):
            idx = dsa.dsa_topk_select(torch.from_numpy(scores).cuda(), ctx, k, flags=flags)
            torch.cuda.synchronize()
            assert np.array_equal(idx.cpu().numpy(), ref), (scores.shape[1], k, flags)


def test_sparse_attn_standalone_with_skipped_entries(torch, dsa):
    c, (rs, ri, ro) = case("ctx16k")
    d = dev_inputs(torch, c)
    note("sparse_attn ctx16k")
    out = dsa.dsa_sparse_attn(d["q"], d["kv"], torch.from_numpy(ri).cuda(), c["Dv"], c["scale"])
    torch.cuda.synchronize()
    check_attention(out.cpu().numpy(), ro, "sparse_attn ctx16k")
    # -1 entries are skipped; out-of-range entries are skipped and counted
    idx = ri.copy()
    idx[0, 100:300] = -1
    idx[0, 5] = c["N"] + 3
    idx[0, 7] = -9
    ws = dsa.new_workspace(1, c["N"], c["k"], c["Hq"], c["Dv"])
    out = dsa.dsa_sparse_attn(d["q"], d["kv"], torch.from_numpy(idx).cuda(), c["Dv"], c["scale"],
                              workspace=ws)
    torch.cuda.synchronize()
    valid = idx.copy()
    valid[0, 5] = -1
    valid[0, 7] = -1
    ref = oracle.sparse_attn(c["q"], c["kv"], valid, c["Dv"], c["scale"])
    check_attention(out.cpu().numpy(), ref, "sparse_attn with skips")
    assert dsa.dsa_read_stats(ws, 1)[0]["bad_indices"] == 2


def test_constant_row_takes_chunk_fallback(torch, dsa):
    # Every score of a 40,000-position row is 0. Each chunk of the one-row score pass
    # (five interleaved 32-position units, 160 positions) then stages all of its
    # positions, more than m + 64, and takes the radix fallback, whose positions step
    # by G units; its chunk summary gives the whole score range, and the selection
    # narrows one 8,000-way tie by position. Chunk c keeps the row's unit c, so the
    # candidates still cover the top k (positions 0 .. k-1) and the fast path holds.
    c = inputs.random_case(4242, B=1, N=40000, k=2048, Hi=64, Di=128, Hq=16, Dk=576, Dv=512)
    c["iq"][...] = 0
    note("constant row: N=40000 k=2048, zero indexer query")
    rs, ri, ro = oracle.decode_step(c["iq"], c["iw"], c["ik"], c["q"], c["kv"], c["ctx_len"], c["k"],
                                    c["Dv"], c["scale"])
    assert np.array_equal(ri[0], np.arange(2048))
    d = dev_inputs(torch, c)
    s, i, o, stats = run_step(torch, dsa, c, d)
    check_scores(s, rs, c["ctx_len"], "constant row")
    assert np.array_equal(i, ri)
    check_attention(o, ro, "constant row")
    st = stats[0]
    assert st["path"] == 0 and st["selected"] == 2048 and st["tied_at_kth"] == 2048 and st["kth_score"] == 0


# ---------------------------------------------------------------- shapes and edge cases

EDGE = [
    # (label, kwargs for random_case)
    ("tiny-N1-k1", dict(B=1, N=1, k=1, Hi=4, Di=32, Hq=2, Dk=64, Dv=64)),
    ("n-below-k", dict(B=1, N=100, k=256, Hi=64, Di=128, Hq=16, Dk=576, Dv=512)),
    ("ragged-rows", dict(B=3, N=9000, k=2048, Hi=64, Di=128, Hq=16, Dk=576, Dv=512,
                         ctx_len=[9000, 4500, 7])),
    ("odd-heads-dims", dict(B=2, N=12345, k=512, Hi=40, Di=96, Hq=20, Dk=192, Dv=128)),
    ("di-256-k4096", dict(B=1, N=50000, k=4096, Hi=64, Di=256, Hq=64, Dk=576, Dv=512)),
    ("hq1-small-dk", dict(B=2, N=5000, k=300, Hi=4, Di=32, Hq=1, Dk=64, Dv=64)),
    ("dk1024-sb32", dict(B=1, N=20000, k=1000, Hi=32, Di=64, Hq=16, Dk=1024, Dv=512)),
    ("generic-bf16", dict(B=2, N=3000, k=200, Hi=16, Di=64, Hq=6, Dk=80, Dv=40)),
    ("generic-f32", dict(B=2, N=70000, k=2048, Hi=8, Di=64, Hq=8, Dk=64, Dv=64, dtype="f32")),
    ("verify-rows", dict(B=8, N=40000, k=2048, Hi=64, Di=128, Hq=16, Dk=576, Dv=512,
                         ctx_len=[39993 + r for r in range(8)])),
    ("many-rows", dict(B=16, N=20000, k=2048, Hi=64, Di=128, Hq=16, Dk=576, Dv=512)),
    # indexer dims that are a multiple of 16 but not of 32 (the last matrix-core step
    # takes a zero query half)
    ("di-48-one-row", dict(B=1, N=30000, k=1024, Hi=24, Di=48, Hq=4, Dk=64, Dv=64)),
    ("di-80-rows", dict(B=3, N=12000, k=700, Hi=64, Di=80, Hq=16, Dk=576, Dv=512, ctx_len=[12000, 9000, 50])),
    ("di-16", dict(B=1, N=5000, k=256, Hi=1, Di=16, Hq=1, Dk=32, Dv=32)),
    # FP8 E4M3 latent cache with bf16 queries: every matrix-core tiling (one to four
    # 16-head tiles; three or five 16-byte loads per thread) and rows of 32 bytes
    ("fp8-hq64-k4096", dict(B=1, N=50000, k=4096, Hi=64, Di=128, Hq=64, Dk=576, Dv=512, dtype="fp8")),
    ("fp8-dk1024", dict(B=2, N=20000, k=1000, Hi=32, Di=64, Hq=16, Dk=1024, Dv=512, dtype="fp8")),
    ("fp8-hq40-rows", dict(B=3, N=9000, k=2048, Hi=64, Di=128, Hq=40, Dk=192, Dv=128, dtype="fp8",
                           ctx_len=[9000, 4500, 7])),
    ("fp8-dk32", dict(B=1, N=5000, k=256, Hi=4, Di=32, Hq=1, Dk=32, Dv=32, dtype="fp8")),
]


@pytest.mark.parametrize("label,kw", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(torch, dsa, label, kw):
    c = inputs.random_case(zlib.crc32(label.encode()) % 100000, **kw)
    note("edge", label)
    rs, ri, ro = oracle.decode_step(c["iq"], c["iw"], c["ik"], c["q"], c["kv"], c["ctx_len"], c["k"],
                                    c["Dv"], c["scale"])
    d = dev_inputs(torch, c)
    outs = []
    for flags in (0, 1):
        s, i, o, stats = run_step(torch, dsa, c, d, flags)
        check_scores(s, rs, c["ctx_len"], label)
        assert np.array_equal(i, ri), "%s indices differ (flags %d)" % (label, flags)
        check_attention(o, ro, "%s flags %d" % (label, flags))
        # the row record comes from the attention split that holds the kk-th best key
        ties = expected_ties(rs, ri, c["ctx_len"], c["k"])
        for b, st in enumerate(stats):
            kk = min(c["k"], int(c["ctx_len"][b]))
            assert (st["selected"], st["kth_score"], st["tied_at_kth"]) == (kk, int(rs[b, ri[b, kk - 1]]), ties[b]), \
                "%s row %d record %s (flags %d)" % (label, b, st, flags)
            if flags:
                assert st["path"] == 1 and st["reason"] == 1
        outs.append(o)
    assert bits_equal(outs[0], outs[1]), label + ": fast path and exhaustive path outputs differ"


def test_row_longer_than_candidate_pass(torch, dsa):
    # A row of 2^21 + 1,000 positions is longer than the one-row candidate pass takes
    # (256 chunks of at most 8,192 positions): it is scored without candidates and
    # selected by the exhaustive path (reason 3). Small indexer and attention shapes
    # keep the caches at about 200 MB.
    N = (1 << 21) + 1000
    c = inputs.random_case(2121, B=1, N=N, k=2048, Hi=4, Di=32, Hq=2, Dk=64, Dv=64, key_range=3)
    note("long row: N=%d k=2048 Hi=4 Di=32 Hq=2 Dk=64" % N)
    rs, ri, ro = oracle.decode_step(c["iq"], c["iw"], c["ik"], c["q"], c["kv"], c["ctx_len"], c["k"],
                                    c["Dv"], c["scale"])
    d = dev_inputs(torch, c)
    s, i, o, stats = run_step(torch, dsa, c, d)
    check_scores(s, rs, c["ctx_len"], "long row")
    assert np.array_equal(i, ri), "long row indices differ"
    check_attention(o, ro, "long row")
    assert stats[0]["path"] == 1 and stats[0]["reason"] == 3
    assert stats[0]["tied_at_kth"] == expected_ties(rs, ri, c["ctx_len"], c["k"])[0]
