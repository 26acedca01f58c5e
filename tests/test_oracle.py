"""Pins for the CPU oracle, checked against things other than the oracle itself:
hand-worked examples (tests/golden), closed forms, brute force with a different
algorithm (rank counting), a library routine (torch's scaled_dot_product_attention
in float64) and invariants. No GPU is needed."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from sparse_attention_decode_scores_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- indexer scores

def test_hand8_scores():
    g = load_golden("hand8.json")
    iq = np.array(g["iq"], np.int8)
    iw = np.array(g["iw"], np.int8)
    ik = np.array(g["ik"], np.int8)
    s = oracle.index_scores(iq, iw, ik, np.array([8], np.int32))
    assert s[0].tolist() == g["scores"]


def test_zero_query_gives_zero_scores():
    c = inputs.random_case(3, B=2, N=300, k=8, Hi=5, Di=16, Hq=1, Dk=8, Dv=8)
    s = oracle.index_scores(np.zeros_like(c["iq"]), c["iw"], c["ik"], c["ctx_len"])
    assert not s.any()


def test_one_hot_query_reads_one_key_column():
    rng = np.random.default_rng(7)
    ik = rng.integers(-128, 128, size=(257, 32), dtype=np.int8)
    for d in (0, 5, 31):
        iq = np.zeros((1, 1, 32), np.int8)
        iq[0, 0, d] = 1
        s = oracle.index_scores(iq, np.ones((1, 1), np.int8), ik, np.array([257], np.int32))
        assert s[0].tolist() == [max(0, int(v)) for v in ik[:, d]]


def test_relu_then_signed_weights_closed_form():
    # heads +e_d and -e_d with weights a and b: score = a*max(0,x) + b*max(0,-x)
    rng = np.random.default_rng(8)
    ik = rng.integers(-128, 128, size=(100, 4), dtype=np.int8)
    iq = np.zeros((1, 2, 4), np.int8)
    iq[0, 0, 2], iq[0, 1, 2] = 1, -1
    a, b = 3, -7
    s = oracle.index_scores(iq, np.array([[a, b]], np.int8), ik, np.array([100], np.int32))
    x = ik[:, 2].astype(int)
    assert s[0].tolist() == [a * v if v > 0 else b * (-v) for v in x]


def test_scores_per_row_query_and_weights():
    # two rows with different queries/weights must each use their own
    c = inputs.random_case(11, B=2, N=64, k=8, Hi=3, Di=8, Hq=1, Dk=8, Dv=8)
    s = oracle.index_scores(c["iq"], c["iw"], c["ik"], np.array([64, 40], np.int32))
    for b in range(2):
        sb = oracle.index_scores(c["iq"][b:b + 1], c["iw"][b:b + 1], c["ik"],
                                 np.array([64], np.int32))
        n = 64 if b == 0 else 40
        assert (s[b, :n] == sb[0, :n]).all()


def test_scores_invariant_under_head_and_dim_permutations():
    c = inputs.random_case(12, B=1, N=500, k=8, Hi=6, Di=24, Hq=1, Dk=8, Dv=8, qk_range=100,
                           key_range=100, w_range=(-20, 20))
    base = oracle.index_scores(c["iq"], c["iw"], c["ik"], c["ctx_len"])
    rng = np.random.default_rng(0)
    hp, dp = rng.permutation(6), rng.permutation(24)
    perm = oracle.index_scores(c["iq"][:, hp][:, :, dp], c["iw"][:, hp],
                               np.ascontiguousarray(c["ik"][:, dp]), c["ctx_len"])
    assert (base == perm).all()


def test_scores_bigint_brute_force():
    # positions outer, dims-major accumulation in Python integers, full int8 range
    rng = np.random.default_rng(13)
    B, Hi, Di, N = 2, 3, 16, 50
    iq = rng.integers(-128, 128, size=(B, Hi, Di), dtype=np.int8)
    iw = rng.integers(-128, 128, size=(B, Hi), dtype=np.int8)
    ik = rng.integers(-128, 128, size=(N, Di), dtype=np.int8)
    ctx = np.array([50, 17], np.int32)
    s = oracle.index_scores(iq, iw, ik, ctx)
    for b in range(B):
        for p in range(int(ctx[b])):
            dots = [0] * Hi
            for d in range(Di):
                for h in range(Hi):
                    dots[h] += int(iq[b, h, d]) * int(ik[p, d])
            assert s[b, p] == sum(int(iw[b, h]) * (dots[h] if dots[h] > 0 else 0) for h in range(Hi))
        assert not s[b, int(ctx[b]):].any()  # never written past the row's length


def test_scores_overflow_is_reported():
    iq = np.full((1, 64, 128), 127, np.int8)
    ik = np.full((4, 128), 127, np.int8)
    with pytest.raises(ValueError):
        oracle.index_scores(iq, np.full((1, 64), 127, np.int8), ik, np.array([4], np.int32))


# ---------------------------------------------------------------- ordered top-k

def test_hand8_selection():
    g = load_golden("hand8.json")
    s = np.array([g["scores"]], np.int32)
    for case in g["cases"]:
        idx = oracle.topk_select(s, np.array([case["ctx_len"]], np.int32), case["k"])
        assert idx[0].tolist() == case["idx"], case
    idx = oracle.topk_select(s, np.array([8], np.int32), 8)
    assert idx[0].tolist() == g["full_order"]


def rank_count_select(row, n, k):
    """Brute force by rank counting (no sorting): position i is at output slot
    #{j < n: s_j > s_i or (s_j == s_i and j < i)} when that is below k."""
    out = [-1] * k
    for i in range(n):
        r = sum(1 for j in range(n) if row[j] > row[i] or (row[j] == row[i] and j < i))
        if r < k:
            assert out[r] == -1
            out[r] = i
    return out


@pytest.mark.parametrize("seed", range(6))
def test_selection_matches_rank_counting(seed):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(1, 400))
    B = 3
    span = [3, 50, 1 << 30][seed % 3]  # heavy ties, some ties, almost none
    s = rng.integers(-span, span, size=(B, N)).astype(np.int32)
    ctx = rng.integers(1, N + 1, size=B).astype(np.int32)
    for k in (1, 7, 64, 512):
        idx = oracle.topk_select(s, ctx, k)
        for b in range(B):
            assert idx[b].tolist() == rank_count_select(s[b].tolist(), int(ctx[b]), k)


def test_all_equal_scores_give_first_positions():
    s = np.zeros((1, 5000), np.int32)
    idx = oracle.topk_select(s, np.array([5000], np.int32), 2048)
    assert idx[0].tolist() == list(range(2048))


def test_length_at_most_k_returns_every_position():
    rng = np.random.default_rng(5)
    s = rng.integers(0, 1000, size=(1, 2048)).astype(np.int32)
    idx = oracle.topk_select(s, np.array([2048], np.int32), 2048)
    assert sorted(idx[0].tolist()) == list(range(2048))
    idx = oracle.topk_select(s, np.array([1000], np.int32), 2048)
    assert sorted(idx[0, :1000].tolist()) == list(range(1000))
    assert (idx[0, 1000:] == -1).all()


def test_selection_order_properties_on_workload():
    c = inputs.make("tiny_4k")
    s = oracle.index_scores(c["iq"], c["iw"], c["ik"], c["ctx_len"])
    idx = oracle.topk_select(s, c["ctx_len"], c["k"])[0]
    sel = s[0, idx]
    assert (np.diff(sel) <= 0).all()
    for a, b in zip(idx[:-1], idx[1:]):
        if s[0, a] == s[0, b]:
            assert a < b
    last = (int(s[0, idx[-1]]), -int(idx[-1]))
    chosen = set(idx.tolist())
    for p in range(c["N"]):
        if p not in chosen:
            assert (int(s[0, p]), -p) < last


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("case", load_golden("attn_closed_forms.json")["cases"],
                         ids=lambda c: c["name"])
def test_attention_closed_forms(case):
    q = np.array([[case["q"]]], np.float32)
    kv = np.array(case["kv"], np.float32)
    idx = np.array([case["idx"]], np.int32)
    out = oracle.sparse_attn(q, kv, idx, case["Dv"], case["scale"])
    assert np.abs(out[0, 0] - np.array(case["out"])).max() <= case["tol"]


def test_identical_rows_give_that_row():
    rng = np.random.default_rng(2)
    row = rng.standard_normal(40).astype(np.float32)
    kv = np.stack([row] * 6 + [rng.standard_normal(40).astype(np.float32)])
    q = rng.standard_normal((1, 3, 40)).astype(np.float32)
    out = oracle.sparse_attn(q, kv, np.array([[0, 1, 2, 3, 4, 5]], np.int32), 32, 0.7)
    assert np.abs(out[0] - row[:32].astype(np.float64)).max() < 1e-12


def sdpa64(q, kv, rows, Dv, scale):
    import torch
    qt = torch.from_numpy(np.asarray(q, np.float64))[None]              # [1, H, Dk]
    k = torch.from_numpy(np.asarray(kv[rows], np.float64))[None, None]   # [1, 1, n, Dk]
    v = k[..., :Dv].contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(
        qt[:, :, None, :], k.expand(1, qt.shape[1], -1, -1), v.expand(1, qt.shape[1], -1, -1),
        scale=scale)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_matches_torch_sdpa_over_whole_context(dtype):
    # n <= k: the selection is every position, so the result is dense attention
    c = inputs.random_case(21, B=2, N=300, k=512, Hi=2, Di=16, Hq=4, Dk=72, Dv=64, dtype=dtype)
    idx = np.tile(np.arange(512, dtype=np.int32), (2, 1))
    idx[:, 300:] = -1
    out = oracle.sparse_attn(c["q"], c["kv"], idx, 64, c["scale"])
    qf = c["q"] if dtype == "f32" else inputs.bf16_bits_to_f32(c["q"])
    kvf = c["kv"] if dtype == "f32" else inputs.bf16_bits_to_f32(c["kv"])
    for b in range(2):
        ref = sdpa64(qf[b], kvf, np.arange(300), 64, c["scale"])
        assert np.abs(out[b] - ref).max() < 1e-12


# ---------------------------------------------------------------- FP8 E4M3 latent cache

def test_e4m3_decode_closed_forms():
    # from the format's definition (1 sign, 4 exponent bits, bias 7, 3 mantissa bits,
    # no infinities, all-ones exponent and mantissa = NaN)
    v = oracle.e4m3_to_f64(np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x40, 0x7E, 0xFE, 0xB8,
                                     0x7F, 0xFF, 0x78], np.uint8))
    assert v[0] == 0.0 and not np.signbit(v[0]) and v[1] == 0.0 and np.signbit(v[1])
    assert v[2] == 2.0 ** -9 and v[3] == 7 * 2.0 ** -9       # subnormals m * 2^-9
    assert v[4] == 2.0 ** -6                                 # smallest normal
    assert v[5] == 1.0 and v[6] == 1.5 and v[7] == 2.0
    assert v[8] == 448.0 and v[9] == -448.0 and v[10] == -1.0
    assert np.isnan(v[11]) and np.isnan(v[12])
    assert v[13] == 256.0                                    # exponent 15 is finite below m = 7


def test_e4m3_decode_matches_torch_on_every_code():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_fp8_cache_attention_equals_fp32_attention_on_the_decoded_values():
    # bf16 queries and e4m3 cache codes are exact in fp32, so the fp8 path must equal
    # the fp32 path given the decoded values, bit for bit
    c = inputs.random_case(41, B=2, N=900, k=256, Hi=2, Di=16, Hq=5, Dk=96, Dv=64, dtype="fp8")
    assert c["q"].dtype == np.uint16 and c["kv"].dtype == np.uint8
    rng = np.random.default_rng(42)
    idx = rng.choice(900, size=(2, 256), replace=False).astype(np.int32)
    idx[1, 200:] = -1
    out = oracle.sparse_attn(c["q"], c["kv"], idx, c["Dv"], c["scale"])
    q32 = inputs.bf16_bits_to_f32(c["q"])
    kv32 = oracle.e4m3_to_f64(c["kv"]).astype(np.float32)
    assert np.array_equal(kv32.astype(np.float64), oracle.e4m3_to_f64(c["kv"]))
    assert np.array_equal(out, oracle.sparse_attn(q32, kv32, idx, c["Dv"], c["scale"]))


def test_fp8_workload_shares_the_bf16_workload_draws():
    # ctx16k_fp8kv: the ctx16k seed, so the same indexer inputs and queries, and the
    # cache is the e4m3 rounding of the same normal draws (within e4m3's half step)
    a, b = inputs.make("ctx16k"), inputs.make("ctx16k_fp8kv")
    for key in ("iq", "iw", "ik", "q"):
        assert np.array_equal(a[key], b[key])
    x = inputs.bf16_bits_to_f32(a["kv"][:2048]).astype(np.float64)
    y = oracle.e4m3_to_f64(b["kv"][:2048])
    # e4m3 rounds the draw within half a step (2^-4 relative, 2^-10 absolute below 2^-6),
    # bf16 within 2^-9 relative
    assert np.all(np.abs(y - x) <= np.abs(x) * (2.0 ** -4 + 2.0 ** -8) + 2.0 ** -10)


def test_attention_permutation_invariance_and_minus_one_skipping():
    c = inputs.make("tiny_4k")
    rng = np.random.default_rng(4)
    idx = rng.choice(c["N"], size=(1, 256), replace=False).astype(np.int32)
    out = oracle.sparse_attn(c["q"], c["kv"], idx, c["Dv"], c["scale"])
    perm = idx[:, rng.permutation(256)]
    out2 = oracle.sparse_attn(c["q"], c["kv"], perm, c["Dv"], c["scale"])
    assert np.abs(out - out2).max() < 1e-12
    padded = np.concatenate([idx[:, :100], -np.ones((1, 156), np.int32)], axis=1)
    out3 = oracle.sparse_attn(c["q"], c["kv"], padded, c["Dv"], c["scale"])
    ref = sdpa64(c["q"][0], c["kv"], idx[0, :100], c["Dv"], c["scale"])
    assert np.abs(out3[0] - ref).max() < 1e-12


def test_attention_rejects_out_of_range_index():
    q = np.zeros((1, 1, 4), np.float32)
    kv = np.zeros((5, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.sparse_attn(q, kv, np.array([[5]], np.int32), 4, 1.0)


# ---------------------------------------------------------------- whole step

def test_decode_step_on_hand8_example():
    g = load_golden("hand8.json")
    iq = np.array(g["iq"], np.int8)
    iw = np.array(g["iw"], np.int8)
    ik = np.array(g["ik"], np.int8)
    rng = np.random.default_rng(9)
    kv = rng.standard_normal((8, 6)).astype(np.float32)
    q = rng.standard_normal((1, 2, 6)).astype(np.float32)
    scores, idx, out = oracle.decode_step(iq, iw, ik, q, kv, np.array([8], np.int32), 3, 4, 0.5)
    assert scores[0].tolist() == g["scores"]
    assert idx[0].tolist() == [2, 6, 3]
    ref = sdpa64(q[0], kv, np.array([2, 6, 3]), 4, 0.5)
    assert np.abs(out[0] - ref).max() < 1e-12


def test_workload_generator_is_deterministic():
    a, b = inputs.make("tiny_4k"), inputs.make("tiny_4k")
    for key in ("iq", "iw", "ik", "q", "kv", "ctx_len"):
        assert (a[key] == b[key]).all()
    assert inputs.ctx_lengths("verify8_ctx131k").tolist() == [131065 + r for r in range(8)]
    assert inputs.ctx_lengths("verify16_ctx131k").tolist() == [131057 + r for r in range(16)]


def test_openmp_build_gives_identical_results():
    # the all-core build (same source, -fopenmp) splits independent loops only
    c = inputs.random_case(31, B=2, N=6000, k=512, Hi=16, Di=64, Hq=6, Dk=96, Dv=64, ctx_len=[6000, 3333])
    args = (c["iq"], c["iw"], c["ik"], c["q"], c["kv"], c["ctx_len"], c["k"], c["Dv"], c["scale"])
    a = oracle.decode_step(*args)
    b = oracle.decode_step(*args, omp=True)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    with pytest.raises(ValueError):  # 64 heads x 128 dims of 127s overflow int32
        oracle.index_scores(np.full((1, 64, 128), 127, np.int8), np.full((1, 64), 127, np.int8),
                            np.full((10, 128), 127, np.int8), np.array([10], np.int32), omp=True)


# ---------------------------------------------------------------- paged caches

def test_gather_pages_hand_example():
    # three pool pages of 4 rows; the sequence's logical pages are pool pages 2 then 0,
    # and it holds 7 positions: rows 8..11 of the pool, then rows 0..2
    pool = np.arange(12, dtype=np.int32).reshape(12, 1)
    got = oracle.gather_pages(pool, np.array([2, 0], np.int32), 7, page=4)
    assert got[:, 0].tolist() == [8, 9, 10, 11, 0, 1, 2]


@pytest.mark.parametrize("N", [1, 255, 256, 257, 3000])
def test_gather_pages_reads_whole_pages_in_table_order(N):
    # every pool row holds its own row number; the gathered cache must be the table's
    # pages laid end to end (256 consecutive rows each), cut at N
    pages = 17
    pool = np.stack([np.arange(pages * 256, dtype=np.int64), -np.arange(pages * 256, dtype=np.int64)], axis=1)
    table = np.random.default_rng(N).permutation(pages)[:(N + 255) // 256].astype(np.int32)
    expect = np.concatenate([np.arange(256 * p, 256 * p + 256) for p in table])[:N]
    got = oracle.gather_pages(pool, table, N)
    assert got[:, 0].tolist() == expect.tolist()
    assert (got[:, 1] == -got[:, 0]).all()


def test_gather_pages_rejects_entries_outside_the_pool():
    pool = np.zeros((512, 4), np.int8)
    for bad in (-1, 2):
        with pytest.raises(ValueError):
            oracle.gather_pages(pool, np.array([0, bad], np.int32), 300)


def test_paged_step_equals_step_on_the_described_cache():
    # pages scattered over a pool whose other rows are decoys: the paged step is the
    # contiguous step on the cache the table describes, and an identity table over a
    # pool that is the cache itself changes nothing
    c = inputs.random_case(41, B=2, N=1000, k=128, Hi=8, Di=32, Hq=4, Dk=64, Dv=32, dtype="f32",
                           ctx_len=[1000, 617])
    args = (c["q"], c["ctx_len"], c["k"], c["Dv"], c["scale"])
    ref = oracle.decode_step(c["iq"], c["iw"], c["ik"], c["q"], c["kv"], *args[1:])
    p = inputs.paged(c, seed=5)
    got = oracle.decode_step_paged(c["iq"], c["iw"], p["ik_pool"], c["q"], p["kv_pool"], p["page_table"],
                                   *args[1:], N=c["N"])
    for x, y in zip(ref, got):
        assert np.array_equal(x, y)
    # the identity table over the (whole-page) cache itself
    ik = np.concatenate([c["ik"], np.zeros((24, 32), np.int8)])
    kv = np.concatenate([c["kv"], np.zeros((24, 64), np.float32)])
    ident = oracle.decode_step_paged(c["iq"], c["iw"], ik, c["q"], kv, np.arange(4, dtype=np.int32),
                                     *args[1:], N=c["N"])
    for x, y in zip(ref, ident):
        assert np.array_equal(x, y)


def test_paged_inputs_place_every_page_once():
    c = inputs.make("tiny_4k")
    p = inputs.paged(c)
    t = p["page_table"]
    assert len(set(t.tolist())) == len(t) == 16 and p["pool_pages"] == 35
    assert t.min() >= 0 and t.max() < p["pool_pages"]
    # pool pages the sequence does not own hold only decoys (latent rows of 8.0)
    free = sorted(set(range(p["pool_pages"])) - set(t.tolist()))
    assert (p["kv_pool"].reshape(p["pool_pages"], 256, -1)[free] == 8.0).all()
