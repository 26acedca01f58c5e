"""dsa_decode_step_noalloc (the static per-device scratch) against dsa_decode_step (a
caller workspace), through the C ABI: identical bytes on two calls in a row, the
second with a smaller input, so the scratch keeps the first call's contents when the
second runs."""
import sys

import numpy as np
import pytest

from sparse_attention_decode_scores_amd import inputs

pytestmark = pytest.mark.gpu


def note(*a):
    print("[no-alloc]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def dev(torch, c):
    d = {}
    for key in ("iq", "iw", "ik"):
        d[key] = torch.from_numpy(np.ascontiguousarray(c[key])).cuda()
    for key in ("q", "kv"):
        a = np.ascontiguousarray(c[key])
        d[key] = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16
                  else torch.from_numpy(a)).cuda()
    return d


def outputs(torch, c):
    scores = torch.full((c["B"], c["N"]), -7, dtype=torch.int32, device="cuda")
    idx = torch.full((c["B"], c["k"]), -7, dtype=torch.int32, device="cuda")
    out = torch.full((c["B"], c["Hq"], c["Dv"]), -7.0, dtype=torch.float32, device="cuda")
    return scores, idx, out


def test_noalloc_matches_workspace_call(torch):
    from sparse_attention_decode_scores_amd import binding
    binding.load_library()
    cases = [inputs.make("ctx16k"),
             inputs.random_case(777, B=3, N=9000, k=1024, Hi=64, Di=128, Hq=16, Dk=576, Dv=512,
                                ctx_len=[9000, 6000, 40])]
    for n, c in enumerate(cases):
        note("call %d: B=%d N=%d k=%d" % (n + 1, c["B"], c["N"], c["k"]))
        d = dev(torch, c)
        ref = binding.dsa_decode_step(d["iq"], d["iw"], d["ik"], d["q"], d["kv"], c["ctx_len"], c["k"],
                                      c["Dv"], c["scale"], *outputs(torch, c))
        got = binding.dsa_decode_step_noalloc(d["iq"], d["iw"], d["ik"], d["q"], d["kv"], c["ctx_len"],
                                              c["k"], c["Dv"], c["scale"], *outputs(torch, c))
        torch.cuda.synchronize()
        for name, a, b in zip(("scores", "idx", "out"), ref, got):
            a, b = a.cpu().numpy(), b.cpu().numpy()
            if name == "scores":  # only positions below each row's ctx_len are written
                for r, m in enumerate(c["ctx_len"]):
                    assert np.array_equal(a[r, :m], b[r, :m]), (n, name, r)
            else:
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (n, name)
        # and the forced exhaustive path on the static scratch
        got = binding.dsa_decode_step_noalloc(d["iq"], d["iw"], d["ik"], d["q"], d["kv"], c["ctx_len"],
                                              c["k"], c["Dv"], c["scale"], *outputs(torch, c),
                                              flags=binding.FLAG_FORCE_FALLBACK)
        torch.cuda.synchronize()
        assert np.array_equal(ref[1].cpu().numpy(), got[1].cpu().numpy()), (n, "fallback idx")
        assert np.array_equal(ref[2].cpu().numpy().view(np.uint8), got[2].cpu().numpy().view(np.uint8)), \
            (n, "fallback out")
