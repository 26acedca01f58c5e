"""Host-side checks of the C ABI: the library loads, exports every function that
include/dsa.h declares, and rejects bad arguments before touching the GPU (these
calls return from the validators, so no device is needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

from sparse_attention_decode_scores_amd import binding  # noqa: E402

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x100000  # an aligned, never dereferenced stand-in for a device pointer


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.skip("libdsa.so not built")
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dsa_status|size_t|const char\*)\s+(dsa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert binding.dsa_status_string(0) == "DSA_OK"
    for code in (1, 2, 3, 4):
        assert binding.dsa_status_string(code).startswith(binding.STATUS_NAMES[code])
    assert "unknown" in binding.dsa_status_string(99)


def test_workspace_size(lib):
    ws = binding.dsa_workspace_size
    assert ws(0, 100, 8) == 0 and ws(17, 100, 8) == 0 and ws(1, 0, 8) == 0
    assert ws(1, 100, 0) == 0 and ws(1, 100, 4097) == 0 and ws(1, 1 << 31, 8) == 0
    a, b = ws(1, 16384, 2048, 16, 512), ws(1, 300000, 2048, 16, 512)
    # the workspace does not grow with the context (no full-row scratch)
    assert 0 < a == b == ws(1, (1 << 31) - 1, 2048, 16, 512)
    assert ws(8, 131072, 2048, 16, 512) > ws(1, 131072, 2048, 16, 512)
    assert a % 256 == 0


def lens(*v):
    arr = (ctypes.c_int32 * len(v))(*v)
    return ctypes.cast(arr, ctypes.c_void_p), arr


def scores_call(lib, B=1, Hi=64, Di=128, N=1000, ctx=None, iq=FAKE, ik=FAKE, out=FAKE):
    p, keep = lens(*(ctx or [N] * B))
    return lib.dsa_index_scores(iq, FAKE, ik, p, B, Hi, Di, N, out, None)


def test_index_scores_validation(lib):
    assert scores_call(lib, B=0) == INVALID
    assert scores_call(lib, B=17, ctx=[10] * 17) == INVALID
    assert scores_call(lib, Hi=0) == INVALID
    assert scores_call(lib, Di=40) == INVALID and scores_call(lib, Di=8) == INVALID
    # valid shapes that no built kernel covers
    assert scores_call(lib, Hi=65) == UNSUPPORTED and scores_call(lib, Di=288) == UNSUPPORTED
    assert scores_call(lib, ctx=[0]) == INVALID and scores_call(lib, ctx=[1001]) == INVALID
    assert scores_call(lib, iq=None) == INVALID and scores_call(lib, out=None) == INVALID
    assert scores_call(lib, ik=FAKE + 8) == INVALID  # keys must be 16-byte aligned
    p, keep = lens(10)
    assert lib.dsa_index_scores(FAKE, FAKE, FAKE, None, 1, 64, 128, 1000, FAKE, None) == INVALID


def topk_call(lib, k=2048, ws_bytes=None, flags=0, N=20000, ctx=None, B=1, ws=FAKE):
    p, keep = lens(*(ctx or [N] * B))
    need = binding.dsa_workspace_size(B, N, max(1, min(k, 4096)), 1, 1)
    return lib.dsa_topk_select(FAKE, p, B, N, k, FAKE, ws, need if ws_bytes is None else ws_bytes,
                               flags, None)


def test_topk_validation(lib):
    assert topk_call(lib, k=0) == INVALID and topk_call(lib, k=4097) == INVALID
    assert topk_call(lib, flags=2) == INVALID
    assert topk_call(lib, ctx=[20001]) == INVALID
    assert topk_call(lib, ws=None) == WORKSPACE
    assert topk_call(lib, ws=FAKE + 16) == WORKSPACE  # 256-byte alignment
    assert topk_call(lib, ws_bytes=1024) == WORKSPACE


def attn_call(lib, Hq=16, Dk=576, Dv=512, dt=1, scale=1 / 24, k=2048, N=20000, ws_bytes=None,
              q=FAKE):
    need = binding.dsa_workspace_size(1, N, k, Hq, max(1, Dv))
    return lib.dsa_sparse_attn(q, FAKE, FAKE, 1, Hq, Dk, Dv, N, k, scale, dt, FAKE, FAKE,
                               need if ws_bytes is None else ws_bytes, None)


def test_attention_validation(lib):
    assert attn_call(lib, Hq=0) == INVALID and attn_call(lib, Dk=100, Dv=64) == INVALID
    assert attn_call(lib, Dv=600) == INVALID and attn_call(lib, Dk=0, Dv=1) == INVALID
    assert attn_call(lib, dt=7) == INVALID
    assert attn_call(lib, scale=float("inf")) == INVALID and attn_call(lib, scale=float("nan")) == INVALID
    assert attn_call(lib, q=FAKE + 4) == INVALID
    assert attn_call(lib, q=None) == INVALID
    # valid shapes that no built kernel covers
    assert attn_call(lib, Hq=64, Dk=1000, Dv=500) == UNSUPPORTED
    assert attn_call(lib, Hq=65) == UNSUPPORTED and attn_call(lib, Dk=2048, Dv=512) == UNSUPPORTED
    assert attn_call(lib, ws_bytes=100) == WORKSPACE
    # bf16 queries with an FP8 E4M3 cache (dt 2): matrix-core shapes only; a valid shape
    # passes validation and stops at the short workspace (nothing is launched)
    assert attn_call(lib, dt=2, ws_bytes=100) == WORKSPACE
    assert attn_call(lib, dt=2, Hq=6, Dk=80, Dv=40) == UNSUPPORTED
    assert attn_call(lib, dt=2, Hq=65) == UNSUPPORTED
    assert attn_call(lib, dt=3) == INVALID


def test_decode_step_validation(lib):
    p, keep = lens(300000)
    need = binding.dsa_workspace_size(1, 300000, 2048, 16, 512)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, p, 1, 64, 128, 16, 576, 512, 300000, 2048, 1 / 24, 1,
            FAKE, FAKE, FAKE, FAKE, need, 0, None]
    bad = list(args)
    bad[13] = 0  # k
    assert lib.dsa_decode_step(*bad) == INVALID
    bad = list(args)
    bad[8] = 100  # Di
    assert lib.dsa_decode_step(*bad) == INVALID
    bad = list(args)
    bad[20] = need - 1
    assert lib.dsa_decode_step(*bad) == WORKSPACE
    # Di = 48 (a multiple of 16) passes the indexer checks: the short workspace is
    # what the call reports (and nothing is launched on these stand-in pointers)
    bad[8] = 48
    assert lib.dsa_decode_step(*bad) == WORKSPACE
    bad[7] = 65  # Hi beyond the built kernels
    assert lib.dsa_decode_step(*bad) == UNSUPPORTED
    bad = list(args)
    bad[21] = 8  # unknown flag
    assert lib.dsa_decode_step(*bad) == INVALID
    bad[21] = 2  # the table-in-memory flag is for paged calls only
    assert lib.dsa_decode_step(*bad) == INVALID


def test_paged_validation(lib):
    # every call below is rejected by the host checks (a short workspace where the
    # paging arguments pass), so nothing is launched on the stand-in pointers
    p, keep = lens(300000)
    need = binding.dsa_workspace_size(1, 300000, 2048, 16, 512)
    step = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2400, p, 1, 64, 128, 16, 576, 512, 300000, 2048, 1 / 24, 1,
            FAKE, FAKE, FAKE, FAKE, need - 1, 0, None, None]

    def run(**kw):
        a = list(step)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.dsa_decode_step_paged(*a)

    assert run() == WORKSPACE           # paging accepted; the short workspace stops it
    assert run(a5=None) == INVALID      # no page table
    assert run(a5=FAKE + 2) == INVALID  # misaligned table
    assert run(a6=0) == INVALID         # empty pool
    assert run(a6=(1 << 31) // 256) == UNSUPPORTED  # pool rows beyond int32
    assert run(a6=65536) == UNSUPPORTED  # 65,536 pages x 256 x 128 B of keys reach 2^31
    assert run(a14=8192 * 256 + 1) == UNSUPPORTED  # beyond DSA_MAX_PAGES pages
    assert run(a14=8192 * 256) == WORKSPACE          # the largest paged sequence passes
    assert run(a23=2) == WORKSPACE                   # the table-in-memory testing flag
    assert run(a23=4) == INVALID                     # an unknown flag

    def scores(**kw):
        a = [FAKE, FAKE, FAKE, FAKE, 2400, p, 1, 64, 128, 300000, FAKE, None]
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.dsa_index_scores_paged(*a)

    assert scores(a3=None) == INVALID
    assert scores(a4=0) == INVALID
    assert scores(a4=65536) == UNSUPPORTED
    assert scores(a9=8192 * 256 + 1) == UNSUPPORTED
    assert scores(a8=100) == INVALID  # Di

    def attn(**kw):
        a = [FAKE, FAKE, FAKE, 2400, FAKE, 1, 16, 576, 512, 300000, 2048, 1 / 24, 1, FAKE, FAKE, need - 1, None]
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.dsa_sparse_attn_paged(*a)

    assert attn() == WORKSPACE
    assert attn(a3=65536) == WORKSPACE  # the latent pool has no 2^31-byte offset limit
    assert attn(a2=None) == INVALID
    assert attn(a3=-1) == INVALID
    assert attn(a9=8192 * 256 + 1) == UNSUPPORTED


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    # B=16, k=4096, 64 heads x 512 values needs far more than the static scratch: a clear
    # workspace error before anything touches the device (the stand-in pointers are
    # never read)
    p, keep = lens(*([300000] * 16))
    rc = lib.dsa_decode_step_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, p, 16, 64, 128, 64, 576, 512, 300000,
                                     4096, 1 / 24, 1, FAKE, FAKE, FAKE, 0, None)
    assert rc == WORKSPACE
    assert binding.dsa_workspace_size(16, 300000, 4096, 64, 512) > 64 << 20
    rc = lib.dsa_decode_step_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, p, 16, 64, 128, 64, 576, 512, 300000,
                                     0, 1 / 24, 1, FAKE, FAKE, FAKE, 0, None)
    assert rc == INVALID


def test_read_stats_validation(lib):
    arr = (binding.RowStats * 2)()
    assert lib.dsa_read_stats(None, 4096, 1, ctypes.cast(arr, ctypes.c_void_p), None) == INVALID
    assert lib.dsa_read_stats(FAKE, 4096, 0, ctypes.cast(arr, ctypes.c_void_p), None) == INVALID
    assert lib.dsa_read_stats(FAKE, 8, 2, ctypes.cast(arr, ctypes.c_void_p), None) == WORKSPACE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(binding.DSAError):
        binding.load_library()
