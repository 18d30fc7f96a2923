"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid arguments before launching anything
(no GPU needed: every call here returns before the first HIP call).

The argument-validation tests pass made-up device addresses and rely on the
host checks failing first; on a machine with a visible GPU a regression in a
check would launch kernels on those addresses, so there they are skipped (the
GPU tests exercise the same checks with real buffers)."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                            reason="made-up device addresses: host-only test")

HEADER = os.path.join(ROOT, "include", "kvq.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import rotated_int2_kv_kvq_amd as kvq
    if not os.path.exists(kvq.LIB_PATH):
        pytest.skip("libkvq.so not built")
    return kvq.lib()


def test_header_declares_the_entry_points():
    assert declared_symbols() == sorted([
        "kvq_append", "kvq_append_decode", "kvq_append_decode_window", "kvq_decode_attn",
        "kvq_decode_attn_noalloc", "kvq_decode_attn_staged", "kvq_decode_attn_window",
        "kvq_decode_plan", "kvq_decode_workspace_bytes",
        "kvq_page_bytes", "kvq_status_string", "kvq_window_bytes", "kvq_window_write"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_status_strings_and_page_bytes(lib):
    import rotated_int2_kv_kvq_amd as kvq
    assert kvq.status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5, 7):
        assert kvq.status_string(s)
    assert "scratch" in kvq.status_string(-5)
    assert kvq.page_bytes(128, 128) == 1152
    assert kvq.page_bytes(128, 64) == 1280
    assert kvq.page_bytes(128, 32) == 0
    assert kvq.page_bytes(64, 64) == 0


def test_workspace_bytes(lib):
    import rotated_int2_kv_kvq_amd as kvq
    a = kvq.decode_workspace_bytes(4, 32, 8, 8192)
    b = kvq.decode_workspace_bytes(64, 32, 8, 32768)
    assert 0 < a < b
    assert kvq.decode_workspace_bytes(4, 30, 8, 8192) == 0          # Hq % Hkv
    assert kvq.decode_workspace_bytes(4, 32, 8, 8192, split_pages=12) == 0
    assert kvq.decode_workspace_bytes(4, 32, 8, 8192, split_pages=512) > 0
    assert kvq.decode_workspace_bytes(4, 32, 8, 8192, split_pages=520) == 0  # above 512
    assert kvq.decode_workspace_bytes(4, 32, 8, 8192, head_dim=64) == 0
    assert kvq.decode_workspace_bytes(4, 32, 8, 0) > 0
    # workspace grows with the number of splits
    assert kvq.decode_workspace_bytes(1, 32, 8, 131072, split_pages=8) > \
        kvq.decode_workspace_bytes(1, 32, 8, 131072, split_pages=64)


def test_decode_plan(lib):
    """The host plan query: splits of round(pages / split_pages), at least one
    for a non-empty context; the operand built in the scan only while the grid
    (splits x KV heads x query tiles x batch) is at most 1024 workgroups."""
    import rotated_int2_kv_kvq_amd as kvq
    p = kvq.decode_plan(16, 32, 8, 16384 + 64)
    assert p == {"num_splits": 8, "split_pages": 128, "operand_in_scan": True}   # 1024 WGs
    p = kvq.decode_plan(32, 32, 8, 16384)
    assert p["num_splits"] * 8 * 32 > 1024 and not p["operand_in_scan"]
    p = kvq.decode_plan(4, 32, 8, 1000, split_pages=64)    # 63 pages: one split of 64
    assert p["num_splits"] == 1 and p["split_pages"] == 64 and p["operand_in_scan"]
    p = kvq.decode_plan(4, 32, 8, 1000, split_pages=8)     # 63 / 8 -> 8 splits
    assert p["num_splits"] == 8
    p = kvq.decode_plan(1, 64, 8, 131072)                  # two query tiles per KV head
    assert p["num_splits"] * 8 * 2 <= 1024 and p["operand_in_scan"]
    assert kvq.decode_plan(4, 32, 8, 0)["num_splits"] == 0
    assert not kvq.decode_plan(4, 32, 8, 0)["operand_in_scan"]
    with pytest.raises(kvq.KvqError):
        kvq.decode_plan(4, 30, 8, 8192)                    # Hq % Hkv
    with pytest.raises(kvq.KvqError):
        kvq.decode_plan(4, 32, 8, 8192, head_dim=64)
    # null outputs are allowed
    assert lib.kvq_decode_plan(4, 32, 8, 128, 8192, 0, None, None, None) == 0


def _append(lib, **kw):
    args = dict(pages=1 << 20, num_blocks=4, hkv=8, d=128, g=128, table=1 << 21, maxb=4,
                start=1 << 22, B=1, T=1, k=1 << 23, v=1 << 24, dt=1, mu=1 << 25, rk=1 << 26,
                rv=1 << 27, ck=0.9, cv=0.9)
    args.update(kw)
    return lib.kvq_append(args["pages"], args["num_blocks"], args["hkv"], args["d"], args["g"],
                          args["table"], args["maxb"], args["start"], args["B"], args["T"],
                          args["k"], args["v"], args["dt"], args["mu"], args["rk"], args["rv"],
                          args["ck"], args["cv"], None)


@no_gpu
def test_append_rejects_invalid_arguments(lib):
    assert _append(lib, g=32) == -1
    assert _append(lib, d=64, g=64) == -2
    assert _append(lib, ck=0.0) == -1
    assert _append(lib, cv=1.5) == -1
    assert _append(lib, dt=5) == -1
    assert _append(lib, hkv=0) == -1
    assert _append(lib, k=None) == -1
    assert _append(lib, pages=(1 << 20) + 4) == -1          # misaligned
    assert _append(lib, start=(1 << 22) + 2) == -1           # int32 array alignment
    assert _append(lib, B=0) == 0 and _append(lib, T=0) == 0  # no-ops


def _decode(lib, **kw):
    args = dict(pages=1 << 20, nb=4, hkv=8, d=128, g=128, table=1 << 21, maxb=4, ctx=1 << 22,
                maxctx=64, B=1, hq=32, q=1 << 23, qdt=1, rk=1 << 24, rv=1 << 25, scale=0.088,
                out=1 << 26, ws=1 << 27, wsb=1 << 30, sp=0)
    args.update(kw)
    return lib.kvq_decode_attn(args["pages"], args["nb"], args["hkv"], args["d"], args["g"],
                               args["table"], args["maxb"], args["ctx"], args["maxctx"], args["B"],
                               args["hq"], args["q"], args["qdt"], args["rk"], args["rv"],
                               args["scale"], args["out"], args["ws"], args["wsb"], args["sp"], None)


@no_gpu
def test_decode_rejects_invalid_arguments(lib):
    assert _decode(lib, hq=30) == -1
    assert _decode(lib, maxctx=65) == -1                     # beyond the block table
    assert _decode(lib, maxctx=-1) == -1
    assert _decode(lib, qdt=3) == -1
    assert _decode(lib, sp=4) == -1
    assert _decode(lib, scale=float("nan")) == -1
    assert _decode(lib, out=None) == -1
    assert _decode(lib, d=64, g=64) == -2
    assert _decode(lib, wsb=16) == -3
    assert _decode(lib, ws=None) == -3
    assert _decode(lib, ws=(1 << 27) + 16) == -3             # workspace alignment
    assert _decode(lib, q=(1 << 23) + 4) == -1               # q read as 64-bit words
    assert _decode(lib, out=(1 << 26) + 8) == -1             # out alignment
    assert _decode(lib, ctx=(1 << 22) + 2) == -1             # int32 array alignment
    assert _decode(lib, table=(1 << 21) + 1) == -1
    assert _decode(lib, B=0) == 0
    # staged variant: stage mask is validated first
    base = [1 << 20, 4, 8, 128, 128, 1 << 21, 4, 1 << 22, 64, 1, 32, 1 << 23, 1, 1 << 24, 1 << 25,
            0.088, 1 << 26, 1 << 27, 1 << 30, 0]
    assert lib.kvq_decode_attn_staged(*base, 0, None) == -1
    assert lib.kvq_decode_attn_staged(*base, 8, None) == -1
    bad = list(base)
    bad[10] = 30
    assert lib.kvq_decode_attn_staged(*bad, 7, None) == -1


def _append_decode(lib, **kw):
    args = dict(pages=1 << 20, nb=4, hkv=8, d=128, g=128, table=1 << 21, maxb=4, start=1 << 22,
                ctx=1 << 22, maxctx=64, B=1, k=1 << 23, v=1 << 24, kdt=1, mu=1 << 25, ck=0.9,
                cv=0.9, hq=32, q=1 << 26, qdt=1, rk=1 << 27, rv=1 << 28, scale=0.088, out=1 << 29,
                ws=1 << 30, wsb=1 << 30, sp=0)
    args.update(kw)
    a = args
    return lib.kvq_append_decode(a["pages"], a["nb"], a["hkv"], a["d"], a["g"], a["table"],
                                 a["maxb"], a["start"], a["ctx"], a["maxctx"], a["B"], a["k"],
                                 a["v"], a["kdt"], a["mu"], a["ck"], a["cv"], a["hq"], a["q"],
                                 a["qdt"], a["rk"], a["rv"], a["scale"], a["out"], a["ws"],
                                 a["wsb"], a["sp"], None)


@no_gpu
def test_append_decode_rejects_invalid_arguments(lib):
    # the append's checks
    assert _append_decode(lib, ck=0.0) == -1
    assert _append_decode(lib, kdt=5) == -1
    assert _append_decode(lib, k=None) == -1
    assert _append_decode(lib, mu=(1 << 25) + 4) == -1         # misaligned
    # the decode's checks
    assert _append_decode(lib, hq=30) == -1
    assert _append_decode(lib, maxctx=65) == -1
    assert _append_decode(lib, qdt=3) == -1
    assert _append_decode(lib, sp=520) == -1
    assert _append_decode(lib, out=None) == -1
    assert _append_decode(lib, d=64, g=64) == -2
    assert _append_decode(lib, wsb=16) == -3
    assert _append_decode(lib, B=0) == 0


@no_gpu
def test_window_entry_points_reject_invalid_arguments(lib):
    import rotated_int2_kv_kvq_amd as kvq
    assert kvq.window_bytes(16, 8) == 16 * 8 * 2 * 320 * 128 * 2
    assert kvq.window_bytes(1, 8, head_dim=64) == 0
    w = lib.kvq_window_write
    assert w(None, 8, 128, 1, 1 << 21, 4, 1 << 22, 1 << 23, 1, None) == -1
    assert w(1 << 20, 8, 128, 1, 1 << 21, 4, 1 << 22, 1 << 23, 7, None) == -1   # dtype
    assert w(1 << 20, 8, 64, 1, 1 << 21, 4, 1 << 22, 1 << 23, 1, None) == -2
    assert w(1 << 20, 8, 128, 0, 1 << 21, 4, 1 << 22, 1 << 23, 1, None) == 0    # no-op
    assert w(1 << 20, 8, 128, 1, 1 << 21, 0, 1 << 22, 1 << 23, 1, None) == 0    # no-op
    d = [1 << 20, 4, 8, 128, 128, 1 << 21, 4, 1 << 22, 1 << 23, 1 << 24, 64, 1, 32, 1 << 25, 1,
         1 << 26, 1 << 27, 0.088, 1 << 28, 1 << 29, 1 << 30, 0, None]
    bad = list(d)
    bad[7] = None                                             # window
    assert lib.kvq_decode_attn_window(*bad) == -1
    bad = list(d)
    bad[8] = None                                             # mu
    assert lib.kvq_decode_attn_window(*bad) == -1
    bad = list(d)
    bad[12] = 30                                              # Hq % Hkv
    assert lib.kvq_decode_attn_window(*bad) == -1
    bad = list(d)
    bad[11] = 0                                               # batch 0: no-op
    assert lib.kvq_decode_attn_window(*bad) == 0
    a = [1 << 20, 4, 8, 128, 128, 1 << 21, 4, 1 << 22, 1 << 23, 1 << 23, 64, 1, 1 << 24, 1 << 25, 1,
         1 << 26, 0.9, 0.9, 32, 1 << 27, 1, 1 << 28, 1 << 29, 0.088, 1 << 30, 1 << 31, 1 << 30, 0,
         None]
    bad = list(a)
    bad[7] = None                                             # window
    assert lib.kvq_append_decode_window(*bad) == -1
    bad = list(a)
    bad[16] = 0.0                                             # clip
    assert lib.kvq_append_decode_window(*bad) == -1
    bad = list(a)
    bad[26] = 16                                              # workspace too small
    assert lib.kvq_append_decode_window(*bad) == -3


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """With the library file absent the binding raises; there is no fallback."""
    import rotated_int2_kv_kvq_amd._lib as L
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "libkvq.so"))
    with pytest.raises(RuntimeError, match="not built"):
        L.lib()
    with pytest.raises(RuntimeError, match="not built"):
        L.page_bytes(128, 128)


@no_gpu
def test_noalloc_validates_before_touching_the_device(lib):
    """Invalid arguments are rejected first (no device lookup, no launch); a
    plan larger than the static scratch is KVQ_ERR_SCRATCH."""
    f = lib.kvq_decode_attn_noalloc
    base = [1 << 20, 4, 8, 128, 128, 1 << 21, 4, 1 << 22, 64, 1, 32, 1 << 23, 1, 1 << 24, 1 << 25,
            0.088, 1 << 26, 0, None]
    bad = list(base)
    bad[10] = 30                                              # Hq % Hkv
    assert f(*bad) == -1
    bad = list(base)
    bad[16] = None                                            # out
    assert f(*bad) == -1
    bad = list(base)
    bad[11] = (1 << 23) + 4                                   # q alignment
    assert f(*bad) == -1
    bad = list(base)
    bad[9] = 0                                                # batch 0: no-op
    assert f(*bad) == 0
    big = [1 << 20, 4, 8, 128, 128, 1 << 21, 8192, 1 << 22, 131072, 64, 32, 1 << 23, 1, 1 << 24,
           1 << 25, 0.088, 1 << 26, 8, None]
    assert f(*big) == -5


def test_build_rejects_kernels_with_a_private_segment():
    """build.py's check of the compiler's resource-usage remarks."""
    from rotated_int2_kv_kvq_amd.build import scratch_users
    remarks = """x.hip:1:1: remark: Function Name: _ZN3kvq1aEv [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark: Function Name: _ZN3kvq1bEv [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     ScratchSize [bytes/lane]: 120 [-Rpass-analysis=kernel-resource-usage]
"""
    assert scratch_users(remarks) == ["_ZN3kvq1bEv: 120 bytes/lane"]
