"""Host-side pieces of bench.py that run without a GPU: the oracle's CPU
baseline (one BLAS thread, then one per core) on a tiny cache."""
from types import SimpleNamespace

import numpy as np
import torch

import bench
import oracle as O


def _tiny_cache(batch=2, n=40, hkv=2, hq=8, group=64, seed=5):
    rng = np.random.default_rng(seed)
    d = O.HEAD_DIM
    n_pages = (n + 15) // 16
    table = rng.permutation(batch * n_pages).astype(np.int32).reshape(batch, n_pages)
    cache = np.zeros((batch * n_pages, hkv * O.page_bytes(d, group)), np.uint8)
    rot = np.stack([np.linalg.qr(rng.standard_normal((d, d)))[0] for _ in range(hkv)])
    k = rng.standard_normal((batch, n, hkv, d))
    v = rng.standard_normal((batch, n, hkv, d))
    mu = k.mean(axis=(0, 1))
    O.append(cache, table, np.zeros(batch, np.int64), k, v, mu, rot, rot, group, 0.9, 0.9)
    w = SimpleNamespace(batch=batch, num_kv_heads=hkv, num_q_heads=hq, group=group)
    st = SimpleNamespace(rot_k=[rot], rot_v=[rot])
    q = torch.from_numpy(rng.standard_normal((batch, hq, d)).astype(np.float32))
    ctx = torch.full((batch,), n, dtype=torch.int32)
    return w, st, torch.from_numpy(cache), torch.from_numpy(table), ctx, q


def test_cpu_baseline_fields():
    w, st, pages, table, ctx, q = _tiny_cache()
    per = bench.cache_bytes_per_token_head(w.group)
    # two (layer, step) samples of the same layer-0 cache
    samples = [(0, 5, pages, ctx, q), (0, 7, pages, ctx - 3, q)]
    res = bench.cpu_baseline(w, st, samples, table, per, 0.3, 1.0 / np.sqrt(O.HEAD_DIM))
    assert res["kind"] == "oracle" and res["unit"] == "GB/s" and res["cores"] == 1
    assert res["value"] > 0 and "1 thread;" in res["sample"]
    assert "layer 0 step 5, layer 0 step 7" in res["sample"]
    assert isinstance(res["cpu_model"], str) and res["cpu_model"]
    import os
    if (os.cpu_count() or 1) > 1:
        allc = res["all_cores"]
        assert allc["cores"] == min(os.cpu_count(), 16) and allc["value"] > 0


def test_bits_and_context_fields():
    assert bench.bits_per_element(128) == 2.25 and bench.bits_per_element(64) == 2.5
    w = SimpleNamespace(group=128)
    ctx = bench.pages_context(w, np.array([16384]), 72, {"overhead_pct": {"x": 1.0}})
    figs = {f["figure"]: f["value"] for f in ctx["pages"]}
    assert figs["decode speed-up vs BF16 FlashDecoding-v2"] == "up to 3.0x"
    assert figs["effective bits per cache element"] == 2.32
    tb = ctx["this_library"]
    assert tb["bits_per_element"] == 2.25 and tb["prefill_overhead_pct"] == {"x": 1.0}
    # 16,064 body tokens at 2.25 bits and 320 window tokens at 16 bits over 16,384
    assert abs(tb["bits_per_element_with_bf16_windows"] - (16064 * 2.25 + 320 * 16) / 16384) < 1e-4


def test_traffic_summary_filters_kernel_and_grid(tmp_path):
    """The counter summary averages only the named kernel's dispatches on the
    timed grid, and scales each counter by the copy kernel's known bytes."""
    from rotated_int2_kv_kvq_amd import traffic

    def write(path, counter, rows):
        with open(path, "w") as f:
            f.write("Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n")
            for name, grid, val in rows:
                f.write(f'"{name}",{grid},{counter},{val}\n')

    scan = "void kvq::split_kernel<1, false, false, true>(int)"
    other = "void kvq::split_kernel<1, false, false, false>(int)"
    copy = "void at::native::neg_kernel(int)"
    fetch, write_ = tmp_path / "f.csv", tmp_path / "w.csv"
    # copy of 2048 bytes: FETCH reads 1 KiB (factor 2), WRITE 2 KiB (factor 1)
    write(fetch, "FETCH_SIZE", [(copy, 4096, 1.0), (scan, 1024 * 256, 10.0),
                                (scan, 1024 * 256, 14.0), (scan, 1152 * 256, 99.0),
                                (other, 1024 * 256, 99.0)])
    write(write_, "WRITE_SIZE", [(copy, 4096, 2.0), (scan, 1024 * 256, 3.0),
                                 (scan, 1152 * 256, 99.0)])
    res = traffic.summarize(str(fetch), str(write_), 2048, 1000.0,
                            "split_kernel<1, false, false, true>", 1024 * 256)
    assert res["dispatches"]["fetch"] == 2 and res["dispatches"]["write"] == 1
    assert res["fetch_bytes"] == 12.0 * 1024 * 2
    assert res["write_bytes"] == 3.0 * 1024
    assert res["traffic_over_algorithmic"] == (12.0 * 2048 + 3.0 * 1024) / 1000.0
    # no grid given: every dispatch of the kernel
    res_all = traffic.summarize(str(fetch), str(write_), 2048, 1000.0,
                                "split_kernel<1, false, false, true>")
    assert res_all["dispatches"]["fetch"] == 3


def test_kernel_source_hash_ignores_comments_only():
    """The recorded traffic stays valid across comment edits, not code edits."""
    from rotated_int2_kv_kvq_amd.traffic import _code_only

    base = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    assert _code_only(base) == _code_only("/* doc */\nint f(int x) {\n\n    return x + 1;\n}\n")
    assert _code_only(base) != _code_only(base.replace("x + 1", "x + 2"))
