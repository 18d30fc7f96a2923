"""Host-side checks of the Python binding: wrong dtypes, shapes, page sizes
and head counts raise ValueError before any pointer reaches the library.

The checks run on host tensors: dtype and shape are validated before the
device, so every case below fails on the argument it names (a host tensor with
the right dtype and shape is then rejected as not on the device)."""
import pytest
import torch

import rotated_int2_kv_kvq_amd as kvq


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import os
    if not os.path.exists(kvq.LIB_PATH):
        pytest.skip("libkvq.so not built")


B, HKV, HQ, D = 2, 2, 8, 128


def _append_args(**kw):
    a = dict(pages=torch.zeros(8, HKV, 1152, dtype=torch.uint8),
             block_table=torch.zeros(B, 4, dtype=torch.int32),
             start_pos=torch.zeros(B, dtype=torch.int32),
             k=torch.zeros(B, 3, HKV, D, dtype=torch.bfloat16),
             v=torch.zeros(B, 3, HKV, D, dtype=torch.bfloat16),
             mu=torch.zeros(HKV, D), rot_k=torch.zeros(HKV, D, D), rot_v=torch.zeros(HKV, D, D),
             group=128, clip_k=0.9, clip_v=0.9)
    a.update(kw)
    return a


def _decode_args(**kw):
    a = dict(pages=torch.zeros(8, HKV, 1152, dtype=torch.uint8),
             block_table=torch.zeros(B, 4, dtype=torch.int32),
             ctx_len=torch.zeros(B, dtype=torch.int32), max_ctx_len=64,
             q=torch.zeros(B, HQ, D, dtype=torch.bfloat16), rot_k=torch.zeros(HKV, D, D),
             rot_v=torch.zeros(HKV, D, D), group=128)
    a.update(kw)
    return a


@pytest.mark.parametrize("bad, match", [
    (dict(block_table=torch.zeros(B, 4, dtype=torch.int64)), "block_table must be torch.int32"),
    (dict(start_pos=torch.zeros(B, dtype=torch.int64)), "start_pos must be torch.int32"),
    (dict(pages=torch.zeros(8, HKV, 1152, dtype=torch.int8)), "pages must be torch.uint8"),
    (dict(mu=torch.zeros(HKV, D, dtype=torch.float64)), "mu must be torch.float32"),
    (dict(rot_k=torch.zeros(HKV, D, D, dtype=torch.float64)), "rot_k must be torch.float32"),
    (dict(rot_v=torch.zeros(HKV, D, D, dtype=torch.bfloat16)), "rot_v must be torch.float32"),
    (dict(k=torch.zeros(B, 3, HKV, D, dtype=torch.float16)), "k must be"),
    (dict(v=torch.zeros(B, 3, HKV, D, dtype=torch.float32)), "v must be torch.bfloat16"),
    (dict(group=64), "a group-64 page is 1280 bytes"),
    (dict(k=torch.zeros(B, 3, HKV + 1, D, dtype=torch.bfloat16)), "k must have shape"),
    (dict(start_pos=torch.zeros(B + 1, dtype=torch.int32)), "start_pos must have shape"),
    (dict(rot_k=torch.zeros(HKV + 1, D, D)), "rot_k must have shape"),
    (dict(block_table=torch.zeros(B - 1, 4, dtype=torch.int32)), "rows for a batch"),
    ({}, "must be a device tensor"),
])
def test_append_binding_rejects(bad, match):
    with pytest.raises(ValueError, match=match):
        kvq.append(**_append_args(**bad))


@pytest.mark.parametrize("bad, match", [
    (dict(ctx_len=torch.zeros(B, dtype=torch.int64)), "ctx_len must be torch.int32"),
    (dict(q=torch.zeros(B, HQ, D, dtype=torch.float16)), "q must be"),
    (dict(q=torch.zeros(B, HQ + 1, D, dtype=torch.bfloat16)), "do not group"),
    (dict(out=torch.zeros(B, HQ, D, dtype=torch.bfloat16)), "out must be torch.float32"),
    (dict(out=torch.zeros(B, HQ, D + 1)), "out must have shape"),
    (dict(workspace=torch.zeros(16, dtype=torch.float32)), "workspace must be torch.uint8"),
    (dict(workspace=torch.zeros(16, dtype=torch.uint8)), "the call needs"),
    (dict(pages=torch.zeros(8, HKV, 1280, dtype=torch.uint8)), "a group-128 page is 1152"),
    (dict(max_ctx_len=64, split_pages=12), "no decode plan"),
    ({}, "must be a device tensor"),
])
def test_decode_binding_rejects(bad, match):
    with pytest.raises(ValueError, match=match):
        kvq.decode(**_decode_args(**bad))


def test_window_binding_rejects():
    a = _decode_args()
    a.pop("max_ctx_len")
    win = torch.zeros(B, HKV, 2, 320, D, dtype=torch.float32)
    with pytest.raises(ValueError, match="window must be torch.bfloat16"):
        kvq.decode_window(window=win, mu=torch.zeros(HKV, D), max_ctx_len=64, **a)
    with pytest.raises(ValueError, match="mu must be torch.float32"):
        kvq.decode_window(window=win.bfloat16(), mu=torch.zeros(HKV, D, dtype=torch.float64),
                          max_ctx_len=64, **a)
    k = torch.zeros(B, 1, HKV, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="start_pos must be torch.int32"):
        kvq.window_write(win.bfloat16(), torch.zeros(B, dtype=torch.int64), k, k)


class _FakeLib:
    """Stands in for libkvq: records each call's arguments, returns a status."""

    def __init__(self, status=0):
        self.calls = []
        self.status = status

    def __getattr__(self, name):
        if not name.startswith("kvq_"):
            raise AttributeError(name)

        def call(*args):
            if name == "kvq_status_string":
                return b"status text"
            self.calls.append((name, args))
            return self.status
        return call


@pytest.fixture
def fake(monkeypatch):
    import rotated_int2_kv_kvq_amd._lib as L
    f = _FakeLib()
    monkeypatch.setattr(L, "lib", lambda: f)
    monkeypatch.setattr(L, "page_bytes", lambda d=128, g=128: 1024 + 128 * (128 // g))
    monkeypatch.setattr(L, "decode_workspace_bytes", lambda *a, **k: 4096)
    monkeypatch.setattr(L, "_same_device", lambda **t: None)       # host tensors stand in
    monkeypatch.setattr(L, "_ptr", lambda t: None if t is None else t.data_ptr())
    monkeypatch.setattr(L, "_stream", lambda s: 0)
    return f


def test_append_marshals_every_argument(fake):
    a = _append_args(rot_v=None)
    kvq.append(**a)
    (name, args), = fake.calls
    assert name == "kvq_append"
    assert args[1:5] == (8, HKV, D, 128)                     # num_blocks, Hkv, head_dim, group
    assert args[6] == 4 and args[8:10] == (B, 3)             # max blocks, batch, num_new
    assert args[12] == kvq.KVQ_BF16 and args[15] is None     # kv dtype, folded R_V
    assert args[10] == a["k"].data_ptr() and args[14] == a["rot_k"].data_ptr()
    assert abs(args[16] - 0.9) < 1e-7 and abs(args[17] - 0.9) < 1e-7


def test_decode_marshals_and_raises_on_a_status(fake):
    a = _decode_args(rot_k=None)
    out = kvq.decode(**a, out=torch.zeros(B, HQ, D), workspace=torch.zeros(4096, dtype=torch.uint8))
    (name, args), = fake.calls
    assert name == "kvq_decode_attn" and args[13] is None     # unrotated keys
    assert args[9:11] == (B, HQ) and args[8] == 64 and args[16] == out.data_ptr()
    assert abs(args[15] - 1 / 128 ** 0.5) < 1e-7               # default softmax scale
    fake.status = -3
    with pytest.raises(kvq.KvqError, match="status -3"):
        kvq.decode(**a)
