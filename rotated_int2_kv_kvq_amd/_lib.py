"""Thin ctypes binding of libkvq (argument marshalling only).

Every step of the hot path runs in the HIP kernels behind the C ABI declared
in include/kvq.h; this module turns torch tensors into device pointers and
shapes into integers, and raises on a non-zero status.  torch is imported
first so that libkvq binds to the HIP runtime torch already loaded (both are
libamdhip64.so.7): device pointers and streams are then shared.

rot_v=None selects the folded form: the value rotation lives in the caller's
W_V and W_O, values are encoded as given and outputs stay in that basis.
rot_k=None encodes keys (less their mean) unrotated and scores with the
unrotated query: with both None the cache is plain per-group INT2, the
baseline the rotations are measured against.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_F32, KVQ_BF16 = 0, 1
_DTYPES = {torch.float32: KVQ_F32, torch.bfloat16: KVQ_BF16}

_lib = None

c_i32, c_i64, c_f32, c_sz, c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                   ctypes.c_size_t, ctypes.c_void_p)
SIGNATURES = {
    "kvq_status_string": ([c_i32], ctypes.c_char_p),
    "kvq_page_bytes": ([c_i32, c_i32], c_sz),
    "kvq_append": ([c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32, c_i32, c_vp,
                    c_vp, c_i32, c_vp, c_vp, c_vp, c_f32, c_f32, c_vp], c_i32),
    "kvq_decode_workspace_bytes": ([c_i32, c_i32, c_i32, c_i32, c_i32, c_i32], c_sz),
    "kvq_decode_plan": ([c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp], c_i32),
    "kvq_decode_attn": ([c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32, c_i32,
                         c_i32, c_vp, c_i32, c_vp, c_vp, c_f32, c_vp, c_vp, c_sz, c_i32, c_vp],
                        c_i32),
    "kvq_decode_attn_staged": ([c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32,
                                c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_f32, c_vp, c_vp, c_sz,
                                c_i32, c_i32, c_vp], c_i32),
    "kvq_append_decode": ([c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_i32,
                           c_i32, c_vp, c_vp, c_i32, c_vp, c_f32, c_f32, c_i32, c_vp, c_i32,
                           c_vp, c_vp, c_f32, c_vp, c_vp, c_sz, c_i32, c_vp], c_i32),
    "kvq_decode_attn_noalloc": ([c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32,
                                 c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_f32, c_vp, c_i32, c_vp],
                                c_i32),
    "kvq_window_bytes": ([c_i32, c_i32, c_i32], c_sz),
    "kvq_window_write": ([c_vp, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_i32, c_vp], c_i32),
    "kvq_decode_attn_window": ([c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_vp,
                                c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_f32, c_vp, c_vp,
                                c_sz, c_i32, c_vp], c_i32),
    "kvq_append_decode_window": ([c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp,
                                  c_vp, c_i32, c_i32, c_vp, c_vp, c_i32, c_vp, c_f32, c_f32,
                                  c_i32, c_vp, c_i32, c_vp, c_vp, c_f32, c_vp, c_vp, c_sz, c_i32,
                                  c_vp], c_i32),
}
STAGE_PREPARE, STAGE_SPLITS, STAGE_MERGE, STAGE_ALL = 1, 2, 4, 7
WINDOW_SINK, WINDOW_RECENT = 64, 256


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libkvq.so (built in-tree); raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m rotated_int2_kv_kvq_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().kvq_status_string(int(status)).decode()


def page_bytes(head_dim: int = 128, group: int = 128) -> int:
    return int(lib().kvq_page_bytes(head_dim, group))


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("kvq operates on device tensors")
    if not t.is_contiguous():
        raise ValueError("kvq expects contiguous tensors")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(status: int, where: str) -> None:
    if status != 0:
        raise KvqError(status, where)


def _need(name: str, t, dtype, shape=None) -> None:
    """Raise ValueError unless t is a tensor of the given dtype (one dtype or a
    tuple of them) and shape (None entries match any size)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dts)}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and s != n for s, n in zip(shape, t.shape)):
            want = "[" + ", ".join("*" if s is None else str(s) for s in shape) + "]"
            raise ValueError(f"{name} must have shape {want}, got {list(t.shape)}")


def _same_device(**tensors) -> None:
    """Every given tensor (None skipped) on the current CUDA device, together."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if dev is None:
            dev = t.device
            if dev.index is not None and dev.index != torch.cuda.current_device():
                raise ValueError(f"{name} is on {dev}, not on the current device, whose "
                                 "stream the launches use")
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other arguments on {dev}")


_FLOATS = (torch.float32, torch.bfloat16)


def _check_cache(pages, group: int, block_table, batch: int):
    """The cache buffer and block table of a call; returns (num_blocks, Hkv)."""
    _need("pages", pages, torch.uint8, (None, None, None))
    if group not in (64, 128):
        raise ValueError(f"group must be 64 or 128, got {group}")
    pb = page_bytes(128, group)
    if pages.shape[2] != pb:
        raise ValueError(f"pages.shape[2] is {pages.shape[2]}; a group-{group} page is {pb} bytes")
    _need("block_table", block_table, torch.int32, (None, None))
    if block_table.shape[0] < batch:
        raise ValueError(f"block_table has {block_table.shape[0]} rows for a batch of {batch}")
    return pages.shape[0], pages.shape[1]


def _check_rotations(mu, rot_k, rot_v, hkv: int, need_mu: bool = True) -> None:
    if need_mu or mu is not None:
        _need("mu", mu, torch.float32, (hkv, 128))
    if rot_k is not None:
        _need("rot_k", rot_k, torch.float32, (hkv, 128, 128))
    if rot_v is not None:
        _need("rot_v", rot_v, torch.float32, (hkv, 128, 128))


def _check_kv(k, v, batch, hkv, num_new=None) -> None:
    _need("k", k, _FLOATS, (batch, num_new, hkv, 128))
    _need("v", v, k.dtype, tuple(k.shape))


def _check_query_out(q, out, hkv):
    """q [B][Hq][128] (fp32 or bf16) and out fp32 [B][Hq][128]; returns (B, Hq)."""
    _need("q", q, _FLOATS, (None, None, 128))
    B, Hq, _ = q.shape
    if Hq < hkv or Hq % hkv:
        raise ValueError(f"{Hq} query heads do not group over {hkv} KV heads")
    if out is not None:
        _need("out", out, torch.float32, (B, Hq, 128))
    return B, Hq


def _check_workspace(ws, need: int) -> None:
    _need("workspace", ws, torch.uint8)
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, the call needs {need}")


def append(pages: torch.Tensor, block_table: torch.Tensor, start_pos: torch.Tensor,
           k: torch.Tensor, v: torch.Tensor, mu: torch.Tensor, rot_k: torch.Tensor,
           rot_v: torch.Tensor | None, group: int, clip_k: float, clip_v: float, stream=None) -> None:
    """kvq_append: pages uint8 [num_blocks][Hkv][page_bytes]; k, v [B][T][Hkv][128]."""
    _need("k", k, _FLOATS, (None, None, None, 128))
    B = k.shape[0]
    num_blocks, hkv = _check_cache(pages, group, block_table, B)
    _check_kv(k, v, B, hkv)
    _need("start_pos", start_pos, torch.int32, (B,))
    _check_rotations(mu, rot_k, rot_v, hkv)
    _same_device(pages=pages, block_table=block_table, start_pos=start_pos, k=k, v=v, mu=mu,
                 rot_k=rot_k, rot_v=rot_v)
    T = k.shape[1]
    _check(lib().kvq_append(_ptr(pages), num_blocks, hkv, k.shape[-1], group, _ptr(block_table),
                            block_table.shape[1], _ptr(start_pos), B, T, _ptr(k), _ptr(v),
                            _DTYPES[k.dtype], _ptr(mu), _ptr(rot_k), _ptr(rot_v), clip_k, clip_v,
                            _stream(stream)), "kvq_append")


def decode_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, max_ctx_len: int,
                           head_dim: int = 128, split_pages: int = 0) -> int:
    return int(lib().kvq_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                max_ctx_len, split_pages))


def decode_plan(batch: int, num_q_heads: int, num_kv_heads: int, max_ctx_len: int,
                head_dim: int = 128, split_pages: int = 0) -> dict:
    """kvq_decode_plan: {"num_splits", "split_pages", "operand_in_scan"}."""
    ns, sp, ins = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().kvq_decode_plan(batch, num_q_heads, num_kv_heads, head_dim, max_ctx_len,
                                 split_pages, ctypes.byref(ns), ctypes.byref(sp),
                                 ctypes.byref(ins)), "kvq_decode_plan")
    return {"num_splits": ns.value, "split_pages": sp.value, "operand_in_scan": bool(ins.value)}


def _decode_common(pages, block_table, ctx_len, max_ctx_len, q, rot_k, rot_v, group, sm_scale,
                   out, workspace, split_pages, mu=None, need_mu=False, window=None,
                   new_kv=None, workspace_needed=True):
    """Checks shared by the decode entry points (with the window store and the
    appended token's (k, v, start_pos) when given), every tensor's dtype and
    shape before any device; returns (num_blocks, Hkv, B, Hq, sm_scale, out,
    workspace)."""
    _need("q", q, _FLOATS, (None, None, 128))
    num_blocks, hkv = _check_cache(pages, group, block_table, q.shape[0])
    B, Hq = _check_query_out(q, out, hkv)
    _need("ctx_len", ctx_len, torch.int32, (B,))
    _check_rotations(mu, rot_k, rot_v, hkv, need_mu=need_mu)
    need = decode_workspace_bytes(B, Hq, hkv, max_ctx_len, 128, split_pages)
    if need == 0 and B > 0:
        raise ValueError(f"no decode plan for batch {B}, {Hq}/{hkv} heads, max_ctx_len "
                         f"{max_ctx_len}, split_pages {split_pages}")
    if workspace is not None:
        _check_workspace(workspace, need)
    if window is not None:
        _check_window(window, B, hkv)
    k = v = start_pos = None
    if new_kv is not None:
        k, v, start_pos = new_kv
        _check_kv(k, v, B, hkv, num_new=1)
        _need("start_pos", start_pos, torch.int32, (B,))
    _same_device(pages=pages, block_table=block_table, ctx_len=ctx_len, q=q, out=out, mu=mu,
                 rot_k=rot_k, rot_v=rot_v, workspace=workspace, window=window, k=k, v=v,
                 start_pos=start_pos)
    dev = pages.device
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    if out is None:
        out = torch.empty(B, Hq, 128, dtype=torch.float32, device=dev)
    if workspace is None and workspace_needed:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    return num_blocks, hkv, B, Hq, sm_scale, out, workspace


def decode(pages: torch.Tensor, block_table: torch.Tensor, ctx_len: torch.Tensor,
           max_ctx_len: int, q: torch.Tensor, rot_k: torch.Tensor, rot_v: torch.Tensor | None,
           group: int, sm_scale: float | None = None, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None, split_pages: int = 0,
           stages: int = STAGE_ALL, stream=None) -> torch.Tensor:
    """kvq_decode_attn (or kvq_decode_attn_staged when stages != all):
    q [B][Hq][128] -> out float32 [B][Hq][128]."""
    num_blocks, hkv, B, Hq, sm_scale, out, workspace = _decode_common(
        pages, block_table, ctx_len, max_ctx_len, q, rot_k, rot_v, group, sm_scale, out,
        workspace, split_pages)
    d = q.shape[-1]
    args = (_ptr(pages), num_blocks, hkv, d, group, _ptr(block_table), block_table.shape[1],
            _ptr(ctx_len), max_ctx_len, B, Hq, _ptr(q), _DTYPES[q.dtype], _ptr(rot_k),
            _ptr(rot_v), sm_scale, _ptr(out), _ptr(workspace), workspace.numel(), split_pages)
    if stages == STAGE_ALL:
        _check(lib().kvq_decode_attn(*args, _stream(stream)), "kvq_decode_attn")
    else:
        _check(lib().kvq_decode_attn_staged(*args, stages, _stream(stream)),
               "kvq_decode_attn_staged")
    return out


def append_decode(pages: torch.Tensor, block_table: torch.Tensor, start_pos: torch.Tensor,
                  ctx_len: torch.Tensor, max_ctx_len: int, k: torch.Tensor, v: torch.Tensor,
                  mu: torch.Tensor, q: torch.Tensor, rot_k: torch.Tensor, rot_v: torch.Tensor | None,
                  group: int, clip_k: float, clip_v: float, sm_scale: float | None = None,
                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  split_pages: int = 0, stream=None) -> torch.Tensor:
    """kvq_append_decode: k, v [B][1][Hkv][128] appended at start_pos, then
    q [B][Hq][128] attends over ctx_len tokens -> out float32 [B][Hq][128]."""
    num_blocks, hkv, B, Hq, sm_scale, out, workspace = _decode_common(
        pages, block_table, ctx_len, max_ctx_len, q, rot_k, rot_v, group, sm_scale, out,
        workspace, split_pages, mu=mu, need_mu=True, new_kv=(k, v, start_pos))
    d = q.shape[-1]
    _check(lib().kvq_append_decode(
        _ptr(pages), num_blocks, hkv, d, group, _ptr(block_table), block_table.shape[1],
        _ptr(start_pos), _ptr(ctx_len), max_ctx_len, B, _ptr(k), _ptr(v), _DTYPES[k.dtype],
        _ptr(mu), clip_k, clip_v, Hq, _ptr(q), _DTYPES[q.dtype], _ptr(rot_k), _ptr(rot_v),
        sm_scale, _ptr(out), _ptr(workspace), workspace.numel(), split_pages, _stream(stream)),
        "kvq_append_decode")
    return out


SCRATCH_BYTES = 32 << 20  # KVQ_SCRATCH_BYTES of include/kvq.h


def decode_noalloc(pages: torch.Tensor, block_table: torch.Tensor, ctx_len: torch.Tensor,
                   max_ctx_len: int, q: torch.Tensor, rot_k: torch.Tensor | None,
                   rot_v: torch.Tensor | None, group: int, sm_scale: float, out: torch.Tensor,
                   split_pages: int = 0, stream=None) -> torch.Tensor:
    """kvq_decode_attn_noalloc: kvq_decode_attn with the library's static
    scratch as its workspace; `out` must be given (nothing is allocated)."""
    _need("out", out, torch.float32)
    num_blocks, hkv, B, Hq, sm_scale, out, _ = _decode_common(
        pages, block_table, ctx_len, max_ctx_len, q, rot_k, rot_v, group, sm_scale, out,
        None, split_pages, workspace_needed=False)
    _check(lib().kvq_decode_attn_noalloc(
        _ptr(pages), num_blocks, hkv, q.shape[-1], group, _ptr(block_table),
        block_table.shape[1], _ptr(ctx_len), max_ctx_len, B, Hq, _ptr(q), _DTYPES[q.dtype],
        _ptr(rot_k), _ptr(rot_v), sm_scale, _ptr(out), split_pages, _stream(stream)),
        "kvq_decode_attn_noalloc")
    return out


# ----------------------------------------------------------------- BF16 windows
def window_bytes(batch: int, num_kv_heads: int, head_dim: int = 128) -> int:
    return int(lib().kvq_window_bytes(batch, num_kv_heads, head_dim))


def new_window(batch: int, num_kv_heads: int, device="cuda") -> torch.Tensor:
    """A window store: bfloat16 [B][Hkv][2][320][128] (contents unspecified)."""
    return torch.empty(batch, num_kv_heads, 2, WINDOW_SINK + WINDOW_RECENT, 128,
                       dtype=torch.bfloat16, device=device)


def _check_window(window, batch, hkv) -> None:
    _need("window", window, torch.bfloat16, (batch, hkv, 2, WINDOW_SINK + WINDOW_RECENT, 128))


def window_write(window: torch.Tensor, start_pos: torch.Tensor, k: torch.Tensor,
                 v: torch.Tensor, stream=None) -> None:
    """kvq_window_write: k, v [B][T][Hkv][128] at positions start_pos[b] + tau."""
    _need("k", k, _FLOATS, (None, None, None, 128))
    B, T, hkv, d = k.shape
    _check_kv(k, v, B, hkv)
    _check_window(window, B, hkv)
    _need("start_pos", start_pos, torch.int32, (B,))
    _same_device(window=window, start_pos=start_pos, k=k, v=v)
    _check(lib().kvq_window_write(_ptr(window), hkv, d, B, _ptr(start_pos), T, _ptr(k), _ptr(v),
                                  _DTYPES[k.dtype], _stream(stream)), "kvq_window_write")


def decode_window(pages: torch.Tensor, block_table: torch.Tensor, window: torch.Tensor,
                  mu: torch.Tensor, ctx_len: torch.Tensor, max_ctx_len: int, q: torch.Tensor,
                  rot_k: torch.Tensor, rot_v: torch.Tensor | None, group: int,
                  sm_scale: float | None = None, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, split_pages: int = 0,
                  stream=None) -> torch.Tensor:
    """kvq_decode_attn_window: attention over BF16 sinks + INT2 body + BF16 recent."""
    num_blocks, hkv, B, Hq, sm_scale, out, workspace = _decode_common(
        pages, block_table, ctx_len, max_ctx_len, q, rot_k, rot_v, group, sm_scale, out,
        workspace, split_pages, mu=mu, need_mu=True, window=window)
    d = q.shape[-1]
    _check(lib().kvq_decode_attn_window(
        _ptr(pages), num_blocks, hkv, d, group, _ptr(block_table), block_table.shape[1],
        _ptr(window), _ptr(mu), _ptr(ctx_len), max_ctx_len, B, Hq, _ptr(q), _DTYPES[q.dtype],
        _ptr(rot_k), _ptr(rot_v), sm_scale, _ptr(out), _ptr(workspace), workspace.numel(),
        split_pages, _stream(stream)), "kvq_decode_attn_window")
    return out


def append_decode_window(pages: torch.Tensor, block_table: torch.Tensor, window: torch.Tensor,
                         start_pos: torch.Tensor, ctx_len: torch.Tensor, max_ctx_len: int,
                         k: torch.Tensor, v: torch.Tensor, mu: torch.Tensor, q: torch.Tensor,
                         rot_k: torch.Tensor, rot_v: torch.Tensor | None, group: int, clip_k: float,
                         clip_v: float, sm_scale: float | None = None,
                         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         split_pages: int = 0, stream=None) -> torch.Tensor:
    """kvq_append_decode_window: one decode step with BF16 windows."""
    num_blocks, hkv, B, Hq, sm_scale, out, workspace = _decode_common(
        pages, block_table, ctx_len, max_ctx_len, q, rot_k, rot_v, group, sm_scale, out,
        workspace, split_pages, mu=mu, need_mu=True, window=window,
        new_kv=(k, v, start_pos))
    d = q.shape[-1]
    _check(lib().kvq_append_decode_window(
        _ptr(pages), num_blocks, hkv, d, group, _ptr(block_table), block_table.shape[1],
        _ptr(window), _ptr(start_pos), _ptr(ctx_len), max_ctx_len, B, _ptr(k), _ptr(v),
        _DTYPES[k.dtype], _ptr(mu), clip_k, clip_v, Hq, _ptr(q), _DTYPES[q.dtype], _ptr(rot_k),
        _ptr(rot_v), sm_scale, _ptr(out), _ptr(workspace), workspace.numel(), split_pages,
        _stream(stream)), "kvq_append_decode_window")
    return out
