"""Thin ctypes binding of libkvq (argument marshalling only).

Every step of the hot path runs in the HIP kernels behind the C ABI declared
in include/kvq.h; this module turns torch tensors into device pointers and
shapes into integers, and raises on a non-zero status.  torch is imported
first so that libkvq binds to the HIP runtime torch already loaded (both are
libamdhip64.so.7): device pointers and streams are then shared.

rot_v=None selects the folded form: the value rotation lives in the caller's
W_V and W_O, values are encoded as given and outputs stay in that basis.
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
    "kvq_decode_attn": ([c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32, c_i32,
                         c_i32, c_vp, c_i32, c_vp, c_vp, c_f32, c_vp, c_vp, c_sz, c_i32, c_vp],
                        c_i32),
    "kvq_decode_attn_staged": ([c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32,
                                c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_f32, c_vp, c_vp, c_sz,
                                c_i32, c_i32, c_vp], c_i32),
    "kvq_append_decode": ([c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_i32,
                           c_i32, c_vp, c_vp, c_i32, c_vp, c_f32, c_f32, c_i32, c_vp, c_i32,
                           c_vp, c_vp, c_f32, c_vp, c_vp, c_sz, c_i32, c_vp], c_i32),
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


def append(pages: torch.Tensor, block_table: torch.Tensor, start_pos: torch.Tensor,
           k: torch.Tensor, v: torch.Tensor, mu: torch.Tensor, rot_k: torch.Tensor,
           rot_v: torch.Tensor | None, group: int, clip_k: float, clip_v: float, stream=None) -> None:
    """kvq_append: pages uint8 [num_blocks][Hkv][page_bytes]; k, v [B][T][Hkv][128]."""
    num_blocks, hkv, _ = pages.shape
    B, T = k.shape[0], k.shape[1]
    if k.dtype not in _DTYPES or v.dtype != k.dtype:
        raise ValueError("k and v must both be float32 or bfloat16")
    _check(lib().kvq_append(_ptr(pages), num_blocks, hkv, k.shape[-1], group, _ptr(block_table),
                            block_table.shape[1], _ptr(start_pos), B, T, _ptr(k), _ptr(v),
                            _DTYPES[k.dtype], _ptr(mu), _ptr(rot_k), _ptr(rot_v), clip_k, clip_v,
                            _stream(stream)), "kvq_append")


def decode_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, max_ctx_len: int,
                           head_dim: int = 128, split_pages: int = 0) -> int:
    return int(lib().kvq_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                max_ctx_len, split_pages))


def decode(pages: torch.Tensor, block_table: torch.Tensor, ctx_len: torch.Tensor,
           max_ctx_len: int, q: torch.Tensor, rot_k: torch.Tensor, rot_v: torch.Tensor | None,
           group: int, sm_scale: float | None = None, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None, split_pages: int = 0,
           stages: int = STAGE_ALL, stream=None) -> torch.Tensor:
    """kvq_decode_attn (or kvq_decode_attn_staged when stages != all):
    q [B][Hq][128] -> out float32 [B][Hq][128]."""
    num_blocks, hkv, _ = pages.shape
    B, Hq, d = q.shape
    if q.dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, Hq, hkv, max_ctx_len, d, split_pages)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
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
    num_blocks, hkv, _ = pages.shape
    B, Hq, d = q.shape
    if k.dtype not in _DTYPES or v.dtype != k.dtype:
        raise ValueError("k and v must both be float32 or bfloat16")
    if q.dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    if k.shape[1] != 1:
        raise ValueError("append_decode appends exactly one token per sequence")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, Hq, hkv, max_ctx_len, d, split_pages)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().kvq_append_decode(
        _ptr(pages), num_blocks, hkv, d, group, _ptr(block_table), block_table.shape[1],
        _ptr(start_pos), _ptr(ctx_len), max_ctx_len, B, _ptr(k), _ptr(v), _DTYPES[k.dtype],
        _ptr(mu), clip_k, clip_v, Hq, _ptr(q), _DTYPES[q.dtype], _ptr(rot_k), _ptr(rot_v),
        sm_scale, _ptr(out), _ptr(workspace), workspace.numel(), split_pages, _stream(stream)),
        "kvq_append_decode")
    return out


# ----------------------------------------------------------------- BF16 windows
def window_bytes(batch: int, num_kv_heads: int, head_dim: int = 128) -> int:
    return int(lib().kvq_window_bytes(batch, num_kv_heads, head_dim))


def new_window(batch: int, num_kv_heads: int, device="cuda") -> torch.Tensor:
    """A window store: bfloat16 [B][Hkv][2][320][128] (contents unspecified)."""
    return torch.empty(batch, num_kv_heads, 2, WINDOW_SINK + WINDOW_RECENT, 128,
                       dtype=torch.bfloat16, device=device)


def window_write(window: torch.Tensor, start_pos: torch.Tensor, k: torch.Tensor,
                 v: torch.Tensor, stream=None) -> None:
    """kvq_window_write: k, v [B][T][Hkv][128] at positions start_pos[b] + tau."""
    B, T, hkv, d = k.shape
    if k.dtype not in _DTYPES or v.dtype != k.dtype:
        raise ValueError("k and v must both be float32 or bfloat16")
    _check(lib().kvq_window_write(_ptr(window), hkv, d, B, _ptr(start_pos), T, _ptr(k), _ptr(v),
                                  _DTYPES[k.dtype], _stream(stream)), "kvq_window_write")


def decode_window(pages: torch.Tensor, block_table: torch.Tensor, window: torch.Tensor,
                  mu: torch.Tensor, ctx_len: torch.Tensor, max_ctx_len: int, q: torch.Tensor,
                  rot_k: torch.Tensor, rot_v: torch.Tensor | None, group: int,
                  sm_scale: float | None = None, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, split_pages: int = 0,
                  stream=None) -> torch.Tensor:
    """kvq_decode_attn_window: attention over BF16 sinks + INT2 body + BF16 recent."""
    num_blocks, hkv, _ = pages.shape
    B, Hq, d = q.shape
    if q.dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, Hq, hkv, max_ctx_len, d, split_pages)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
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
    num_blocks, hkv, _ = pages.shape
    B, Hq, d = q.shape
    if k.dtype not in _DTYPES or v.dtype != k.dtype or q.dtype not in _DTYPES:
        raise ValueError("k, v and q must be float32 or bfloat16")
    if k.shape[1] != 1:
        raise ValueError("append_decode_window appends exactly one token per sequence")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, Hq, hkv, max_ctx_len, d, split_pages)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().kvq_append_decode_window(
        _ptr(pages), num_blocks, hkv, d, group, _ptr(block_table), block_table.shape[1],
        _ptr(window), _ptr(start_pos), _ptr(ctx_len), max_ctx_len, B, _ptr(k), _ptr(v),
        _DTYPES[k.dtype], _ptr(mu), clip_k, clip_v, Hq, _ptr(q), _DTYPES[q.dtype], _ptr(rot_k),
        _ptr(rot_v), sm_scale, _ptr(out), _ptr(workspace), workspace.numel(), split_pages,
        _stream(stream)), "kvq_append_decode_window")
    return out
