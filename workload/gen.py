"""Seeded synthetic inputs shaped like the attention of the models the pages study.

Recipe (inputs only; nothing here centres, rotates, quantises or attends):

* Rotations: a Haar-random orthogonal matrix (QR of a Gaussian, columns
  sign-fixed by the diagonal of R) or, for the Qwen3-8B-shaped workloads, the
  normalised Sylvester Hadamard matrix times a Haar matrix; or, in the pages'
  parameterisation of a corrected rotation, R0 exp(A - A^T) with R0 the
  normalised Hadamard matrix and A a seeded Gaussian matrix (entries
  N(0, 0.01^2); the calibration that would fit A is out of scope).  Drawn in
  float64, stored as float32.  Key and value rotations are drawn separately
  per (layer, KV head).
* Keys and values: N(0, 1) per element; the same 4 seeded channels per
  (layer, KV head) are multiplied by 20 in both K and V; keys then get a
  per-channel offset drawn once from N(0, sigma) (sigma 3, or 5 for the
  long-context workload); optional sink positions multiply the whole key
  vector after the offset.  Cast to the storage dtype with round-to-nearest-even.
* Queries: N(0, 1), cast to the query dtype.
* Context lengths: fixed, or uniform integers in [lo, hi].
* Paging: 16-token blocks; a random permutation of all physical blocks is
  dealt to the sequences in order (identity for the contiguous workload).

Small parts (rotations, outlier channels, offsets, lengths, block tables) come
from numpy PCG64 streams; bulk keys, values and queries come from torch
generators, one per (layer, sequence, 1024-token chunk), so any token range of
any sequence can be regenerated on any device without drawing the rest.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np
import torch

CHUNK = 1024  # tokens per independently seeded generator stream


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    ctx_min: int
    ctx_max: int
    head_dim: int = 128
    group: int = 128
    clip_k: float = 0.9
    clip_v: float = 0.9
    block_size: int = 16
    kv_dtype: str = "bf16"
    q_dtype: str = "bf16"
    rotation: str = "hadamard_haar"
    key_offset_std: float = 3.0
    outliers: int = 4
    outlier_scale: float = 20.0
    sink_tokens: int = 0
    sink_scale: float = 1.0
    paged: bool = True
    layers: int = 1
    steps: int = 0
    seed: int = 1000

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads


WORKLOADS = {
    w.name: w
    for w in [
        # Single layer, contiguous cache, fp32 K/V and query, Haar rotation.
        Workload("single_layer_b1_h8x2_ctx1k_f32", batch=1, num_q_heads=8, num_kv_heads=2,
                 ctx_min=1024, ctx_max=1024, kv_dtype="f32", q_dtype="f32",
                 rotation="haar", paged=False, seed=1000),
        # Qwen3-8B attention shape, paged, 8K context.
        Workload("qwen3_8b_b4_ctx8k", batch=4, num_q_heads=32, num_kv_heads=8,
                 ctx_min=8192, ctx_max=8192, seed=1001),
        # Decode-heavy ragged batch, group 64 (2.5 bits/element).
        Workload("qwen3_8b_b64_ctx1k_32k_g64", batch=64, num_q_heads=32, num_kv_heads=8,
                 ctx_min=1024, ctx_max=32768, group=64, seed=1002),
        # Long context with a heavy key mean and x50 sink tokens.
        Workload("qwen3_8b_b1_ctx128k_sinks", batch=1, num_q_heads=32, num_kv_heads=8,
                 ctx_min=131072, ctx_max=131072, key_offset_std=5.0, sink_tokens=4,
                 sink_scale=50.0, seed=1003),
        # Append-plus-decode stream over 36 layers.
        Workload("qwen3_8b_36l_b16_ctx16k_stream", batch=16, num_q_heads=32, num_kv_heads=8,
                 ctx_min=16384, ctx_max=16384, layers=36, steps=256, seed=1004),
    ]
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields changed (for smaller parity cases)."""
    return dataclasses.replace(w, **changes)


# --------------------------------------------------------------------------- rotations
def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("Hadamard order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def haar_orthogonal(rng: np.random.Generator, d: int) -> np.ndarray:
    """Haar-distributed orthogonal matrix: QR of a Gaussian, sign-fixed."""
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


# Standard deviation of the entries of the generator A of a corrected rotation.
EXPM_SCALE = 0.01


def corrected_rotation(r0: np.ndarray, a: np.ndarray) -> np.ndarray:
    """R0 exp(A - A^T): a base rotation times the exponential of a
    skew-symmetric generator ("Output-Aware Rotation for INT2 KV-Cache
    Quantization", "What carries the argument", mechanism 1; "Assumptions &
    free parameters": the exponential of a skew-symmetric matrix is
    orthogonal).  Float64, scipy's matrix exponential."""
    from scipy.linalg import expm
    a = np.asarray(a, np.float64)
    return np.asarray(r0, np.float64) @ expm(a - a.T)


def _rotation(rng: np.random.Generator, d: int, kind: str) -> np.ndarray:
    if kind == "haar":
        return haar_orthogonal(rng, d)
    if kind == "hadamard_haar":
        return (hadamard(d) / math.sqrt(d)) @ haar_orthogonal(rng, d)
    if kind == "hadamard_expm":
        return corrected_rotation(hadamard(d) / math.sqrt(d),
                                  EXPM_SCALE * rng.standard_normal((d, d)))
    if kind == "identity":
        return np.eye(d)
    raise ValueError(kind)


# --------------------------------------------------------------------------- static parts
@dataclass
class Static:
    rot_k: np.ndarray        # [L][Hkv][d][d] float32, x_rot = x @ R
    rot_v: np.ndarray        # [L][Hkv][d][d] float32
    outlier_ch: np.ndarray   # [L][Hkv][outliers] int
    key_offset: np.ndarray   # [L][Hkv][d] float64
    ctx_lens: np.ndarray     # [B] int32 (prior context per sequence)
    block_table: np.ndarray  # [B][max_blocks] int32
    num_blocks: int


def ctx_lens_for(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.ctx_min == w.ctx_max:
        return np.full(w.batch, w.ctx_min, dtype=np.int32)
    return rng.integers(w.ctx_min, w.ctx_max + 1, size=w.batch).astype(np.int32)


def block_table_for(w: Workload, rng: np.random.Generator, capacity: np.ndarray):
    """Deal a random permutation of all physical blocks to the sequences in order.

    capacity[b] is the number of token slots sequence b must be able to hold.
    Entries past a sequence's last block are 0 (never read).
    """
    P = w.block_size
    need = (capacity.astype(np.int64) + P - 1) // P
    max_blocks = int(max(1, need.max()))
    if not w.paged:
        table = np.arange(w.batch * max_blocks, dtype=np.int32).reshape(w.batch, max_blocks)
        return table, w.batch * max_blocks
    total = int(need.sum())
    perm = rng.permutation(total).astype(np.int32)
    table = np.zeros((w.batch, max_blocks), dtype=np.int32)
    off = 0
    for b in range(w.batch):
        table[b, : need[b]] = perm[off: off + need[b]]
        off += need[b]
    return table, max(total, 1)


def make_static(w: Workload) -> Static:
    """Draw the small seeded parts in a fixed order: rotations, outlier channels,
    offsets, context lengths, block table."""
    rng = np.random.default_rng(w.seed)
    L, H, d = w.layers, w.num_kv_heads, w.head_dim
    rot_k = np.empty((L, H, d, d), np.float32)
    rot_v = np.empty((L, H, d, d), np.float32)
    for layer in range(L):
        for h in range(H):
            rot_k[layer, h] = _rotation(rng, d, w.rotation)
            rot_v[layer, h] = _rotation(rng, d, w.rotation)
    outl = np.stack([
        np.stack([rng.choice(d, size=w.outliers, replace=False) for _ in range(H)])
        for _ in range(L)
    ]) if w.outliers else np.zeros((L, H, 0), np.int64)
    offset = rng.normal(0.0, w.key_offset_std, size=(L, H, d)) if w.key_offset_std else np.zeros((L, H, d))
    ctx = ctx_lens_for(w, rng)
    table, nblk = block_table_for(w, rng, ctx + w.steps)
    return Static(rot_k, rot_v, outl, offset, ctx, table, nblk)


# --------------------------------------------------------------------------- bulk tensors
def _seed(*parts: int) -> int:
    return int(np.random.SeedSequence([int(p) for p in parts]).generate_state(1)[0])


_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def kv_for_sequence(w: Workload, st: Static, layer: int, seq: int, start: int, count: int,
                    device="cpu"):
    """Keys and values of positions [start, start+count) of one sequence, shaped
    [count][Hkv][d] in the workload's storage dtype."""
    H, d = w.num_kv_heads, w.head_dim
    ks, vs = [], []
    pos = start
    end = start + count
    off = torch.as_tensor(st.key_offset[layer], dtype=torch.float32, device=device)
    scale = torch.ones(H, d, dtype=torch.float32, device=device)
    for h in range(H):
        scale[h, torch.as_tensor(st.outlier_ch[layer, h], device=device)] = w.outlier_scale
    while pos < end:
        c = pos // CHUNK
        g = torch.Generator(device=device)
        g.manual_seed(_seed(w.seed, layer, seq, c, 1))
        kc = torch.randn(CHUNK, H, d, generator=g, device=device, dtype=torch.float32)
        vc = torch.randn(CHUNK, H, d, generator=g, device=device, dtype=torch.float32)
        lo = pos - c * CHUNK
        hi = min(end - c * CHUNK, CHUNK)
        kc, vc = kc[lo:hi] * scale, vc[lo:hi] * scale
        kc = kc + off
        if w.sink_tokens and pos < w.sink_tokens:
            n = min(w.sink_tokens - pos, hi - lo)
            kc[:n] *= w.sink_scale
        ks.append(kc)
        vs.append(vc)
        pos = c * CHUNK + hi
    if not ks:
        z = torch.zeros(0, H, d, device=device)
        return z.to(_DT[w.kv_dtype]), z.to(_DT[w.kv_dtype])
    return torch.cat(ks).to(_DT[w.kv_dtype]), torch.cat(vs).to(_DT[w.kv_dtype])


def query_for(w: Workload, layer: int, step: int, device="cpu"):
    """Queries [B][Hq][d] for one decode step of one layer."""
    g = torch.Generator(device=device)
    g.manual_seed(_seed(w.seed, layer, step, 2))
    q = torch.randn(w.batch, w.num_q_heads, w.head_dim, generator=g, device=device,
                    dtype=torch.float32)
    return q.to(_DT[w.q_dtype])


def key_mean(w: Workload, st: Static, layer: int, sample_tokens: int = 2048, device="cpu"):
    """Per-(KV head, channel) key mean standing in for the calibration mean:
    the float64 mean of the stored (dtype-cast) keys at positions
    [0, min(ctx, sample_tokens)) of every sequence; returned as float32 [Hkv][d]."""
    acc = torch.zeros(w.num_kv_heads, w.head_dim, dtype=torch.float64, device=device)
    n = 0
    for b in range(w.batch):
        cnt = int(min(st.ctx_lens[b], sample_tokens))
        if cnt == 0:
            continue
        k, _ = kv_for_sequence(w, st, layer, b, 0, cnt, device)
        acc += k.to(torch.float64).sum(0)
        n += cnt
    return (acc / max(n, 1)).to(torch.float32)
