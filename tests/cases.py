"""Build seeded cases on the GPU through the C ABI and read them back for the oracle."""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle as O
import rotated_int2_kv_kvq_amd as kvq
from workload import key_mean, kv_for_sequence, make_static, query_for


@dataclass
class Case:
    w: object
    st: object
    layer: int
    device: str
    pages: torch.Tensor
    initial: torch.Tensor | None
    table: torch.Tensor
    mu: torch.Tensor
    rot_k: torch.Tensor
    rot_v: torch.Tensor
    ctx: np.ndarray
    written: dict = field(default_factory=dict)  # b -> number of positions written
    # value rotation folded into the caller's W_V / W_O: rot_v passed as None
    folded: bool = False
    # no key rotation either (rot_k passed as None): plain per-group INT2
    unrotated: bool = False

    @property
    def rk(self):
        """R_K as the library takes it (None when unrotated)."""
        return None if self.unrotated else self.rot_k

    @property
    def rk_host(self):
        """R_K as the oracle takes it (None when unrotated)."""
        return None if self.unrotated else self.st.rot_k[self.layer]

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.w.head_dim)

    @property
    def rv(self):
        """R_V as the library takes it (None when folded)."""
        return None if self.folded else self.rot_v

    @property
    def rv_host(self):
        """R_V as the oracle takes it (None when folded)."""
        return None if self.folded else self.st.rot_v[self.layer]


def new_case(w, layer=0, device="cuda", fill_seed=7, keep_initial=True) -> Case:
    st = make_static(w)
    pb = kvq.page_bytes(w.head_dim, w.group)
    g = torch.Generator(device=device)
    g.manual_seed(fill_seed)
    # arbitrary prior contents: slots that are never written must never be read
    pages = torch.randint(0, 256, (st.num_blocks, w.num_kv_heads, pb), generator=g,
                          dtype=torch.uint8, device=device)
    initial = pages.clone() if keep_initial else None
    table = torch.from_numpy(st.block_table).to(device)
    mu = key_mean(w, st, layer, device=device).contiguous()
    rot_k = torch.from_numpy(st.rot_k[layer]).to(device).contiguous()
    rot_v = torch.from_numpy(st.rot_v[layer]).to(device).contiguous()
    return Case(w, st, layer, device, pages, initial, table, mu, rot_k, rot_v, st.ctx_lens.copy())


def append_range(case: Case, seqs, start: int, count: int):
    """Append positions [start, start+count) of the given sequences in one call."""
    w = case.w
    ks, vs = [], []
    for b in seqs:
        k, v = kv_for_sequence(w, case.st, case.layer, b, start, count, case.device)
        ks.append(k)
        vs.append(v)
    k = torch.stack(ks).contiguous()
    v = torch.stack(vs).contiguous()
    idx = torch.as_tensor(list(seqs), device=case.device, dtype=torch.long)
    table = case.table.index_select(0, idx).contiguous()
    sp = torch.full((len(seqs),), start, dtype=torch.int32, device=case.device)
    kvq.append(case.pages, table, sp, k, v, case.mu, case.rk, case.rv, w.group, w.clip_k,
               w.clip_v)
    for b in seqs:
        case.written[b] = max(case.written.get(b, 0), start + count)


def fill_context(case: Case, pieces=None):
    """Append every sequence's context; pieces = list of chunk sizes (cycled)."""
    by_len = {}
    for b, n in enumerate(case.ctx):
        by_len.setdefault(int(n), []).append(b)
    for n, seqs in by_len.items():
        pos = 0
        i = 0
        while pos < n:
            step = n - pos if not pieces else min(pieces[i % len(pieces)], n - pos)
            append_range(case, seqs, pos, step)
            pos += step
            i += 1


def host_pages(case: Case, b: int, n_tokens: int):
    """(cache, table) on the host holding only sequence b's first pages."""
    n_pages = max(1, (n_tokens + 15) // 16)
    blocks = case.table[b, :n_pages].long()
    cache = case.pages.index_select(0, blocks).cpu().numpy()
    table = np.arange(n_pages, dtype=np.int32)[None, :]
    return cache, table


def oracle_encode(case: Case, b: int, start: int, count: int):
    # the same tensors the GPU appended (generated on the case's device)
    k, v = kv_for_sequence(case.w, case.st, case.layer, b, start, count, case.device)
    k, v = k.cpu(), v.cpu()
    return O.encode_tokens(k.double().numpy(), v.double().numpy(), case.mu.cpu().double().numpy(),
                           case.rk_host, case.rv_host, case.w.group,
                           case.w.clip_k, case.w.clip_v)


def decode(case: Case, q: torch.Tensor, ctx: np.ndarray | None = None, split_pages: int = 0,
           max_ctx: int | None = None):
    ctx = case.ctx if ctx is None else ctx
    ctx_t = torch.from_numpy(np.asarray(ctx, np.int32)).to(case.device)
    max_ctx = int(max(ctx.max(), 0)) if max_ctx is None else max_ctx
    return kvq.decode(case.pages, case.table, ctx_t, max_ctx, q, case.rk, case.rv,
                      case.w.group, case.sm_scale, split_pages=split_pages)


def oracle_decode(case: Case, q: torch.Tensor, pairs, ctx=None):
    """Float64 decode of the GPU's own cache for the listed (b, hq) pairs."""
    ctx = case.ctx if ctx is None else ctx
    qh = q.float().cpu().double().numpy()
    out = {}
    for b in sorted({p[0] for p in pairs}):
        n = int(ctx[b])
        cache, table = host_pages(case, b, n)
        heads = [hq for (bb, hq) in pairs if bb == b]
        o = O.decode(cache, table, [n], qh[b:b + 1], case.rk_host,
                     case.rv_host, case.sm_scale, case.w.num_kv_heads, case.w.group,
                     pairs=[(0, hq) for hq in heads])
        for hq in heads:
            out[(b, hq)] = o[0, hq]
    return out


def query(case: Case, step: int = 0):
    return query_for(case.w, case.layer, step, case.device).contiguous()
