"""Float64 CPU oracle: what the rotated INT2 KV-cache hot path computes.

TEST INFRASTRUCTURE ONLY -- imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.  Plain numpy in
float64; no blocking, no split-K, no code shared with the HIP library.

Sources (web pages; cited by title and section):
  [OptR] "Output-Aware Rotation for INT2 KV-Cache Quantization", Pith review of
         arXiv 2608.02691: sections "The reading", "What carries the argument",
         "Core claim", "If this is right", "Assumptions & free parameters",
         and the abstract.
The pages describe the method in prose only; where they leave a step open the
reading taken here is stated at the function that takes it.

What the oracle computes
------------------------
Append ([OptR] "What carries the argument": the key is centred by a
per-channel mean, then rotation, clipping, grouping, rounding; "Core claim":
one rotation per KV head and layer):
    x = (k - mu_h) @ R_K[h]          keys   (row vectors, x_rot = x @ R)
    y =  v         @ R_V[h]          values (no centring)
    per group of `group` rotated channels of one token:
        lo = c * min, hi = c * max,  s = (hi - lo) / 3,  z = lo
        s16 = fp16(s), z16 = fp16(z)  (round to nearest even, saturating)
        code = clamp(rint((x - z16) / s16), 0, 3), or 0 when s16 == 0
Decode ([OptR] "What carries the argument": dequantisation, then inverse
rotation; the abstract: attention over the quantised cache):
    q_r = q @ R_K[h]; x_hat = s16 * code + z16
    p = softmax(sm_scale * q_r . k_hat_t) over t < ctx_len
    o = (sum_t p_t v_hat_t) @ R_V[h].T
An empty context gives o = 0.

Cache layout (ours; the pages only say the paged KV-cache format is kept,
[OptR] "If this is right" and the abstract).  One byte buffer per layer,
[num_blocks][Hkv][page_bytes], 16 tokens per block, head_dim 128, G = 128/group:
    [0, 512)        K codes, token-row major: token t, channel i at byte
                    32*t + i//4, bits 2*(i%4)
    [512, 1024)     V codes, 128 little-endian 32-bit words, one per
                    channel: channel i at byte 512 + 4*(8*(i%16) + i//16),
                    its 16 tokens inside the word at code positions
                    u = 3t mod 16 (bits 2u)
    [1024, +64G)    K fp16 (scale, zero) pairs, [token][group]
    [.., +64G)      V fp16 (scale, zero) pairs, [token][group]
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128
BLOCK = 16
LEVELS = 3.0  # 2**2 - 1 steps of a 2-bit grid
F16_MAX = 65504.0

__all__ = [
    "HEAD_DIM", "BLOCK", "F16_MAX", "fp16_sat", "page_bytes", "bits_per_element",
    "rotate", "encode_groups", "quantize_on_grid", "encode_tokens", "k_code_site", "v_code_site",
    "sz_site", "write_tokens", "read_tokens", "dequant", "attend", "decode",
    "append", "plain_attention", "SINK", "RECENT", "WINDOW", "window_slot", "window_parts",
    "bf16_round", "window_write", "append_windowed", "decode_windowed", "dequantized_kv",
    "eq8_decomposition", "value_rotation", "key_rotation",
]


# --------------------------------------------------------------------------- scalars
def fp16_sat(x):
    """Nearest fp16 value (round half to even) as float64, saturating at +-65504.

    Reading: the pages only say "fp16 scale/zero"; out-of-range values are
    outside the method's contract and are saturated rather than sent to inf.
    """
    x = np.clip(np.asarray(x, dtype=np.float64), -F16_MAX, F16_MAX)
    return x.astype(np.float16).astype(np.float64)


def page_bytes(head_dim: int = HEAD_DIM, group: int = 128) -> int:
    """Bytes of one (block, KV head) page: 2-bit K and V codes for 16 tokens plus
    one fp16 (scale, zero) pair per token, group and K/V."""
    G = head_dim // group
    return 2 * BLOCK * head_dim // 4 + 2 * BLOCK * G * 4


def bits_per_element(head_dim: int = HEAD_DIM, group: int = 128) -> float:
    """Stored bits per cached K or V element."""
    return page_bytes(head_dim, group) * 8 / (2 * BLOCK * head_dim)


# --------------------------------------------------------------------------- append
def rotate(x, R):
    """Row-vector rotation x @ R for x [..., Hkv, d] and R [Hkv, d, d]
    ([OptR] "Core claim": one orthogonal rotation per KV head).  R None is the
    identity: no rotation (the unrotated INT2 cache the rotations are
    compared against)."""
    x = np.asarray(x, np.float64)
    if R is None:
        return x.copy()
    R = np.asarray(R, np.float64)
    return np.einsum("...hi,hij->...hj", x, R)


def encode_groups(x, group: int, clip: float):
    """Clipped asymmetric INT2 round-to-nearest over groups of the last axis
    ([OptR] "What carries the argument": clipping, grouping, rounding;
    "Assumptions & free parameters": clipping ratios c_K, c_V).

    Readings: clipping scales both group end points by c (lo = c*min,
    hi = c*max); the grid is z + s*{0,1,2,3} with s = (hi-lo)/3, z = lo, both
    stored as fp16; codes are taken against the stored fp16 s16/z16 with
    round-half-even and clamped to [0, 3]; a group whose s16 is 0 stores
    code 0 everywhere.

    Returns (s16, z16, codes, s_raw, z_raw) where s_raw/z_raw are the float64
    values before fp16 rounding.
    """
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    G = d // group
    xg = x.reshape(x.shape[:-1] + (G, group))
    lo = np.float64(clip) * xg.min(axis=-1)
    hi = np.float64(clip) * xg.max(axis=-1)
    s_raw = (hi - lo) / LEVELS
    z_raw = lo
    s16 = fp16_sat(s_raw)
    z16 = fp16_sat(z_raw)
    codes = quantize_on_grid(x, s16, z16, group)
    return s16, z16, codes, s_raw, z_raw


def quantize_on_grid(x, s16, z16, group: int):
    """Codes of x [..., d] on the grid z16 + s16*{0..3} of each group
    ([..., G] each): clamp(rint((x - z16)/s16), 0, 3), 0 where s16 == 0."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    G = d // group
    xg = x.reshape(x.shape[:-1] + (G, group))
    s16 = np.asarray(s16, np.float64)[..., None]
    z16 = np.asarray(z16, np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (xg - z16) / s16
    codes = np.clip(np.rint(t), 0, 3)
    codes = np.where(s16 == 0, 0, codes).astype(np.uint8)
    return codes.reshape(x.shape)


def key_rotation(rot_k, h, d: int = HEAD_DIM):
    """R_K of KV head h as float64; rot_k None (keys encoded unrotated) is the
    identity."""
    if rot_k is None:
        return np.eye(d)
    return np.asarray(rot_k[h], np.float64)


def value_rotation(rot_v, h, d: int = HEAD_DIM):
    """R_V of KV head h as float64; rot_v None is the folded form ([OptR]
    "If this is right": the value rotations are folded into W_V and W_O), where
    the values arrive already rotated and the output stays in that basis, i.e.
    the identity here."""
    if rot_v is None:
        return np.eye(d)
    return np.asarray(rot_v[h], np.float64)


def encode_tokens(k, v, mu, rot_k, rot_v, group: int, clip_k: float, clip_v: float):
    """Centre, rotate and quantise new tokens.

    k, v: [..., Hkv, d]; mu: [Hkv, d]; rot_k, rot_v: [Hkv, d, d] (rot_v None:
    values folded, encoded as given; rot_k None: centred keys unrotated).
    Key centring subtracts mu before rotation ([OptR] "What carries the
    argument", mechanism 2); values are not centred.
    """
    x = rotate(np.asarray(k, np.float64) - np.asarray(mu, np.float64), rot_k)
    y = rotate(v, rot_v)
    ks, kz, kc, ks_raw, kz_raw = encode_groups(x, group, clip_k)
    vs, vz, vc, vs_raw, vz_raw = encode_groups(y, group, clip_v)
    return dict(x=x, y=y, k_s=ks, k_z=kz, k_codes=kc, v_s=vs, v_z=vz, v_codes=vc,
                k_s_raw=ks_raw, k_z_raw=kz_raw, v_s_raw=vs_raw, v_z_raw=vz_raw)


# --------------------------------------------------------------------------- layout
def k_code_site(t, i):
    """(byte offset in page, bit shift) of K code of token t, channel i."""
    t = np.asarray(t)
    i = np.asarray(i)
    return 32 * t + i // 4, 2 * (i % 4)


def v_code_site(t, i):
    """(byte offset in page, bit shift) of V code of token t, channel i."""
    t = np.asarray(t)
    i = np.asarray(i)
    word = 8 * (i % 16) + i // 16  # one 32-bit word per channel and page
    u = (3 * t) % 16               # code position of token t in the word
    return 512 + 4 * word + u // 4, 2 * (u % 4)


def sz_site(t, gidx, group: int, which: str):
    """Byte offset in page of the fp16 scale of (token t, group gidx) of K or V;
    the zero follows at +2."""
    G = HEAD_DIM // group
    base = 1024 if which == "k" else 1024 + 64 * G
    return base + (np.asarray(t) * G + np.asarray(gidx)) * 4


def _page_base(block_table, b, pos, h, Hkv, pb):
    blk = np.asarray(block_table)[b, pos // BLOCK].astype(np.int64)
    return (blk * Hkv + h) * pb


def write_tokens(cache, block_table, b, positions, h, enc_idx, enc, Hkv, group):
    """Store encoded tokens enc[...][enc_idx] of KV head h at the given positions
    of sequence b into the flat uint8 cache (in place)."""
    pb = page_bytes(HEAD_DIM, group)
    flat = cache.reshape(-1)
    positions = np.asarray(positions, np.int64)
    base = _page_base(block_table, b, positions, h, Hkv, pb)          # [n]
    t = positions % BLOCK
    ch = np.arange(HEAD_DIM)
    G = HEAD_DIM // group
    for which, codes_key, site in (("k", "k_codes", k_code_site), ("v", "v_codes", v_code_site)):
        codes = enc[codes_key][enc_idx].astype(np.uint8)               # [n][d]
        byte, sh = site(t[:, None], ch[None, :])
        idx = (base[:, None] + byte).reshape(-1)
        sh = np.broadcast_to(sh, codes.shape).reshape(-1).astype(np.uint8)
        np.bitwise_and.at(flat, idx, (~(np.uint8(3) << sh)).astype(np.uint8))
        np.bitwise_or.at(flat, idx, (codes.reshape(-1) << sh).astype(np.uint8))
        s = enc[which + "_s"][enc_idx].astype(np.float16)              # [n][G]
        z = enc[which + "_z"][enc_idx].astype(np.float16)
        off = base[:, None] + sz_site(t[:, None], np.arange(G)[None, :], group, which)
        pair = np.stack([s, z], axis=-1).view(np.uint8)                # [n][G][4]
        for k in range(4):
            flat[(off + k).reshape(-1)] = pair[..., k].reshape(-1)


def read_tokens(cache, block_table, b, positions, h, Hkv, group):
    """Codes and fp16 scale/zero of KV head h at positions of sequence b.
    Returns dict with k_codes, v_codes [n][d] and k_s, k_z, v_s, v_z [n][G]."""
    pb = page_bytes(HEAD_DIM, group)
    flat = cache.reshape(-1)
    positions = np.asarray(positions, np.int64)
    base = _page_base(block_table, b, positions, h, Hkv, pb)
    t = positions % BLOCK
    ch = np.arange(HEAD_DIM)
    G = HEAD_DIM // group
    out = {}
    for which, site in (("k", k_code_site), ("v", v_code_site)):
        byte, sh = site(t[:, None], ch[None, :])
        out[which + "_codes"] = (flat[base[:, None] + byte] >> sh) & 3
        off = base[:, None] + sz_site(t[:, None], np.arange(G)[None, :], group, which)
        raw = np.stack([flat[off + k] for k in range(4)], axis=-1).astype(np.uint8)
        sz = raw.view(np.float16).astype(np.float64)                  # [n][G][2]
        out[which + "_s"] = sz[..., 0]
        out[which + "_z"] = sz[..., 1]
    return out


def append(cache, block_table, start_pos, k, v, mu, rot_k, rot_v, group, clip_k, clip_v):
    """Encode k, v [B][T][Hkv][d] and store token tau of sequence b at position
    start_pos[b] + tau.  Returns the encoding dict (for parity checks)."""
    k = np.asarray(k, np.float64)
    B, T, Hkv, _ = k.shape
    enc = encode_tokens(k, v, mu, rot_k, rot_v, group, clip_k, clip_v)
    for b in range(B):
        pos = int(start_pos[b]) + np.arange(T)
        for h in range(Hkv):
            sel = {key: val[b, :, h] for key, val in enc.items()}
            write_tokens(cache, block_table, b, pos, h, slice(None), sel, Hkv, group)
    return enc


# --------------------------------------------------------------------------- decode
def dequant(s16, z16, codes, group: int):
    """x_hat = s16 * code + z16 per group ([OptR] "What carries the argument":
    dequantisation)."""
    codes = np.asarray(codes, np.float64)
    d = codes.shape[-1]
    cg = codes.reshape(codes.shape[:-1] + (d // group, group))
    return (np.asarray(s16)[..., None] * cg + np.asarray(z16)[..., None]).reshape(codes.shape)


def attend(q_r, k_hat, v_hat, sm_scale: float):
    """Exact softmax attention of one query over N keys/values (float64,
    max-subtracted).  N = 0 gives a zero vector."""
    k_hat = np.asarray(k_hat, np.float64)
    v_hat = np.asarray(v_hat, np.float64)
    if k_hat.shape[0] == 0:
        return np.zeros(v_hat.shape[-1])
    logits = np.float64(sm_scale) * (k_hat @ np.asarray(q_r, np.float64))
    p = np.exp(logits - logits.max())
    p /= p.sum()
    return p @ v_hat


def plain_attention(q, k, v, sm_scale: float):
    """Unquantised attention of one query over raw keys/values (information)."""
    return attend(q, k, v, sm_scale)


def decode(cache, block_table, ctx_len, q, rot_k, rot_v, sm_scale: float, num_kv_heads: int,
           group: int, pairs=None):
    """Decode attention over the INT2 paged cache.

    q: [B][Hq][d]; rot_k, rot_v: [Hkv][d][d]; ctx_len: [B].
    Query head hq reads KV head hq // (Hq/Hkv) (grouped-query attention; the
    pages do not state the grouping, consecutive heads share a KV head here).
    pairs: optional list of (b, hq) to compute; others are left as NaN.
    Returns o [B][Hq][d] float64.
    """
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hg = Hq // num_kv_heads
    out = np.full((B, Hq, d), np.nan)
    want = set(pairs) if pairs is not None else None
    for b in range(B):
        n = int(ctx_len[b])
        for h in range(num_kv_heads):
            heads = [hq for hq in range(h * Hg, (h + 1) * Hg) if want is None or (b, hq) in want]
            if not heads:
                continue
            tok = read_tokens(cache, block_table, b, np.arange(n), h, num_kv_heads, group)
            k_hat = dequant(tok["k_s"], tok["k_z"], tok["k_codes"], group)
            v_hat = dequant(tok["v_s"], tok["v_z"], tok["v_codes"], group)
            Rk = key_rotation(rot_k, h, d)
            Rv = value_rotation(rot_v, h, d)
            for hq in heads:
                q_r = q[b, hq] @ Rk
                o_r = attend(q_r, k_hat, v_hat, sm_scale)
                out[b, hq] = o_r @ Rv.T
    return out


# --------------------------------------------------------------------------- Eq. 8
# [OptR] abstract, "What carries the argument" and "Core claim": the error of
# the attention output after the output projection W_O splits exactly into a
# key-induced term (the quantised keys move the attention distribution, the
# change weighted by the exact values) and a value-induced term (the value
# errors weighted by the quantised-key distribution):
#     y  = (sum_s p_s v_s) W_O^T,   y~ = (sum_s p~_s v~_s) W_O^T
#     y~ - y = (sum_s (p~_s - p_s) v_s) W_O^T + (sum_s p~_s (v~_s - v_s)) W_O^T
# with p = softmax(sm_scale q . k_s), p~ = softmax(sm_scale q . k~_s).
def dequantized_kv(cache, block_table, b, n, h, num_kv_heads, group, mu, rot_k, rot_v):
    """Keys and values of KV head h, positions [0, n) of sequence b, as the
    INT2 cache represents them in the original basis: k~ = k_hat R_K^T + mu,
    v~ = v_hat R_V^T (the inverse of the append's centring and rotations)."""
    tok = read_tokens(cache, block_table, b, np.arange(n), h, num_kv_heads, group)
    k_hat = dequant(tok["k_s"], tok["k_z"], tok["k_codes"], group)
    v_hat = dequant(tok["v_s"], tok["v_z"], tok["v_codes"], group)
    Rk = key_rotation(rot_k, h)
    Rv = value_rotation(rot_v, h)
    return k_hat @ Rk.T + np.asarray(mu[h], np.float64), v_hat @ Rv.T


def _softmax_weights(q, keys, sm_scale):
    logits = np.float64(sm_scale) * (np.asarray(keys, np.float64) @ np.asarray(q, np.float64))
    p = np.exp(logits - logits.max())
    return p / p.sum()


def eq8_decomposition(q, k, v, k_tilde, v_tilde, w_o, sm_scale: float):
    """Post-W_O error of one query's attention over N tokens and its two terms.

    q [d]; k, v [N][d] exact keys and values; k_tilde, v_tilde [N][d] their
    quantised versions in the same basis; w_o [D][d] (y = o W_O^T).
    Returns y, y_tilde, key_term, value_term (each [D]) and e_out = |y~ - y|^2.
    """
    p = _softmax_weights(q, k, sm_scale)
    p_t = _softmax_weights(q, k_tilde, sm_scale)
    v = np.asarray(v, np.float64)
    v_t = np.asarray(v_tilde, np.float64)
    w_o = np.asarray(w_o, np.float64)
    y = (p @ v) @ w_o.T
    y_t = (p_t @ v_t) @ w_o.T
    key_term = ((p_t - p) @ v) @ w_o.T
    value_term = (p_t @ (v_t - v)) @ w_o.T
    return {"y": y, "y_tilde": y_t, "key_term": key_term, "value_term": value_term,
            "e_out": float(np.sum((y_t - y) ** 2))}


# --------------------------------------------------------------------------- BF16 windows
# [OptR] "Assumptions & free parameters": the deployed cache keeps 64 sink
# tokens and the 256 most recent tokens in BF16 beside the INT2 body.  The
# pages give only the two sizes; the readings taken here:
#   - a context of n tokens splits into sinks [0, min(64, n)), the recent
#     window [max(64, n - 256), n) and the INT2 body [64, n - 256) between;
#   - window tokens are kept as given (uncentred, unrotated), rounded to BF16;
#     their logits subtract the key mean too, q . (k - mu), so that every
#     logit of the context carries the same -q . mu shift as the centred body
#     keys (softmax-invariant, "What carries the argument", mechanism 2);
#   - a token leaving the recent window is encoded into the INT2 body from its
#     BF16 window copy;
#   - window store: slot of position p is p for p < 64, else
#     64 + (p - 64) mod 256 (a ring).
SINK = 64
RECENT = 256
WINDOW = SINK + RECENT


def window_slot(pos):
    """Window-store slot of a token position (sinks first, then the ring)."""
    pos = np.asarray(pos)
    return np.where(pos < SINK, pos, SINK + (pos - SINK) % RECENT)


def window_parts(n: int):
    """(sink, body, recent) position ranges of a context of n tokens."""
    n = int(n)
    sink = range(0, min(SINK, n))
    recent = range(max(SINK, n - RECENT), n)
    body = range(SINK, max(SINK, n - RECENT))
    return sink, body, recent


def bf16_round(x):
    """Nearest bfloat16 value (round half to even) as float64."""
    f = np.asarray(x, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return (r.astype(np.uint32)).view(np.float32).astype(np.float64)


def window_write(win_k, win_v, start_pos, k, v):
    """Store tokens k, v [B][T][Hkv][d] at positions start_pos[b] + tau into the
    window store win_k, win_v [B][Hkv][WINDOW][d] (float64 holding BF16
    values), later positions winning a shared ring slot."""
    k = np.asarray(k, np.float64)
    B, T = k.shape[:2]
    for b in range(B):
        for tau in range(T):
            slot = int(window_slot(int(start_pos[b]) + tau))
            win_k[b, :, slot] = bf16_round(k[b, tau])
            win_v[b, :, slot] = bf16_round(np.asarray(v, np.float64)[b, tau])


def append_windowed(cache, block_table, win_k, win_v, start_pos, k, v, mu, rot_k, rot_v,
                    group, clip_k, clip_v):
    """One token per sequence (k, v [B][1][Hkv][d]) at position p = start_pos[b]:
    when p >= WINDOW the token it displaces from the ring, position p - RECENT,
    is encoded into the INT2 body from its window copy; then the new token
    takes the slot."""
    B = np.asarray(k).shape[0]
    for b in range(B):
        p = int(start_pos[b])
        slot = int(window_slot(p))
        if p >= WINDOW:
            old_k = win_k[b:b + 1, :, slot][:, None]
            old_v = win_v[b:b + 1, :, slot][:, None]
            append(cache, block_table[b:b + 1], [p - RECENT], old_k, old_v, mu, rot_k, rot_v,
                   group, clip_k, clip_v)
        window_write(win_k[b:b + 1], win_v[b:b + 1], [p], np.asarray(k)[b:b + 1],
                     np.asarray(v)[b:b + 1])


def decode_windowed(cache, block_table, ctx_len, q, rot_k, rot_v, mu, win_k, win_v,
                    sm_scale: float, num_kv_heads: int, group: int, pairs=None):
    """Decode attention over sinks + INT2 body + recent window: one softmax over
    the whole context.  Body tokens as in decode(); window token t scores
    sm_scale * q . (k_t - mu_h) and contributes its value as stored.
    Returns o [B][Hq][d] float64 (NaN for pairs not requested)."""
    q = np.asarray(q, np.float64)
    mu = np.asarray(mu, np.float64)
    B, Hq, d = q.shape
    Hg = Hq // num_kv_heads
    out = np.full((B, Hq, d), np.nan)
    want = set(pairs) if pairs is not None else None
    for b in range(B):
        sink, body, recent = window_parts(int(ctx_len[b]))
        wpos = np.array(list(sink) + list(recent), dtype=np.int64)
        bpos = np.array(list(body), dtype=np.int64)
        for h in range(num_kv_heads):
            heads = [hq for hq in range(h * Hg, (h + 1) * Hg) if want is None or (b, hq) in want]
            if not heads:
                continue
            slots = window_slot(wpos)
            kw = np.asarray(win_k[b, h], np.float64)[slots] - mu[h]
            vw = np.asarray(win_v[b, h], np.float64)[slots]
            tok = read_tokens(cache, block_table, b, bpos, h, num_kv_heads, group)
            k_hat = dequant(tok["k_s"], tok["k_z"], tok["k_codes"], group)
            v_hat = dequant(tok["v_s"], tok["v_z"], tok["v_codes"], group)
            Rk = key_rotation(rot_k, h)
            Rv = value_rotation(rot_v, h)
            for hq in heads:
                if len(wpos) + len(bpos) == 0:
                    out[b, hq] = 0.0
                    continue
                logits = np.float64(sm_scale) * np.concatenate(
                    [kw @ q[b, hq], k_hat @ (q[b, hq] @ Rk)])
                p = np.exp(logits - logits.max())
                p /= p.sum()
                nw = len(wpos)
                out[b, hq] = p[:nw] @ vw + (p[nw:] @ v_hat) @ Rv.T
    return out
