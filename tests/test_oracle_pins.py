"""Pins of the float64 oracle to facts fixed outside the oracle itself.

Each test checks the oracle against something it does not compute by the same
formula: IEEE binary16 facts, values already on the INT2 grid, brute-force
nearest-grid-point search, hand-worked examples, closed forms of softmax on
one or two keys, exact invariances (key centring, orthogonal rotation), and
hand-computed byte positions of the cache layout.

Sources: "Output-Aware Rotation for INT2 KV-Cache Quantization" (Pith review
of arXiv 2608.02691) -- "What carries the argument" (key centring is
attention-equivalent; rotation, clipping, grouping, rounding, dequantisation
and inverse rotation), "Core claim" (one rotation per KV head and layer),
"Assumptions & free parameters" (clip ratios; centring leaves full-precision
softmax unchanged; exp of a skew-symmetric matrix is orthogonal).
"""
import math
import os

import numpy as np
import pytest

import oracle as O
from workload import EXPM_SCALE, WORKLOADS, corrected_rotation, haar_orthogonal, hadamard, \
    make_static, scaled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- fp16 rounding
def test_fp16_rounding_ieee_facts():
    # binary16: 1/3 -> 0x3555 = 1365/4096; ties to even around 1.0; saturation.
    assert O.fp16_sat(1 / 3) == 1365 / 4096
    assert O.fp16_sat(1 + 2 ** -11) == 1.0                 # tie -> even mantissa
    assert O.fp16_sat(1 + 3 * 2 ** -11) == 1 + 2 ** -9     # tie -> even mantissa
    assert O.fp16_sat(65519.0) == 65504.0
    assert O.fp16_sat(1e9) == 65504.0 and O.fp16_sat(-1e9) == -65504.0
    assert O.fp16_sat(2 ** -24) == 2 ** -24                 # smallest subnormal
    assert O.fp16_sat(2 ** -26) == 0.0


# ----------------------------------------------------------------- quantiser
def _grid_group(rng, group, s16, z16):
    q = rng.integers(0, 4, size=group)
    q[rng.integers(group)] = 0
    q[(rng.integers(group - 1) + 1 + np.flatnonzero(q == 0)[0]) % group] = 3
    return q, z16 + s16 * q


def test_on_grid_values_round_trip():
    """Values already on a dyadic fp16 grid re-quantise to themselves (c = 1)."""
    rng = np.random.default_rng(1)
    for group in (64, 128):
        for s16, z16 in [(0.25, -1.5), (2.0, 3.0), (0.0078125, -0.5), (16.0, -24.0)]:
            rows = []
            codes = []
            for _ in range(128 // group):
                q, x = _grid_group(rng, group, s16, z16)
                rows.append(x)
                codes.append(q)
            x = np.concatenate(rows)
            s, z, c, _, _ = O.encode_groups(x, group, 1.0)
            assert np.all(s == s16) and np.all(z == z16)
            assert np.array_equal(c, np.concatenate(codes))


def test_codes_are_nearest_grid_point_brute_force():
    """RTN + clamp equals the exhaustive argmin over the 4 grid points."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((500, 128)) * rng.uniform(0.1, 30, size=(500, 1))
    for group in (64, 128):
        for clip in (1.0, 0.9):
            s, z, c, _, _ = O.encode_groups(x, group, clip)
            G = 128 // group
            grid = z.reshape(500, G, 1, 1) + s.reshape(500, G, 1, 1) * np.arange(4).reshape(1, 1, 1, 4)
            dist = np.abs(x.reshape(500, G, group, 1) - grid)
            best = dist.argmin(-1).reshape(500, 128)
            srt = np.sort(dist, axis=-1).reshape(500, 128, 4)
            clear = srt[..., 1] - srt[..., 0] > 1e-9   # no tie
            assert clear.mean() > 0.99
            assert np.array_equal(c[clear], best[clear])


def test_clip_scales_end_points_hand_example():
    """c = 0.5 on a group spanning [-4, 8]: lo = -2, hi = 4, s = 2, z = -2."""
    x = np.zeros(64)
    x[:6] = [-4.0, 8.0, 0.0, 1.0, 3.0, 2.5]
    x[6:] = 2.0
    s, z, c, s_raw, z_raw = O.encode_groups(x, 64, 0.5)
    assert s_raw[0] == 2.0 and z_raw[0] == -2.0 and s[0] == 2.0 and z[0] == -2.0
    # -4 clamps to 0; 8 clamps to 3; 0 -> 1; 1 -> rint(1.5) = 2 (tie to even);
    # 3 -> rint(2.5) = 2 (tie to even); 2.5 -> rint(2.25) = 2; 2 -> 2
    assert list(c[:7]) == [0, 3, 1, 2, 2, 2, 2]


def test_degenerate_group_stores_zero_codes():
    x = np.full(128, 3.25)
    s, z, c, _, _ = O.encode_groups(x, 128, 1.0)
    assert s[0] == 0.0 and z[0] == 3.25 and not c.any()
    s, z, c, _, _ = O.encode_groups(np.full(128, 1e-9) + np.arange(128) * 1e-12, 128, 1.0)
    assert s[0] == 0.0 and not c.any()                   # s underflows fp16


def test_scale_zero_are_fp16_rounded():
    x = np.linspace(-1.0, 2.0 / 3.0 + 1e-3, 128)
    s, z, c, s_raw, z_raw = O.encode_groups(x, 128, 1.0)
    assert s_raw[0] != s[0]
    assert s[0] == float(np.float16(s_raw[0])) and z[0] == float(np.float16(z_raw[0]))


# ----------------------------------------------------------------- rotation
def _signed_perm(rng, d):
    sigma = rng.permutation(d)
    while np.all(sigma[sigma] == np.arange(d)):
        sigma = rng.permutation(d)
    sign = rng.choice([-1.0, 1.0], size=d)
    R = np.zeros((d, d))
    R[np.arange(d), sigma] = sign          # e_i -> sign_i e_sigma(i)
    return R, sigma, sign


def test_rotation_is_row_vector_times_R():
    """x_rot = x @ R: with R[i, sigma(i)] = sign_i, x_rot[sigma(i)] = sign_i x[i]."""
    rng = np.random.default_rng(3)
    R, sigma, sign = _signed_perm(rng, 128)
    x = rng.standard_normal((3, 1, 128))
    xr = O.rotate(x, R[None])
    expect = np.empty_like(x)
    expect[..., sigma] = x * sign
    assert np.array_equal(xr, expect)


def test_generated_rotations_are_orthogonal_and_preserve_dot_products():
    rng = np.random.default_rng(4)
    for R in (haar_orthogonal(rng, 128), hadamard(128) / math.sqrt(128) @ haar_orthogonal(rng, 128)):
        assert np.abs(R.T @ R - np.eye(128)).max() < 1e-12
        q, k = rng.standard_normal(128), rng.standard_normal(128)
        assert abs((q @ R) @ (k @ R) - q @ k) <= 1e-12 * np.abs(q).sum() * np.abs(k).sum()
    H = hadamard(8)
    assert np.array_equal(H @ H.T, 8 * np.eye(8))


# ----------------------------------------------------------------- attention
def test_attention_closed_forms():
    rng = np.random.default_rng(5)
    q = rng.standard_normal(16)
    k = rng.standard_normal((2, 16))
    v = rng.standard_normal((2, 16))
    scale = 0.25
    # N = 1: the value itself
    assert np.allclose(O.attend(q, k[:1], v[:1], scale), v[0], rtol=0, atol=0)
    # N = 2: logistic weights
    l0, l1 = scale * sum(q[i] * k[0, i] for i in range(16)), scale * sum(q[i] * k[1, i] for i in range(16))
    p0 = 1.0 / (1.0 + math.exp(l1 - l0))
    assert np.allclose(O.attend(q, k, v, scale), p0 * v[0] + (1 - p0) * v[1], rtol=1e-14, atol=1e-14)
    # identical keys: mean of values
    kk = np.repeat(k[:1], 5, axis=0)
    vv = rng.standard_normal((5, 16))
    assert np.allclose(O.attend(q, kk, vv, scale), vv.mean(0), rtol=1e-14, atol=1e-14)
    # huge logit gap: one-hot, no overflow
    big = np.stack([k[0] * 0, k[0] * 0])
    big[0, 0] = 1e4
    qq = np.zeros(16)
    qq[0] = 1.0
    assert np.array_equal(O.attend(qq, big, v, 1.0), v[0])
    # empty context
    assert np.array_equal(O.attend(q, k[:0], v[:0], scale), np.zeros(16))


def test_key_centring_leaves_softmax_unchanged_exactly():
    """Subtracting one vector from every key shifts all logits by q.mu; with
    small integers every dot product is exact, so softmax is bit-identical."""
    rng = np.random.default_rng(6)
    q = rng.integers(-4, 5, size=32).astype(float)
    k = rng.integers(-8, 9, size=(40, 32)).astype(float)
    v = rng.standard_normal((40, 32))
    mu = rng.integers(-6, 7, size=32).astype(float)
    a = O.attend(q, k, v, 1 / 8)
    b = O.attend(q, k - mu, v, 1 / 8)
    assert np.array_equal(a, b)
    # Gaussian inputs: a few ulp
    qg, kg, mug = rng.standard_normal(32), rng.standard_normal((40, 32)), rng.standard_normal(32) * 3
    a, b = O.attend(qg, kg, v, 0.2), O.attend(qg, kg - mug, v, 0.2)
    assert np.abs(a - b).max() <= 1e-13 * np.abs(a).max()


# ----------------------------------------------------------------- layout
def test_layout_golden_examples():
    lines = [ln.split() for ln in open(os.path.join(GOLDEN, "layout_examples.txt"))
             if ln.strip() and not ln.startswith("#")]
    assert len(lines) == 9
    for kind, t, i, code, byte, value in lines:
        t, i, code, byte, value = int(t), int(i), int(code), int(byte), int(value, 16)
        site = O.k_code_site if kind == "k" else O.v_code_site
        off, sh = site(t, i)
        assert int(off) == byte and (code << int(sh)) == value
        # through the page writer: one page, one head, one token with one code
        enc = {key: np.zeros((1, 128) if "codes" in key else (1, 1)) for key in
               ("k_codes", "v_codes", "k_s", "k_z", "v_s", "v_z")}
        enc[kind + "_codes"][0, i] = code
        cache = np.zeros((1, 1, O.page_bytes(128, 128)), np.uint8)
        O.write_tokens(cache, np.zeros((1, 1), np.int32), 0, [t], 0, slice(None), enc, 1, 128)
        nz = np.flatnonzero(cache.reshape(-1))
        assert list(nz) == [byte] and cache.reshape(-1)[byte] == value
    # the worked K byte: codes [1, 2, 3, 0] on channels 0..3 -> 0x39
    enc = {key: np.zeros((1, 128) if "codes" in key else (1, 1)) for key in
           ("k_codes", "v_codes", "k_s", "k_z", "v_s", "v_z")}
    enc["k_codes"][0, :4] = [1, 2, 3, 0]
    cache = np.zeros((1, 1, O.page_bytes()), np.uint8)
    O.write_tokens(cache, np.zeros((1, 1), np.int32), 0, [0], 0, slice(None), enc, 1, 128)
    assert cache.reshape(-1)[0] == 0x39


def test_scale_zero_sites_and_page_size():
    assert O.page_bytes(128, 128) == 1152 and O.page_bytes(128, 64) == 1280
    assert int(O.sz_site(3, 1, 64, "k")) == 1052 and int(O.sz_site(3, 1, 64, "v")) == 1180
    assert int(O.sz_site(15, 0, 128, "v")) == 1024 + 64 + 60
    enc = {key: np.zeros((1, 128) if "codes" in key else (1, 2)) for key in
           ("k_codes", "v_codes", "k_s", "k_z", "v_s", "v_z")}
    enc["v_s"][0, 1] = 0.75      # fp16 0x3A00
    enc["v_z"][0, 1] = -2.0      # fp16 0xC000
    cache = np.zeros((1, 1, O.page_bytes(128, 64)), np.uint8)
    O.write_tokens(cache, np.zeros((1, 1), np.int32), 0, [3], 0, slice(None), enc, 1, 64)
    flat = cache.reshape(-1)
    assert list(flat[1180:1184]) == [0x00, 0x3A, 0x00, 0xC0]


def test_pack_unpack_identity_over_all_byte_values():
    """Every byte value of every code site survives write -> read."""
    rng = np.random.default_rng(7)
    for group in (64, 128):
        cache = np.zeros((3, 2, O.page_bytes(128, group)), np.uint8)
        table = np.array([[2, 0, 1]], np.int32)
        pos = np.arange(48)
        G = 128 // group
        enc = {"k_codes": rng.integers(0, 4, (48, 128)), "v_codes": rng.integers(0, 4, (48, 128)),
               "k_s": O.fp16_sat(rng.standard_normal((48, G))), "k_z": O.fp16_sat(rng.standard_normal((48, G))),
               "v_s": O.fp16_sat(rng.standard_normal((48, G))), "v_z": O.fp16_sat(rng.standard_normal((48, G)))}
        for h in range(2):
            O.write_tokens(cache, table, 0, pos, h, slice(None), enc, 2, group)
        for h in range(2):
            got = O.read_tokens(cache, table, 0, pos, h, 2, group)
            for key in enc:
                assert np.array_equal(got[key], enc[key]), key
    # every byte value 0..255 at a K byte and at a V byte: the four codes that
    # share the byte are written (as four tokens/channels) and read back
    for val in range(256):
        four = [(val >> (2 * i)) & 3 for i in range(4)]
        for kind in ("k", "v"):
            cache = np.zeros((1, 1, O.page_bytes()), np.uint8)
            table = np.zeros((1, 1), np.int32)
            site = O.k_code_site if kind == "k" else O.v_code_site
            target = (32 * (val % 16) + val // 16) if kind == "k" else 512 + 2 * val + (val % 2)
            # the four (token, channel) codes stored in byte `target`, ordered by bit
            sites = sorted((int(site(tt, ii)[1]), tt, ii) for tt in range(16) for ii in range(128)
                           if int(site(tt, ii)[0]) == target)
            assert [sh for sh, _, _ in sites] == [0, 2, 4, 6]
            toks = [tt for _, tt, _ in sites]
            chans = [ii for _, _, ii in sites]
            for tok, ch, code in zip(toks, chans, four):
                enc = {key: np.zeros((1, 128) if "codes" in key else (1, 1)) for key in
                       ("k_codes", "v_codes", "k_s", "k_z", "v_s", "v_z")}
                old = O.read_tokens(cache, table, 0, [tok], 0, 1, 128)
                enc[kind + "_codes"][0] = old[kind + "_codes"][0]
                enc[kind + "_codes"][0, ch] = code
                O.write_tokens(cache, table, 0, [tok], 0, slice(None), enc, 1, 128)
            assert cache.reshape(-1)[target] == val
            got = O.read_tokens(cache, table, 0, toks, 0, 1, 128)[kind + "_codes"]
            assert [int(got[n, chans[n]]) for n in range(4)] == four
    # overwriting one token leaves its neighbours' bits untouched
    cache = np.full((1, 1, O.page_bytes()), 0xFF, np.uint8)
    enc = {key: np.zeros((1, 128) if "codes" in key else (1, 1)) for key in
           ("k_codes", "v_codes", "k_s", "k_z", "v_s", "v_z")}
    O.write_tokens(cache, np.zeros((1, 1), np.int32), 0, [9], 0, slice(None), enc, 1, 128)
    got = O.read_tokens(cache, np.zeros((1, 1), np.int32), 0, np.arange(16), 0, 1, 128)
    assert not got["v_codes"][9].any() and np.all(got["v_codes"][np.arange(16) != 9] == 3)
    assert not got["k_codes"][9].any() and np.all(got["k_codes"][np.arange(16) != 9] == 3)


def test_bits_per_element_closed_form():
    # group 64 stores 2.5 bits/element (stated for the decode-heavy workload); group 128: 2.25
    assert O.bits_per_element(128, 64) == 2.5
    assert O.bits_per_element(128, 128) == 2.25


# ----------------------------------------------------------------- end to end
def _one_layer(rng, Hkv, group, R_k, R_v):
    cache = np.zeros((4, Hkv, O.page_bytes(128, group)), np.uint8)
    table = np.array([[3, 1, 0, 2]], np.int32)
    return cache, table


def test_value_path_single_token_returns_value_exactly():
    """Append v with y = v @ R_V on a dyadic grid, decode with one token: the
    output is v exactly (p = 1, dequantisation exact, inverse rotation exact for
    a signed permutation)."""
    rng = np.random.default_rng(8)
    R_v, _, _ = _signed_perm(rng, 128)
    R_k, _, _ = _signed_perm(rng, 128)
    for group in (64, 128):
        y = np.concatenate([_grid_group(rng, group, 0.5, -1.0)[1] for _ in range(128 // group)])
        v = y @ R_v.T
        k = rng.integers(-3, 4, size=128).astype(float)
        cache, table = _one_layer(rng, 1, group, R_k, R_v)
        O.append(cache, table, [37], k[None, None, None], v[None, None, None], np.zeros((1, 128)),
                 R_k[None], R_v[None], group, 0.9, 1.0)
        table_full = table
        q = rng.standard_normal((1, 1, 128))
        # ctx 38 would include unwritten slots; read the single written token
        tok = O.read_tokens(cache, table_full, 0, [37], 0, 1, group)
        v_hat_r = O.dequant(tok["v_s"], tok["v_z"], tok["v_codes"], group)[0]
        assert np.array_equal(v_hat_r, y)
        o_r = O.attend(q[0, 0] @ R_k, O.dequant(tok["k_s"], tok["k_z"], tok["k_codes"], group), v_hat_r[None], 0.1)
        assert np.array_equal(o_r @ R_v.T, v)
        # decode over a context of one token
        cache2, _ = _one_layer(rng, 1, group, R_k, R_v)
        O.append(cache2, table, [0], k[None, None, None], v[None, None, None], np.zeros((1, 128)),
                 R_k[None], R_v[None], group, 0.9, 1.0)
        o = O.decode(cache2, table, [1], q, R_k[None], R_v[None], 0.1, 1, group)
        assert np.array_equal(o[0, 0], v)


def test_key_centring_is_applied_before_rotation():
    """k = mu + x with x on the grid (R = I, c = 1): the stored grid is x's."""
    rng = np.random.default_rng(9)
    x = _grid_group(rng, 128, 0.25, -0.75)[1]
    mu = rng.integers(-64, 64, size=128) / 8.0
    k = mu + x
    enc = O.encode_tokens(k[None, None], np.zeros((1, 1, 128)), mu[None], np.eye(128)[None],
                          np.eye(128)[None], 128, 1.0, 1.0)
    assert enc["k_s"][0, 0, 0] == 0.25 and enc["k_z"][0, 0, 0] == -0.75
    assert np.array_equal(enc["k_codes"][0, 0], ((x + 0.75) / 0.25).astype(int))
    # values are not centred
    assert np.array_equal(enc["y"], np.zeros((1, 1, 128)))


def test_decode_scores_with_rotated_query_and_maps_gqa_heads():
    """Keys on the grid in the rotated basis, R_K a non-involutive signed
    permutation: decode logits equal sm_scale * q . k (rotation preserved), so
    two-token outputs follow the logistic closed form; query head hq reads KV
    head hq // (Hq/Hkv)."""
    rng = np.random.default_rng(10)
    Hkv, Hq, group, scale = 2, 4, 128, 0.3
    Rk = np.stack([_signed_perm(rng, 128)[0] for _ in range(Hkv)])
    Rv = np.stack([_signed_perm(rng, 128)[0] for _ in range(Hkv)])
    cache = np.zeros((2, Hkv, O.page_bytes(128, group)), np.uint8)
    table = np.array([[1]], np.int32)
    ys_k = np.stack([[_grid_group(rng, 128, 0.5, -1.0)[1] for _ in range(Hkv)] for _ in range(2)])
    ys_v = np.stack([[_grid_group(rng, 128, 0.25, -0.5)[1] for _ in range(Hkv)] for _ in range(2)])
    k = np.einsum("thj,hij->thi", ys_k, Rk)   # k = y_k @ R_K^T
    v = np.einsum("thj,hij->thi", ys_v, Rv)
    O.append(cache, table, [0], k[None], v[None], np.zeros((Hkv, 128)), Rk, Rv, group, 1.0, 1.0)
    q = rng.standard_normal((1, Hq, 128))
    o = O.decode(cache, table, [2], q, Rk, Rv, scale, Hkv, group)
    for hq in range(Hq):
        h = hq // (Hq // Hkv)
        l0 = scale * float(np.dot(q[0, hq], k[0, h]))
        l1 = scale * float(np.dot(q[0, hq], k[1, h]))
        p0 = 1.0 / (1.0 + math.exp(l1 - l0))
        expect = p0 * v[0, h] + (1 - p0) * v[1, h]
        assert np.allclose(o[0, hq], expect, rtol=1e-12, atol=1e-12)
    # empty context -> zeros
    o0 = O.decode(cache, table, [0], q, Rk, Rv, scale, Hkv, group)
    assert np.array_equal(o0, np.zeros_like(o0))


# ----------------------------------------------------------------- BF16 windows
# [OptR] "Assumptions & free parameters": 64 sink and 256 recent tokens kept in
# BF16 beside the INT2 body.  The slot mapping, the part boundaries and the
# key-mean convention for window keys are readings stated in the oracle.
def test_window_slots_and_parts_hand_examples():
    assert O.SINK == 64 and O.RECENT == 256 and O.WINDOW == 320
    pos = [0, 1, 63, 64, 65, 319, 320, 321, 575, 576, 1000]
    slot = [0, 1, 63, 64, 65, 319, 64, 65, 319, 64, 64 + (1000 - 64) % 256]
    assert list(O.window_slot(pos)) == slot
    for n, parts in [(0, (0, 0, 0)), (10, (10, 0, 0)), (64, (64, 0, 0)), (65, (64, 0, 1)),
                     (320, (64, 0, 256)), (321, (64, 1, 256)), (400, (64, 80, 256))]:
        s, b, r = O.window_parts(n)
        assert (len(s), len(b), len(r)) == parts, n
        assert sorted(list(s) + list(b) + list(r)) == list(range(n))


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal(4096) * 10.0 ** rng.integers(-8, 8, 4096),
                        [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 65504.0, 3.0e38]])
    ref = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_round(x), ref)
    assert O.bf16_round(1 + 2 ** -8) == 1.0 and O.bf16_round(1 + 3 * 2 ** -8) == 1 + 2 ** -6


def _windowed_layer(rng, n_blocks=40, Hkv=1, group=128):
    cache = np.zeros((n_blocks, Hkv, O.page_bytes(128, group)), np.uint8)
    table = rng.permutation(n_blocks).astype(np.int32)[None]
    return cache, table


def test_windowed_single_token_returns_its_value():
    rng = np.random.default_rng(22)
    cache, table = _windowed_layer(rng)
    win_k = np.zeros((1, 1, O.WINDOW, 128))
    win_v = np.zeros_like(win_k)
    k = rng.standard_normal((1, 1, 1, 128))
    v = rng.standard_normal((1, 1, 1, 128))
    O.window_write(win_k, win_v, [0], k, v)
    q = rng.standard_normal((1, 2, 128))
    R = np.eye(128)[None]
    o = O.decode_windowed(cache, table, [1], q, R, R, rng.standard_normal((1, 128)), win_k, win_v,
                          0.1, 1, 128)
    assert np.array_equal(o[0, 0], O.bf16_round(v[0, 0, 0]))
    assert np.array_equal(o[0, 1], O.bf16_round(v[0, 0, 0]))


def test_windowed_equal_keys_give_the_mean_of_all_values():
    """Every key equals the key mean: window logits q . (k - mu) are 0, and the
    body keys encode to zero codes with scale 0 and zero 0, so every logit is 0
    and the output is the plain mean of the window values (as stored) and the
    dequantised, inverse-rotated body values."""
    rng = np.random.default_rng(23)
    n, group = 400, 128
    Rk = _signed_perm(rng, 128)[0][None]
    Rv = np.linalg.qr(rng.standard_normal((128, 128)))[0][None]
    mu = rng.integers(-40, 40, size=(1, 128)) / 8.0
    cache, table = _windowed_layer(rng)
    win_k = np.zeros((1, 1, O.WINDOW, 128))
    win_v = np.zeros_like(win_k)
    vals = rng.standard_normal((n, 128))
    for p in range(n):
        O.append_windowed(cache, table, win_k, win_v, [p], mu[None, None], vals[p][None, None, None],
                          mu, Rk, Rv, group, 0.9, 0.9)
    q = rng.standard_normal((1, 2, 128))
    o = O.decode_windowed(cache, table, [n], q, Rk, Rv, mu, win_k, win_v, 0.2, 1, group)
    body = np.arange(O.SINK, n - O.RECENT)
    tok = O.read_tokens(cache, table, 0, body, 0, 1, group)
    assert not tok["k_codes"].any() and not tok["k_s"].any() and not tok["k_z"].any()
    v_body = O.dequant(tok["v_s"], tok["v_z"], tok["v_codes"], group) @ Rv[0].T
    win = np.concatenate([np.arange(O.SINK), np.arange(n - O.RECENT, n)])
    expect = np.concatenate([O.bf16_round(vals[win]), v_body]).mean(0)
    assert np.allclose(o[0, 0], expect, rtol=1e-12, atol=1e-12)
    assert np.allclose(o[0, 1], expect, rtol=1e-12, atol=1e-12)


def test_windowed_key_mean_shift_is_softmax_invariant_without_a_body():
    rng = np.random.default_rng(24)
    n = 300
    cache, table = _windowed_layer(rng)
    win_k = np.zeros((1, 1, O.WINDOW, 128))
    win_v = np.zeros_like(win_k)
    O.window_write(win_k, win_v, [0], rng.standard_normal((1, n, 1, 128)),
                   rng.standard_normal((1, n, 1, 128)))
    q = rng.standard_normal((1, 1, 128))
    R = np.eye(128)[None]
    mu = rng.standard_normal((1, 128))
    o1 = O.decode_windowed(cache, table, [n], q, R, R, mu, win_k, win_v, 0.3, 1, 128)
    o2 = O.decode_windowed(cache, table, [n], q, R, R, mu + 5.0, win_k, win_v, 0.3, 1, 128)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)


def test_windowed_stream_keeps_windows_and_encodes_evicted_tokens_like_bulk():
    """Tokens appended one at a time: the window store holds the BF16 sinks and
    the last 256 tokens in their ring slots, and the body holds exactly what a
    bulk append of the BF16-rounded body tokens writes."""
    rng = np.random.default_rng(25)
    n, group, Hkv = 420, 64, 2
    Rk = np.stack([np.linalg.qr(rng.standard_normal((128, 128)))[0] for _ in range(Hkv)])
    Rv = np.stack([np.linalg.qr(rng.standard_normal((128, 128)))[0] for _ in range(Hkv)])
    mu = rng.standard_normal((Hkv, 128))
    k = rng.standard_normal((n, Hkv, 128)) * 3
    v = rng.standard_normal((n, Hkv, 128))
    cache, table = _windowed_layer(rng, Hkv=Hkv, group=group)
    win_k = np.zeros((1, Hkv, O.WINDOW, 128))
    win_v = np.zeros_like(win_k)
    for p in range(n):
        O.append_windowed(cache, table, win_k, win_v, [p], k[p][None, None], v[p][None, None], mu,
                          Rk, Rv, group, 0.9, 0.8)
    for p in list(range(O.SINK)) + list(range(n - O.RECENT, n)):
        s = int(O.window_slot(p))
        assert np.array_equal(win_k[0, :, s], O.bf16_round(k[p]))
        assert np.array_equal(win_v[0, :, s], O.bf16_round(v[p]))
    body = np.arange(O.SINK, n - O.RECENT)
    bulk, _ = _windowed_layer(np.random.default_rng(0), Hkv=Hkv, group=group)
    O.append(bulk, table, [O.SINK], O.bf16_round(k[body])[None], O.bf16_round(v[body])[None], mu,
             Rk, Rv, group, 0.9, 0.8)
    for h in range(Hkv):
        a = O.read_tokens(cache, table, 0, body, h, Hkv, group)
        b = O.read_tokens(bulk, table, 0, body, h, Hkv, group)
        for key in a:
            assert np.array_equal(a[key], b[key]), key


# ----------------------------------------------------------------- corrected rotations R0 exp(A - A^T)
def test_corrected_rotation_of_a_single_plane_is_a_givens_rotation():
    """A = theta e_i e_j^T: exp(A - A^T) turns the (i, j) plane by theta
    (closed form cos/sin) and leaves every other axis fixed; A = 0 gives R0."""
    d = 16
    for (i, j, theta) in [(0, 1, 0.3), (5, 2, -1.1), (3, 15, 2.5)]:
        a = np.zeros((d, d))
        a[i, j] = theta
        r = corrected_rotation(np.eye(d), a)
        want = np.eye(d)
        want[i, i] = want[j, j] = math.cos(theta)
        want[i, j] = math.sin(theta)
        want[j, i] = -math.sin(theta)
        assert np.allclose(r, want, rtol=0, atol=1e-14)
    r0 = hadamard(d) / 4.0
    assert np.array_equal(corrected_rotation(r0, np.zeros((d, d))), r0)


def test_corrected_rotations_are_orthogonal_with_unit_determinant():
    rng = np.random.default_rng(21)
    r0 = hadamard(128) / math.sqrt(128)
    for scale in (EXPM_SCALE, 0.3):
        a = scale * rng.standard_normal((128, 128))
        e = corrected_rotation(np.eye(128), a)
        assert np.abs(e.T @ e - np.eye(128)).max() < 1e-12
        assert abs(np.linalg.det(e) - 1.0) < 1e-9          # exp(trace S) = 1
        r = corrected_rotation(r0, a)
        assert np.abs(r.T @ r - np.eye(128)).max() < 1e-12
    # the workload's corrected rotations, stored float32, stay orthogonal and
    # near their Hadamard base
    w = scaled(WORKLOADS["qwen3_8b_b4_ctx8k"], rotation="hadamard_expm", batch=1, ctx_min=16,
               ctx_max=16)
    st = make_static(w)
    for rk in (st.rot_k[0, 0], st.rot_v[0, 0]):
        rk = rk.astype(np.float64)
        assert np.abs(rk.T @ rk - np.eye(128)).max() < 1e-5
        dist = np.abs(rk - r0).max()
        assert 1e-4 < dist < 0.1


# ----------------------------------------------------------------- Eq. 8 error decomposition
def test_eq8_hand_example():
    """d = 1, two tokens: p = (1/2, 1/2) from equal keys; the quantised keys
    give logits (ln 3, 0), so p~ = (3/4, 1/4); v = (1, 3), v~ = (1, 2),
    W_O = [2].  y = 4, y~ = 2.5; key term ((1/4) 1 - (1/4) 3) 2 = -1; value
    term (3/4 * 0 + 1/4 * (-1)) 2 = -1/2; the two add to y~ - y = -3/2."""
    r = O.eq8_decomposition(np.array([1.0]), np.array([[0.0], [0.0]]), np.array([[1.0], [3.0]]),
                            np.array([[math.log(3.0)], [0.0]]), np.array([[1.0], [2.0]]),
                            np.array([[2.0]]), 1.0)
    assert math.isclose(r["y"][0], 4.0, rel_tol=1e-15)
    assert math.isclose(r["y_tilde"][0], 2.5, rel_tol=1e-15)
    assert math.isclose(r["key_term"][0], -1.0, rel_tol=1e-14)
    assert math.isclose(r["value_term"][0], -0.5, rel_tol=1e-14)
    assert math.isclose(r["e_out"], 2.25, rel_tol=1e-14)


def test_eq8_terms_add_up_and_vanish_in_the_special_cases():
    rng = np.random.default_rng(22)
    n, d, D = 40, 128, 96
    q = rng.standard_normal(d)
    k = 3 * rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    kt = k + 0.2 * rng.standard_normal((n, d))
    vt = v + 0.2 * rng.standard_normal((n, d))
    w_o = rng.standard_normal((D, d)) / math.sqrt(d)
    sm = 1 / math.sqrt(d)
    r = O.eq8_decomposition(q, k, v, kt, vt, w_o, sm)
    dy = r["y_tilde"] - r["y"]
    assert np.abs(r["key_term"] + r["value_term"] - dy).max() <= 1e-13 * np.abs(dy).max()
    assert r["e_out"] > 0
    # exact keys: the key-induced term is zero; exact values: the value-induced one
    r = O.eq8_decomposition(q, k, v, k, vt, w_o, sm)
    assert not r["key_term"].any()
    assert np.allclose(r["value_term"], r["y_tilde"] - r["y"], rtol=0, atol=1e-13)
    r = O.eq8_decomposition(q, k, v, kt, v, w_o, sm)
    assert not r["value_term"].any()
    # one token: p = p~ = 1, so only the value error remains
    r = O.eq8_decomposition(q, k[:1], v[:1], kt[:1], vt[:1], w_o, sm)
    assert not r["key_term"].any()
    assert np.allclose(r["y_tilde"] - r["y"], (vt[0] - v[0]) @ w_o.T, rtol=0, atol=1e-13)
    # adding one vector to every quantised key (the key mean) changes nothing
    r2 = O.eq8_decomposition(q, k, v, kt + 5.0 * rng.standard_normal(d), vt, w_o, sm)
    r1 = O.eq8_decomposition(q, k, v, kt, vt, w_o, sm)
    assert np.allclose(r2["key_term"], r1["key_term"], rtol=1e-9, atol=1e-12)


def test_dequantized_kv_inverts_centring_and_rotations_exactly_on_grid():
    """Keys k = x P^T + mu and values v = y P'^T with x, y on dyadic grids and
    P, P' signed permutations: the cache represents them exactly, so the
    original-basis keys and values read back are k and v themselves."""
    rng = np.random.default_rng(23)
    for group in (64, 128):
        R_k, _, _ = _signed_perm(rng, 128)
        R_v, _, _ = _signed_perm(rng, 128)
        mu = rng.integers(-64, 64, size=128) / 8.0
        n = 5
        x = np.stack([np.concatenate([_grid_group(rng, group, 0.25, -0.5)[1]
                                      for _ in range(128 // group)]) for _ in range(n)])
        y = np.stack([np.concatenate([_grid_group(rng, group, 0.5, -1.0)[1]
                                      for _ in range(128 // group)]) for _ in range(n)])
        k = x @ R_k.T + mu
        v = y @ R_v.T
        cache, table = _one_layer(rng, 1, group, R_k, R_v)
        O.append(cache, table, [0], k[None, :, None], v[None, :, None], mu[None], R_k[None],
                 R_v[None], group, 1.0, 1.0)
        kt, vt = O.dequantized_kv(cache, table, 0, n, 0, 1, group, mu[None], R_k[None], R_v[None])
        assert np.array_equal(kt, k) and np.array_equal(vt, v)


# ----------------------------------------------------------------- value rotation folded into W_V / W_O
def test_folded_value_rotation_writes_the_same_cache_and_output_through_the_weights():
    """Folded form (rot_v None): the caller's values are h (W_V R_V) and its
    output projection W_O R_V.  With R_V a signed permutation the folded
    append of v R_V writes exactly the bytes the unfolded append of v does;
    the folded decode is the unfolded one before the inverse rotation, and
    after the folded output projection both give the same y."""
    rng = np.random.default_rng(24)
    d, Hkv, Hq, group, n = 128, 2, 4, 64, 40
    R_k = np.stack([haar_orthogonal(rng, d) for _ in range(Hkv)])
    R_v = np.stack([_signed_perm(rng, d)[0] for _ in range(Hkv)])
    mu = rng.standard_normal((Hkv, d))
    h_in = rng.standard_normal((1, n, Hkv, 96))
    w_v = rng.standard_normal((Hkv, 96, d)) / math.sqrt(96)
    k = 2 * rng.standard_normal((1, n, Hkv, d)) + mu
    v = np.einsum("btki,kid->btkd", h_in, w_v)                 # h W_V
    v_fold = np.einsum("btki,kid->btkd", h_in, w_v @ R_v)      # h (W_V R_V)
    assert np.array_equal(v_fold, np.einsum("btkd,kde->btke", v, R_v))
    table = np.array([[2, 0, 1]], np.int32)
    c_unf = np.zeros((3, Hkv, O.page_bytes(d, group)), np.uint8)
    c_fold = np.zeros_like(c_unf)
    O.append(c_unf, table, [0], k, v, mu, R_k, R_v, group, 0.9, 0.9)
    O.append(c_fold, table, [0], k, v_fold, mu, R_k, None, group, 0.9, 0.9)
    assert np.array_equal(c_unf, c_fold)
    q = rng.standard_normal((1, Hq, d))
    o_unf = O.decode(c_unf, table, [n], q, R_k, R_v, 0.1, Hkv, group)
    o_fold = O.decode(c_fold, table, [n], q, R_k, None, 0.1, Hkv, group)
    w_o = rng.standard_normal((64, d))
    for hq in range(Hq):
        kv = hq // (Hq // Hkv)
        assert np.array_equal(o_fold[0, hq] @ R_v[kv].T, o_unf[0, hq])
        y = o_unf[0, hq] @ w_o.T
        y_fold = o_fold[0, hq] @ (w_o @ R_v[kv]).T
        assert np.allclose(y_fold, y, rtol=1e-12, atol=1e-12)


def test_unrotated_cache_is_textbook_per_group_rtn_and_decodes_with_the_plain_query():
    """rot_k = rot_v = None (the cache the rotations are compared against):
    the keys less their mean and the values as given are coded by the
    exhaustive nearest grid point of per-token, per-group asymmetric min/max
    INT2 (c = 1, fp16 scale (max - min)/3 and zero min), and the decode of an
    on-grid cache with one token returns that token's value, scoring with the
    unrotated query."""
    rng = np.random.default_rng(11)
    k = rng.standard_normal((1, 9, 2, 128)) * 3
    v = rng.standard_normal((1, 9, 2, 128))
    mu = rng.standard_normal((2, 128))
    enc = O.encode_tokens(k, v, mu, None, None, 64, 1.0, 1.0)
    for x, key in ((k[0] - mu[None], "k"), (v[0], "v")):
        xg = x.reshape(9, 2, 2, 64)                       # [token][head][group][64]
        s = np.float16((xg.max(-1) - xg.min(-1)) / 3).astype(np.float64)
        z = np.float16(xg.min(-1)).astype(np.float64)
        assert np.array_equal(enc[key + "_s"][0], s) and np.array_equal(enc[key + "_z"][0], z)
        grid = z[..., None, None] + s[..., None, None] * np.arange(4)
        dist = np.abs(xg[..., None] - grid)
        srt = np.sort(dist, axis=-1)
        clear = (srt[..., 1] - srt[..., 0] > 1e-9).reshape(9, 2, 128)
        best = dist.argmin(-1).reshape(9, 2, 128)
        assert clear.mean() > 0.99
        assert np.array_equal(enc[key + "_codes"][0][clear], best[clear])
    # one cached token on the grid: the output is its value; a rotation given
    # explicitly as the identity is the same cache and output
    cache = np.zeros((1, 2, O.page_bytes(128, 128)), np.uint8)
    tab = np.zeros((1, 1), np.int32)
    kk = (rng.integers(0, 4, (1, 1, 2, 128)) * 0.5 - 1.0)
    vv = (rng.integers(0, 4, (1, 1, 2, 128)) * 0.25 + 0.5)
    kk[..., 0], kk[..., 1] = -1.0, 0.5                    # both end points in the group
    vv[..., 0], vv[..., 1] = 0.5, 1.25
    O.append(cache, tab, [0], kk, vv, np.zeros((2, 128)), None, None, 128, 1.0, 1.0)
    eye = np.broadcast_to(np.eye(128), (2, 128, 128))
    cache2 = np.zeros_like(cache)
    O.append(cache2, tab, [0], kk, vv, np.zeros((2, 128)), eye, eye, 128, 1.0, 1.0)
    assert np.array_equal(cache, cache2)
    q = rng.standard_normal((1, 4, 128))
    o = O.decode(cache, tab, [1], q, None, None, 1 / math.sqrt(128), 2, 128)
    assert np.array_equal(o[0, :2], np.broadcast_to(vv[0, 0, 0], (2, 128)))
    assert np.array_equal(o[0, 2:], np.broadcast_to(vv[0, 0, 1], (2, 128)))
