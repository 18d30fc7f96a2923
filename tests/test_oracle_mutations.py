"""Planted mistakes in the oracle, each caught by at least one pin.

Every case below replaces one oracle function by a plausible wrong version:

- a transposed operand;
- a dropped step (centring, clipping, fp16 rounding, the inverse value
  rotation, the softmax scale);
- a wrong rounding mode, scale divisor or sign;
- a wrong head mapping;
- a wrong bit or word order;
- a wrong weighting in the Eq. 8 split;
- a wrong window slot or window boundary;
- bfloat16 truncation instead of rounding.

It then runs the pins of test_oracle_pins and requires that one of them
fails.  This shows the pins constrain each part of the oracle, not only its
happy path.  The mistakes are planted in the oracle on the CPU; nothing here
touches the GPU.
"""
import numpy as np
import pytest

import oracle
import oracle.kvq_oracle as K
import test_oracle_pins as pins

ORIG = {name: getattr(K, name) for name in (
    "rotate", "encode_tokens", "encode_groups", "quantize_on_grid", "fp16_sat",
    "value_rotation", "attend", "k_code_site", "v_code_site", "dequant", "decode",
    "eq8_decomposition", "window_slot", "window_parts", "bf16_round")}


def _rotate_transposed(x, R):
    return np.einsum("...hi,hji->...hj", np.asarray(x, np.float64), np.asarray(R, np.float64))


def _encode_tokens_uncentred(k, v, mu, rot_k, rot_v, group, clip_k, clip_v):
    mu0 = np.zeros_like(np.asarray(mu, np.float64))
    return ORIG["encode_tokens"](k, v, mu0, rot_k, rot_v, group, clip_k, clip_v)


def _encode_groups_unclipped(x, group, clip):
    return ORIG["encode_groups"](x, group, 1.0)


def _encode_groups_divisor(levels):
    def enc(x, group, clip):
        x = np.asarray(x, np.float64)
        xg = x.reshape(x.shape[:-1] + (x.shape[-1] // group, group))
        lo, hi = clip * xg.min(axis=-1), clip * xg.max(axis=-1)
        s16, z16 = K.fp16_sat((hi - lo) / levels), K.fp16_sat(lo)
        return s16, z16, K.quantize_on_grid(x, s16, z16, group), (hi - lo) / levels, lo
    return enc


def _quantize_floor(x, s16, z16, group):
    x = np.asarray(x, np.float64)
    xg = x.reshape(x.shape[:-1] + (x.shape[-1] // group, group))
    s = np.asarray(s16, np.float64)[..., None]
    z = np.asarray(z16, np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.clip(np.floor((xg - z) / s), 0, 3)
    return np.where(s == 0, 0, c).astype(np.uint8).reshape(x.shape)


def _fp16_unrounded(x):
    return np.clip(np.asarray(x, np.float64), -K.F16_MAX, K.F16_MAX)


def _value_rotation_transposed(rot_v, h, d=K.HEAD_DIM):
    return ORIG["value_rotation"](rot_v, h, d).T


def _attend_unscaled(q_r, k_hat, v_hat, sm_scale):
    return ORIG["attend"](q_r, k_hat, v_hat, 1.0)


def _k_code_site_msb_first(t, i):
    off, sh = ORIG["k_code_site"](t, i)
    return off, 6 - sh


def _v_code_site_other_words(t, i):
    t, i = np.asarray(t), np.asarray(i)
    word = 16 * (i % 8) + i // 8  # a different bijection of channels onto words
    u = (3 * t) % 16
    return 512 + 4 * word + u // 4, 2 * (u % 4)


def _dequant_zero_subtracted(s16, z16, codes, group):
    return ORIG["dequant"](s16, -np.asarray(z16, np.float64), codes, group)


def _decode_gqa_interleaved(cache, block_table, ctx_len, q, rot_k, rot_v, sm_scale,
                            num_kv_heads, group, pairs=None):
    # query head hq read KV head hq % Hkv instead of hq // Hg
    q = np.asarray(q, np.float64)
    Hq = q.shape[1]
    Hg = Hq // num_kv_heads
    pi = np.array([(hq % num_kv_heads) * Hg + hq // num_kv_heads for hq in range(Hq)])
    q2 = np.empty_like(q)
    q2[:, pi] = q
    pairs2 = None if pairs is None else [(b, int(pi[hq])) for (b, hq) in pairs]
    return ORIG["decode"](cache, block_table, ctx_len, q2, rot_k, rot_v, sm_scale,
                          num_kv_heads, group, pairs=pairs2)[:, pi]


def _eq8_terms_with_exact_weights(q, k, v, k_tilde, v_tilde, w_o, sm_scale):
    # the value term weighted by the exact-key distribution instead of p~
    r = ORIG["eq8_decomposition"](q, k, v, k_tilde, v_tilde, w_o, sm_scale)
    p = K._softmax_weights(q, k, sm_scale)
    dv = np.asarray(v_tilde, np.float64) - np.asarray(v, np.float64)
    r["value_term"] = (p @ dv) @ np.asarray(w_o, np.float64).T
    return r


def _window_slot_no_sinks(pos):
    return np.asarray(pos) % (K.SINK + K.RECENT)


def _window_parts_recent_short(n):
    sink, body, recent = ORIG["window_parts"](n)
    if len(recent) > 0:  # the last recent token counted in the body
        body = range(body.start, max(body.stop, recent.start + 1))
        recent = range(recent.start + 1, recent.stop)
    return sink, body, recent


def _bf16_truncated(x):
    f = np.asarray(x, np.float32)
    u = f.view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


MUTATIONS = {
    "rotation_transposed": ("rotate", _rotate_transposed),
    "key_centring_dropped": ("encode_tokens", _encode_tokens_uncentred),
    "clip_ignored": ("encode_groups", _encode_groups_unclipped),
    "scale_over_4": ("encode_groups", _encode_groups_divisor(4.0)),
    "scale_over_2": ("encode_groups", _encode_groups_divisor(2.0)),
    "codes_floored": ("quantize_on_grid", _quantize_floor),
    "fp16_rounding_dropped": ("fp16_sat", _fp16_unrounded),
    "inverse_value_rotation_transposed": ("value_rotation", _value_rotation_transposed),
    "softmax_scale_dropped": ("attend", _attend_unscaled),
    "k_bits_msb_first": ("k_code_site", _k_code_site_msb_first),
    "v_words_permuted": ("v_code_site", _v_code_site_other_words),
    "zero_point_sign": ("dequant", _dequant_zero_subtracted),
    "gqa_interleaved": ("decode", _decode_gqa_interleaved),
    "eq8_value_term_weights": ("eq8_decomposition", _eq8_terms_with_exact_weights),
    "window_slot_without_sinks": ("window_slot", _window_slot_no_sinks),
    "window_recent_one_short": ("window_parts", _window_parts_recent_short),
    "bf16_truncated": ("bf16_round", _bf16_truncated),
}

PINS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


def test_pins_pass_called_directly():
    """Control: the unmodified oracle passes every pin when called this way."""
    for pin in PINS:
        pin()


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    func, fake = MUTATIONS[name]
    monkeypatch.setattr(K, func, fake)
    monkeypatch.setattr(oracle, func, fake, raising=False)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # an assertion, or the mistake breaking a pin outright
            caught.append(pin.__name__)
            break
    assert caught, f"no pin fails with {name}"
    print(f"{name}: caught by {caught[0]}")
