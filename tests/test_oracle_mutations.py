"""The oracle's pins catch plausible mistakes. Each case plants one mistake in
the oracle (on the CPU, by replacing one oracle function with a wrong
variant for the duration of the test) and runs the pins of that part: at
least one of them must fail. Mistakes: a swapped nibble order, scales
written before the data, a dropped global scale, ties rounded away from
zero, a block scale that truncates or is off by a factor of two, a wrong
E2M1 value table, a lost sign, a wrong query-to-kv-head mapping, an
off-by-one causal limit, a dropped softmax scale and K dequantised with V's
scale."""
import numpy as np
import pytest

from oracle import nvfp4_oracle as O
import test_oracle_attention as A
import test_oracle_format as F

CODEC_PINS = [
    F.test_e2m1_decode_all_codes,
    F.test_e2m1_encode_matches_bruteforce,
    F.test_e4m3_decode_matches_torch,
    F.test_e4m3_encode_matches_torch_cast,
    F.test_golden_rows,
    F.test_block_scale_is_nearest_e4m3,
    F.test_codes_are_nearest_multiple_of_step,
    F.test_representable_blocks_round_trip,
]
ATTN_PINS = [
    lambda: A.test_attention_matches_torch_sdpa(True),
    lambda: A.test_attention_matches_torch_sdpa(False),
    A.test_attention_bruteforce_loops,
    A.test_constant_values_and_single_key,
    A.test_causal_prefix_ignores_later_keys,
]


def _swap_nibbles(orig):
    def f(x_bits, g):
        out = orig(x_bits, g).copy()
        D = np.asarray(x_bits).shape[-1]
        d = out[..., : D // 2]
        out[..., : D // 2] = ((d >> np.uint8(4)) | (d << np.uint8(4))).astype(np.uint8)
        return out
    return f


def _scales_first(orig):
    def f(x_bits, g):
        out = orig(x_bits, g)
        D = np.asarray(x_bits).shape[-1]
        return np.concatenate([out[..., D // 2:], out[..., : D // 2]], axis=-1)
    return f


def _global_scale_dropped(orig):
    return lambda x_bits, g: orig(x_bits, 1.0)


def _ties_away(orig):
    def f(v):
        v = np.asarray(v, np.float32)
        return orig((v * np.float32(1 + 2.0 ** -20)).astype(np.float32))
    return f


def _e4m3_truncates(orig):
    table = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0x00 .. 0x7E, increasing

    def f(s):
        s = np.asarray(s, np.float64)
        return (np.searchsorted(table, s, side="right") - 1).clip(0, 0x7E).astype(np.uint8)
    return f


def _e4m3_scale_doubled(orig):
    return lambda s: orig((np.asarray(s, np.float32) * np.float32(2)).astype(np.float32))


def _e2m1_table_swapped(orig):
    def f(code):
        code = np.asarray(code, dtype=np.int64)
        swapped = np.where((code & 7) == 3, (code & 8) | 4, np.where((code & 7) == 4, (code & 8) | 3, code))
        return orig(swapped)
    return f


def _sign_lost(orig):
    return lambda rows, g, head_size: np.abs(orig(rows, g, head_size))


def _dequant_without_g(orig):
    return lambda rows, g, head_size: orig(rows, 1.0, head_size)


def _gqa_modulo(orig):
    """q head h reads kv head h % Hkv instead of h // (Hq / Hkv)."""
    def f(pool, q, cu_q, bt, lens, ks, vs, sm, D, causal=True, kv_dtype="nvfp4"):
        Hq, Hkv = q.shape[1], pool.shape[3]
        G = Hq // Hkv
        perm = np.array([(h % Hkv) * G + h // Hkv for h in range(Hq)])  # h -> head h' with h' // G == h % Hkv
        q2 = np.empty_like(q)
        q2[:, perm] = q
        out = orig(pool, q2, cu_q, bt, lens, ks, vs, sm, D, causal, kv_dtype)
        return out[:, perm]
    return f


def _causal_off_by_one(orig):
    """Every query misses its last visible key."""
    def f(pool, q, cu_q, bt, lens, ks, vs, sm, D, causal=True, kv_dtype="nvfp4"):
        return orig(pool, q, cu_q, bt, np.maximum(np.asarray(lens) - 1, 0), ks, vs, sm, D, causal, kv_dtype)
    return f


def _sm_scale_dropped(orig):
    def f(pool, q, cu_q, bt, lens, ks, vs, sm, D, causal=True, kv_dtype="nvfp4"):
        return orig(pool, q, cu_q, bt, lens, ks, vs, 1.0, D, causal, kv_dtype)
    return f


def _k_with_v_scale(orig):
    def f(pool, q, cu_q, bt, lens, ks, vs, sm, D, causal=True, kv_dtype="nvfp4"):
        return orig(pool, q, cu_q, bt, lens, vs, vs, sm, D, causal, kv_dtype)
    return f


MUTANTS = {
    "nibble order swapped": ("quantize_rows", _swap_nibbles, CODEC_PINS),
    "scales before data": ("quantize_rows", _scales_first, CODEC_PINS),
    "global scale dropped": ("quantize_rows", _global_scale_dropped, CODEC_PINS),
    "E2M1 ties away from zero": ("e2m1_encode", _ties_away, CODEC_PINS),
    "E4M3 truncates": ("e4m3_encode_sat", _e4m3_truncates, CODEC_PINS),
    "E4M3 scale doubled": ("e4m3_encode_sat", _e4m3_scale_doubled, CODEC_PINS),
    "E2M1 values 1.5 and 2 swapped": ("e2m1_decode", _e2m1_table_swapped, CODEC_PINS),
    "dequant loses the sign": ("dequantize_rows", _sign_lost, CODEC_PINS),
    "dequant drops g": ("dequantize_rows", _dequant_without_g, CODEC_PINS),
    "GQA head modulo": ("paged_attention", _gqa_modulo, ATTN_PINS),
    "causal limit off by one": ("paged_attention", _causal_off_by_one, ATTN_PINS),
    "softmax scale dropped": ("paged_attention", _sm_scale_dropped, ATTN_PINS),
    "K dequantised with V's scale": ("paged_attention", _k_with_v_scale, ATTN_PINS),
}


def test_pins_pass_on_the_oracle():
    for pin in CODEC_PINS + ATTN_PINS:
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, make, pins = MUTANTS[name]
    monkeypatch.setattr(O, attr, make(getattr(O, attr)))
    caught = []
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught.append(getattr(pin, "__name__", "lambda"))
    assert caught, f"no pin fails when the oracle has this mistake: {name}"
