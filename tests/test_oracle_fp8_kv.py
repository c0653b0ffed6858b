"""Pins of the oracle's FP8 KV cache formats [P40177 "Key source snippets":
fp8 / fp8_e4m3 / fp8_e5m2 cache dtypes, mapped to float8_e4m3fn and
float8_e5m2]: E5M2 decoding against IEEE half precision (E5M2 is the top
byte of a binary16), both encoders against a brute-force nearest search over
every finite code, exact round trips, and attention on an FP8 cache against
torch's fp64 attention on values decoded independently of the oracle."""
import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from workloads import make_workload

KINDS = {"e4m3": (448.0, 0x7E), "e5m2": (57344.0, 0x7B)}


def _finite_magnitudes(kind):
    codes = np.arange(KINDS[kind][1] + 1)
    return codes, O.fp8_decode(codes, kind)


def test_e5m2_decode_is_half_precision_top_byte():
    codes = np.arange(256, dtype=np.uint16)
    half = (codes << np.uint16(8)).view(np.float16).astype(np.float64)
    got = O.e5m2_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(half))
    ok = ~np.isnan(half)
    assert np.array_equal(got[ok], half[ok])


def _nearest(x, kind):
    """Brute force: the finite code whose value is nearest to |x|, ties to
    the even code, |x| >= max -> the largest code; sign copied from x."""
    codes, mags = _finite_magnitudes(kind)
    maxv, maxcode = KINDS[kind]
    a = np.abs(x.astype(np.float64))
    d = np.abs(mags[None, :] - a[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes take the even one
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    mag = np.where(a >= maxv, maxcode, codes[pick])
    sign = (x.astype(np.float32).view(np.uint32) >> 31).astype(np.uint8)
    return (sign << 7) | mag.astype(np.uint8)


@pytest.mark.parametrize("kind", ["e4m3", "e5m2"])
def test_encoder_matches_bruteforce_nearest(kind):
    _, mags = _finite_magnitudes(kind)
    mids = (mags[1:] + mags[:-1]) / 2
    xs = [mags, mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
          np.nextafter(mids.astype(np.float32), np.float32(0)), [KINDS[kind][0] * 1.01, 1e30, np.inf]]
    x = np.concatenate([np.asarray(v, np.float64) for v in xs]).astype(np.float32)
    # every finite bf16 pattern too
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    bf = bits.view(np.float32)
    x = np.concatenate([x, -x, bf[np.isfinite(bf)], np.float32([0.0, -0.0])])
    assert np.array_equal(O.fp8_encode(x, kind), _nearest(x, kind))


@pytest.mark.parametrize("kind", ["e4m3", "e5m2"])
def test_rows_round_trip_exact(kind):
    """Values that are FP8 values times a power-of-two scale come back
    exactly; everything from the largest value up saturates to it."""
    rng = np.random.default_rng(3)
    codes, mags = _finite_magnitudes(kind)
    g = np.float32(2.0 ** -4)
    pick = rng.integers(0, len(codes), (6, 64))
    x = (mags[pick] * rng.choice([-1.0, 1.0], pick.shape) * float(g)).astype(np.float32)
    bits = O.f32_to_bf16(x)
    assert np.array_equal(O.bf16_to_f32(bits), x)  # the test values are bf16-exact
    rows = O.quantize_rows_fp8(bits, g, kind)
    assert np.array_equal(O.dequantize_rows_fp8(rows, g, kind), x)
    big = O.f32_to_bf16(np.float32([3e38, -3e38, KINDS[kind][0] * 2.0 * float(g)] + [0.0] * 13))
    r = O.quantize_rows_fp8(big, g, kind)
    assert r[0] == KINDS[kind][1] and r[1] == 0x80 | KINDS[kind][1] and r[2] == KINDS[kind][1]


def _decode_independent(rows, kind):
    if kind == "e5m2":
        return (rows.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    # E4M3FN spelled out: exponent bias 7, subnormal step 2^-9
    r = rows.astype(np.int64)
    e, m = (r >> 3) & 15, r & 7
    mag = np.where(e == 0, m / 512.0, (8 + m) * 2.0 ** (e - 10))
    return np.where(r & 0x80, -mag, mag)


@pytest.mark.parametrize("kind", ["e4m3", "e5m2"])
def test_attention_on_fp8_cache(kind):
    kv = "fp8_" + kind
    lens, qls, hq, hkv, D, bs = [37, 5, 70], [1, 5, 9], 8, 2, 64, 16
    w = make_workload(seed=31, name="t", seq_lens=lens, q_lens=qls, num_q_heads=hq, num_kv_heads=hkv,
                      head_size=D, block_size=bs)
    pool = np.zeros(O.pool_shape(w.num_blocks, bs, hkv, D, kv), np.uint8)
    assert pool.shape[-1] == D
    O.append(pool, w.key, w.value, w.slot_mapping, w.k_scale, w.v_scale, kv)
    sm = np.float32(0.125)
    out = O.paged_attention(pool, w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale, sm, D,
                            kv_dtype=kv)
    for b in range(len(lens)):
        L, nq = lens[b], qls[b]
        j = np.arange(L)
        rk = pool[w.block_table[b][j // bs], 0, j % bs]
        rv = pool[w.block_table[b][j // bs], 1, j % bs]
        K = _decode_independent(rk, kind) * float(w.k_scale)
        V = _decode_independent(rv, kind) * float(w.v_scale)
        q = torch.from_numpy(O.bf16_to_f32(w.query[w.cu_q[b]: w.cu_q[b + 1]]).astype(np.float64)).permute(1, 0, 2)
        k = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
        v = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
        mask = torch.arange(L)[None, :] <= (L - nq + torch.arange(nq)[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=float(sm))
        got = out[w.cu_q[b]: w.cu_q[b + 1]].transpose(1, 0, 2)
        # the oracle rounds fp8 * g to fp32 before fp64 attention: 2^-24 relative per value
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("kind", ["e4m3", "e5m2"])
def test_quotient_is_one_rounded_division(kind):
    """code = FP8(RN32(x / g)): the fp32 quotient is the fp64 quotient rounded
    once to fp32 (exact, since 53 >= 2 * 24 + 2 bits), and differs from
    RN32(x * RN32(1 / g)) on some of these inputs, which this separates."""
    rng = np.random.default_rng(9)
    g = np.float32(3.0) if kind == "e4m3" else np.float32(0.37)
    x = O.f32_to_bf16(rng.standard_normal(4096).astype(np.float32) * 50)
    xf = O.bf16_to_f32(x).astype(np.float64)
    q = (xf / float(g)).astype(np.float32)
    want = _nearest(q, kind)
    assert np.array_equal(O.quantize_rows_fp8(x, g, kind), want)
    recip = (O.bf16_to_f32(x) * (np.float32(1.0) / g)).astype(np.float32)
    assert np.any(recip != q)
