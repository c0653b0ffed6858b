"""Pins of the oracle's NVFP4 codec against things other than itself:
closed-form format definitions, torch's own fp8/bf16 casts, brute-force
nearest-value searches, hand-derived golden bytes and lossless round trips."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_rows.txt")


def _bf16_bits(vals):
    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# --- layout ----------------------------------------------------------------

def test_full_dim_formula():
    # row width D/2 + D/16 (get_kv_cache_shape); about 3.56x smaller than bf16 at D=128
    assert [O.full_dim(d) for d in (64, 128, 256)] == [36, 72, 144]
    assert O.pool_shape(7, 16, 2, 128) == (7, 2, 16, 2, 72)
    assert 2 * 128 / O.full_dim(128) == pytest.approx(3.5556, rel=1e-4)


# --- E2M1 ------------------------------------------------------------------

def _e2m1_closed_form(code):
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -mag if s else mag


def test_e2m1_decode_all_codes():
    codes = np.arange(16)
    got = O.e2m1_decode(codes)
    want = np.array([_e2m1_closed_form(int(c)) for c in codes])
    assert np.array_equal(got, want)
    assert sorted(set(np.abs(got).tolist())) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def _e2m1_bruteforce(v):
    """nearest of the 8 magnitudes; ties to the code with mantissa bit 0;
    above 6 -> 6; sign copied from v."""
    a = abs(float(v))
    mags = [_e2m1_closed_form(c) for c in range(8)]
    d = [abs(a - m) for m in mags]
    best = min(d)
    cands = [c for c in range(8) if d[c] == best]
    idx = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    if a > 6:
        idx = 7
    return (8 if math.copysign(1.0, float(v)) < 0 else 0) | idx


def test_e2m1_encode_matches_bruteforce():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1, 1.5, 2, 3, 4]
    vals = [0.0, -0.0, 7.0, 1e30, -1e30, 1e-40]
    for m in mids:
        f = np.float32(m)
        vals += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(10))]
    rng = np.random.default_rng(0)
    vals += list(rng.uniform(-8, 8, 4000).astype(np.float32))
    vals += list(np.linspace(-7, 7, 2801).astype(np.float32))
    v = np.array(vals, np.float32)
    v = np.concatenate([v, -v])
    got = O.e2m1_encode(v)
    want = np.array([_e2m1_bruteforce(x) for x in v], np.uint8)
    assert np.array_equal(got, want)


# --- E4M3 ------------------------------------------------------------------

def test_e4m3_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(b)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert O.e4m3_decode(np.array([0x7E]))[0] == 448.0


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_cast():
    vals = O.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))  # all finite non-negative
    pts = []
    for a, b in zip(vals[:-1], vals[1:]):
        mid = np.float32((a + b) / 2)
        pts += [np.float32(a), mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    rng = np.random.default_rng(1)
    pts += list(np.exp2(rng.uniform(-14, np.log2(447.9), 200000)).astype(np.float32))
    pts += [np.float32(2.0 ** -10), np.float32(2.0 ** -11), np.float32(1e-30), np.float32(0.0)]
    x = np.array(pts, np.float32)
    x = x[x < 448]
    assert np.array_equal(O.e4m3_encode_sat(x), _torch_e4m3(x))


def test_e4m3_encode_saturates():
    x = np.array([448.0, 449.0, 463.99, 464.0, 500.0, 1e20, np.inf], np.float32)
    assert np.all(O.e4m3_encode_sat(x) == 0x7E)
    # just below the saturation point rounding still applies (the binade
    # [256, 512) steps by 32): 420 -> 416 (0x7D); 432 ties between 416 and 448
    # and goes to the even mantissa, 448 (0x7E)
    assert O.e4m3_encode_sat(np.array([420.0], np.float32))[0] == 0x7D
    assert O.e4m3_encode_sat(np.array([432.0], np.float32))[0] == 0x7E
    # torch agrees up to 464 (the tie between 448 and the missing 480 goes to
    # the even 448) and returns NaN (0x7F) past it
    assert np.all(_torch_e4m3(x[:4]) == 0x7E) and _torch_e4m3(x[4:5])[0] == 0x7F


# --- bf16 --------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 100,
                        np.array([1.00390625, 1.01171875, -3.0000001, 65504.0, 1e-39], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16(x), want)
    assert np.array_equal(O.bf16_to_f32(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


# --- golden rows -------------------------------------------------------------

def _load_golden():
    rows, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line == "[row]":
            cur = {}
            rows.append(cur)
            continue
        k, v = [s.strip() for s in line.split("=", 1)]
        cur[k] = v
    return rows


def test_golden_rows():
    rows = _load_golden()
    assert len(rows) == 2
    for r in rows:
        D = int(r["head_size"])
        g = np.array([int(r["g"], 16)], np.uint32).view(np.float32)[0]
        x = np.array([float(t) for t in r["x"].split()], np.float32)
        assert x.size == D
        xb = _bf16_bits(x)
        assert np.array_equal(O.bf16_to_f32(xb), x), "inputs must be bf16-exact"
        want = np.array([int(t, 16) for t in r["bytes"].split()], np.uint8)
        got = O.quantize_rows(xb[None], g)[0]
        assert got.tolist() == want.tolist()
        deq = np.array([float(t) for t in r["dequant"].split()], np.float32)
        assert np.array_equal(O.dequantize_rows(want[None], g, D)[0], deq)


# --- properties of the quantiser checked by brute force ----------------------

def _random_rows(rng, n, D, spread=True):
    x = rng.standard_normal((n, D)).astype(np.float32)
    if spread:
        x *= np.exp2(rng.integers(-12, 8, size=(n, D // 16, 1))).repeat(16, axis=2).reshape(n, D)
    return _bf16_bits(x)


def test_block_scale_is_nearest_e4m3():
    """The scale byte is the E4M3 value nearest the exact amax/(6g) (ties to
    even), saturating at 448 — checked against all 127 finite E4M3 values in
    fp64, skipping ratios within 2^-20 of a midpoint (where the fp32 steps of
    the oracle may legitimately go either way)."""
    rng = np.random.default_rng(3)
    D = 128
    xb = _random_rows(rng, 400, D)
    x = O.bf16_to_f32(xb).astype(np.float64)
    g = np.float32(0.0123)
    rows = O.quantize_rows(xb, g)
    scales = rows[:, D // 2:]
    table = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    amax = np.abs(x.reshape(400, D // 16, 16)).max(-1)
    ratio = amax / (6.0 * float(g))
    checked = 0
    for i in range(400):
        for j in range(D // 16):
            rt = ratio[i, j]
            if rt >= 448:
                assert scales[i, j] == 0x7E
                continue
            d = np.abs(table - rt)
            order = np.argsort(d, kind="stable")
            if abs(d[order[0]] - d[order[1]]) <= 2.0 ** -20 * max(rt, 2.0 ** -9):
                continue
            assert scales[i, j] == order[0], (i, j, rt)
            checked += 1
    assert checked > 2500


def test_codes_are_nearest_multiple_of_step():
    """Each element's dequantised value c*s*g is the nearest of the 15
    candidates x' = m*d (d the block step) to the exact x, ties excluded."""
    rng = np.random.default_rng(4)
    D = 64
    xb = _random_rows(rng, 300, D)
    x = O.bf16_to_f32(xb).astype(np.float64).reshape(300, D // 16, 16)
    g = np.float32(0.37)
    rows = O.quantize_rows(xb, g)
    deq = O.dequantize_rows(rows, g, D).astype(np.float64).reshape(300, D // 16, 16)
    step = O.e4m3_decode(rows[:, D // 2:]).astype(np.float64) * float(g)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6.0])
    cand = np.concatenate([-mags[::-1], mags[1:]])
    n = 0
    for i in range(300):
        for j in range(D // 16):
            dstep = step[i, j]
            if dstep == 0:
                assert np.all(deq[i, j] == 0)
                continue
            for k in range(16):
                vals = cand * dstep
                err = np.abs(vals - x[i, j, k])
                o = np.argsort(err, kind="stable")
                if err[o[1]] - err[o[0]] <= 1e-6 * dstep:
                    continue
                assert math.isclose(deq[i, j, k], vals[o[0]], rel_tol=2 ** -22, abs_tol=1e-38), (i, j, k)
                n += 1
    assert n > 15000


def test_representable_blocks_round_trip():
    """Blocks built as code * s * g (g a power of two, one |code| = 6 per
    block so that s is the block's own scale) come back bit-exactly."""
    rng = np.random.default_rng(5)
    fails = 0
    for trial in range(300):
        D = int(rng.choice([64, 128, 256]))
        g = np.float32(2.0 ** int(rng.integers(-14, 4)))
        nb = D // 16
        s_bytes = rng.integers(1, 0x7F, size=nb)
        s = O.e4m3_decode(s_bytes)
        codes = rng.integers(0, 16, size=(nb, 16))
        codes[np.arange(nb), rng.integers(0, 16, size=nb)] = rng.choice([7, 15], size=nb)
        x = (O.e2m1_decode(codes) * s[:, None] * float(g)).reshape(D).astype(np.float32)
        xb = _bf16_bits(x)
        assert np.array_equal(O.bf16_to_f32(xb), x)
        row = O.quantize_rows(xb[None], g)[0]
        back = O.f32_to_bf16(O.dequantize_rows(row[None], g, D)[0])
        # -0 and +0 both count as the same input zero
        fails += int(not np.array_equal(O.bf16_to_f32(back), x))
        assert np.array_equal(row[D // 2:], s_bytes.astype(np.uint8))
    assert fails == 0


def test_append_and_gather_follow_slot_mapping():
    """Slot -> (block, row) addressing and the skip of out-of-pool slots."""
    rng = np.random.default_rng(6)
    nb, bs, hkv, D = 5, 16, 2, 64
    pool = np.zeros(O.pool_shape(nb, bs, hkv, D), np.uint8)
    k = _random_rows(rng, 7 * hkv, D).reshape(7, hkv, D)
    v = _random_rows(rng, 7 * hkv, D).reshape(7, hkv, D)
    slots = np.array([0, 17, 79, -1, 80, 33, 5])
    O.append(pool, k, v, slots, np.float32(0.1), np.float32(0.2))
    for t, s in enumerate(slots):
        if 0 <= s < nb * bs:
            assert np.array_equal(pool[s // bs, 0, s % bs], O.quantize_rows(k[t], np.float32(0.1)))
            assert np.array_equal(pool[s // bs, 1, s % bs], O.quantize_rows(v[t], np.float32(0.2)))
    written = sum(1 for s in slots if 0 <= s < nb * bs)
    assert np.count_nonzero(pool.reshape(-1, O.full_dim(D)).any(axis=1)) == 2 * hkv * written
