"""Pins of the oracle's page-form dequantize and quantize-dequantize (QDQ)
emulation against things other than the oracle's own quantiser: a brute-force
search over every E4M3 scale and E2M1 code decoded from the format's closed
form, torch's bf16 cast, lossless round trips of representable blocks, and
the gather-form dequantize of the same pages."""
import numpy as np
import torch

from oracle import nvfp4_oracle as O


def _bf16_bits(vals):
    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_vals(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).float().numpy()


def _e4m3_closed_form(b):
    e, m = (b >> 3) & 15, b & 7
    return (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)


def _e2m1_closed_form(code):
    e, m = (code >> 1) & 3, code & 1
    return 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)


E4M3 = [(_e4m3_closed_form(b), b) for b in range(0x7F)]       # 0 .. 448, no NaN
E2M1 = [(_e2m1_closed_form(c), c) for c in range(8)]


def _nearest(table, v):
    """Nearest table value to v; ties to the even code; saturates at the top."""
    best = None
    for val, code in table:
        key = (abs(val - v), code & 1)
        if best is None or key < best[0]:
            best = (key, val)
    return best[1]


def _qdq_bruteforce(x, g):
    """QDQ of one 16-element block (fp32 inputs): scale = nearest E4M3 to the
    fp32 quotient amax / fp32(6 g); step d = fp32(s g); code = nearest E2M1 to
    fp32(x * fp32(1 / d)) keeping the sign; value = fp32(code * s * g) (the
    product code * s is exact), then bf16 by torch's cast."""
    f32 = np.float32
    amax = f32(np.max(np.abs(x)))
    s = _nearest(E4M3, float(f32(amax / f32(f32(6.0) * f32(g)))))
    d = f32(f32(s) * f32(g))
    r = f32(0.0) if d == 0 else f32(f32(1.0) / d)
    out = []
    for xi in x:
        q = float(f32(f32(xi) * r))
        c = _nearest(E2M1, abs(q))
        out.append(np.float32(np.float32(np.sign(q) * c * s) * f32(g)))
    return _bf16_vals(_bf16_bits(out))


def test_qdq_matches_bruteforce_search():
    rng = np.random.default_rng(71)
    for trial in range(40):
        D = int(rng.choice([64, 128]))
        g = np.float32(rng.choice([1.0, 0.37, 2.0 ** -9, 3.5e-3]))
        x = (rng.standard_normal(D) * rng.choice([0.01, 1.0, 40.0])).astype(np.float32)
        x[rng.integers(0, D)] *= 8.0
        xb = _bf16_bits(x)
        xf = _bf16_vals(xb)
        got = _bf16_vals(O.qdq_rows(xb[None], g, D)[0])
        want = np.concatenate([_qdq_bruteforce(xf[16 * j:16 * j + 16], g) for j in range(D // 16)])
        # -0 and +0 are the same value for this comparison
        assert np.array_equal(got, want), trial


def test_qdq_is_lossless_on_representable_blocks():
    """Blocks built as code * s * g with a power-of-two g and one |code| = 6
    per block come back unchanged, and QDQ is then idempotent."""
    rng = np.random.default_rng(72)
    for trial in range(200):
        D = int(rng.choice([64, 128, 256]))
        g = np.float32(2.0 ** int(rng.integers(-12, 3)))
        nb = D // 16
        s = np.array([_e4m3_closed_form(int(b)) for b in rng.integers(8, 0x70, size=nb)])
        codes = rng.integers(0, 16, size=(nb, 16))
        codes[np.arange(nb), rng.integers(0, 16, size=nb)] = rng.choice([7, 15], size=nb)
        mags = np.array([_e2m1_closed_form(int(c) & 7) for c in codes.reshape(-1)]).reshape(nb, 16)
        x = (np.where(codes >= 8, -mags, mags) * s[:, None] * float(g)).reshape(D).astype(np.float32)
        xb = _bf16_bits(x)
        assert np.array_equal(_bf16_vals(xb), x)
        once = O.qdq_rows(xb[None], g, D)[0]
        assert np.array_equal(_bf16_vals(once), x), trial
        assert np.array_equal(O.qdq_rows(once[None], g, D)[0], once)


def test_dequant_pages_agrees_with_the_gather_form():
    """Page p of the page-form output holds, at (kv, row, head), what the
    gather-form dequantize returns for the token stored there."""
    rng = np.random.default_rng(73)
    nb, bs, hkv, D = 9, 16, 2, 128
    lens = np.array([37, 50, 5])
    pages = (lens + bs - 1) // bs
    perm = rng.permutation(nb)[: pages.sum()]
    bt = np.full((3, pages.max()), -1, np.int64)
    o = 0
    for b in range(3):
        bt[b, : pages[b]] = perm[o:o + pages[b]]
        o += pages[b]
    slots = np.concatenate([bt[b, np.arange(L) // bs] * bs + np.arange(L) % bs for b, L in enumerate(lens)])
    T = int(lens.sum())
    k = _bf16_bits(rng.standard_normal((T, hkv, D)).astype(np.float32))
    v = _bf16_bits(rng.standard_normal((T, hkv, D)).astype(np.float32))
    pool = np.zeros(O.pool_shape(nb, bs, hkv, D), np.uint8)
    gk, gv = np.float32(0.02), np.float32(0.05)
    O.append(pool, k, v, slots, gk, gv)
    ids = np.concatenate([perm, [int(rng.integers(0, nb))]])   # every used page plus a repeat
    got = O.dequant_pages(pool, ids, gk, gv, D)
    assert got.shape == (len(ids), 2, bs, hkv, D) and got.dtype == np.uint16
    ok, ov = O.dequant_paged(pool, bt, lens, gk, gv, D)
    t = 0
    for b, L in enumerate(lens):
        for j in range(L):
            p = int(np.nonzero(ids == bt[b, j // bs])[0][0])
            assert np.array_equal(got[p, 0, j % bs], ok[t])
            assert np.array_equal(got[p, 1, j % bs], ov[t])
            t += 1
    # and a stored row equals the QDQ of the row that was appended
    assert np.array_equal(got[int(np.nonzero(ids == bt[0, 0])[0][0]), 0, 0], O.qdq_rows(k[0], gk, D))
