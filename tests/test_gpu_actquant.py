"""Parity of the activation quantiser (through the C ABI) with the oracle:
codes and scales bit-exact, in both scale layouts, with guard bytes around
the outputs to catch stray writes."""
import numpy as np
import pytest
import torch

import bit_quantized_paged_amd as nvk
from oracle import nvfp4_oracle as O
from workloads import make_activations

pytestmark = pytest.mark.gpu

GUARD = 256
FILL = 0xA5


def _run(bits: np.ndarray, g, swizzled: bool, row_pad: int = 0):
    """Quantise bf16 bits [m, k] on the device (rows padded by row_pad
    elements in memory) into guarded output buffers; return codes, scales and
    whether the guard bytes survived."""
    m, k = bits.shape
    xs = torch.zeros((m, k + row_pad), dtype=torch.int16, device="cuda")
    xs[:, :k] = torch.from_numpy(bits.view(np.int16)).cuda()
    x = xs.view(torch.bfloat16)[:, :k]
    nsf = nvk.quant_activations_scale_bytes(m, k, swizzled)
    cbuf = torch.full((m * k // 2 + 2 * GUARD,), FILL, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((nsf + 2 * GUARD,), FILL, dtype=torch.uint8, device="cuda")
    codes = cbuf[GUARD:GUARD + m * k // 2].view(m, k // 2)
    scales = sbuf[GUARD:GUARD + nsf] if swizzled else sbuf[GUARD:GUARD + nsf].view(m, k // 16)
    gs = torch.tensor([float(np.float32(g))], dtype=torch.float32, device="cuda")
    nvk.quant_activations(x, gs, swizzled, codes, scales)
    torch.cuda.synchronize()
    c, s = cbuf.cpu().numpy(), sbuf.cpu().numpy()
    guards_ok = (np.all(c[:GUARD] == FILL) and np.all(c[GUARD + m * k // 2:] == FILL)
                 and np.all(s[:GUARD] == FILL) and np.all(s[GUARD + nsf:] == FILL))
    return codes.cpu().numpy(), scales.cpu().numpy(), guards_ok


SHAPES = [(1, 16), (33, 80), (128, 64), (200, 272), (257, 1040), (300, 4096), (129, 4112)]


@pytest.mark.parametrize("swizzled", [True, False])
@pytest.mark.parametrize("m,k", SHAPES)
def test_act_quant_bitexact(m, k, swizzled):
    bits, g = make_activations(seed=m * 7 + k, m=m, k=k)
    codes, scales, guards = _run(bits, g, swizzled, row_pad=24 if m % 2 else 0)
    want_c, want_s = O.quant_activations(bits, g, swizzled)
    assert guards, "write outside the output buffers"
    assert np.array_equal(codes, want_c), f"codes differ at {np.argwhere(codes != want_c)[:4].tolist()}"
    assert np.array_equal(scales.reshape(want_s.shape), want_s), \
        f"scales differ at {np.argwhere(scales.reshape(want_s.shape) != want_s)[:4].tolist()}"


def test_act_quant_ties_and_extremes():
    """Exact E2M1 midpoints (ties go to the even code), zero and sign-only
    blocks, bf16 subnormals, saturating blocks and a tiny global scale."""
    m, k = 160, 96
    rng = np.random.default_rng(5)
    x = rng.standard_normal((m, k)).astype(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    # g = 1/8 and amax 6 * 2^e give a power-of-two block step, so x * r hits
    # the midpoints exactly
    for r in range(0, 32):
        e = (r % 7) - 3
        x[r] = rng.choice(np.concatenate([mids, -mids]), k) * np.float32(2.0 ** e)
        x[r, ::16] = 6.0 * 2.0 ** e
    x[32:40] = 0.0
    x[40:44] = -1e-3 * np.abs(x[40:44])
    x[44:52] *= 1e-39
    x[52:60] *= 1e30
    x[60:64, ::16] = 3e38
    bits = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for g in (np.float32(0.125), np.float32(2.0 ** -20), np.float32(7.5e-3), np.float32(1e-30)):
        for swz in (True, False):
            codes, scales, guards = _run(bits, g, swz)
            want_c, want_s = O.quant_activations(bits, g, swz)
            assert guards
            assert np.array_equal(codes, want_c), (float(g), swz, np.argwhere(codes != want_c)[:4].tolist())
            assert np.array_equal(scales.reshape(want_s.shape), want_s), (float(g), swz)


def test_act_quant_chunked_prefill_rows_sampled():
    """The benchmark's shape (the 8192 hidden-state rows of a 4 x 2048 token
    prefill chunk, hidden size 4096, swizzled scales): every row in a sample
    that covers the first and last rows of row tiles matches the oracle on
    that row, at its swizzled scale offsets."""
    m, k = 8192, 4096
    bits, g = make_activations(seed=4, m=m, k=k)
    codes, scales, guards = _run(bits, g, True)
    assert guards
    rows = np.unique(np.concatenate([[0, 31, 32, 127, 128, 4095, 8191],
                                     np.random.default_rng(0).integers(0, m, 57)]))
    want_c, want_s = O.quant_activations(bits[rows], g, False)
    assert np.array_equal(codes[rows], want_c)
    c = np.arange(k // 16)
    for i, r in enumerate(rows):
        assert np.array_equal(scales[O.sf_swizzle_offset(r, c, k)], want_s[i]), int(r)


def test_act_quant_empty_and_rejects():
    gs = torch.ones(1, dtype=torch.float32, device="cuda")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    codes, scales = nvk.quant_activations(x, gs, True)
    assert codes.shape == (0, 32) and scales.numel() == 0
    with pytest.raises(ValueError):
        nvk.quant_activations(torch.zeros((4, 40), dtype=torch.bfloat16, device="cuda"), gs, True)
