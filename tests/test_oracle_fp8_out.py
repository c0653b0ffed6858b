"""Pins of the oracle's FP8-E4M3 attention output and its bf16 epilogue
against torch's own float8_e4m3fn and bfloat16 casts."""
import numpy as np
import torch

from oracle import nvfp4_oracle as O


def _bf16_vals(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).float().numpy()


def test_fp8_out_matches_torch_cast_below_saturation():
    """Signed values inside the E4M3 range (including exact midpoints and
    their neighbours) encode as torch's round-to-nearest-even cast; the
    output scale divides first."""
    rng = np.random.default_rng(81)
    mags = O.e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    x = np.concatenate([mags.astype(np.float32), mids, np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(1e9)),
                        (rng.standard_normal(4000) * rng.choice([1e-3, 1.0, 50.0], 4000)).astype(np.float32)])
    x = np.concatenate([x, -x])
    x = x[np.abs(x) < 448]
    for s in (1.0, 0.25, 3.0):
        s32 = np.float32(s)
        q = (x.astype(np.float32) / s32).astype(np.float32)
        keep = np.abs(q) < 448
        want = torch.from_numpy(q[keep]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = O.fp8_out(x[keep].astype(np.float64), s)
        assert np.array_equal(got, want), s


def test_fp8_out_saturates_and_keeps_the_sign():
    got = O.fp8_out(np.array([500.0, -500.0, 1e30, -1e30, 0.0, -0.0]), 1.0)
    assert list(got) == [0x7E, 0xFE, 0x7E, 0xFE, 0x00, 0x80]
    # with a scale, 448 * s is the largest value kept
    assert O.fp8_out(np.array([896.0, 1000.0]), 2.0).tolist() == [0x7E, 0x7E]


def test_fp8_epilogue_matches_torch_for_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    for s in (1.0, 0.125, 1.7):
        want = (torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * torch.tensor(np.float32(s))
                ).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(O.fp8_to_bf16(codes, s), want), s


def test_fp8_roundtrip_error_is_within_half_a_step():
    """Through FP8 and back, a value moves by at most half an E4M3 step (plus
    the bf16 rounding of the result): the extra rounding the FP8 output adds."""
    rng = np.random.default_rng(82)
    o = rng.standard_normal(20000) * 2.0
    back = _bf16_vals(O.fp8_to_bf16(O.fp8_out(o, 1.0), 1.0)).astype(np.float64)
    a = np.abs(o)
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(np.abs(back - o) <= step / 2 + np.abs(o) * 2.0 ** -8 + 1e-12)


def test_fp8_output_parity_bound_holds_and_has_no_slack():
    """The bound the GPU tests put on FP8 attention outputs
    (gpu_util.fp8_out_bound: half the E4M3 step at the decoded value's binade
    plus the attention tolerance) against brute force on the oracle's own
    encoder: for fp32 results y anywhere within the attention tolerance of a
    reference, the decoded code stays inside it, including references just
    below a power of two whose y rounds up into the next binade; and the
    worst case reaches at least 97% of it, so the bound carries no padding."""
    from gpu_util import fp8_out_bound
    rng = np.random.default_rng(85)
    for os in (1.0, 0.25, 0.03125):
        edges = 2.0 ** np.arange(-12, 8)
        ref = np.concatenate([edges * (1 - 1e-3), edges, edges * (1 + 1e-3), rng.uniform(-1, 1, 20000) *
                              2.0 ** rng.integers(-12, 7, 20000)]) * os
        ref = np.concatenate([ref, -ref])
        ref = ref[np.abs(ref) < 400 * os]
        tol = 2e-3 + 1e-2 * np.abs(ref)
        worst = 0.0
        for t in np.concatenate([np.linspace(-0.999, 0.999, 41), rng.uniform(-0.999, 0.999, 8)]):
            y = (ref + t * tol).astype(np.float32)
            got = O.e4m3_decode(O.fp8_out(y.astype(np.float64), os)) * os
            ratio = np.abs(got - ref) / fp8_out_bound(got, ref, os)
            assert np.all(ratio <= 1.0), (os, t, float(ratio.max()))
            worst = max(worst, float(ratio.max()))
        assert worst > 0.97, (os, worst)
