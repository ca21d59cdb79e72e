"""Comparison helpers for GPU-vs-oracle parity tests.

Tolerances (floating point): the output bar is a max-abs error of 2e-2 *
RMS(oracle) for bf16 activations and 1e-5 * RMS for fp32, checked on the
layer output against the oracle's unrounded float64 value, not counting the
half ulp that storing the output in the activation type costs (assert_bar).  Intermediate
tensors that the layer stores in the activation type (latent rows, expert
outputs, combined rows) are checked element by element.  bf16: both sides
round almost the same value, so an element may differ by one unit in the last
place; a one-ulp flip of a stored input (a hidden activation, say) moves the
next stage's value by about 2^-8 |h w|: with a 1536-wide hidden layer whose
fp32 sums flip a few percent of the bf16 hidden values, an output element
moves by about 6e-4 RMS, more than its own ulp when it is near zero.  Every
element must satisfy |d| <= ulp(v) + 2e-2 RMS (one ulp plus the bar), and
the error's RMS must stay within 2^-7 RMS (storage rounding of both sides,
about 2^-8 RMS, plus the propagated flips).  fp32: tensors differ by the
float32 summation error of their dot products, bounded by the same 1e-5 RMS
as the output: |d| <= 4 ulp + 1e-5 RMS.
"""

import numpy as np
import torch

BAR = {"bf16": 2e-2, "f32": 1e-5}


def host(t):
    """Device tensor -> numpy (bf16 -> float64 values, others as is)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    return t.cpu().numpy()


def ulp(v, act):
    v = np.abs(np.asarray(v, dtype=np.float64))
    bits = 8 if act == "bf16" else 24
    e = np.floor(np.log2(np.maximum(v, 1e-38)))
    return 2.0 ** (e - (bits - 1))


def assert_stored_close(gpu, ref, act, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if ref.size == 0:
        return
    rms = float(np.sqrt(np.mean(ref ** 2))) or 1.0
    err = np.abs(gpu - ref)
    if act == "bf16":
        u = ulp(ref, act)
        hard = err > u + 2e-2 * rms
        assert not hard.any(), (f"{what}: {int(hard.sum())} of {ref.size} elements beyond ulp + 2e-2 rms; "
                                f"worst |d|={err.max():.3g}, rms={rms:.3g}")
        err_rms = float(np.sqrt(np.mean(err ** 2)))
        assert err_rms <= 2.0 ** -7 * rms, f"{what}: error rms {err_rms:.3g} > 2^-7 rms ({rms:.3g})"
    else:
        bad = err > 4 * ulp(ref, act) + 1e-5 * rms
        assert not bad.any(), (f"{what}: {int(bad.sum())} of {ref.size} elements outside tolerance; "
                               f"worst |d|={err.max():.3g}, rms={rms:.3g}")


def assert_bar(gpu, ref_exact, act, what):
    """Output bar: the error beyond the stored output's own rounding,
    max(|gpu - exact| - ulp(exact)/2, 0), is at most BAR[act] * RMS(exact).

    A value stored in the activation type cannot be nearer than half an ulp
    to the exact result; for outputs whose largest values are several times
    the RMS that half ulp alone can exceed 2e-2 RMS, so it is not counted
    against the bar.  Returns (bar ratio, raw max|d|/rms)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref_exact, dtype=np.float64)
    if ref.size == 0:
        return 0.0, 0.0
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(gpu - ref)
    if rms == 0.0:
        # an all-zero exact output (every assignment of every token dropped and
        # no shared experts): the bar has no scale, the result must be zero
        assert not err.any(), f"{what}: exact output is all zero, the result is not (max |d| {err.max():.3g})"
        return 0.0, 0.0
    beyond = np.maximum(err - 0.5 * ulp(ref, act), 0.0)
    ratio = float(beyond.max()) / rms
    raw = float(err.max()) / rms
    assert ratio <= BAR[act], f"{what}: error beyond rounding max/rms = {ratio:.3g} > {BAR[act]} (raw {raw:.3g})"
    return ratio, raw


def unambiguous_tokens(oracle_logits, gpu_logits, k):
    """Tokens whose ordered top-(k+1) oracle logits are separated by more than
    twice the largest GPU-vs-oracle logit difference: their top-k list cannot
    depend on the summation order.  Returns (mask, max difference)."""
    ol = np.asarray(oracle_logits, dtype=np.float64)
    delta = float(np.max(np.abs(np.asarray(gpu_logits, dtype=np.float64) - ol))) if ol.size else 0.0
    srt = -np.sort(-ol, axis=1)[:, :k + 1]
    gaps = srt[:, :-1] - srt[:, 1:]
    return np.all(gaps > 2 * delta, axis=1), delta
