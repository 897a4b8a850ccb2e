"""Shared test helpers: tolerances and device/oracle plumbing (no method arithmetic)."""
import numpy as np

from oracle.numerics import to_f64

# NaN fill bits of the caches on both sides (torch's canonical NaN per dtype)
NAN_BITS = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00)}


def tolerance_report(got, ref, dtype):
    """Elementwise and per-row checks of decode outputs.

    fp32: |got - ref| <= 1e-6 + 1e-5 |ref|.
    bf16/fp16: |got - ref| <= 5e-3 + 2e-2 |ref| elementwise, and per (seq, head)
    ||got - ref||_2 <= 2e-2 ||ref||_2 (the elementwise bar alone is loose once
    outputs shrink like 1/sqrt(len) at long contexts).
    Returns (ok, details).
    """
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    if dtype == "f32":
        bound = 1e-6 + 1e-5 * np.abs(ref)
        ok = bool(np.all(err <= bound))
        return ok, {"max_abs": float(err.max(initial=0)), "worst_ratio":
                    float((err / bound).max(initial=0))}
    bound = 5e-3 + 2e-2 * np.abs(ref)
    ok_elem = bool(np.all(err <= bound))
    d = got.shape[-1]
    num = np.sqrt(((got - ref) ** 2).reshape(-1, d).sum(1))
    den = np.sqrt((ref ** 2).reshape(-1, d).sum(1))
    rel = np.where(den > 0, num / np.maximum(den, 1e-300), num)
    ok_l2 = bool(np.all(rel <= 2e-2))
    return ok_elem and ok_l2, {"max_abs": float(err.max(initial=0)),
                               "worst_ratio": float((err / bound).max(initial=0)),
                               "max_rel_l2": float(rel.max(initial=0))}


def assert_close(got_bits, ref, dtype, what=""):
    got = to_f64(got_bits, dtype)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ok, info = tolerance_report(got, ref, dtype)
    assert ok, f"{what}: {info}"
    return info


def bits_of(t):
    """A torch tensor's storage bits as numpy (uint16 for 2-byte dtypes)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
