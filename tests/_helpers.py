"""Shared test helpers: moving seeded inputs to the device, error metrics and the parity bars."""
import numpy as np
import torch

# Bars: bf16 inputs with fp32 accumulation -> max-abs <= 2e-2 and mean-abs <= 2e-3 against the float64 oracle on the
# same rounded inputs; fp32 path -> 1e-5 relative (max |O - O_ref| / max |O_ref|). A normalised rms error above 1e-2
# would mean a bug even inside those bars (the expected value for a correct kernel is about 2e-3).
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_NRMS = 1e-2
F32_REL = 1e-5


def to_dev(q, device="cuda"):
    """A workloads.Quantised tensor -> device tensor holding exactly the same values."""
    if q.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(q.raw).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(q.raw))
    return t.to(device)


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    rms_ref = float(np.sqrt(np.mean(np.square(ref)))) or 1.0
    return {"max_abs": float(d.max()), "mean_abs": float(d.mean()),
            "nrms": float(np.sqrt(np.mean(np.square(d)))) / rms_ref,
            "rel": float(d.max() / max(np.abs(ref).max(), 1e-300))}


def assert_bf16_parity(got, ref, what=""):
    e = errors(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS and e["nrms"] <= BF16_NRMS, f"{what}: {e}"
    return e


def assert_f32_parity(got, ref, what=""):
    e = errors(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert e["rel"] <= F32_REL, f"{what}: {e}"
    return e
