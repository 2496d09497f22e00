"""Shared helpers of the parity tests: uploads and the parity metrics.

Parity bars (from the OSDN forward's stated tolerances):
  * float32 inputs: d and k~ within 1e-5, o and S within 1e-4, relative, measured
    element-wise as |x - ref| / max(|ref|, rms(ref));
  * bfloat16 inputs with fp32 accumulation: o and S within 2e-2 max-abs error
    normalised by the output RMS, where "output" is one readout vector o_t (one
    (b,t,h) row over V) and one head's final state S (V x K).  Rounding the
    exact result to bf16 alone costs up to 2^-9 * max/rms of the normalising
    group; per row that stays near 1%, while a tensor-wide RMS would fail even a
    correctly rounded result whenever outputs decay over the sequence.  Rows
    whose RMS falls below 1% of the tensor RMS are judged against that floor;
  * d (fp32 arithmetic) within 1e-5 relative; k~ rounded to bf16 on the device
    within one bf16 ulp of the fp64 value.
"""
import numpy as np

from workloads import bf16_ulp

F32_D, F32_KT, F32_OS = 1e-5, 1e-5, 1e-4
BF16_OS = 2e-2


def rms(x):
    x = np.asarray(x, np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def rel_err(x, ref):
    """max_i |x_i - ref_i| / max(|ref_i|, rms(ref))."""
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = np.maximum(np.abs(ref), max(rms(ref), 1e-30))
    return float(np.max(np.abs(x - ref) / den))


def rms_err(x, ref):
    """max|x - ref| / rms(ref)."""
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(x - ref)) / max(rms(ref), 1e-30))


def group_err(x, ref, ndim=1, floor=1e-2):
    """max over groups of max|x - ref| / rms(ref group); a group is the last
    `ndim` axes (1: one output vector o_t, 2: one head's state).  Group RMS is
    floored at `floor` times the whole tensor's RMS."""
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    axes = tuple(range(ref.ndim - ndim, ref.ndim))
    err = np.max(np.abs(x - ref), axis=axes)
    grp = np.sqrt(np.mean(ref * ref, axis=axes))
    den = np.maximum(grp, floor * max(rms(ref), 1e-30))
    return float(np.max(err / den))


def o_err(x, ref):
    """bf16 parity metric of the readout o [..., V]."""
    return group_err(x, ref, 1)


def s_err(x, ref):
    """bf16 parity metric of a state S [..., V, K] (per head)."""
    return group_err(x, ref, 2)


def ulp_err(x, ref):
    """max |x - ref| in units of the bf16 spacing at ref."""
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(x - ref) / bf16_ulp(ref)))


def to_dev(x, dtype, device="cuda:0"):
    """numpy float32 array -> torch tensor of `dtype` ('f32'/'bf16'/'float32')."""
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    if dtype in ("bf16", torch.bfloat16):
        t = t.to(torch.bfloat16)
    return t.to(device).contiguous()


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def dtype_round(x, dtype):
    """The values a device tensor of `dtype` holds for float data x."""
    from workloads import bf16_round
    x = np.asarray(x, np.float32)
    return bf16_round(x) if dtype == "bf16" else x
