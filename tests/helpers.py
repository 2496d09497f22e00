"""Shared helpers of the parity tests: uploads and the parity metrics.

Parity bars (from the OSDN forward's stated tolerances):
  * float32 inputs: d and k~ within 1e-5, o and S within 1e-4, relative, measured
    element-wise as |x - ref| / max(|ref|, rms(ref));
  * bfloat16 inputs with fp32 accumulation: o and S within 2e-2 of
    max|x - ref| / rms(ref) over the whole tensor (``tw_err``).  S is float32.
    For o this bar is asserted on the float32 readout (o_f32), i.e. on the
    kernel arithmetic before the final rounding to bf16: rounding the exact
    readout to bf16 alone (unit roundoff 2^-8) already costs up to 2^-8 max|o| /
    rms(o), which over whole tensors of the sequence workloads reaches 0.019 to
    0.031 (``round_floor``, printed beside every error).  The bf16 readout must
    then be the round-to-nearest-even of that float32 readout, bit for bit.
    The float32 readout must also meet 2e-2 within each (b,h) sequence
    (``seq_err``) and the state within each head (``s_err``: max|x - ref| over
    the group's RMS, floored at 1% of the tensor RMS).  The same ratio per
    output vector o_t (``o_err``) is printed, not asserted: an output vector
    far smaller than its sequence's RMS meets it only with absolute errors far
    below the stated bar;
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
    """max|x - ref| / rms(ref) (the tensor-wide metric)."""
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(x - ref)) / max(rms(ref), 1e-30))


tw_err = rms_err


def round_floor(ref):
    """Tensor-wide error of the exact values rounded to bf16 (nearest even):
    what the output rounding alone costs under ``tw_err``."""
    from workloads import bf16_round
    ref = np.asarray(ref, np.float64)
    return rms_err(bf16_round(ref.astype(np.float32)), ref)


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


def seq_err(x, ref):
    """max over (b,h) sequences of max|x - ref| / rms(ref) within the sequence:
    the tensor-wide metric applied to each head's readout [T, V] of a
    [B,T,H,V] tensor (each head of a packed [1,total,H,V] one)."""
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    err = np.max(np.abs(x - ref), axis=(1, 3))
    den = np.sqrt(np.mean(ref * ref, axis=(1, 3)))
    return float(np.max(err / np.maximum(den, 1e-30)))


def check_bf16_readout(o16, o32, ref, label=""):
    """bf16 parity of a readout o [B,T,H,V]: the float32 readout (same call
    with o_f32) within 2e-2 tensor-wide and per (b,h) sequence; the bf16
    readout equal to its nearest-even rounding bit for bit.  Prints the
    errors of both forms, what the rounding to bf16 alone costs, and the
    per-output-vector form (diagnostic)."""
    from workloads import bf16_bits
    o16, o32, ref = (np.asarray(x, np.float64) for x in (o16, o32, ref))
    e32, e16, fl = tw_err(o32, ref), tw_err(o16, ref), round_floor(ref)
    q32, g32 = seq_err(o32, ref), o_err(o32, ref)
    print("%s o: tensor-wide f32 %.3e  bf16 %.3e (rounding floor %.3e)  per-sequence f32 %.3e  "
          "per-row f32 %.3e" % (label, e32, e16, fl, q32, g32))
    assert e32 <= BF16_OS, (label, "f32 readout tensor-wide", e32)
    assert q32 <= BF16_OS, (label, "f32 readout per sequence", q32)
    rounded = bf16_bits(bf16_round32(o32))
    assert np.array_equal(rounded, bf16_bits(o16.astype(np.float32))), (label, "bf16 readout is not RNE(f32 readout)")
    return e32, e16, fl, q32


def check_bf16_state(S, ref, label=""):
    """bf16-input parity of a float32 state: 2e-2 tensor-wide and per head."""
    et, eh = tw_err(S, ref), s_err(S, ref)
    print("%s S: tensor-wide %.3e  per-head %.3e" % (label, et, eh))
    assert et <= BF16_OS, (label, "S tensor-wide", et)
    assert eh <= BF16_OS, (label, "S per-head", eh)
    return et, eh


def bf16_round32(x):
    from workloads import bf16_round
    return bf16_round(np.asarray(x, np.float32))
