"""Helpers shared by the GPU tests: device tensors from the seeded inputs and
comparisons against the CPU oracle."""
import numpy as np


def torch_mod():
    import torch
    return torch


def to_device(x_f32, dtype="bf16"):
    """fp32 numpy array (already bf16-representable when dtype is bf16) ->
    device tensor of that dtype."""
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.to("cuda:0")


def q_to_host(q):
    return {
        "codes": q.codes.cpu().numpy(),
        "scales": q.scales.cpu().numpy(),
        "ts": float(q.tensor_scale.cpu().numpy()[0]),
    }


def nibbles(codes):
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = c & 15
    out[..., 1::2] = c >> 4
    return out


def assert_bit_exact(gpu, ref, what=""):
    assert gpu["ts"] == ref["ts"] or (np.isnan(gpu["ts"]) and np.isnan(ref["ts"])), \
        f"{what}: tensor scale {gpu['ts']!r} != {ref['ts']!r}"
    sd = np.flatnonzero(gpu["scales"].ravel() != ref["scales"].ravel())
    assert sd.size == 0, f"{what}: {sd.size} scale bytes differ, first at {sd[:5]}"
    cd = np.flatnonzero(gpu["codes"].ravel() != ref["codes"].ravel())
    assert cd.size == 0, f"{what}: {cd.size} code bytes differ, first at {cd[:5]}"


def assert_rotated_close(gpu, ref, frac=1e-5, what=""):
    """Rotation on: codes may differ by one adjacent level for at most `frac`
    of the elements (a zero code of either sign counts as equal), scales by
    one E4M3 step for at most `frac` of the blocks, the tensor scale within
    1e-5 relative.  IF4 (scale bit 7 = INT flag): a block whose FP4/INT4
    choice differs -- a decision at a tie that rounding moves, such as the
    INT scale of the block holding the tensor maximum, a/7 / s_t = 384
    exactly, rounded up -- counts as one differing scale, and its codes,
    which lie on the other grid, are not compared."""
    assert abs(gpu["ts"] - ref["ts"]) <= 1e-5 * abs(ref["ts"]), f"{what}: ts {gpu['ts']} vs {ref['ts']}"
    gs, rs = gpu["scales"].astype(np.int32), ref["scales"].astype(np.int32)
    flip = ((gs ^ rs) & 0x80) != 0
    ds = np.where(flip, 0, np.abs((gs & 0x7F) - (rs & 0x7F)))
    nd = np.count_nonzero(ds) + np.count_nonzero(flip)
    assert ds.max(initial=0) <= 1 and nd <= max(1, frac * ds.size), \
        f"{what}: {nd} scales differ (max {ds.max(initial=0)} steps, {np.count_nonzero(flip)} IF4 choices)"
    gn, rn = nibbles(gpu["codes"]).astype(np.int32), nibbles(ref["codes"]).astype(np.int32)
    same_sign = (gn >> 3) == (rn >> 3)
    dm = np.abs((gn & 7) - (rn & 7))
    # +0 and -0 are the same value: a rotated output that cancels to zero
    # may carry either sign, depending on the order of the additions
    zeros = ((gn & 7) == 0) & ((rn & 7) == 0)
    skip = np.repeat(flip, 16, axis=-1).reshape(gn.shape) if flip.any() else np.zeros(gn.shape, bool)
    bad = ~(((dm == 0) & same_sign) | zeros | skip)
    # one adjacent level: magnitudes differ by one (zero may flip sign)
    adj = (dm == 1) & (same_sign | ((gn & 7) == 0) | ((rn & 7) == 0))
    assert np.all(~bad | adj), f"{what}: codes differ by more than one level"
    assert np.count_nonzero(bad) <= max(1, frac * bad.size), f"{what}: {np.count_nonzero(bad)} codes differ"


def assert_rotation_values_close(z, ref, tol=1e-5, what=""):
    """Rotated fp32 values: in every 128-group along the last axis, each value
    within tol times the group's largest magnitude of the reference (a value
    that cancels to near zero has no meaningful relative error of its own;
    the coding of a block is relative to its largest magnitude)."""
    z = np.asarray(z, dtype=np.float64).reshape(-1, 128)
    r = np.asarray(ref, dtype=np.float64).reshape(-1, 128)
    scale = np.abs(r).max(axis=1, keepdims=True)
    err = np.abs(z - r)
    bad = err > tol * scale
    assert not bad.any(), (f"{what}: {np.count_nonzero(bad)} rotated values off by more than {tol} of their "
                           f"group's maximum (worst {float((err / np.maximum(scale, 1e-300)).max()):.3g})")
