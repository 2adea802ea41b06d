"""Comparison helpers shared by the GPU parity tests."""
import numpy as np
import torch

# Tolerances for bf16 operands (fp32 accumulation): relative L2 error over the
# whole tensor and max-abs error relative to the largest reference magnitude.
BF16_REL_L2 = 5e-3
BF16_MAX_ABS_FRAC = 2e-2
# fp32 operands: no bf16 rounding anywhere on the path; the remaining error is
# fp32 accumulation plus the hardware exp2 (about 1 ulp).
F32_REL_L2 = 1e-5
F32_MAX_ABS_FRAC = 1e-4


def to_np(t):
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def errors(got, ref):
    got, ref = to_np(got), to_np(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU result"
    d = got - ref
    rl2 = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
    mabs = np.max(np.abs(d)) / max(np.max(np.abs(ref)), 1e-300)
    return rl2, mabs


def assert_close(got, ref, io_dtype, what=""):
    rl2, mabs = errors(got, ref)
    if io_dtype in ("bf16", torch.bfloat16):
        tl2, tabs = BF16_REL_L2, BF16_MAX_ABS_FRAC
    else:
        tl2, tabs = F32_REL_L2, F32_MAX_ABS_FRAC
    assert rl2 <= tl2 and mabs <= tabs, \
        "%s: rel-L2 %.3e (limit %.1e), max-abs/max|ref| %.3e (limit %.1e)" % (what, rl2, tl2, mabs, tabs)
    return rl2, mabs


class WholeTensorError:
    """rel-L2 and max-abs/max|ref| of a whole tensor, accumulated over slices.

    add(got, ref) takes matching slices (any partition of the tensor);
    result() gives the same two numbers as ``errors`` on the whole tensor.
    """

    def __init__(self):
        self.d2 = 0.0
        self.r2 = 0.0
        self.dmax = 0.0
        self.rmax = 0.0

    def add(self, got, ref):
        got, ref = to_np(got), to_np(ref)
        assert got.shape == ref.shape, (got.shape, ref.shape)
        assert np.all(np.isfinite(got)), "non-finite values in the GPU result"
        d = got - ref
        self.d2 += float(np.sum(d * d))
        self.r2 += float(np.sum(ref * ref))
        self.dmax = max(self.dmax, float(np.max(np.abs(d))))
        self.rmax = max(self.rmax, float(np.max(np.abs(ref))))

    def result(self):
        return (np.sqrt(self.d2) / max(np.sqrt(self.r2), 1e-300),
                self.dmax / max(self.rmax, 1e-300))

    def check(self, io_dtype, what=""):
        rl2, mabs = self.result()
        if io_dtype in ("bf16", torch.bfloat16):
            tl2, tabs = BF16_REL_L2, BF16_MAX_ABS_FRAC
        else:
            tl2, tabs = F32_REL_L2, F32_MAX_ABS_FRAC
        assert rl2 <= tl2 and mabs <= tabs, \
            "%s: rel-L2 %.3e (limit %.1e), max-abs/max|ref| %.3e (limit %.1e)" % (
                what, rl2, tl2, mabs, tabs)
        return rl2, mabs
