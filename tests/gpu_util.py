"""Helpers shared by the GPU parity tests: device copies of the seeded
inputs and the comparison rules.

Tolerance for fp16 outputs with fp32 accumulation (fixed by the workload
definition): relative L2 error <= 1e-3 and max |gpu - ref| <=
5e-3 * max |ref|, with the oracle's float64 result as ref.
"""
import numpy as np

REL_L2 = 1e-3
MAX_ABS_FRAC = 5e-3
# bf16 outputs (derived, no stated bar): a bf16 has 8 significant bits, so
# rounding an output is off by at most 2**-8 = 3.9e-3 relative and by about
# 1.6e-3 RMS over a spread of mantissas (measured 1.2e-3 to 1.9e-3 for the
# GEMV, which multiplies the exact codes); the GEMM also rounds each
# dequantized weight to bf16 once, about 1.5e-3 more (measured 2.2e-3 in
# total).  Bars: rel-L2 <= 4e-3 (the per-element bound) and max-abs <=
# 1.6e-2 * max|ref| (four times it).
REL_L2_BF16 = 4e-3
MAX_ABS_FRAC_BF16 = 1.6e-2
# bf16 routed-expert layer (derived the same way): its output passes through
# seven independent bf16 roundings the oracle does not share - the gate and
# the up weights (both enter act = SiLU(gate) * up), act on each side (the
# two round different pre-values), the down weights, ydown and the output -
# each about 1.6e-3 RMS relative, so sqrt(7) * 1.6e-3 = 4.2e-3 RMS (measured
# 4.0e-3 to 4.2e-3 for out).  Bars: rel-L2 <= 6e-3 and max-abs <= 2.4e-2 *
# max|ref| (four times it), for act, ydown and out alike.
REL_L2_BF16_MOE = 6e-3
MAX_ABS_FRAC_BF16_MOE = 2.4e-2


def dev():
    import torch
    return torch.device("cuda:0")


def t(a, device=None):
    """numpy -> torch on the GPU (uint32 / uint16 arrays travel as int32 /
    int16 bit patterns)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device or dev())


def w4_dev(W):
    return {"qweight": t(W["qweight"]), "scales": t(W["scales"]), "biases": t(W["biases"]),
            "K": int(W["K"]), "N": int(W["N"])}


def host(x):
    return x.detach().cpu().numpy()


def errors(gpu, ref):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    den = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / den if den > 0 else np.linalg.norm(g - r)
    mref = np.abs(r).max() if r.size else 0.0
    mabs = np.abs(g - r).max() if r.size else 0.0
    return rel, mabs, mref


def assert_close(gpu, ref, what="", rel_l2=REL_L2, max_abs_frac=MAX_ABS_FRAC):
    rel, mabs, mref = errors(gpu, ref)
    assert np.all(np.isfinite(np.asarray(gpu, dtype=np.float64))), f"{what}: non-finite output"
    assert rel <= rel_l2, f"{what}: rel-L2 {rel:.3e} > {rel_l2}"
    assert mabs <= max_abs_frac * mref + 1e-30, f"{what}: max-abs {mabs:.3e} > {max_abs_frac}*{mref:.3e}"
    return rel, mabs / max(mref, 1e-30)


def assert_close_bf16(gpu_bits, ref, what="", rel_l2=REL_L2_BF16, max_abs_frac=MAX_ABS_FRAC_BF16):
    """gpu_bits: bf16 patterns (uint16 / int16 array); ref: float64."""
    g = (np.asarray(gpu_bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return assert_close(g, ref, what, rel_l2, max_abs_frac)


def say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# Guard regions around outputs.  An output tensor is carved out of a larger
# buffer: the bytes before and after it hold GUARD_BYTE and must still hold
# it after the call (a write past either end of an output, by a ragged tile,
# the scatter or a tile-map entry, changes them); the output itself starts
# as FILL_BYTE (NaN in fp16 / fp32, -1 in int32), so an element no kernel
# wrote shows up as NaN or -1.
# ---------------------------------------------------------------------------
GUARD_BYTE = 0x5A
FILL_BYTE = 0xFF
GUARD_PAD = 4096  # bytes on each side (keeps the output 256-byte aligned)


class Guarded:
    """An output tensor with guard regions; ``check()`` asserts the guards
    are intact.  ``t`` is the output view."""

    def __init__(self, shape, dtype, device=None):
        import torch
        shape = tuple(int(s) for s in (shape if isinstance(shape, (tuple, list)) else (shape,)))
        elem = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) if shape else 1
        self.pad = GUARD_PAD // elem
        self.n = n
        self.elem = elem
        self.buf = torch.empty((2 * self.pad + n,), dtype=dtype, device=device or dev())
        raw = self.buf.view(torch.uint8)
        raw.fill_(GUARD_BYTE)
        raw[self.pad * elem:(self.pad + n) * elem].fill_(FILL_BYTE)
        self.t = self.buf[self.pad:self.pad + n].view(shape)

    def check(self, what=""):
        raw = self.buf.view(__import__("torch").uint8).cpu().numpy()
        head = raw[:self.pad * self.elem]
        tail = raw[(self.pad + self.n) * self.elem:]
        bad_h = np.flatnonzero(head != GUARD_BYTE)
        bad_t = np.flatnonzero(tail != GUARD_BYTE)
        assert bad_h.size == 0, f"{what}: {bad_h.size} bytes written before the output (first at -{head.size - bad_h[0]})"
        assert bad_t.size == 0, f"{what}: {bad_t.size} bytes written after the output (first at +{bad_t[0]})"


def guarded(shape, dtype, device=None) -> Guarded:
    return Guarded(shape, dtype, device)


def assert_close_nan(gpu, ref, what="", rel_l2=REL_L2, max_abs_frac=MAX_ABS_FRAC):
    """NaN-aware comparison: NaN exactly where the reference is NaN, and the
    finite entries within the bars.  Returns the number of NaN entries."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    gn, rn = np.isnan(g), np.isnan(r)
    assert np.array_equal(gn, rn), f"{what}: NaN at {int((gn & ~rn).sum())} extra and {int((rn & ~gn).sum())} missing positions"
    if (~rn).any():
        assert_close(g[~rn], r[~rn], what, rel_l2, max_abs_frac)
    return int(rn.sum())
