"""Helpers shared by the GPU parity tests: device copies of the seeded
inputs and the comparison rules.

Tolerance for fp16 outputs with fp32 accumulation (fixed by the workload
definition): relative L2 error <= 1e-3 and max |gpu - ref| <=
5e-3 * max |ref|, with the oracle's float64 result as ref.
"""
import numpy as np

REL_L2 = 1e-3
MAX_ABS_FRAC = 5e-3


def dev():
    import torch
    return torch.device("cuda:0")


def t(a, device=None):
    """numpy -> torch on the GPU (uint32 arrays travel as int32 bit patterns)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
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


def assert_close(gpu, ref, what=""):
    rel, mabs, mref = errors(gpu, ref)
    assert np.all(np.isfinite(np.asarray(gpu, dtype=np.float64))), f"{what}: non-finite output"
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > {REL_L2}"
    assert mabs <= MAX_ABS_FRAC * mref + 1e-30, f"{what}: max-abs {mabs:.3e} > {MAX_ABS_FRAC}*{mref:.3e}"
    return rel, mabs / max(mref, 1e-30)


def say(*a):
    print(*a, flush=True)
