"""Shared helpers of the GPU tests: upload a synthetic workload, run the HIP
path through the C ABI, and compare against the oracle with the stated
tolerances."""
from __future__ import annotations

import numpy as np

# Tolerances (bf16 inputs; the oracle is fed the same bf16-rounded values):
BF16_ABS = 2e-2       # max-abs on outputs and gradients
BF16_LSE_REL = 1e-3   # |dLSE| <= tol * max(1, |LSE|)
BF16_FROB = 1e-2      # relative Frobenius error, guards small-magnitude outputs
F32_ABS = 1e-5        # fp32: max-abs on outputs, same relative form on LSE


def to_device(w, name, dev):
    import torch
    x = getattr(w, name)
    if w.is_bf16:
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(x).to(dev)


def to_np64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def make_path(w, dev, **kw):
    import torch
    from block_sparse_draft_amd import SplitKVAttention
    c = w.cfg
    dt = torch.bfloat16 if w.is_bf16 else torch.float32
    kw.setdefault("fwd_runs_per_worker", None)  # one partial per chunk unless a test asks for runs
    return SplitKVAttention(w.q_off, w.kv_off, w.anchors, c.block, c.hq, c.hkv, c.d, c.chunk, w.sm_scale, dt, dev,
                            with_bwd=kw.pop("with_bwd", c.bwd and w.is_bf16), **kw)


def rel_frob(x, ref):
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def assert_close(name, x, ref, abs_tol, frob_tol=None, mask=None):
    if mask is not None:
        x, ref = x[mask], ref[mask]
    assert np.isfinite(x).all(), f"{name}: non-finite values"
    err = float(np.max(np.abs(x - ref))) if x.size else 0.0
    fr = rel_frob(x, ref)
    msg = f"{name}: max-abs {err:.3e} (tol {abs_tol:.1e}), rel-frob {fr:.3e}, max|ref| {np.max(np.abs(ref)) if ref.size else 0:.3e}"
    print(msg)
    assert err <= abs_tol, msg
    if frob_tol is not None:
        assert fr <= frob_tol, msg


def assert_lse(name, x, ref, rel_tol):
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(x)), f"{name}: -inf pattern differs"
    assert np.array_equal(x[~fin], ref[~fin]), f"{name}: infinite values differ"
    d = np.abs(x[fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin]))
    err = float(d.max()) if d.size else 0.0
    print(f"{name}: max rel {err:.3e} (tol {rel_tol:.1e})")
    assert err <= rel_tol, f"{name}: {err}"
