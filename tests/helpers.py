"""Comparison metrics and device helpers shared by the GPU parity tests."""

import numpy as np

# Parity bar for fp16 inputs with fp32 accumulation against the fp64 oracle.
TOL_MAX_ABS = 1e-3
TOL_REL_L2 = 5e-3


def metrics(out, ref):
    """max abs, mean abs, relative L2 (whole tensor) and cosine of out vs ref."""
    o = np.asarray(out, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    d = o - r
    nr = np.linalg.norm(r)
    return dict(
        max_abs=float(np.abs(d).max()) if d.size else 0.0,
        mean_abs=float(np.abs(d).mean()) if d.size else 0.0,
        rel_l2=float(np.linalg.norm(d) / nr) if nr > 0 else float(np.linalg.norm(d)),
        cosine=float((o * r).sum() / (np.linalg.norm(o) * nr)) if nr > 0 else 1.0,
        finite=bool(np.isfinite(o).all()),
    )


def assert_parity(out, ref, label=""):
    m = metrics(out, ref)
    print(f"[parity] {label} {m}", flush=True)
    assert m["finite"], f"{label}: non-finite output"
    assert m["max_abs"] <= TOL_MAX_ABS, f"{label}: max abs {m['max_abs']:.3e} > {TOL_MAX_ABS}"
    assert m["rel_l2"] <= TOL_REL_L2, f"{label}: rel L2 {m['rel_l2']:.3e} > {TOL_REL_L2}"
    return m


def to_dev(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def to_host(t):
    import torch

    torch.cuda.synchronize()
    return t.cpu().numpy()
