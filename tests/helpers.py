"""Comparison metrics and device helpers shared by the GPU parity tests."""

import numpy as np

# Parity bar for fp16 inputs with fp32 accumulation against the fp64 oracle:
# max abs error 1e-3 beyond the rounding of the result to the fp16 output
# format (unit roundoff 2^-11 of |O|, at most half an fp16 ulp), and relative
# L2 error 5e-3 over the whole tensor.  The long-prefill page's 1e-3 envelope
# (Test Result) compares two fp16 outputs, which share that rounding; against
# the unrounded fp64 oracle it has to be allowed for explicitly, since an fp16
# value of magnitude 2..4 is already up to 9.8e-4 from the exact result.
TOL_MAX_ABS = 1e-3
TOL_REL_L2 = 5e-3
FP16_UNIT_ROUNDOFF = 2.0 ** -11


def metrics(out, ref):
    """max abs, mean abs, relative L2 (whole tensor) and cosine of out vs ref."""
    o = np.asarray(out, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    d = o - r
    nr = np.linalg.norm(r)
    excess = np.abs(d) - FP16_UNIT_ROUNDOFF * np.abs(r)
    i = int(np.argmax(np.abs(d))) if d.size else 0
    return dict(
        max_abs=float(np.abs(d).max()) if d.size else 0.0,
        max_abs_beyond_fp16_rounding=float(excess.max()) if d.size else 0.0,
        ref_at_max_abs=float(r.reshape(-1)[i]) if d.size else 0.0,
        mean_abs=float(np.abs(d).mean()) if d.size else 0.0,
        rel_l2=float(np.linalg.norm(d) / nr) if nr > 0 else float(np.linalg.norm(d)),
        cosine=float((o * r).sum() / (np.linalg.norm(o) * nr)) if nr > 0 else 1.0,
        finite=bool(np.isfinite(o).all()),
    )


def assert_parity(out, ref, label=""):
    m = metrics(out, ref)
    print(f"[parity] {label} {m}", flush=True)
    assert m["finite"], f"{label}: non-finite output"
    assert m["max_abs_beyond_fp16_rounding"] <= TOL_MAX_ABS, (
        f"{label}: max abs error beyond fp16 output rounding {m['max_abs_beyond_fp16_rounding']:.3e} > {TOL_MAX_ABS}")
    assert m["rel_l2"] <= TOL_REL_L2, f"{label}: rel L2 {m['rel_l2']:.3e} > {TOL_REL_L2}"
    return m


def to_dev(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def to_host(t):
    import torch

    torch.cuda.synchronize()
    return t.cpu().numpy()
