"""Shared helpers for the GPU parity tests (not collected by pytest)."""

import sys

import numpy as np
import torch

# Tolerances (max-abs error against the fp64 oracle): fp32 inputs 1e-5 on out
# and lse; bf16 inputs with fp32 accumulation 2e-2 on out and 1e-3 on lse.
TOL = {torch.float32: (1e-5, 1e-5), torch.bfloat16: (2e-2, 1e-3)}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rand(shape, seed, dtype):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


def gpu(*ts):
    return [t.to("cuda") for t in ts]


def maxerr(got, want):
    """Max-abs error; matching infinities (lse of an empty row) count as equal."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert not np.isnan(got).any(), "NaN in GPU result"
    same_inf = np.isinf(got) & np.isinf(want) & (np.sign(got) == np.sign(want))
    with np.errstate(invalid="ignore"):
        d = np.where(same_inf, 0.0, np.abs(got - want))
    return float(d.max()) if d.size else 0.0


def to_np(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def check(out, lse, ref_out, ref_lse, dtype, what=""):
    tol_o, tol_l = TOL[dtype]
    eo = maxerr(to_np(out), ref_out)
    el = maxerr(to_np(lse), ref_lse)
    log(f"  {what}: max|out err| = {eo:.3e} (tol {tol_o}), max|lse err| = {el:.3e} (tol {tol_l})")
    assert eo <= tol_o, f"{what}: out error {eo} > {tol_o}"
    assert el <= tol_l, f"{what}: lse error {el} > {tol_l}"
    return eo, el
