"""Comparison helpers shared by the GPU parity tests.

The spec's float bound is max|err| <= tol x RMS(ref): tol = 2e-2 for bfloat16
storage, 1e-5 for float32.  A stored result is rounded to its format, and one
rounding step of a value v is up to half a unit in the last place of v; for
bfloat16 that exceeds 2e-2 x RMS once |v| is past about 5 x RMS, and a result
whose float32 accumulation lands on the other side of a rounding midpoint than
the exact value (or whose inputs did) is one whole unit away.  So an element may
exceed the plain bound by at most one storage unit of its own magnitude; such
elements are counted, must be rare (at most max(2, 0.1%) of a comparison), and
every comparison's figures -- max|err|/RMS against the plain bound, the number
of elements past it and max|ref|/RMS -- are recorded and printed at the end of
the session.  The layer's output y and the pool's unpermuted output are held to
the plain bound with no allowance (strict): the allowance serves the stored
intermediate stages (h, Y, c), whose rare large elements are rounded to bf16 by
more than the bound.
"""
import json
import os

import numpy as np

TOL = {"bf16": 2e-2, "f32": 1e-5}
# explicit mantissa bits of each storage format
MANT = {"bf16": 7, "f32": 23}

RECORDS = []


def rms(a) -> float:
    return float(np.sqrt(np.mean(np.square(np.asarray(a, np.float64)))))


def storage_ulp(ref, dt: str) -> np.ndarray:
    """One unit in the last place of each |ref| in the storage format dt."""
    a = np.abs(np.asarray(ref, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - MANT[dt]), 0.0)


def record(what: str, **stats):
    rec = dict(what=what, **stats)
    RECORDS.append(rec)
    path = os.environ.get("MOE_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")
    return rec


def assert_close(got, ref, dt: str, what: str, strict: bool = False) -> dict:
    """The spec's bound on every element, except that an element past it may be
    off by one storage unit of its own magnitude more; such elements are rare.
    strict: the plain bound on every element, with no allowance (used for the
    layer's output and the pool's unpermuted output).  Returns (and records) the
    comparison's figures."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.size == 0:
        return record(what, dt=dt, n=0, err_rms=0.0, n_beyond=0, max_ref_rms=0.0)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    r = rms(ref)
    err = np.abs(got - ref)
    base = TOL[dt] * r
    beyond = err > base
    n_beyond = int(beyond.sum())
    stats = dict(dt=dt, n=int(err.size), err_rms=float(err.max() / r) if r > 0 else 0.0,
                 n_beyond=n_beyond, max_ref_rms=float(np.abs(ref).max() / r) if r > 0 else 0.0)
    if n_beyond:
        # how far out the elements past the plain bound sit
        stats["beyond_min_ref_rms"] = float(np.abs(ref[beyond]).min() / r)
    record(what, **stats)
    if strict:
        assert n_beyond == 0, (
            f"{what}: max|err| {err.max():.3e} = {err.max() / r:.3e} x RMS exceeds "
            f"{TOL[dt]:g} x RMS")
    allow = base + storage_ulp(ref, dt)
    worst = int(np.argmax(err - allow))
    assert np.all(err <= allow), (
        f"{what}: |err| {err.flat[worst]:.3e} at |ref| {abs(ref.flat[worst]):.3e} exceeds "
        f"{TOL[dt]:g} x RMS {r:.3e} plus one storage unit")
    assert n_beyond <= max(2, 1e-3 * err.size), \
        f"{what}: {n_beyond} of {err.size} elements past {TOL[dt]:g} x RMS"
    return stats


def summary_lines():
    """One line per recorded comparison, for the end-of-session report."""
    out = []
    for rec in RECORDS:
        extra = (f", {rec['n_beyond']} past the bound (|ref| >= "
                 f"{rec['beyond_min_ref_rms']:.1f} x RMS)" if rec.get("n_beyond") else "")
        out.append(f"{rec['what']}: {rec.get('n', 0)} values, max|err| = "
                   f"{rec.get('err_rms', 0):.3g} x RMS (bound {TOL.get(rec.get('dt'), 0):g}), "
                   f"max|ref| = {rec.get('max_ref_rms', 0):.1f} x RMS{extra}")
    return out
