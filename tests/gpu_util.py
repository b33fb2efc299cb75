"""Comparison helpers shared by the GPU parity tests."""
import numpy as np

TOL = {"bf16": 2e-2, "f32": 1e-5}
# One unit in the last place of a stored value, relative to its magnitude: a
# correctly rounded result may sit one storage unit from the exact value (the
# rounding step itself, or a neighbouring rounding decision taken from a float32
# value that differs from the double one in its last bits).
STORE_ULP = {"bf16": 2.0 ** -7, "f32": 2.0 ** -23}


def rms(a) -> float:
    return float(np.sqrt(np.mean(np.square(np.asarray(a, np.float64)))))


def assert_close(got, ref, dt: str, what: str) -> dict:
    """The spec's bound, max|err| <= tol x RMS(ref), where each element may in
    addition be off by one storage unit of its own magnitude.  Elements that need
    that allowance are counted and must be rare; the statistics are returned so
    callers can report them."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.size == 0:
        return dict(err_rms=0.0, n_beyond=0)
    r = rms(ref)
    err = np.abs(got - ref)
    base = TOL[dt] * r
    allow = base + STORE_ULP[dt] * np.abs(ref)
    worst = int(np.argmax(err - allow))
    assert np.all(err <= allow), (
        f"{what}: |err| {err.flat[worst]:.3e} at |ref| {abs(ref.flat[worst]):.3e} exceeds "
        f"{TOL[dt]:g} x RMS {r:.3e} + one storage ulp")
    n_beyond = int(np.sum(err > base))
    assert n_beyond <= max(2, 1e-3 * err.size), f"{what}: {n_beyond} elements beyond the bound"
    return dict(err_rms=float(err.max() / r) if r > 0 else 0.0, n_beyond=n_beyond,
                max_over_rms=float(np.abs(ref).max() / r) if r > 0 else 0.0)
