"""Error measures of the GPU parity tests (shared by the test modules).

The bar of the operator's statement is max |gpu - oracle| / RMS(oracle):
2e-2 for bf16 I/O with fp32 accumulation, 1e-4 for fp32 I/O.  Every case
drawn from the workload recipe is held to it as it stands (`plain`).

Named stress inputs (random gates, random RMSNorm weights, a sharpened
softmax) and gradients have heavy-tailed outputs: their largest element is
several times the RMS (`peak` = max|ref| / RMS(ref)), and rounding one bf16
output to nearest moves it by up to 2^-9 of itself, i.e. up to 2^-9 * peak of
the RMS before any arithmetic error.  For those cases only, the same bar is
applied to the error in excess of each element's own half-ulp (`excess`);
the plain error may then exceed the bar only when peak >= 5, where output
rounding alone takes at least half of it.  Each such case logs all three.

A quantity formed as one floating-point sum of many products whose signs
cancel (the gradient of a write strength, dbeta) cannot be computed in fp32
to better than about unit roundoff times the total absolute size of its
terms (`mass`, from the oracle): the standard error bound of an inner
product.  For it, `check_sum` adds SUM_SLACK * 2^-24 * mass to each
element's allowance; where the terms do not cancel that addition is a small
fraction of the bar.
"""
import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}
STRESS_PEAK = 5.0
SUM_SLACK = 16.0


def rel_err(got, ref):
    """max |got - ref| / RMS(ref); where ref is exactly zero, max |got|."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return err / rms if rms > 0 else err


def excess_err(got, ref, dtype):
    """max(|got - ref| - ulp/2(ref), 0) / RMS(ref); plain rel_err for fp32."""
    if dtype != "bf16":
        return rel_err(got, ref)
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    exc = np.maximum(np.abs(got - ref) - 2.0 ** -9 * np.abs(ref), 0.0)
    return float(np.max(exc) / np.sqrt(np.mean(ref * ref)))


def peak(ref):
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(ref)) / np.sqrt(np.mean(ref * ref)))


def check(log, tag, got, ref, dtype, stress=False, tol=None):
    """Assert the bar on one output; returns the plain error.  stress=True
    marks a named stress input or a gradient (see the module docstring)."""
    tol = TOL[dtype] if tol is None else tol
    plain = rel_err(got, ref)
    if not stress:
        log(f"  {tag}: rel err {plain:.3e} (tol {tol})")
        assert plain <= tol, (tag, plain)
        return plain
    exc = excess_err(got, ref, dtype)
    pk = peak(ref)
    log(f"  {tag} [stress]: rel err {plain:.3e}, beyond output rounding {exc:.3e}, max/RMS {pk:.2f} (tol {tol})")
    assert exc <= tol, (tag, exc)
    assert plain <= tol or pk >= STRESS_PEAK, (tag, plain, pk)
    return plain


def check_sum(log, tag, got, ref, mass, dtype, tol=None):
    """The bar for an fp32 sum of products whose absolute values total `mass`
    (per element): |got - ref| <= tol * RMS(ref) + SUM_SLACK * 2^-24 * mass."""
    tol = TOL[dtype] if tol is None else tol
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    mass = np.asarray(mass, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    allow = tol * rms + SUM_SLACK * 2.0 ** -24 * mass
    plain = float(np.max(err)) / rms if rms > 0 else float(np.max(err))
    cond = float(np.max(mass) / max(float(np.max(np.abs(ref))), 1e-300))
    log(f"  {tag}: rel err {plain:.3e} (tol {tol}), term mass / max|ref| {cond:.3g}, "
        f"max err / allowance {float(np.max(err / allow)):.3g}")
    assert np.all(err <= allow), (tag, plain, cond)
    return plain
