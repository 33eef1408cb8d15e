"""Accuracy budgets of the deterministic package, applied against the FP64 oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The page "restore the K1 weight-gradient routes that meet the deterministic
package's absolute FP64 budgets" (description and commit message) states them:

* BF16 output: atol = rtol = 1e-2 with zero violations, read in the allclose
  form |out - ref| <= atol + rtol*|ref| for every element, ref the unrounded
  FP64 value;
* FP32 output: relative Frobenius error <= 5e-5 and max |out - ref| <=
  1e-3 * max |ref|.

Every output must also be finite.
"""
import numpy as np

BF16_ATOL = 1e-2
BF16_RTOL = 1e-2
F32_REL_FRO = 5e-5
F32_MAX_ABS_REL = 1e-3


def check_bf16(out, ref):
    """out: float64 values of the BF16 output; ref: FP64 oracle.  Returns a report dict."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(out - ref)
    bound = BF16_ATOL + BF16_RTOL * np.abs(ref)
    finite = bool(np.all(np.isfinite(out)))
    viol = int(np.count_nonzero(~(err <= bound)))
    worst = float(np.max(err / bound)) if err.size else 0.0
    return {"ok": finite and viol == 0, "violations": viol, "worst_ratio": worst, "finite": finite,
            "max_abs": float(err.max()) if err.size else 0.0}


def check_f32(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    finite = bool(np.all(np.isfinite(out)))
    d = out - ref
    nref = float(np.linalg.norm(ref))
    rel_fro = float(np.linalg.norm(d)) / nref if nref > 0 else float(np.linalg.norm(d))
    mref = float(np.max(np.abs(ref))) if ref.size else 0.0
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    ok = finite and rel_fro <= F32_REL_FRO and max_abs <= F32_MAX_ABS_REL * mref
    return {"ok": ok, "rel_fro": rel_fro, "max_abs": max_abs, "max_ref": mref, "finite": finite}


def check(out, ref, out_dtype):
    return check_bf16(out, ref) if out_dtype == "bf16" else check_f32(out, ref)
