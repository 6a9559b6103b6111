"""Error metric of the parity tests.

Outputs of long-context attention are small and cross zero, so an
element-wise relative error is ill-posed.  The gate is row-normwise: for
every output row (b, i, h), max_v |gpu - ref| / max_v |ref|, and the test
takes the maximum over rows.
"""

import numpy as np

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 5e-2}


def row_rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den)) if num.size else 0.0


def tol_for(cfg) -> float:
    if cfg.kv_dtype == "fp8":
        return TOL["fp8"]
    return TOL[cfg.q_dtype]


# Per-stage errors of every parity case, printed in the terminal summary so
# that the margins against the gates appear in the tail of a quiet run.
RECORDED: list = []


def record(label: str, errs: dict, tol: float) -> None:
    RECORDED.append((label, dict(errs), float(tol)))
