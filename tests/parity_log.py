"""Max-abs errors of the GPU parity checks, per test.

``record`` keeps the largest error each test measured against the oracle
(with the tolerance it was held to, and for bf16 outputs the distance in bf16
steps from the oracle's own rounding) and prints it; ``dump`` writes the table
as JSON to the path in the environment variable PA_PARITY_LOG, when set.
"""
from __future__ import annotations

import json
import os

CURRENT = "?"
ERRORS: dict = {}


def record(err: float, tol=None, ulp=None) -> None:
    """err: max-abs error against the oracle; ulp: for bf16 outputs, the largest
    distance in bf16 steps from the oracle's own bf16 rounding."""
    prev = ERRORS.setdefault(CURRENT, {"max_abs": err, "tol": tol, "max_ulp": ulp})
    prev["max_abs"] = max(prev["max_abs"], err)
    if ulp is not None:
        prev["max_ulp"] = ulp if prev["max_ulp"] is None else max(prev["max_ulp"], ulp)
    print(f"[max-abs] {err:.3e}" + ("" if tol is None else f" (tol {tol:g})") +
          ("" if ulp is None else f", {ulp} bf16 steps from the rounded oracle"), flush=True)


def dump() -> None:
    path = os.environ.get("PA_PARITY_LOG")
    if not path or not ERRORS:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(ERRORS, f, indent=1, sort_keys=True)
