"""Max-abs errors of the GPU parity checks, per test.

``record`` keeps the largest error each test measured against the oracle
(with the tolerance it was held to, and for bf16 outputs the error beyond the
oracle's own rounding to bf16) and prints it; ``dump`` writes the table
as JSON to the path in the environment variable PA_PARITY_LOG, when set.
"""
from __future__ import annotations

import json
import os

CURRENT = "?"
ERRORS: dict = {}


def record(err: float, tol=None, excess=None) -> None:
    """err: max-abs error against the oracle; excess: for bf16 outputs, the largest
    error beyond the oracle's own rounding to bf16 (the kernel's share)."""
    prev = ERRORS.setdefault(CURRENT, {"max_abs": err, "tol": tol, "max_excess": excess})
    prev["max_abs"] = max(prev["max_abs"], err)
    if excess is not None:
        prev["max_excess"] = excess if prev["max_excess"] is None else max(prev["max_excess"], excess)
    print(f"[max-abs] {err:.3e}" + ("" if tol is None else f" (tol {tol:g})") +
          ("" if excess is None else f", {excess:.3e} beyond the bf16 rounding of the oracle"),
          flush=True)


def dump() -> None:
    path = os.environ.get("PA_PARITY_LOG")
    if not path or not ERRORS:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(ERRORS, f, indent=1, sort_keys=True)
