"""Worst errors the GPU parity tests observed, per test and quantity.

The GPU tests call `record` with every max-abs error they check against a
bound; at the end of the session the conftest writes the collected maxima to
gpurun_out/parity_errors.json, so the error figures quoted for the kernels
have a record behind them. Nothing here touches the GPU or the oracle.
"""
from __future__ import annotations

import json
import os

_ERRS: dict = {}


def record(quantity: str, value: float, bound: float | None = None) -> None:
    """Keep the largest `value` seen for `quantity` in the running test."""
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    entry = _ERRS.setdefault(test, {})
    cur = entry.get(quantity)
    if cur is None or float(value) > cur["max"]:
        entry[quantity] = {"max": float(value), "bound": bound}


def dump(path: str) -> bool:
    """Write the collected maxima to `path` (JSON); False if nothing was recorded."""
    if not _ERRS:
        return False
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(_ERRS, f, indent=1, sort_keys=True)
    return True
