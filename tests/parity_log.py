"""Measured parity margins: every GPU parity check records what it measured next to its bound,
so the headroom under each bar is visible (printed in pytest's summary, and written as JSON to
the path in SPECACHE_PARITY_LOG when that is set)."""
from __future__ import annotations

import os

RECORDS: list = []


def record(kind: str, value: float, bound: float, what: str = "") -> None:
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    RECORDS.append({"test": test, "kind": kind, "what": what, "value": float(value), "bound": float(bound)})
