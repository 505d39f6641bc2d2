"""Record of every GPU-vs-oracle comparison of a test session (test id, what
was compared, max |error|, tolerance), printed as a summary at the end of the
run so that the margins show even under `pytest -q`; with PA_PARITY_LOG set,
also written there as JSON."""
import json
import os

current = ""          # node id of the running test (set by an autouse fixture)
records = []


def add(what, err, tol):
    records.append({"test": current, "what": what, "max_abs_err": float(err),
                    "tol": float(tol)})


def summary_lines():
    if not records:
        return []
    lines = ["GPU parity: %d comparisons against the float64 oracle in %d tests"
             % (len(records), len({r["test"] for r in records}))]
    for tol in sorted({r["tol"] for r in records}):
        rs = [r for r in records if r["tol"] == tol]
        worst = max(rs, key=lambda r: r["max_abs_err"])
        lines.append("  tol %.0e: %d comparisons, worst max|err| %.3e (%.1f%% of tol) in %s [%s]"
                     % (tol, len(rs), worst["max_abs_err"], 100 * worst["max_abs_err"] / tol,
                        worst["test"], worst["what"]))
    path = os.environ.get("PA_PARITY_LOG")
    if path:
        with open(path, "w") as f:
            json.dump(records, f, indent=1)
        lines.append("  all comparisons written to %s" % path)
    return lines
