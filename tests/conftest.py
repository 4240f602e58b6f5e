import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")


@pytest.fixture(scope="session")
def repo_root():
    return ROOT


def pytest_terminal_summary(terminalreporter):
    """Worst forward parity figures of the run, raw and beyond the bf16
    output rounding, printed (also under -q) when any forward comparison
    ran, and written as JSON to the path in ATTN_PARITY_REPORT when that is
    set."""
    import json
    try:
        from tests import gpu_util
    except Exception:
        return
    rows = gpu_util.REPORT
    if not rows:
        return
    worst = {key: max(rows, key=lambda r: r[key])
             for key in ("o_max_abs_raw", "o_max_abs_beyond_bf16", "o_rel_l2", "lse_max_abs")}
    tr = terminalreporter
    tr.write_line(f"forward parity over {len(rows)} comparisons (bars: O max|err| beyond "
                  f"bf16 rounding <= {gpu_util.O_MAX_ABS}, rel-L2 <= {gpu_util.O_REL_L2}, "
                  f"lse <= {gpu_util.LSE_MAX_ABS}, {gpu_util.LSE_MAX_ABS_PADDED} for "
                  f"padded head dims):")
    for key, r in worst.items():
        tr.write_line(f"  worst {key} = {r[key]:.3e}  ({r['what']})")
    path = os.environ.get("ATTN_PARITY_REPORT")
    if not path:
        return
    try:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            json.dump({"worst": {k: {"value": r[k], "case": r["what"]} for k, r in worst.items()},
                       "comparisons": rows}, f, indent=1)
    except OSError:
        pass
