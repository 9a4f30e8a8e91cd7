import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _device_hygiene(request):
    """GPU tests: caches and workspaces sit between guard bands of a known byte
    pattern, and outputs and workspaces are NaN-filled before every call; after
    the test every guard must be intact."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import gc
    from decode_attention_wushkv_amd.device_cache import DeviceCache
    DeviceCache.guard_bytes = 4096
    DeviceCache.poison = True
    del DeviceCache.guard_failures[:]
    yield
    gc.collect()   # closes the caches the test dropped (each checks its guards)
    bad = [f"{name} of a live cache" for dc in list(DeviceCache.live) if dc.handle
           for name in dc.check_guards()]
    bad += DeviceCache.guard_failures
    assert not bad, f"guard bands overwritten: {bad}"


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Parity statistics of every GPU check that ran: one line per test, then
    the worst attention margin and the totals."""
    try:
        import gpu_checks
    except ImportError:
        return
    stats = gpu_checks.STATS
    if not stats:
        return
    tr = terminalreporter
    tr.section("parity statistics")
    worst, worst_id = 0.0, None
    n_codes = n_mism = 0
    s_rel = z_rel = 0.0
    for tid, st in stats.items():
        tr.write_line(f"{tid}: {gpu_checks.summarize(st)}")
        for a in st.get("A", []):
            if a["max_err_over_tol"] > worst:
                worst, worst_id = a["max_err_over_tol"], tid
        for q in st.get("Q", []):
            n_codes += q["codes"]
            n_mism += q["mismatch"]
            s_rel = max(s_rel, q["max_scale_rel"])
            z_rel = max(z_rel, q["max_zero_rel"])
    match = 100.0 * (1 - n_mism / n_codes) if n_codes else 100.0
    tr.write_line(f"parity totals: {len(stats)} tests; {n_codes} codes {match:.5f}% equal "
                  f"({n_mism} one level off at a tie); max scale rel err {s_rel:.1e}, "
                  f"max zero rel err {z_rel:.1e}; worst attention err/tol {worst:.3f} "
                  f"({worst_id})")
