import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    # SANATAN_TEST_LIB: run the tests against another build of the library (the host-ASan build of
    # test_abi_asan.py); the package itself always loads its in-tree libsanatan.so
    alt = os.environ.get("SANATAN_TEST_LIB")
    if alt:
        import root_parity_gated_amd as rpg

        rpg.LIB_PATH = alt

    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests against the CPU oracle")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    import parity_log

    if not parity_log.ERRORS:
        return
    terminalreporter.write_sep("-", "achieved parity errors (max row error against the oracle, and the bar)")
    for name, rec in sorted(parity_log.ERRORS.items()):
        terminalreporter.write_line(f"{name:60s} {rec['max_err']:.3e}  bar {rec['bar']:.0e}")
    path = os.environ.get("SANATAN_PARITY_LOG")
    if path:
        with open(path, "w") as f:
            json.dump(parity_log.ERRORS, f, indent=1, sort_keys=True)
