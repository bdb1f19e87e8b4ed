import os
import sys

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library)")


def pytest_runtest_logreport(report):
    """With MOE_TEST_TIMES set, append each test's call duration and outcome
    to that file as soon as the test ends."""
    path = os.environ.get("MOE_TEST_TIMES")
    if path and report.when == "call":
        with open(path, "a") as fh:
            fh.write(f"{report.duration:8.2f} {report.outcome} {report.nodeid}\n")
