import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped (not failed) when no GPU is visible, so that the
    # CPU suite can run with or without -m "not gpu".
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


# Errors against the oracle, collected from what each passed GPU test printed
# (a figure in scientific notation right after the word "err"), so that the
# margin to each test's bar shows in the run's summary and not only in its
# captured output.
_ERR_FIGURE = re.compile(r"\berr\w*\s*[:=]?\s*([0-9]\.[0-9]+e[-+][0-9]+)")
_ERRORS = []


def pytest_runtest_logreport(report):
    if report.when != "call" or not report.passed or "gpu" not in report.keywords:
        return
    figures = []
    for name, text in report.sections:
        if not name.startswith("Captured"):
            continue
        figures += [float(x) for x in _ERR_FIGURE.findall(text)]
    if figures:
        _ERRORS.append((report.nodeid.split("::", 1)[-1], max(figures), len(figures)))


def pytest_terminal_summary(terminalreporter):
    if not _ERRORS:
        return
    terminalreporter.section("largest error figure printed by each passed GPU test")
    for test, worst, count in _ERRORS:
        terminalreporter.write_line(f"{worst:.3e}  ({count:3d} figures)  {test}")
