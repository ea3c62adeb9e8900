import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU on this host (reported as skipped, not passed)")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """The parity hash lines (GPU, oracle and stored SHA-256 per full-size
    workload and mode), shown whatever the verbosity, and kept in
    gpurun_out/parity_sha256.txt."""
    mod = sys.modules.get("gpu_util")
    lines = getattr(mod, "HASH_LINES", None) if mod else None
    if not lines:
        return
    out = ["parity sha256 (workload mode: gpu / oracle / stored)"]
    for workload, mode, gpu, orc, stored in lines:
        same = "equal" if gpu == orc == stored else "DIFFER"
        out.append(f"{workload} {mode}: {gpu} / {orc} / {stored}  {same}")
    terminalreporter.section("parity hashes")
    for line in out:
        terminalreporter.write_line(line)
    try:
        d = os.path.join(ROOT, "gpurun_out")
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "parity_sha256.txt"), "w") as f:
            f.write("\n".join(out) + "\n")
    except OSError:
        pass
