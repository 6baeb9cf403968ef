import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _ensure_cpu_libs():
    """The CPU-side helpers (oracle, host generator) are tiny: build them if absent."""
    import oracle.build as ob
    import synth

    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        ob.build()
    if not os.path.exists(synth.HOST_LIB):
        import subprocess

        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        os.path.join(ROOT, "synth", "synth_host.c"), "-o", synth.HOST_LIB], check=True)


_ensure_cpu_libs()


@pytest.fixture(scope="session")
def orc():
    import oracle

    return oracle.load()


def gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
