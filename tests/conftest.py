import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    # The oracle and the input generator are plain C built with gcc in a second; build
    # them here if a checkout has not been built yet.
    import oracle
    import synth
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    if not os.path.exists(synth.LIB_PATH):
        synth.build()
    # The HIP library (hipcc cross-compiles for gfx950 without a GPU) is built only when no
    # build is present, as __graft_entry__.build() would; the package itself refuses to load
    # without it.
    lib = os.path.join(ROOT, "flatquant_transform_quant_amd", "libfq.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "fq_build", os.path.join(ROOT, "flatquant_transform_quant_amd", "_build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
