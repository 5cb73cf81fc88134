import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    # The HIP library and the oracle are built in-tree; build whichever is
    # missing so a fresh checkout can run the suite (hipcc cross-compiles
    # for gfx950 without a GPU).
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_pdattn_build", os.path.join(ROOT, "paged_kv_split_amd", "build.py"))
    hip_build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(hip_build)
    from oracle import build as oracle_build
    if not os.path.exists(hip_build.LIBRARY):
        hip_build.build()
    if not os.path.exists(oracle_build.LIBRARY):
        oracle_build.build()
