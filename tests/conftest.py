import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads; minutes rather than seconds")


def pytest_collection_modifyitems(config, items):
    """GPU tests must run the library built from the current sources."""
    if not any(item.get_closest_marker("gpu") for item in items):
        return
    import glob

    lib = os.path.join(ROOT, "attention_causal_gqa_amd", "libattn.so")
    srcs = glob.glob(os.path.join(ROOT, "attention_causal_gqa_amd", "csrc", "*")) + [
        os.path.join(ROOT, "include", "attn.h")]
    if not os.path.exists(lib):
        raise RuntimeError(f"{lib} is not built: run python -m attention_causal_gqa_amd.build")
    stale = [s for s in srcs if os.path.getmtime(s) > os.path.getmtime(lib)]
    if stale:
        raise RuntimeError(f"{lib} is older than {stale}: rebuild before running GPU tests")
