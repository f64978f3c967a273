"""The C-ABI checks (tests/test_abi.py) against a build of the host layer with AddressSanitizer and
UndefinedBehaviorSanitizer (attention_causal_gqa_amd/build_sanitized.py), CPU only."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_are_clean_under_address_and_undefined_behaviour_sanitizers():
    from attention_causal_gqa_amd import build_sanitized
    lib = build_sanitized.build()
    with open(lib, "rb") as f:
        assert b"libclang_rt.asan-x86_64.so" in f.read()  # linked against the sanitizer runtime
    env = dict(os.environ, LD_PRELOAD=build_sanitized.runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", ATTN_LIBRARY=lib)
    probe = ("import attention_causal_gqa_amd._binding as b, ctypes; b.load_library(); "
             "print(b.LIB_PATH); print(hasattr(ctypes.CDLL(None), '__asan_init'))")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split() == [lib, "True"]
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join("tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
