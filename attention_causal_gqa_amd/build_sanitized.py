"""Build the host-sanitized variant of libattn.so: the C-ABI layer (attn_api.cpp) compiled with
AddressSanitizer and UndefinedBehaviorSanitizer on the host side only (-Xarch_host), linked with the
regular kernel objects, into _build/asan/libattn.so.  The CPU tests run the ABI checks against it with
the sanitizer runtime preloaded (tests/test_sanitized_abi.py).

    python -m attention_causal_gqa_amd.build_sanitized
"""

import glob
import os
import subprocess

try:
    from . import build as _b
except ImportError:  # run as a script
    import build as _b

OUT_DIR = os.path.join(_b.BUILD, "asan")
LIB = os.path.join(OUT_DIR, "libattn.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime():
    """The shared AddressSanitizer runtime of the ROCm clang, which the host process must preload."""
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    found = sorted(glob.glob(os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under " + root)
    return found[-1]


def build():
    """Compile attn_api.cpp sanitized and link it with the kernel objects of the regular build."""
    os.makedirs(OUT_DIR, exist_ok=True)
    cc = _b.hipcc()
    kernels = [os.path.join(_b.BUILD, s.rsplit(".", 1)[0] + ".o") for s in _b.SOURCES if s != "attn_api.cpp"]
    missing = [k for k in kernels if not os.path.exists(k)]
    if missing:
        _b.build()
    obj = os.path.join(OUT_DIR, "attn_api.o")
    flags = [f for f in _b.FLAGS if f != "-O3"] + ["-O1", "-g"]
    rc, out = _b._run([cc, *flags, *HOST_SAN, "-shared-libsan", "-c",
                       os.path.join(_b.CSRC, "attn_api.cpp"), "-o", obj])
    if rc != 0:
        raise RuntimeError("sanitized compile of attn_api.cpp failed:\n" + out)
    # The runtime (which carries the UndefinedBehaviorSanitizer handlers too)
    # is linked by path, so no sanitizer flag reaches the device link.
    rc, out = _b._run([cc, f"--offload-arch={_b.ARCH}", "-shared", "-fPIC", obj, *kernels, runtime(), "-o", LIB])
    if rc != 0:
        raise RuntimeError("link of the sanitized library failed:\n" + out)
    return LIB


if __name__ == "__main__":
    print(build())
