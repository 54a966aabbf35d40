"""The host side of the C ABI (argument validation, workspace sizing, layout
arithmetic) under AddressSanitizer, on the CPU: the library's host-sanitizer
flavour (mixture_experts_layer_21_amd/build.py --asan: every host object
built with -fsanitize=address, the device code as usual) is built, and the
ABI tests (tests/test_abi.py) run against it in a subprocess with the
sanitizer runtime preloaded; any report aborts that process and fails here."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def asan_runtime():
    cands = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return cands[-1] if cands else None


@pytest.mark.skipif(asan_runtime() is None or not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs ROCm's hipcc and its AddressSanitizer runtime")
def test_abi_under_address_sanitizer():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "moe_build", os.path.join(ROOT, "mixture_experts_layer_21_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    lib = mod.build(verbose=False, asan=True)
    env = dict(os.environ, LD_PRELOAD=asan_runtime(), MOE_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr, tail
    assert " passed" in r.stdout, tail
