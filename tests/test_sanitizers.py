"""The C ABI's host code (argument checks, workspace carve, launch
sequence) under AddressSanitizer and UndefinedBehaviorSanitizer: the CPU ABI
tests rerun in a child process against libmoe_hostsan.so with the ASan
runtime preloaded; any sanitizer report fails them."""
import os
import subprocess
import sys

from mixture_experts_router_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _fresh():
    """libmoe_hostsan.so, rebuilt if a source is newer."""
    srcs = [os.path.join(b.CSRC, f) for f in os.listdir(b.CSRC)] + [os.path.join(ROOT, "include", "moe.h")]
    if not os.path.exists(b.HOSTSAN_LIB) or os.path.getmtime(b.HOSTSAN_LIB) < max(map(os.path.getmtime, srcs)):
        b.build(hostsan=True)
    return b.HOSTSAN_LIB


def _env():
    env = dict(os.environ)
    env.update(MOE_TEST_LIB=_fresh(), LD_PRELOAD=b.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def test_sanitizer_runtime_is_active():
    """The child really runs with the ASan runtime and the instrumented
    library (else the run below would prove nothing)."""
    code = ("import mixture_experts_router_amd as m, os;"
            "m.load(os.environ['MOE_TEST_LIB']);"
            "maps = open('/proc/self/maps').read();"
            "assert 'libclang_rt.asan' in maps and 'libmoe_hostsan.so' in maps;"
            "print('ok')")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(), capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def test_abi_checks_under_asan_ubsan():
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       cwd=ROOT, env=_env(), capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
