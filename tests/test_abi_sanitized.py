"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer: the argument checks
of every call run the CPU ABI tests against a build whose host side is instrumented (the kernels
are not), in a child process that preloads the sanitizer runtime. Any report aborts the child."""
import importlib.util
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_nf4_build", os.path.join(ROOT, "bit_nf4_quantised_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_checks_are_clean_under_host_sanitizers():
    b = _build_module()
    lib = b.build_sanitized(verbose=False)
    if shutil.which("nm"):   # the host code really is instrumented
        syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": b.asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "NF4_LIBRARY": lib,
    })
    probe = ("import bit_nf4_quantised_amd as q, sys; "
             f"assert q.LIB_PATH == {lib!r}, q.LIB_PATH; "
             "import ctypes; assert ctypes.CDLL(None).__asan_init, 'sanitizer runtime missing'; "
             "sys.exit(__import__('pytest').main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', "
             f"{os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}]))")
    res = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
