"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The library's host side (C ABI, argument validation, launch planning, plan
creation with its injected failures and handle checks) is rebuilt with the
sanitizers on its host pass and runs the boundary, binding and plan-failure
tests; the oracle is rebuilt with gcc's sanitizers and runs its pins.  Each
run is a separate process with the sanitizer runtime preloaded (the two
compilers' runtimes cannot share one process), and first shows that the
instrumented library is the one it mapped.  Any report aborts the process
and fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(REPO, "_build", "sanitize")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(env, args, timeout=600):
    e = dict(os.environ, **SAN_ENV, **env)
    return subprocess.run([sys.executable, *args], cwd=REPO, env=e, capture_output=True, text=True, timeout=timeout)


def _mapped_check(module_expr, path):
    return ["-c", f"import sys; sys.path.insert(0, {REPO!r}); {module_expr}; "
                  f"maps = open('/proc/self/maps').read(); assert {path!r} in maps, 'not mapped'; print('mapped')"]


@pytest.mark.skipif(not shutil.which("gcc") or not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs gcc and hipcc")
def test_library_host_code_under_asan_ubsan():
    sys.path.insert(0, REPO)
    from weight_streaming_gemv_decode_amd import build
    lib = build.build_sanitized(OUT)
    rt = build.asan_runtime()
    assert os.path.exists(rt), rt
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in nm and "__ubsan_" in nm
    env = {"WSGEMV_LIB": lib, "LD_PRELOAD": rt, "WSG_ENABLE_TEST_HOOKS": "1"}
    r = _run(env, _mapped_check("from weight_streaming_gemv_decode_amd import wsgemv; wsgemv.lib()", lib))
    assert r.returncode == 0 and "mapped" in r.stdout, r.stdout + r.stderr
    r = _run(env, ["-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_boundary.py",
                   "tests/test_plan_faults.py", "tests/test_binding_checks.py"])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout


@pytest.mark.skipif(not shutil.which("gcc"), reason="needs gcc")
def test_oracle_under_asan_ubsan():
    sys.path.insert(0, REPO)
    import oracle
    os.makedirs(OUT, exist_ok=True)
    lib = oracle.build(os.path.join(OUT, "liboracle.so"),
                       extra=["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                              "-fno-omit-frame-pointer"])
    pre = " ".join(subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True).stdout.strip()
                   for n in ("libasan.so", "libubsan.so"))
    env = {"WSG_ORACLE_LIB": lib, "LD_PRELOAD": pre}
    r = _run(env, _mapped_check("import oracle; oracle.load()", lib))
    assert r.returncode == 0 and "mapped" in r.stdout, r.stdout + r.stderr
    r = _run(env, ["-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_oracle.py"])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
