"""AddressSanitizer and UndefinedBehaviorSanitizer on the CPU-side code.

Three C/C++ parts run on the host: the fp64 oracle, the seeded input
generator, and the library's host-side argument checks (qsa_api.cpp, with
the kernel launchers' host stubs).  Each is rebuilt with
-fsanitize=address,undefined (undefined behaviour is fatal) and the CPU tests
that exercise it run in a child process with the sanitizer runtime preloaded:
the oracle pins and guards, the generator tests, and the ABI validation
tests.  A report of either sanitizer fails the child, and so this test.

Only host code is instrumented (the sanitizer flags go to the host pass); the
ABI tests call nothing but host code, on a machine without a GPU.  GPU-side
sanitizers are not used.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def _gcc_runtime():
    path = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_runtime():
    try:
        out = subprocess.check_output([os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin",
                                                    "clang"), "-print-file-name="
                                       "libclang_rt.asan-x86_64.so"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    if os.path.exists(out):
        return out
    # the runtime sits under lib/linux of the resource directory
    res = subprocess.check_output([os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin",
                                                "clang"), "-print-resource-dir"], text=True).strip()
    cand = os.path.join(res, "lib", "linux", "libclang_rt.asan-x86_64.so")
    return cand if os.path.exists(cand) else None


def _run_child(tests, env_extra, preload, tmp):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    # reports go to files: pytest's output capture would lose them on an abort
    logs = os.path.join(tmp, "sanitizer_logs")
    os.makedirs(logs, exist_ok=True)
    env["ASAN_OPTIONS"] = ("detect_leaks=0:abort_on_error=1:halt_on_error=1:"
                           f"log_path={logs}/asan")
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={logs}/ubsan"
    env["OMP_NUM_THREADS"] = "2"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *[os.path.join(ROOT, "tests", t) for t in tests]],
                       cwd=tmp, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    for f in sorted(os.listdir(logs)):
        with open(os.path.join(logs, f), errors="replace") as fh:
            out = fh.read() + "\n" + out
    # the sanitizers' own report lines lead the failure message
    reports = [ln for ln in out.splitlines()
               if "ERROR: AddressSanitizer" in ln or "runtime error:" in ln]
    msg = "\n".join(reports[:5]) + "\n" + out[-4000:]
    assert r.returncode == 0, msg
    assert not reports, msg
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_and_generator_under_sanitizers(tmp_path):
    rt = _gcc_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    libs = {}
    for name, src in (("oracle", os.path.join(ROOT, "oracle", "qsa_oracle.c")),
                      ("synth", os.path.join(ROOT, "synth", "synth.c"))):
        so = str(tmp_path / f"lib_{name}_san.so")
        subprocess.check_call(["gcc", *SAN, "-fPIC", "-shared", "-fopenmp", "-std=c11", "-o", so,
                               src, "-lm"])
        libs[name] = so
    _run_child(["test_oracle_pins.py", "test_oracle_guards.py", "test_synth.py"],
               {"QSA_ORACLE_LIB": libs["oracle"], "QSA_SYNTH_LIB": libs["synth"]}, rt,
               str(tmp_path))


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_host_argument_checks_under_sanitizers(tmp_path):
    rt = _clang_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from block_sparse_long_08_amd import _build
    # every sanitizer flag is for the host pass; the GPU pass is built at -O1
    # only to complete the objects (nothing here launches a kernel)
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = [HIPCC, "-std=c++17", "-fPIC", "--offload-arch=gfx950", *host_san,
               "-Xarch_device", "-O1", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument", "-x", "hip", "-c",
               os.path.join(_build.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        return obj, r

    with ThreadPoolExecutor(max_workers=4) as ex:
        done = list(ex.map(compile_one, _build.SOURCES))
    for obj, r in done:
        assert r.returncode == 0, r.stderr[-3000:]
    objs = [obj for obj, _ in done]
    so = str(tmp_path / "libqsa_host_san.so")
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-shared-libasan",
                        "-Xarch_host", "-fsanitize=address,undefined", "-o", so, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    _run_child(["test_abi.py"], {"QSA_ABI_LIB": so}, rt, str(tmp_path))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_sanitizer_harness_catches_a_planted_overflow(tmp_path):
    """The harness is live: a copy of the oracle whose pooled-key scratch is
    one row short (a heap overflow once the rotation writes its second half)
    fails under the sanitizers."""
    rt = _gcc_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = open(os.path.join(ROOT, "oracle", "qsa_oracle.c")).read()
    old = "double *m = (double *)malloc(sizeof(double) * 2 * (size_t)Di);"
    assert src.count(old) == 1
    c_path = tmp_path / "oracle_overflow.c"
    c_path.write_text(src.replace(old, "double *m = (double *)malloc(sizeof(double) * (size_t)Di);"))
    so = str(tmp_path / "lib_oracle_overflow.so")
    subprocess.check_call(["gcc", *SAN, "-fPIC", "-shared", "-fopenmp", "-std=c11", "-o", so,
                           str(c_path), "-lm"])
    with pytest.raises(AssertionError, match="AddressSanitizer"):
        _run_child(["test_oracle_pins.py"], {"QSA_ORACLE_LIB": so}, rt, str(tmp_path))
