"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU (no GPU).

1. The fp64 oracle, built with gcc's sanitizers, runs small forward and
   backward cases in every direction and order (edge sizes included) in a
   Python process that preloads the sanitizer runtimes.
2. The library's host code (every entry point, the argument validation, the
   launch planning and the kernel-choice query), built with hipcc's host-side
   sanitizers and with its kernels replaced by stubs (tests/sanitize), runs
   the C-ABI checks of test_abi_cpu.py in such a process.
3. A positive control: a copy of the oracle with a planted out-of-bounds
   write must be stopped by the sanitizer.

Any sanitizer report ends its process with a non-zero status, which fails
the test.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_ssm2d_amd", "csrc")
ORACLE_SRC = os.path.join(ROOT, "oracle", "ssm2d_oracle.c")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=23",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=23"}


def _gcc_runtimes():
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
        if not os.path.isabs(p) or not os.path.exists(p):
            pytest.skip(f"gcc sanitizer runtime {name} not found")
        libs.append(p)
    return " ".join(libs)


def _clang_runtime():
    hits = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not hits or shutil.which("hipcc") is None:
        pytest.skip("hipcc or clang's ASan runtime not found")
    return hits[0]


def _run(script, preload, timeout=600):
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=preload, PYTHONPATH=ROOT + os.pathsep + os.path.join(ROOT, "tests"))
    return subprocess.run([sys.executable, "-c", script], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def _build_oracle(src, out):
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
                    "-std=c99", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", src, "-o", out, "-lm"], check=True)


ORACLE_SCRIPT = r"""
import sys
import numpy as np
import oracle
from selective_state_space_ssm2d_amd.inputs import make_random_inputs
lib = oracle.load(sys.argv[1] if len(sys.argv) > 1 else {path!r})
ks = ("x", "delta", "A", "B", "C", "D")
for shape in [(1, 1, 1, 1, 1), (2, 3, 5, 7, 9), (1, 2, 0, 3, 4), (1, 2, 3, 1, 6), (1, 2, 3, 6, 1), (2, 1, 4, 5, 5)]:
    t = make_random_inputs(*shape, seed=sum(shape))
    b, d, n, H, W = shape
    for fh in (False, True):
        for fw in (False, True):
            for vf in (False, True):
                y = oracle.fwd(*(t[k] for k in ks), lib=lib, flip_h=fh, flip_w=fw, vertical_first=vf)
                assert y.shape == (b, d, H, W) and np.all(np.isfinite(y))
    h0 = np.random.default_rng(1).standard_normal((b, d, n, W))
    y, hl = oracle.fwd(*(t[k] for k in ks), lib=lib, h_init=h0, return_last=True)
    y4 = oracle.fwd(*(t[k] for k in ks), lib=lib, four_way=True)
    ym = oracle.fwd(*(t[k] for k in ks), lib=lib, maps=[0, b * d - 1])
    dy = np.random.default_rng(2).standard_normal((b, d, H, W))
    if n <= 32:
        for vf in (False, True):
            g = oracle.bwd(*(t[k] for k in ks), dy, lib=lib, vertical_first=vf)
            assert all(np.all(np.isfinite(v)) for v in g.values())
    s = oracle.states(np.full((3, 4), 0.5), np.ones((3, 4)), lib=lib)
print("oracle sanitizer run ok")
"""


def test_oracle_under_sanitizers(tmp_path):
    pre = _gcc_runtimes()
    out = str(tmp_path / "liboracle_san.so")
    _build_oracle(ORACLE_SRC, out)
    r = _run(ORACLE_SCRIPT.format(path=out), pre)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert "oracle sanitizer run ok" in r.stdout


def test_sanitizer_catches_planted_overflow(tmp_path):
    """Positive control: the horizontal pass of a copy of the oracle writes
    one element past its row buffer; the sanitized run must fail with a
    heap-buffer-overflow report."""
    pre = _gcc_runtimes()
    src = open(ORACLE_SRC).read()
    needle = "hh_row[j] = carry;"
    assert needle in src
    bad = src.replace(needle, "hh_row[j + 1] = carry;", 1)
    p = tmp_path / "oracle_planted.c"
    p.write_text(bad)
    out = str(tmp_path / "liboracle_planted.so")
    _build_oracle(str(p), out)
    r = _run(ORACLE_SCRIPT.format(path=out), pre)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr


ABI_SCRIPT = r"""
import sys
import pytest
import selective_state_space_ssm2d_amd as pkg
pkg._lib = pkg.load_library({path!r})
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", "tests/test_abi_cpu.py"]))
"""


def test_host_abi_under_sanitizers(tmp_path):
    rt = _clang_runtime()
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    procs = []
    for src in (os.path.join(CSRC, "ssm2d.hip"), os.path.join(ROOT, "tests", "sanitize", "dispatch_stubs.hip")):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(o)
        procs.append(subprocess.Popen(["hipcc", *flags, "-c", src, "-o", o], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT, text=True))
    for pr in procs:
        out, _ = pr.communicate()
        assert pr.returncode == 0, out[-4000:]
    lib = str(tmp_path / "libssm2d_san.so")
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib,
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"],
                   check=True, capture_output=True)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm  # instrumented
    r = _run(ABI_SCRIPT.format(path=lib), rt)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-6000:]
    assert " passed" in r.stdout
