"""libawq's host-side argument handling under AddressSanitizer and UndefinedBehaviorSanitizer.

Every HIP source is compiled again with the sanitizers applied to its host half only (the
"-Xarch_host" form: device code is built as usual and never runs here), linked into a separate
library in a temporary directory, and driven by tests/host_checks.cpp: each entry point with
rejected arguments (outputs must stay untouched) and every workspace-size query at extreme
sizes.  Needs no GPU; a sanitizer report or a failed expectation fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_only_int4_act_amd", "csrc")
SOURCES = ["awq_api.hip", "awq_stats.hip", "awq_search.hip", "awq_pack.hip", "awq_gemm.hip", "awq_greedy.hip"]
SAN = ["address", "undefined"]


def _tool(name):
    for p in (os.environ.get("HIPCC") if name == "hipcc" else None, shutil.which(name),
              f"/opt/rocm/bin/{name}", f"/opt/rocm/llvm/bin/{name}"):
        if p and os.path.exists(p):
            return p
    pytest.skip(f"{name} not found")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.slow
def test_host_argument_checks_under_sanitizers(tmp_path):
    hipcc, clang = _tool("hipcc"), _tool("clang++")
    host_san = []
    for s in SAN:
        host_san += ["-Xarch_host", f"-fsanitize={s}"]
    host_san += ["-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wno-unused-command-line-argument"]
    procs, objs = [], []
    for src in SOURCES:
        obj = str(tmp_path / (src[:-4] + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([hipcc, *flags, *host_san, "-c", os.path.join(CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p, src in zip(procs, SOURCES):
        out, err = p.communicate()
        assert p.returncode == 0, f"{src}:\n{err[-4000:]}"
    lib = str(tmp_path / "libawq_san.so")
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib])
    exe = str(tmp_path / "host_checks")
    san = ",".join(SAN)
    _run([clang, "-std=c++17", "-O1", "-g", f"-fsanitize={san}", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "tests", "host_checks.cpp"), lib,
          f"-Wl,-rpath,{tmp_path}", "-o", exe])
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "0 failures" in r.stdout, f"{r.stdout[-4000:]}\n{r.stderr[-6000:]}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-6000:]
