"""Host-side AddressSanitizer runs (CPU only, no GPU).

Two instrumented builds, each exercised by the existing CPU tests in a child
process with the sanitizer runtime preloaded (a report or a failing test
fails this test):
  * the C-ABI library with its host code (argument validation, workspace
    plans, the entry points' error paths) built with -fsanitize=address --
    ssd_api.cpp and noalloc.hip recompiled, the kernels' objects reused --
    under the boundary tests;
  * the C oracle (ssd_oracle.c) built with gcc -fsanitize=address, under the
    oracle's pins.
GPU code is never instrumented: -fsanitize= reaches the host compilation only.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "state_space_sequence_03_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


def _gcc_asan():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _instrumented(so):
    """The build calls into the sanitizer runtime (its checks are compiled in)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", so], capture_output=True, text=True,
                         check=True).stdout
    return "__asan_report" in out


def _run_child(tests, env_extra, timeout=600):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider"] + tests,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr, out
    assert r.returncode == 0, out
    return out


@pytest.mark.skipif(not CLANG_RT or not os.path.exists(HIPCC), reason="ROCm clang ASan runtime missing")
def test_library_host_code_under_asan(tmp_path):
    from state_space_sequence_03_amd import build as b
    objs = {os.path.splitext(s)[0]: os.path.join(b.BUILD_DIR, os.path.splitext(s)[0] + ".o")
            for s in b.SOURCES}
    if not all(os.path.exists(o) for o in objs.values()):
        b.build()
    asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    rebuilt = {}
    for src in ("ssd_api.cpp", "noalloc.hip"):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        subprocess.run([HIPCC] + b.COMMON_FLAGS + b.SOURCE_FLAGS.get(src, []) + asan + lang +
                       ["-c", os.path.join(b.CSRC, src), "-o", obj], check=True,
                       capture_output=True, text=True)
        rebuilt[os.path.splitext(src)[0]] = obj
    objs.update(rebuilt)
    so = str(tmp_path / "libssd_asan.so")
    subprocess.run([HIPCC, "--offload-arch=" + b.ARCH, "-shared", "-fPIC", "-shared-libasan",
                    "-fsanitize=address", "-o", so] + list(objs.values()),
                   check=True, capture_output=True, text=True)
    assert _instrumented(so)
    _run_child(["tests/test_boundary.py", "tests/test_boundary_properties.py"],
               {"LD_PRELOAD": CLANG_RT[-1], "SSD_LIBRARY": so})


@pytest.mark.skipif(_gcc_asan() is None, reason="gcc ASan runtime missing")
def test_oracle_under_asan(tmp_path):
    so = str(tmp_path / "libssd_oracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-std=c99", "-fsanitize=address", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "ssd_oracle.c"), "-o", so, "-lm"],
                   check=True, capture_output=True, text=True)
    assert _instrumented(so)
    _run_child(["tests/test_oracle.py"], {"LD_PRELOAD": _gcc_asan(), "SSD_ORACLE_LIBRARY": so})
