"""AddressSanitizer + UndefinedBehaviorSanitizer CPU builds (no GPU needed).

* The oracle (oracle/oracle.c) compiled with gcc's sanitizers into the
  driver tests/sanitize/oracle_asan.c, which runs every storage dtype of
  every stream through two appended chunks, the indexer, the top-k and the
  attention on exactly sized buffers, and every codec over its code space.
* The library's host side (lcca_api.cpp: validation, launch planning, size
  functions) compiled with clang's sanitizers and linked, with the kernels'
  objects of the release build, into tests/sanitize/api_asan.cpp, which
  calls every entry point with arguments the validation must reject and
  sweeps the size functions over their argument range.  No case reaches a
  kernel launch, and the run hides every GPU from the HIP runtime.

Any sanitizer report aborts the driver with a non-zero status."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
HIP_OBJS = tuple(sorted(f[:-4] for f in os.listdir(os.path.join(ROOT, "long_context_compressed_append_amd", "csrc"))
                        if f.endswith(".hip")))

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2", HIP_VISIBLE_DEVICES="",
           ROCR_VISIBLE_DEVICES="")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr)
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-ffp-contract=off", "-Wall", "-o", exe, os.path.join(SAN, "oracle_asan.c"),
          "-lm"])
    out = _run([exe], env=ENV, timeout=300)
    assert "0 failed checks" in out, out


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not installed")
def test_library_host_side_under_asan_and_ubsan(tmp_path):
    objs = [os.path.join(ROOT, "_build", f + ".hip.o") for f in HIP_OBJS]
    if not all(os.path.exists(o) for o in objs):
        from long_context_compressed_append_amd import build
        build.build_one(False)
    san = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", "-I" + os.path.join(ROOT, "include")]
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
                "-fno-sanitize-recover=all"]
    api = str(tmp_path / "api.o")
    drv = str(tmp_path / "drv.o")
    exe = str(tmp_path / "api_asan")
    _run([CLANG, "-x", "hip", "--cuda-host-only", "--offload-arch=gfx950"] + san + host_san +
         ["-c", os.path.join(ROOT, "long_context_compressed_append_amd", "csrc", "lcca_api.cpp"), "-o", api])
    _run([CLANG] + san + ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-c",
                          os.path.join(SAN, "api_asan.cpp"), "-o", drv])
    _run([CLANG, "-fsanitize=address,undefined", "-o", exe, api, drv] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    out = _run([exe], env=ENV, timeout=300)
    assert " 0 failed" in out, out
