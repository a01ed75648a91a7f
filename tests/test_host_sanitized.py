"""Host code under AddressSanitizer (CPU only; no GPU code is instrumented).

* The oracle: gdn_oracle.c rebuilt with gcc's address and undefined-behaviour
  checks, and every pin of tests/oracle_pins.py run against that build in a
  child Python process with the sanitizer runtimes preloaded. Any
  out-of-bounds access, use of freed memory or undefined arithmetic in the
  oracle (e.g. an index overflow on the varlen, L = 0 or ragged-tail paths
  the pins drive) aborts the child with a report.
* The C ABI's host-side validation: csrc/api.hip rebuilt with the address
  checks on its host code only, linked with the other objects of the normal
  build, and tests/test_abi_host.py (argument, overlap, alignment, workspace
  and scratch-limit checks, none of which launches a kernel) run against it
  with clang's runtime preloaded.
The tests fail on a non-zero exit of the child or a report in its output.
"""
import os
import subprocess
import sys

import pytest

import oracle

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def sanitized_oracle(tmp_path_factory):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    out = str(tmp_path_factory.mktemp("asan") / "libgdn_oracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fno-fast-math", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    "-shared", "-fPIC", "-o", out, os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c"),
                    "-lm"], check=True)
    return out, f"{asan}:{ubsan}"


def test_pins_pass_under_sanitizers(sanitized_oracle):
    lib, preload = sanitized_oracle
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import oracle\n"
            "from tests import oracle_pins\n"
            "orc = oracle.Oracle(%r)\n"
            "for pin in oracle_pins.ALL_PINS:\n"
            "    pin(orc)\n"
            "print('pins ok', len(oracle_pins.ALL_PINS))\n") % (REPO, lib)
    env = dict(os.environ, LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=REPO,
                       timeout=600)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert "pins ok" in r.stdout, report


def _clang_asan_runtime():
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def sanitized_hip_host(tmp_path_factory):
    from gated_deltanet_layer_amd import build as hb
    rt = _clang_asan_runtime()
    try:
        hipcc = hb.hipcc()
    except RuntimeError:
        hipcc = None
    if rt is None or hipcc is None:
        pytest.skip("hipcc or clang's ASan runtime not installed")
    d = tmp_path_factory.mktemp("hip_asan")
    flags = [f for f in hb.FLAGS if f != "-O3"]
    objs = []
    for src in sorted(os.listdir(hb.CSRC)):
        if not src.endswith(".hip"):
            continue
        obj = str(d / (src[:-4] + ".o"))
        extra = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"] \
            if src == "api.hip" else ["-O3"]
        subprocess.run([hipcc, *flags, *extra, "-c", os.path.join(hb.CSRC, src), "-o", obj],
                       check=True, capture_output=True)
        objs.append(obj)
    lib = str(d / "libgdn_asan.so")
    subprocess.run([hipcc, "--offload-arch=" + hb.ARCH, "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-o", lib, *objs], check=True, capture_output=True)
    return lib, rt


def test_abi_validation_under_asan(sanitized_hip_host):
    lib, rt = sanitized_hip_host
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from gated_deltanet_layer_amd import binding\n"
            "binding.LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))\n") % (
        REPO, lib, os.path.join(REPO, "tests", "test_abi_host.py"))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:exitcode=23")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=REPO,
                       timeout=900)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr, report
    assert " passed" in r.stdout, report
