"""CPU sanitizer tier: the oracle and the host side of the library under
AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle is rebuilt with gcc -fsanitize=address,undefined and every
  oracle pin test runs against that build (Q8KV_ORACLE_LIB), the sanitizer
  runtime preloaded into the test process; a planted over-read through the
  same build must be reported, so the tier is known to be live.
* The library's host code (argument validation, launch planning, the C ABI
  layer) is rebuilt with -Xarch_host -fsanitize=address,undefined -- device
  code is not instrumented -- and the C ABI tests (tests/test_abi_host.py,
  which launch no kernel) run against it.
Each leg runs in a subprocess of its own, since the sanitizer runtime must be
the first library loaded."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "q8kv_oracle.c")
ORACLE_PINS = [os.path.join(ROOT, "tests", f) for f in
               ("test_oracle_pins.py", "test_oracle_sparse_pins.py", "test_oracle_mirror_pins.py",
                "test_oracle_prefill_pins.py")]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=23",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_asan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


@pytest.fixture(scope="module")
def oracle_asan(tmp_path_factory):
    lib = str(tmp_path_factory.mktemp("orc_san") / "liboracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-o", lib, ORACLE_SRC, "-lm"], check=True)
    return lib, _gcc_asan()


def _run(cmd, preload, extra_env):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV, **extra_env)
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def test_oracle_pins_under_asan_ubsan(oracle_asan):
    lib, rt = oracle_asan
    r = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *ORACLE_PINS], rt,
             {"Q8KV_ORACLE_LIB": lib})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_sanitized_oracle_reports_a_planted_overread(oracle_asan):
    # the exact block sums over 128 elements of a 64-byte key row: an
    # over-read the sanitized build must stop
    lib, rt = oracle_asan
    code = ("import ctypes, numpy as np\n"
            f"l = ctypes.CDLL({lib!r})\n"
            "cq = np.ones(128, np.int8); ck = np.ones(64, np.int8); out = np.zeros(4, np.int32)\n"
            "p = lambda a: ctypes.c_void_p(a.ctypes.data)\n"
            "l.orc_block_partials(p(cq), p(ck), 128, p(out))\n")
    r = _run([sys.executable, "-c", code], rt, {})
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def _clang_asan():
    import glob
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.skip("the ROCm clang AddressSanitizer runtime is not installed")
    return hits[-1]


def test_abi_host_layer_under_asan_ubsan(tmp_path):
    rt = _clang_asan()
    from decode_attention_int8_kv_amd import build
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    lib = build.build(extra=san, out=str(tmp_path / "libq8kv_hostsan.so"), link_extra=san[:4])
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import decode_attention_int8_kv_amd as m\n"
            "m.LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n") % (
        ROOT, lib, os.path.join(ROOT, "tests", "test_abi_host.py"))
    r = _run([sys.executable, "-c", code], rt, {})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
