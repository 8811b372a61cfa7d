"""CPU sanitizer runs (AddressSanitizer + UndefinedBehaviorSanitizer).

* The C-ABI layer (sda_api.cpp) is built host-only with g++ against stubbed
  kernel launches and device queries (tests/sanitize/sda_api_check.cpp), and
  its validation, plans and argument marshalling run over the workload shapes
  and ~400k randomised argument sets.  "Device" buffers are inaccessible
  mappings, so a host read of device memory would fault.
* The fp64 oracle is rebuilt with the sanitizers (libsda_oracle_san.so) and
  the oracle pin suites run against it in a child process with the sanitizer
  runtimes preloaded.  A planted out-of-bounds read (a problem that claims more
  cache pages than its buffer holds) must be caught, which shows that the
  instrumentation is live.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_paged_decode_02_amd")

ORACLE_PIN_SUITES = ["tests/test_oracle_formats.py", "tests/test_oracle_semantics.py",
                     "tests/test_oracle_swa.py", "tests/test_oracle_select.py",
                     "tests/test_oracle_logits.py"]


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


ASAN, UBSAN = _runtime("libasan.so"), _runtime("libubsan.so")
needs_sanitizers = pytest.mark.skipif(
    not (ASAN and UBSAN and shutil.which("g++")),
    reason="gcc's libasan/libubsan runtimes are not installed")


def build_api_check(out_path: str) -> str:
    """Compile the host-only, sanitized check of the C-ABI layer."""
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(PKG, "csrc"), os.path.join(PKG, "csrc", "sda_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "sda_api_check.cpp"), "-o", out_path]
    subprocess.check_call(cmd)
    return out_path


def _sanitized_env():
    env = dict(os.environ)
    pre = " ".join(p for p in (ASAN, UBSAN, env.get("LD_PRELOAD", "")) if p)
    env.update(LD_PRELOAD=pre, ASAN_OPTIONS="detect_leaks=0", SDA_ORACLE_SANITIZE="1",
               PYTHONDONTWRITEBYTECODE="1")
    return env


@needs_sanitizers
def test_api_layer_under_asan_ubsan(tmp_path):
    exe = build_api_check(str(tmp_path / "sda_api_check"))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "sda_api_check: ok" in r.stdout


@needs_sanitizers
def test_oracle_pins_under_asan_ubsan():
    from oracle import oracle
    oracle.build(force=True, sanitize=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + ORACLE_PIN_SUITES, capture_output=True, text=True,
                       timeout=900, cwd=ROOT, env=_sanitized_env())
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout


@needs_sanitizers
def test_planted_out_of_bounds_read_is_caught():
    # A mistake planted in the oracle's inputs on the CPU: the problem claims
    # 5 cache pages while its buffer holds 4, and a row's region resolves to
    # page 4, just past the end.  The sanitized oracle must abort on the read.
    from oracle import oracle
    oracle.build(sanitize=True)
    code = textwrap.dedent("""
        import ctypes, numpy as np
        from oracle import oracle
        rng = np.random.default_rng(0)
        hp = oracle.HostProblem(
            query=rng.integers(0, 1 << 14, (1, 1, 192)).astype(np.uint16),
            cache=np.zeros((4, 1, 16, 384), dtype=np.uint16),
            regions=np.array([[0]], dtype=np.int32),
            block_table=np.array([[4]], dtype=np.int32),
            positions=np.array([5], dtype=np.int32),
            active=np.array([1], dtype=np.uint8), scale=0.07, query_len=1,
            region_tokens=0, clear_inactive=True, k_scale=1.0, v_scale=1.0, gate=None)
        p = oracle._problem(hp)
        p.num_pages = 5
        out = np.zeros((1, 1, 192))
        oracle.lib().sdo_decode(ctypes.byref(p), out.ctypes.data, 0, 1)
        print("not caught")
    """)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300, cwd=ROOT, env=_sanitized_env())
    assert r.returncode != 0 and "not caught" not in r.stdout
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr
