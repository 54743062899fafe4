"""AddressSanitizer and UndefinedBehaviorSanitizer on the host code, on the CPU (no GPU).

- The oracle (oracle.c) is built with gcc's ASan + UBSan (``ORACLE_SANITIZE=1``, any UB report
  aborts) and every oracle pin runs against that build in a child process with gcc's ASan
  runtime preloaded.
- The C-ABI library is built with its host code instrumented (each sanitizer flag passed to the
  host compilation only; the gfx950 device code is built as usual) and the boundary tests run
  against it with clang's ASan runtime preloaded: every argument check of every entry point
  executes under the sanitizers (none of these calls reaches a launch).
- Each toolchain is first shown to be live: a deliberate heap overflow in a throwaway program
  built with the same flags must be reported.
The child processes print the sanitizers' reports; a report fails the test.
"""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# host-only instrumentation for hipcc: -Xarch_host right before each sanitizer flag
HIPCC_HOST_SAN = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                  "-Xarch_host -fno-sanitize-recover=undefined "
                  "-Xarch_host -fno-omit-frame-pointer -Xarch_host -shared-libsan").split()
SAN_ENV = dict(ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
REPORT_MARKERS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def gcc_asan_runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("gcc's ASan runtime is not installed")
    return p


def clang_asan_runtime():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hits = sorted(glob.glob(os.path.join(rocm, "llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")))
    if not hits:
        pytest.skip("clang's ASan runtime is not installed")
    return hits[-1]


def run_child(args, preload, extra_env=None, cwd=ROOT, timeout=600):
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=preload, PYTHONPATH=ROOT)
    env.update(extra_env or {})
    return subprocess.run(args, capture_output=True, text=True, cwd=cwd, env=env, timeout=timeout)


def assert_clean(r):
    out = r.stdout + r.stderr
    bad = [m for m in REPORT_MARKERS if m in out]
    assert r.returncode == 0 and not bad, f"rc={r.returncode} {bad}\n{out[-4000:]}"


def test_gcc_sanitizers_are_live(tmp_path):
    import oracle
    src = tmp_path / "overflow.c"
    src.write_text(textwrap.dedent("""
        #include <stdlib.h>
        int main(int argc, char** argv) {
            (void)argv;
            int* a = malloc(4 * sizeof(int));
            a[argc + 3] = 1;                  /* one past the end */
            int r = a[0];
            free(a);
            return r;
        }
    """))
    exe = tmp_path / "overflow"
    subprocess.run(["gcc", *oracle.SAN_FLAGS, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True,
                       env=dict(os.environ, **SAN_ENV))
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_oracle_pins_under_asan_and_ubsan():
    import oracle
    path = oracle.build(force=True, sanitize=True)
    asan = gcc_asan_runtime()
    env = dict(ORACLE_SANITIZE="1")
    # the child loads the sanitized build
    r = run_child([sys.executable, "-c", "import oracle; oracle._load(); print(oracle._lib._name)"],
                  asan, env)
    assert_clean(r)
    assert r.stdout.strip() == path
    r = run_child([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                   "tests/test_oracle_pins.py"], asan, env)
    assert_clean(r)
    assert " passed" in r.stdout


def test_hipcc_host_sanitizers_are_live(tmp_path):
    from finalize_residual_rmsnorm_amd import build as mf_build
    src = tmp_path / "overflow.hip"
    src.write_text(textwrap.dedent("""
        #include <cstdlib>
        int main(int argc, char**) {
            int* a = static_cast<int*>(std::malloc(4 * sizeof(int)));
            a[argc + 3] = 1;
            int r = a[0];
            std::free(a);
            return r;
        }
    """))
    exe = tmp_path / "overflow"
    subprocess.run([mf_build.hipcc(), "--offload-arch=gfx950", *HIPCC_HOST_SAN, str(src), "-o",
                    str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True,
                       env=dict(os.environ, **SAN_ENV, LD_PRELOAD=clang_asan_runtime()))
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_c_abi_argument_checks_under_asan_and_ubsan(tmp_path):
    from finalize_residual_rmsnorm_amd import build as mf_build
    lib = str(tmp_path / "libmf_san.so")
    mf_build.build(out=lib, extra_flags=HIPCC_HOST_SAN)
    driver = tmp_path / "driver.py"
    driver.write_text(textwrap.dedent(f"""
        import sys
        import pytest
        import finalize_residual_rmsnorm_amd as mf
        mf.LIB_PATH = {lib!r}
        mf._lib = None
        assert mf.lib()._name == {lib!r}
        sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "tests/test_boundary.py"]))
    """))
    r = run_child([sys.executable, str(driver)], clang_asan_runtime())
    assert_clean(r)
    assert " passed" in r.stdout
