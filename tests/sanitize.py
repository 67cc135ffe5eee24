#!/usr/bin/env python3
"""CPU sanitizer tier: the oracle and the library's host code (argument
checks, planning, workspace layout) built with AddressSanitizer and UBSan,
driven by the CPU tests that exercise them. Runs without a GPU.

    python tests/sanitize.py

1. oracle/ssa_oracle.c built with gcc -fsanitize=address,undefined; the
   oracle's pin tests (tests/test_oracle*.py) run against it with gcc's ASan
   runtime preloaded.
2. libssa.so relinked with api.cpp's host code built the same way (clang);
   the C-ABI host tests (tests/test_abi.py) run against it with clang's ASan
   runtime preloaded.

UBSan reports abort (-fno-sanitize-recover); ASan aborts on its first report.
Leak detection is off: the Python interpreter itself keeps allocations to
exit. Exits non-zero if a run fails or prints a sanitizer report.
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def run(env_extra, tests, what):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *tests]
    print(f"[sanitize] {what}: {' '.join(tests)}", flush=True)
    p = subprocess.run(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = p.stdout
    tail = "\n".join(out.splitlines()[-3:])
    print(tail, flush=True)
    bad = [ln for ln in out.splitlines() if "AddressSanitizer" in ln or "runtime error:" in ln]
    if p.returncode != 0 or bad:
        print(out[-6000:], file=sys.stderr)
        return False
    return True


def main():
    import oracle
    from block_sparse_streaming_amd import build

    ok = True
    lib_oracle = oracle.build(force=True, sanitize=True)
    gcc_asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    tests = sorted(glob.glob(os.path.join("tests", "test_oracle*.py")))
    ok &= run({"LD_PRELOAD": gcc_asan, "SSA_ORACLE_LIB": lib_oracle}, tests, "oracle (gcc ASan + UBSan)")

    lib_ssa = build.build_host_sanitized()
    rt = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        print("[sanitize] clang ASan runtime not found", file=sys.stderr)
        return 1
    ok &= run({"LD_PRELOAD": rt[-1], "SSA_LIB": lib_ssa}, ["tests/test_abi.py"],
              "library host code (clang ASan + UBSan)")
    print("[sanitize] " + ("no sanitizer reports" if ok else "FAILED"), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
