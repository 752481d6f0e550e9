"""CPU-side code under AddressSanitizer and UndefinedBehaviorSanitizer.

* The library's host code (argument checks, the residency manager's policy,
  host state of stacks and segments objects) built with its host part
  instrumented (build.build_sanitized) and driven in plan mode -- no stack, no
  GPU call -- by the residency reference-model workload of
  test_residency_policy.py, in a subprocess with the ASan runtime preloaded.
* The CPU oracle (oracle/lora_oracle.c) built by gcc with both sanitizers and
  run through every oracle pin, in a subprocess with gcc's ASan runtime.

Both runs abort on the first finding (-fno-sanitize-recover=all), so a pass
means no out-of-bounds access, use-after-free or undefined behaviour on those
paths.  Leak checking is off: the Python interpreter itself does not free
everything at exit.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(cmd, env_extra, timeout):
    env = dict(os.environ)
    env.update(env_extra)
    env.setdefault("ASAN_OPTIONS", "detect_leaks=0")
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    return res.returncode, res.stdout + res.stderr


def test_residency_host_code_under_asan_ubsan(tmp_path):
    from rank_adapter_gemm_lora_amd import build as B
    lib = B.build_sanitized(str(tmp_path / "liblora_sanitized.so"))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms, "host code not instrumented"
    rt = B.sanitizer_runtime()
    probe = ("import ctypes, sys; sys.path.insert(0, 'tests'); "
             "from rank_adapter_gemm_lora_amd import binding as lb; lb.load(); "
             "maps = open('/proc/self/maps').read(); "
             "assert 'libclang_rt.asan' in maps and 'liblora_sanitized' in maps; print('loaded')")
    rc, out = _run([sys.executable, "-c", probe],
                   {"LD_PRELOAD": rt, "RANK_ADAPTER_GEMM_LORA_LIB": lib}, 300)
    assert rc == 0 and "loaded" in out, out[-3000:]
    rc, out = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                    "tests/test_residency_policy.py"],
                   {"LD_PRELOAD": rt, "RANK_ADAPTER_GEMM_LORA_LIB": lib}, 600)
    assert rc == 0, out[-5000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-5000:]


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build(out_path=str(tmp_path / "liboracle_sanitized.so"),
                       extra_flags=("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                    "-fno-omit-frame-pointer", "-g"))
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc's ASan runtime not found")
    script = ("import sys; sys.path.insert(0, 'tests'); import oracle; "
              f"lib = oracle.load({lib!r}); import test_oracle_pins as T; "
              "[pin(lib) for pin in T.PINS]; "
              "assert 'libasan' in open('/proc/self/maps').read(); print('pins', len(T.PINS))")
    rc, out = _run([sys.executable, "-c", script], {"LD_PRELOAD": asan}, 600)
    assert rc == 0 and "pins" in out, out[-5000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-5000:]
