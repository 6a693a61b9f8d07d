"""The host side under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the C ABI's validation layer (kda_abi.cpp, built here with g++
-fsanitize=address,undefined and linked with the library's own kernel
objects) runs every host ABI check of test_abi_host.py, and the C oracle
(kda_oracle.c, built with gcc and the same sanitizers) runs every pin.  The
checks run in a child process that preloads the sanitizer runtimes; any report
fails the test.  A copy of the oracle with a one-element out-of-bounds read
planted in it shows the sanitizer is armed.  Nothing here touches a GPU: the
host checks stop at validation."""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_55_amd", "csrc")
BUILD = os.path.join(ROOT, "gated_delta_rule_55_amd", "_build")
OBJS = [os.path.join(BUILD, f"{n}.o") for n in ("kda_conv", "kda_decode", "kda_headscan", "kda_prefill")]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-g", "-O1"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


pytestmark = pytest.mark.skipif(
    not (shutil.which("g++") and shutil.which("gcc") and _runtime("libasan.so")
         and _runtime("libubsan.so") and all(os.path.exists(o) for o in OBJS)),
    reason="needs gcc/g++ with ASan/UBSan runtimes and the library's objects (build first)")


def _build_abi(td):
    obj = os.path.join(td, "kda_abi.o")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    f"-I{ROOT}/include", f"-I{CSRC}", *SAN, "-c", os.path.join(CSRC, "kda_abi.cpp"),
                    "-o", obj], check=True)
    lib = os.path.join(td, "libkda_san.so")
    subprocess.run(["g++", "-shared", *SAN, "-o", lib, obj, *OBJS, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib"], check=True)
    return lib


def _build_oracle(td, src_text, name):
    src = os.path.join(td, name + ".c")
    with open(src, "w") as f:
        f.write(src_text)
    lib = os.path.join(td, "lib" + name + ".so")
    subprocess.run(["gcc", "-std=c99", "-fopenmp", "-fPIC", "-shared", *SAN, src, "-lm", "-o", lib],
                   check=True)
    return lib


def _run_child(td, body):
    script = os.path.join(td, "child.py")
    with open(script, "w") as f:
        f.write(textwrap.dedent(f"""
            import os, sys
            sys.path.insert(0, {ROOT!r})
            sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})
        """) + textwrap.dedent(body))
    env = dict(os.environ)
    env["LD_PRELOAD"] = f"{_runtime('libasan.so')} {_runtime('libubsan.so')}"
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    p = subprocess.run([sys.executable, script], env=env, capture_output=True, text=True, timeout=600)
    return p.returncode, p.stdout + p.stderr


def test_abi_validation_and_oracle_pins_under_sanitizers(tmp_path):
    td = str(tmp_path)
    abi_lib = _build_abi(td)
    orc_lib = _build_oracle(td, open(os.path.join(ROOT, "oracle", "kda_oracle.c")).read(), "oracle_san")
    rc, out = _run_child(td, f"""
        from gated_delta_rule_55_amd import _abi
        _abi.LIB_PATH = {abi_lib!r}
        import pytest
        rc = pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                          {os.path.join(ROOT, 'tests', 'test_abi_host.py')!r}])
        print("host ABI checks:", rc, flush=True)
        if rc != 0:
            sys.exit(int(rc))
        import pins
        from oracle.recurrent import OracleLib
        lib = OracleLib({orc_lib!r})
        for pin in pins.ALL_PINS:
            pin(lib)
        print("oracle pins:", len(pins.ALL_PINS), "ok", flush=True)
    """)
    print(out[-2000:])
    assert rc == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out
    assert "oracle pins:" in out


def test_sanitizer_is_armed(tmp_path):
    """A copy of the oracle that reads one element past h0 must be reported."""
    td = str(tmp_path)
    src = open(os.path.join(ROOT, "oracle", "kda_oracle.c")).read()
    old = "memcpy(S, h0 + c * dk * dv, sizeof(double) * (size_t)(dk * dv));"
    assert old in src
    bad = _build_oracle(td, src.replace(old, "memcpy(S, h0 + c * dk * dv + 1, sizeof(double) * (size_t)(dk * dv));"),
                        "oracle_oob")
    rc, out = _run_child(td, f"""
        import numpy as np
        from oracle.recurrent import OracleLib
        lib = OracleLib({bad!r})
        rng = np.random.default_rng(0)
        T, H, d = 4, 1, 16
        q, k, v, g = (rng.standard_normal((T, H, d)) for _ in range(4))
        lib.prefill(q, k, v, -np.abs(g), np.full((T, H), 0.5), rng.standard_normal((1, H, d, d)))
        print("no report", flush=True)
    """)
    assert rc != 0 and "AddressSanitizer" in out, out[-3000:]
