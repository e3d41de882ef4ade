"""The library's host code (argument validation, workspace sizing and split
plan, the allocation-free entry point's checks, the commit's order checks
and the pipelined scheduler's state machine) under AddressSanitizer: a
build with the host code instrumented runs the CPU ABI and scheduler tests
in a child process, which must pass with no sanitizer report.  No GPU is
needed: every call there fails validation before any launch, and the
scheduler is host code."""

import os
import subprocess
import sys

import pytest

from block_causal_attention_gqa_amd import build as BLD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_under_address_sanitizer(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("the host-side ABI tests run where no GPU is present")
    rt = BLD.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    try:
        lib = BLD.build(asan=True, out=str(tmp_path / "libbc_asan.so"))
    except RuntimeError as e:
        pytest.skip("hipcc unavailable: %s" % e)
    syms = subprocess.run(["nm", "-D", lib], stdout=subprocess.PIPE, text=True).stdout
    assert "__asan_report" in syms, "the host code is not instrumented"
    script = ("import sys; sys.path.insert(0, %r)\n"
              "from block_causal_attention_gqa_amd import binding as B\n"
              "B.LIB_PATH = %r\n"
              "import pytest\n"
              "sys.exit(pytest.main(['-q', '-s', '-p', 'no:cacheprovider', %r, %r]))\n"
              % (ROOT, lib, os.path.join(ROOT, "tests", "test_abi.py"),
                 os.path.join(ROOT, "tests", "test_pipeline_native.py")))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    proc = subprocess.run([sys.executable, "-c", script], env=env, stdout=subprocess.PIPE,
                          stderr=subprocess.STDOUT, text=True, timeout=600)
    assert "AddressSanitizer" not in proc.stdout, proc.stdout[-4000:]
    assert proc.returncode == 0, proc.stdout[-4000:]
    assert " passed" in proc.stdout
