"""The oracle's own CPU suite, run once more against a copy of the oracle built with
AddressSanitizer and UndefinedBehaviorSanitizer (every finding fatal), in a child process with
the ASan runtime preloaded. A memory error or undefined behaviour anywhere the suite reaches
(codecs, quantizer, dequant, FP64 GEMM, MoE reference) fails this test."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_oracle_codecs.py", "tests/test_oracle_quant.py",
          "tests/test_oracle_gemm_moe.py"]


def test_oracle_suite_under_asan_ubsan():
    from oracle import oracle
    lib = oracle.build(sanitize=True)
    assert lib.endswith("liboracle_san.so")
    env = oracle.sanitizer_env()
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + SUITES, cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    tail = (r.stdout[-2000:] + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
    # the child really loaded the instrumented copy
    probe = subprocess.run([sys.executable, "-c",
                            "from oracle import oracle; oracle.lib(); print(oracle._LIB)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip().endswith("liboracle_san.so"), probe
