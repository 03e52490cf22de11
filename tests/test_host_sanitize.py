"""Sanitizer build of the host code, on the CPU: the scheduler
(mla_latent_kv_bf16_amd/csrc/plan.cpp, which has no HIP call) and the C
oracle (oracle/mla_oracle.c), driven by tests/host/sanitize_driver.cpp over
valid, edge-case and invalid inputs, compiled with AddressSanitizer and
UndefinedBehaviorSanitizer. The run must end cleanly: no sanitizer report,
every invariant check passing."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         "-g", "-O1"]


def test_host_code_clean_under_sanitizers(tmp_path):
    oracle_obj = str(tmp_path / "mla_oracle.o")
    subprocess.run(["gcc", *FLAGS, "-c", os.path.join(ROOT, "oracle", "mla_oracle.c"), "-o",
                    oracle_obj], check=True)
    exe = str(tmp_path / "sanitize_driver")
    subprocess.run(["g++", "-std=c++17", *FLAGS,
                    os.path.join(ROOT, "tests", "host", "sanitize_driver.cpp"),
                    os.path.join(ROOT, "mla_latent_kv_bf16_amd", "csrc", "plan.cpp"),
                    oracle_obj, "-o", exe, "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-6000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-6000:]
    assert "all checks passed" in r.stdout
