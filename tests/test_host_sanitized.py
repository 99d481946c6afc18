"""The host half of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

Batch intake, the splitters, placement, commit, n_kv, seq_rm, the sequence
state's host side and the iteration loop do index arithmetic on host
buffers; this builds the library with every -fsanitize flag scoped to the
host compilation (build.py --sanitize) and runs the host parity tests
against it in a child interpreter with the sanitizer runtime preloaded.  Any
report aborts that child, which fails this test.
"""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_tests_pass_under_asan_and_ubsan():
    spec = importlib.util.spec_from_file_location("_kvattn_build", os.path.join(ROOT, "ubatch_attention_paged_amd",
                                                                                  "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    lib = b.build(sanitize=True)
    env = b.sanitize_env()
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host_abi.py"), os.path.join(ROOT, "tests", "test_host_sched.py"),
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    # the child really ran the instrumented build
    probe = subprocess.run([sys.executable, "-c", "import ubatch_attention_paged_amd as K; print(K.LIB_PATH); "
                            "print(any('asan' in l for l in open('/proc/self/maps')))"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.stdout.split() == [lib, "True"], probe.stdout + probe.stderr
