"""The host entry points under AddressSanitizer and UndefinedBehaviorSanitizer.

The tile schedule code (csrc/schedule.cpp, csrc/metadata.cpp: no HIP call,
no device code) is built with g++ and both sanitizers into
tests/fuzz_metadata.cpp, which makes thousands of random calls of
sink_attn_metadata, sink_attn_metadata_padded and sink_attn_metadata_paged,
valid and invalid, with every input array allocated at exactly the size the
header states. The run must end cleanly (a sanitizer report aborts it), and
the same driver linked against the built libsinkattn.so must print the same
statuses, sizes and table hashes, call for call. Host only, no GPU."""
import os
import shutil
import subprocess
from collections import Counter

import pytest

from softmax_sink_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "softmax_sink_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"
FLAGS = ["-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
         "-isystem", ROCM_INCLUDE]


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_schedule_calls_clean_under_sanitizers_and_equal_to_the_library(tmp_path):
    assert os.path.exists(B.LIB_PATH), "build the library first"
    driver = os.path.join(ROOT, "tests", "fuzz_metadata.cpp")
    asan = str(tmp_path / "fuzz_asan")
    subprocess.run(["g++", *FLAGS, "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", os.path.join(CSRC, "schedule.cpp"),
                    os.path.join(CSRC, "metadata.cpp"), driver, "-o", asan],
                   check=True, capture_output=True, text=True)
    lib_dir = os.path.dirname(B.LIB_PATH)
    plain = str(tmp_path / "fuzz_lib")
    subprocess.run(["g++", *FLAGS, driver, "-o", plain, "-L", lib_dir, "-lsinkattn",
                    f"-Wl,-rpath,{lib_dir}"], check=True, capture_output=True, text=True)

    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    for seed in (7, 2024):
        a = subprocess.run([asan, str(seed), "3000"], capture_output=True, text=True, env=env)
        assert a.returncode == 0 and "runtime error" not in a.stderr and \
            "AddressSanitizer" not in a.stderr, a.stderr[-3000:]
        b = subprocess.run([plain, str(seed), "3000"], capture_output=True, text=True, check=True)
        assert a.stdout == b.stdout
        lines = [ln.split() for ln in a.stdout.splitlines() if ln.startswith("case ")]
        assert len(lines) == 3000
        # every family has accepted and refused calls; no status outside the enum
        seen = Counter((int(f[2]), int(f[3]) == 0) for f in lines)
        for family in (0, 1, 2):
            assert seen[(family, True)] > 100 and seen[(family, False)] > 100, seen
        assert {int(f[3]) for f in lines} <= {0, 1, 2, 3, 4}
