"""The C ABI from C: tests/abi_from_c.c, a C11 program that includes only
include/sink_attn.h and links libsinkattn.so, is compiled with gcc and run
(host entry points only, no GPU). Its table must equal, word for word, the
one the Python binding gets for the same problem, and the refused call must
report E_INVALID."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from softmax_sink_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs gcc and the ROCm headers")
def test_c_program_gets_the_same_table_as_the_binding(tmp_path):
    lib_dir = os.path.dirname(B.LIB_PATH)
    assert os.path.exists(B.LIB_PATH), "build the library first"
    exe = str(tmp_path / "abi_from_c")
    # the HIP runtime header needs its platform macro outside hipcc
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", ROCM_INCLUDE,
           os.path.join(ROOT, "tests", "abi_from_c.c"), "-o", exe,
           "-L", lib_dir, "-lsinkattn", f"-Wl,-rpath,{lib_dir}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    lines = dict(line.split(" ", 1) for line in out.strip().splitlines())

    assert int(lines["abi"]) == B.abi_version()
    cu_q = np.array([0, 5, 135, 199], np.int32)
    cu_k = np.array([0, 5, 205, 269], np.int32)
    p = B.make_problem(cu_q, cu_k, 8, 2, 128, True, -1, -1, B.BF16)
    meta, fws, bws = B.sink_attn_metadata(p, cu_q, cu_k)
    words, c_fws, c_bws = map(int, lines["sizes"].split())
    assert (words, c_fws, c_bws) == (len(meta), fws, bws)
    table = np.array(lines["table"].split(), dtype=np.int64)
    assert np.array_equal(table, meta.astype(np.int64))

    code, text = lines["refused"].split(" ", 1)
    assert int(code) == 1 and text == B.status_string(1)
