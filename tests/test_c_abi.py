"""The header is a plain C ABI: a C99 program that includes include/qsdpa.h
compiles with no warnings, links against libqsdpa.so and gets the same host
answers as the Python binding (no GPU call is made)."""
import os
import shutil
import subprocess

import pytest

import precision_attention_qsdpa_amd as qs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include "qsdpa.h"

int main(void) {
  qsdpa_params p = {1, 24, 8704, QSDPA_HEAD_DIM, 128, 64, QSDPA_QK_FP8_E4M3, 16, 0.08838834764831845f};
  qsdpa_layout L;
  if (qsdpa_abi_version() != QSDPA_ABI_VERSION) return 3;
  printf("%d %zu %d ", qsdpa_validate_params(&p), qsdpa_workspace_bytes(&p), qsdpa_workspace_layout(&p, &L));
  printf("%llu %d ", (unsigned long long)L.total, L.n_pad);
  p.head_dim = 64;
  printf("%d %s\n", qsdpa_validate_params(&p), qsdpa_status_string(qsdpa_validate_params(&p)));
  return 0;
}
"""


def test_c_program_uses_the_abi(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(qs.LIB_PATH)
    qs.load()   # the library must be built
    res = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                          str(src), "-o", str(exe), f"-L{libdir}", "-l:libqsdpa.so", f"-Wl,-rpath,{libdir}"],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    st, nbytes, lst, total, npad, bad, msg = run.stdout.split(maxsplit=6)
    params = qs.make_params(1, 24, 8704, fmt="fp8", block_q=128)
    assert (int(st), int(lst)) == (qs.QSDPA_OK, qs.QSDPA_OK)
    assert int(nbytes) == int(total) == qs.qsdpa_workspace_bytes(params)
    assert int(npad) == 8704
    assert int(bad) == qs.QSDPA_ERR_UNSUPPORTED
    assert msg.strip() == qs.status_string(qs.QSDPA_ERR_UNSUPPORTED)
