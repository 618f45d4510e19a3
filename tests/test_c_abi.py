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


SWEEP = r"""
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include "qsdpa.h"
#include "qsdpa_launch.h"

// the kernel launchers are not linked: a call that reached one would be a bug here
namespace qsdpa {
void launch_quantize(const LaunchArgs&, hipStream_t) { std::puts("launched"); std::abort(); }
void launch_attention(const LaunchArgs&, hipStream_t) { std::puts("launched"); std::abort(); }
void launch_vc(const VcArgs&, hipStream_t) { std::puts("launched"); std::abort(); }
}

#define FAIL(...) do { std::printf(__VA_ARGS__); std::puts(""); return 1; } while (0)

int main() {
  const int vals[] = {INT_MIN, -1, 0, 1, 2, 63, 64, 65, 127, 128, 129, 1000, 4096, 65535, 65536,
                      1 << 17, (1 << 22) - 1, 1 << 22, (1 << 22) + 1, INT_MAX};
  const int fmts[] = {0, 1, 2, 3, -1};
  const float scales[] = {0.088f, 0.f, -1.f, 1e30f};
  char* const A = (char*)(1ull << 40);   // fake, 256-byte aligned device addresses (never dereferenced)
  long n = 0, valid = 0;
  for (int b : vals) for (int h : vals) for (int s : vals) for (int f : fmts) for (float sc : scales) {
    qsdpa_params p;
    std::memset(&p, 0, sizeof(p));
    p.batch = b; p.heads = h; p.seq_len = s; p.head_dim = 128; p.block_q = 128; p.block_k = 64;
    p.qk_format = f; p.fp4_group = 16; p.softmax_scale = sc;
    const int st = qsdpa_validate_params(&p);
    const size_t ws = qsdpa_workspace_bytes(&p);
    qsdpa_layout L;
    const int st2 = qsdpa_workspace_layout(&p, &L);
    qsdpa_vc_layout V;
    const int st3 = qsdpa_vc_workspace_layout(&p, 0.005f, &V);
    (void)qsdpa_vc_workspace_bytes(&p, 1.0f);
    ++n;
    if (st2 != st || (st == QSDPA_OK) != (ws > 0)) FAIL("layout status %d vs %d", st2, st);
    if (st != QSDPA_OK) {
      // every entry point refuses the same parameters with the same status, before any launch
      if (qsdpa_forward(&p, A, A, A, A, A, 1, nullptr) != st) FAIL("forward status");
      if (qsdpa_quantize(&p, A, A, A, A, 1, nullptr) != st) FAIL("quantize status");
      if (qsdpa_attention(&p, A, 1, A, nullptr) != st) FAIL("attention status");
      if (qsdpa_attention_bf16q(&p, A, A, 1, A, nullptr) != st) FAIL("bf16q status");
      if (qsdpa_forward_vc(&p, 0.005f, A, A, A, A, A, 1, nullptr) != st) FAIL("vc status");
      continue;
    }
    ++valid;
    if (L.total != ws) FAIL("layout total");
    if (f == 0 && st3 != QSDPA_OK) FAIL("vc layout");
    const unsigned long long t = 2ull * b * h * s * 128;   // bytes of one bf16 tensor
    char* q = A; char* k = q + ((t + 255) / 256) * 256; char* v = k + ((t + 255) / 256) * 256;
    char* o = v + ((t + 255) / 256) * 256; char* w = o + ((t + 255) / 256) * 256;
    // buffer checks, all before any launch
    if (qsdpa_forward(&p, nullptr, k, v, o, w, ws, nullptr) != QSDPA_ERR_INVALID_ARG) FAIL("null q");
    if (qsdpa_forward(&p, q + 8, k, v, o, w, ws, nullptr) != QSDPA_ERR_ALIGNMENT) FAIL("misaligned q");
    if (qsdpa_forward(&p, q, k, v, o, w + 16, ws, nullptr) != QSDPA_ERR_ALIGNMENT) FAIL("misaligned ws");
    if (qsdpa_forward(&p, q, k, v, o, w, ws - 1, nullptr) != QSDPA_ERR_WORKSPACE_TOO_SMALL) FAIL("small ws");
    if (qsdpa_forward(&p, q, k, v, q, w, ws, nullptr) != QSDPA_ERR_ALIAS) FAIL("o aliases q");
    if (qsdpa_forward(&p, q, k, v, o, o, ws, nullptr) != QSDPA_ERR_ALIAS) FAIL("ws aliases o");
    if (qsdpa_attention(&p, w, ws - 1, o, nullptr) != QSDPA_ERR_WORKSPACE_TOO_SMALL) FAIL("attention ws");
  }
  std::printf("%ld %ld\n", n, valid);
  return 0;
}
"""


def test_host_checks_under_sanitizers(tmp_path):
    """The C ABI's host side (argument checks, workspace layout, selective-
    correction plan) built with AddressSanitizer and UndefinedBehaviorSanitizer
    (host code only) over 160000 parameter sets: INT_MIN .. INT_MAX sizes,
    unknown formats, bad scales; every entry point must refuse invalid
    parameters and buffers with the validator's status and never reach a
    kernel launcher (they are replaced here by stubs that abort)."""
    cxx = shutil.which("g++")
    hip_inc = "/opt/rocm/include"
    if cxx is None or not os.path.exists(os.path.join(hip_inc, "hip", "hip_runtime.h")):
        pytest.skip("no g++ or HIP headers")
    src = tmp_path / "sweep.cpp"
    src.write_text(SWEEP)
    exe = tmp_path / "sweep"
    res = subprocess.run([cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                          "-D__HIP_PLATFORM_AMD__", "-I", hip_inc, "-I", os.path.join(ROOT, "include"),
                          "-I", os.path.join(ROOT, "precision_attention_qsdpa_amd", "csrc"),
                          os.path.join(ROOT, "precision_attention_qsdpa_amd", "csrc", "qsdpa_api.cpp"), str(src),
                          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-3000:]
    n, valid = map(int, run.stdout.split())
    assert n == 160000 and valid > 1000
