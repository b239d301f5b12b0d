"""The boundary from plain C (CPU only): include/csakv.h compiles as strict C11, and a C
program linked against libcsakv.so gets the same host-side results (kv_cache_bytes,
csakv_status_string) as the Python binding.  No GPU call is made."""
import os
import shutil
import subprocess

import pytest

import compressed_sparse_kv_csa_amd as ck

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SOURCE = r"""
#include <stdio.h>
#include "csakv.h"

int main(void) {
  kv_cache_spec spec = {0};
  kv_cache_breakdown out;
  uint64_t total;
  int32_t s;
  spec.n_csa = 30; spec.n_hca = 31; spec.n_swa = 0;
  spec.csa_ratio = 4; spec.hca_ratio = 128; spec.window = 128;
  spec.kv_dim = 512; spec.rope_dim = 64; spec.idx_dim = 128;
  spec.kv_fmt = CSAKV_KV_FP8_MIXED; spec.idx_fmt = CSAKV_IDX_FP4;
  spec.count_window = 1; spec.count_scales = 0;
  total = kv_cache_bytes(&spec, 1048576, &out);
  printf("%llu %llu %llu %llu %llu %llu\n", (unsigned long long)total,
         (unsigned long long)out.csa_shared_kv, (unsigned long long)out.csa_indexer,
         (unsigned long long)out.hca_shared_kv, (unsigned long long)out.windows,
         (unsigned long long)out.scales);
  for (s = 0; s >= -4; --s) printf("%d %s\n", (int)s, csakv_status_string(s));
  return 0;
}
"""


@pytest.fixture(scope="module")
def c_program(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    lib = ck.lib_path()
    if not os.path.exists(lib):
        pytest.skip("libcsakv.so is not built")
    d = tmp_path_factory.mktemp("c_abi")
    src = d / "use_csakv.c"
    src.write_text(C_SOURCE)
    exe = d / "use_csakv"
    r = subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                        lib, f"-Wl,-rpath,{os.path.dirname(lib)}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_header_compiles_as_strict_c(c_program):
    assert os.path.exists(c_program)


def test_c_program_matches_the_binding(c_program):
    r = subprocess.run([str(c_program)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.strip().splitlines()
    spec = ck.KvCacheSpec(n_csa=30, n_hca=31, n_swa=0, csa_ratio=4, hca_ratio=128, window=128,
                          kv_dim=512, rope_dim=64, idx_dim=128, kv_fmt=ck.KV_FP8_MIXED,
                          idx_fmt=ck.IDX_FP4, count_window=1, count_scales=0)
    total, b = ck.kv_cache_bytes(spec, 1048576)
    assert lines[0].split() == [str(v) for v in (total, b.csa_shared_kv, b.csa_indexer, b.hca_shared_kv,
                                                 b.windows, b.scales)]
    assert total > 0
    for line, code in zip(lines[1:], range(0, -5, -1)):
        num, text = line.split(" ", 1)
        assert int(num) == code
        assert text == ck.lib().csakv_status_string(code).decode()
