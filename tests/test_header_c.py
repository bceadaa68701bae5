"""include/fa.h is a plain C header: a C99 translation unit that includes it
and takes the address of every entry point compiles, links against
libfa.so with the system C compiler, and reads back the ABI version the
header declares (no GPU needed: nothing is launched)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "flashattention_backward_pass_fa_amd")

C_SOURCE = r"""
#include <stdio.h>
#include "fa.h"

int main(void) {
  typedef void (*entry_fn)(void);
  entry_fn entry[] = {(entry_fn)fa_abi_version, (entry_fn)fa_last_hip_error,
                      (entry_fn)fa_status_string, (entry_fn)fa_fwd, (entry_fn)fa_bwd_preprocess,
                      (entry_fn)fa_bwd_workspace_bytes, (entry_fn)fa_bwd,
                      (entry_fn)fa_bwd_noalloc, (entry_fn)fa_debug_dropout_mask};
  fa_params p = {0};
  fa_tensor t = {0, 0, 0, 0};
  (void)t;
  for (unsigned i = 0; i < sizeof entry / sizeof entry[0]; ++i)
    if (!entry[i]) return 2;
  /* an invalid call is rejected before any HIP call */
  if (fa_bwd_workspace_bytes(&p) != 0) return 3;
  printf("%d %d %s\n", fa_abi_version(), FA_ABI_VERSION, fa_status_string(FA_ERR_INVALID_VALUE));
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_compiles_as_c99_and_links(tmp_path):
    lib = os.path.join(LIB_DIR, "libfa.so")
    if not os.path.exists(lib):
        pytest.skip("libfa.so is not built")
    src = tmp_path / "abi.c"
    src.write_text(C_SOURCE)
    exe = tmp_path / "abi"
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                          str(src), "-L", LIB_DIR, "-lfa", f"-Wl,-rpath,{LIB_DIR}", "-o", str(exe)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert out[0] == out[1], "library and header disagree on the ABI version"
    assert out[2:] == ["invalid", "argument", "value"]
