"""The C ABI header is plain C: a C11 translation unit that includes it compiles with every
warning as an error, links against libmol.so, and calls the host-only entry points (sizing
queries, status strings, version); no GPU is touched."""
import os
import subprocess
import tempfile

from tests import conftest
from virtual_expert_routed_amd import binding as mb

C_SOURCE = r"""
#include <stdio.h>
#include <string.h>
#include "mol.h"

int main(void) {
    if (mol_abi_version() < 1) return 1;
    if (strcmp(mol_status_string(MOL_OK), mol_status_string(MOL_E_ARG)) == 0) return 2;
    /* 184 pairs over 1024 virtual experts in blocks of 64 */
    const int64_t mb = mol_align_max_blocks(184, 1024, 64);
    if (mb != (184 + 184 * 63 + 63) / 64) return 3;
    if (mol_align_max_blocks(10, 8192, 64) != -MOL_E_LIMIT) return 4;
    if (mol_delta_workspace_bytes(184, 64, 1024, 64) < 184 * 64 * 4) return 5;
    /* rejected on the host, before anything is enqueued */
    if (mol_virtual_topk(NULL, NULL, 3, 2, 4, 2, NULL, NULL) != MOL_E_ARG) return 6;
    printf("ok %lld\n", (long long)mb);
    return 0;
}
"""


def test_header_compiles_as_c_and_links():
    lib = mb.lib()  # built
    assert lib is not None
    inc = os.path.join(conftest.ROOT, "include")
    libdir = os.path.dirname(mb.LIB_PATH)
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "use_mol.c")
        exe = os.path.join(d, "use_mol")
        open(src, "w").write(C_SOURCE)
        r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                            "-I", inc, src, "-o", exe, "-L", libdir, "-lmol",
                            f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
        assert run.returncode == 0 and run.stdout.startswith("ok"), (run.returncode, run.stdout,
                                                                      run.stderr)
