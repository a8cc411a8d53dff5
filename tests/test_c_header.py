"""include/epl.h is a C header: a C11 program that includes it compiles
with -Wall -Werror, links against libepl.so and runs the host-only calls
(no GPU needed: none of them touches the HIP runtime)."""
import os
import shutil
import subprocess

import pytest

import permute_ep_layout_amd as epl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include "epl.h"

int main(void)
{
    epl_problem p = {0};
    p.num_tokens = 4096;
    p.num_topk = 8;
    p.num_experts = 256;
    p.num_ranks = 32;
    p.hidden = 7168;
    p.scale_cols = 56;
    p.expert_alignment = 128;
    p.ranks_per_node = 8;
    if (sizeof(epl_problem) != 40)
        return 10;
    if (epl_validate(&p) != EPL_OK)
        return 11;
    printf("version %x\n", epl_version());
    printf("workspace %zu\n", epl_workspace_bytes(&p));
    printf("capacity %lld\n", (long long)epl_capacity_rows(&p));
    printf("ll_workspace %zu\n", epl_ll_workspace_bytes(&p, 128));
    printf("einval %s\n", epl_strerror(EPL_EINVAL));
    p.num_ranks = 30;                     /* 256 % 30 != 0 */
    printf("bad %d\n", epl_validate(&p));
    return 0;
}
"""


@pytest.fixture(scope="module")
def lib():
    epl.ensure_built()
    return epl.lib_path()


def test_c_program_uses_the_header(tmp_path, lib):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use_epl.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_epl"
    libdir = os.path.dirname(lib)
    subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    lib, f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    vals = dict(line.split(" ", 1) for line in out.strip().splitlines())
    assert int(vals["version"], 16) == epl.load().epl_version()
    p = epl.Problem.make(4096, 8, 256, 32, 7168, 56, 128, 8)
    assert int(vals["workspace"]) == epl.epl_workspace_bytes(p)
    assert int(vals["capacity"]) == epl.epl_capacity_rows(p)
    assert int(vals["ll_workspace"]) == epl.epl_ll_workspace_bytes(p, 128) == 0   # alignment
    assert "invalid" in vals["einval"]
    assert int(vals["bad"]) == epl.EPL_EINVAL
