"""include/moe.h as a plain C interface: a C11 program that includes it
compiles with every warning as an error, links against the library, and
calls the host-only entry points (version, shape checks, workspace size,
the error channel) with no C++ or torch in sight. Runs on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "routed_expert_ffn_top_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "moe.h"

static moe_shape olmoe(void)
{
    moe_shape s;
    memset(&s, 0, sizeof s);
    s.T = 4096; s.d = 2048; s.f = 1024; s.E = 64; s.k = 8; s.n_shared = 0;
    s.P = 64; s.capacity = 4096 * 8; s.dtype = MOE_DT_BF16; s.renorm = 1;
    s.ldx = 2048; s.ldy = 2048;
    return s;
}

int main(void)
{
    char msg[512];
    moe_shape s = olmoe();
    size_t ws = moe_workspace_bytes(&s);
    printf("version %s\n", moe_version());
    printf("workspace %zu\n", ws);
    s.k = 65;                                  /* k > E: refused */
    printf("bad_k %zu\n", moe_workspace_bytes(&s));
    moe_status st = moe_last_error(msg, sizeof msg);
    printf("status_k %d\n", (int)st);
    printf("message_k %s\n", msg);
    s = olmoe();
    s.dtype = MOE_DT_BF16; s.d = 2000;         /* bf16 needs d % 64 == 0 */
    printf("bad_d %zu\n", moe_workspace_bytes(&s));
    st = moe_last_error(msg, sizeof msg);
    printf("status_d %d\n", (int)st);
    return ws > 0 ? 0 : 1;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_is_plain_c_and_links(tmp_path):
    lib = os.path.join(LIBDIR, "libmoe_gfx950.so")
    if not os.path.exists(lib):
        pytest.fail("the HIP library is not built (run __graft_entry__.build())")
    src = tmp_path / "use_moe.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_moe"
    cc = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Wpedantic", "-Werror", f"-I{os.path.join(ROOT, 'include')}",
          str(src), "-o", str(exe), f"-L{LIBDIR}", "-lmoe_gfx950", f"-Wl,-rpath,{LIBDIR}"]
    r = subprocess.run(cc, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    out = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    assert out["version"].startswith("routed-expert-ffn-gfx950")
    assert int(out["workspace"]) > 300 << 20          # H and the per-route rows at T = 4096
    assert out["bad_k"] == "0" and out["bad_d"] == "0"      # refused shapes have no workspace
    assert out["status_k"] == "-1" and "k" in out["message_k"]   # MOE_ERR_INVALID_ARG, with a message
    assert out["status_d"] == "-6"                          # MOE_ERR_UNSUPPORTED
