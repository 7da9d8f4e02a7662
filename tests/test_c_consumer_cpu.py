"""The library from plain C: a C99 program that includes include/ra_attn.h, takes the address of
every declared entry point, links against libra_attn.so with the system C compiler (no HIP
compiler, no Python), and calls entry points whose arguments fail validation or describe empty
problems, so that nothing is launched and no GPU is needed."""
import os
import re
import shutil
import subprocess

import pytest

import rational_softmax_tiled_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra_attn.h")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "ra_attn.h"

typedef void (*fn_t)(void);
static fn_t entry_points[] = { %s };

int main(void) {
  const char* s = ra_status_string(RA_ERR_DTYPE);
  if (s == NULL || strncmp(s, "RA_", 3) != 0) return 1;
  /* an unknown dtype is refused before anything is launched */
  int st = ra_attn_fwd(NULL, NULL, NULL, NULL, NULL, 1, 2, 1, 8, 8, 64, RA_CAUSAL_TOP_LEFT, 0.125f,
                       7, NULL);
  if (st != RA_ERR_DTYPE) return 2;
  /* an empty problem succeeds with nothing launched */
  st = ra_attn_fwd(NULL, NULL, NULL, NULL, NULL, 0, 2, 1, 8, 8, 64, RA_CAUSAL_TOP_LEFT, 0.125f,
                   RA_BF16, NULL);
  if (st != RA_OK) return 3;
  st = ra_rope_neox(NULL, NULL, NULL, 2, 8, 63, 10000.0, 0, RA_F32, NULL);
  if (st != RA_ERR_HEADDIM) return 4;
  printf("%%u entry points, %%s\n", (unsigned)(sizeof(entry_points) / sizeof(entry_points[0])), s);
  return 0;
}
"""


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z0-9_]+)\s*\(", text)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_plain_c_program_links_and_calls_the_library(tmp_path):
    if not os.path.exists(ra.library_path()):
        from rational_softmax_tiled_amd import build
        build.build()
    names = _declared_functions()
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM % ", ".join(f"(fn_t){n}" for n in names))
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(ra.library_path())
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe), "-L", libdir, "-lra_attn",
           f"-Wl,-rpath,{libdir}", "-Wl,--allow-shlib-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = os.pathsep.join(p for p in (libdir, "/opt/rocm/lib", env.get("LD_LIBRARY_PATH", "")) if p)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert f"{len(names)} entry points, RA_ERR_DTYPE" in r.stdout
