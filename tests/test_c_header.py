"""The boundary from C (no GPU): include/fa_fwd.h compiles as strict C99, a C program links
against libfa_fwd.so and calls the host entry points (version, error text, device limits,
shared-memory screen, planner, packed-batch check) with the values the Python binding sees."""
import os
import shutil
import subprocess

import pytest

import exact_attention_forward_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SOURCE = r"""
#include <stdio.h>
#include "fa_fwd.h"

int main(void) {
  fa_device_limits_t dev;
  fa_plan_t plan;
  fa_tile_config_t cfg = {128, 128, 128, 128, 2, 2, 0};
  fa_screen_t scr;
  const int cu_ok[6] = {0, 3, 5, 0, 4, 9};  /* two sequences: q lengths 3, 2; k lengths 4, 5 */
  const int cu_bad[6] = {0, 3, 2, 0, 4, 9}; /* query offsets decrease */
  if (fa_gfx950_limits(&dev) != FA_OK) return 10;
  if (fa_smem_screen(&cfg, &dev, &scr) != FA_OK) return 11;
  if (fa_fwd_plan(FA_DTYPE_BF16, 2, 32, 8, 8192, 8192, 0, 128, 128, 1, NULL, &plan) != FA_OK)
    return 12;
  printf("version %d\n", fa_version());
  printf("cus %d %lld\n", dev.num_cus, (long long)dev.lds_bytes_per_block);
  printf("screen %lld %d %d\n", (long long)scr.smem_bytes, scr.fits, scr.blocks_per_cu);
  printf("plan %d %d %lld %lld\n", plan.schedule, plan.waves, (long long)plan.num_workgroups,
         (long long)plan.lds_bytes);
  printf("cu %d %d %d\n", fa_check_cu_seqlens(cu_ok, 2, 3, 5, 5, 9),
         fa_check_cu_seqlens(cu_bad, 2, 3, 5, 5, 9), fa_check_cu_seqlens(NULL, 2, 3, 5, 5, 9));
  printf("null %d\n", fa_fwd(NULL, NULL, NULL, NULL, NULL, 1, 4, 2, 128, 128, NULL, 128, 128,
                             0.1f, 0, NULL, NULL));
  printf("err %s\n", fa_strerror(FA_ERR_INVALID));
  return 0;
}
"""


def test_header_is_c99_and_links(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    lib_dir = os.path.dirname(fa.library_path())
    src, exe = tmp_path / "boundary.c", tmp_path / "boundary"
    src.write_text(C_SOURCE)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I",
                        os.path.join(ROOT, "include"), str(src), "-L", lib_dir, "-lfa_fwd",
                        f"-Wl,-rpath,{lib_dir}", "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    out = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    # the same answers as through the Python binding
    assert int(out["version"]) == fa.fa_version()
    lim = fa.fa_gfx950_limits()
    assert out["cus"] == f"{lim.num_cus} {lim.lds_bytes_per_block}"
    s = fa.fa_smem_screen(fa.TileConfig(tile_m=128, tile_n=128, head_dim=128, head_dim_v=128,
                                        elem_bytes=2, kv_stages=2, q_in_regs=0), lim)
    assert out["screen"] == f"{s.smem_bytes} {s.fits} {s.blocks_per_cu}"
    p = fa.fa_fwd_plan(fa.FA_DTYPE_BF16, 2, 32, 8, 8192, 8192, False, 128, 128, True)
    assert out["plan"] == f"{p.schedule} {p.waves} {p.num_workgroups} {p.lds_bytes}"
    assert out["cu"] == f"{fa.FA_OK} {fa.FA_ERR_INVALID} {fa.FA_ERR_NULL}"
    assert int(out["null"]) == fa.FA_ERR_NULL  # refused before any HIP call
    assert out["err"] == fa.fa_strerror(fa.FA_ERR_INVALID)
