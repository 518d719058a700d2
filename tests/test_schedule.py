"""Host-side check of the kernels' scheduling and tile-range arithmetic.

The bf16 kernels take their workgroup-to-block mapping and the key / query
tile ranges each wave walks from ``exact_io_aware_14_amd/csrc/fa_schedule.h``
(``__host__ __device__`` functions). ``tests/schedule_check.cpp`` compiles
that same header for the host and checks it against the definition of the
mask over many sequence lengths, windows and head groupings: one-to-one
grid mappings, every visible (query, key) pair inside a tile its wave
computes, tiles computed without per-score masks holding only visible pairs
(or rows / keys past N, which are zero-filled), no 32-bit overflow.

Each planted mistake below is a plausible slip in that arithmetic; the
checker must report it, which shows that its checks can fail.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_14_amd", "csrc")
HEADER = os.path.join(CSRC, "fa_schedule.h")
CHECK_SRC = os.path.join(ROOT, "tests", "schedule_check.cpp")


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _build_and_run(header_dir, out_dir):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    exe = os.path.join(out_dir, "schedule_check")
    # host-only compilation of the HIP header: the __host__ __device__
    # functions the kernels call, built for the CPU
    cmd = [hipcc, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17",
           "-I", header_dir, CHECK_SRC, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    return subprocess.run([exe], capture_output=True, text=True, timeout=300)


def test_schedule_arithmetic(tmp_path):
    res = _build_and_run(CSRC, str(tmp_path))
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert " 0 failures" in res.stdout


# (name, text in fa_schedule.h, replacement)
MUTATIONS = [
    ("fwd_wave_tiles_one_short",
     "r.wt_end = r.qw0 >= N ? r.wt_first\n"
     "                        : (masked ? imin(N - 1, r.wave_last + wr) / BC + 1 : ktiles_all);",
     "r.wt_end = r.qw0 >= N ? r.wt_first\n"
     "                        : (masked ? imin(N - 1, r.wave_last + wr) / BC : ktiles_all);"),
    ("fwd_block_tiles_from_wave_row",
     "r.t_first = masked ? imax(0, r.q0 - wl) / BC : 0;",
     "r.t_first = masked ? imax(0, r.qw0 - wl) / BC : 0;"),
    ("fwd_tail_tile_unmasked",
     "return (key0 + BC > N) || (masked &&",
     "return (masked &&"),
    ("fwd_lower_edge_from_first_row",
     "key0 < r.wave_last - wl));",
     "key0 < r.qw0 - wl));"),
    ("fwd_pair_second_block",
     "b.qb_second = pi;",
     "b.qb_second = pi + 1;"),
    ("fwd_xcd_head_order",
     "b.bh = ((slot / group) * 8 + xcd) * group + slot % group;\n    qbr = within / g2;",
     "b.bh = ((slot / group) * 8 + xcd) * group + slot / group % group;\n    qbr = within / g2;"),
    ("grads_rotation_of_partial_group",
     "if ((j | 3) < per_head)",
     "if (j < per_head)"),
    ("grads_dq_head_index",
     "job.bh = kvh * group + rank % group;",
     "job.bh = kvh + rank % group;"),
    ("dkdv_unmasked_one_tile_long",
     "floor_div(r.kw0 + wl - RW * qh - (RW - 1), T) + 1));",
     "floor_div(r.kw0 + wl - RW * qh - (RW - 1), T) + 2));"),
    ("dkdv_visible_first_row_only",
     "return r0 + (RW - 1) >= r.kw0 - wr && r0 <= r.kw0 + 31 + wl;",
     "return r0 >= r.kw0 - wr && r0 <= r.kw0 + 31 + wl;"),
    ("dkdv_wave_rows_fixed_at_32",
     "return r0 + (RW - 1) >= r.kw0 - wr && r0 <= r.kw0 + 31 + wl;",
     "return r0 + 31 >= r.kw0 - wr && r0 <= r.kw0 + 31 + wl;"),
    ("dkdv_first_tile_from_wave_key",
     "r.t0 = masked ? imax(0, r.k0 - wr) / T : 0;",
     "r.t0 = masked ? imax(0, r.kw0 - wr) / T : 0;"),
    ("dq_unmasked_start_floor",
     "r.tm1 = imin(r.ntiles, imax(r.kt0, ceil_div(r.wave_last - wl, T)));",
     "r.tm1 = imin(r.ntiles, imax(r.kt0, floor_div(r.wave_last - wl, T)));"),
    ("dq_rowless_wave_not_skipped",
     "if (r.qw0 >= N) r.tm2 = r.tm1;",
     ""),
    ("floor_div_truncates",
     "return a >= 0 ? a / b : -((b - 1 - a) / b);",
     "return a / b;"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_schedule_check_catches(tmp_path, name, old, new):
    text = open(HEADER).read()
    assert text.count(old) == 1, f"mutation {name}: pattern not found once"
    hdir = tmp_path / "inc"
    hdir.mkdir()
    (hdir / "fa_schedule.h").write_text(text.replace(old, new))
    res = _build_and_run(str(hdir), str(tmp_path))
    assert res.returncode != 0, f"mutation {name} not caught:\n{res.stdout}"
    assert "FAIL" in res.stdout
