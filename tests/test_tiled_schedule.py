"""CPU check of the tiled split GEMM's CU-group schedule.

DAK paper §4.1: disjoint groups of compute units own disjoint output rows and
read one tier each.  The schedule arithmetic (csrc/tiled_schedule.hpp) is plain
constexpr C++ shared with the kernel; this builds it with g++ and checks exact
coverage of host and HBM tiles, host-group co-location on one XCD and the
per-XCD balance over many device sizes and splits."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "tiered_memory_offloading_amd", "csrc")


def test_tiled_schedule_covers_every_tile_once(tmp_path):
    exe = str(tmp_path / "sched")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", CSRC, os.path.join(HERE, "tiled_schedule_check.cpp"),
                    "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr


def test_split_roles_cover_every_work_group_once(tmp_path):
    """The split kernels' role layout (csrc/split_roles.hpp), with and without
    an XCD of the host role's own: every host work-group and every HBM work
    number exactly once, host work-groups only on XCD 0 when it is reserved."""
    exe = str(tmp_path / "roles")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", CSRC, os.path.join(HERE, "split_roles_check.cpp"),
                    "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
