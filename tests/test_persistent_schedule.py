"""The persistent dK/dV schedule (`persistent_tile` in the kernels' band.h),
compiled for the host with g++: every key tile of an XCD's range goes to
exactly one (workgroup, round), for the grids and tile counts the launcher
produces, and on the causal bands of the bench workloads the mirrored rounds
spread the work evenly.  The cost model is the number of 32-query steps of a
tile's band (the band of keys j0 .. j0 + BNK - 1 is queries j0 .. j0 + BNK - 1 + W)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BAND_H = os.path.join(ROOT, "sliding_window_causal_qk_amd", "csrc", "band.h")

DRIVER = r"""
#include <cstdio>
#include "band.h"
int main() {
  int g8, n8, nkt;
  while (std::scanf("%d %d %d", &g8, &n8, &nkt) == 3) {
    const int R = (n8 + g8 - 1) / g8;
    for (int s = 0; s < g8; ++s) {
      for (int i = 0; i < R + 1; ++i) std::printf("%d ", swattn::persistent_tile(i, s, g8, n8, nkt));
      std::printf("\n");
    }
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def schedule_bin(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("sched")
    src = d / "drv.cpp"
    src.write_text(DRIVER)
    exe = d / "drv"
    subprocess.run([gxx, "-O1", "-std=c++17", "-I", os.path.dirname(BAND_H), str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    return str(exe)


def schedule(exe, g8, n8, nkt):
    out = subprocess.run([exe], input=f"{g8} {n8} {nkt}\n", capture_output=True, text=True, check=True).stdout
    return [[int(x) for x in line.split()] for line in out.strip().splitlines()]


def launch_shape(B, T, Hkv, bnk, grid_cap):
    """(g8, n8, xcd ranges) as the kernel derives them from the launch."""
    nkt = -(-T // bnk)
    ntiles = nkt * B * Hkv
    grid = min(grid_cap, ntiles)
    if ntiles % 8 == 0 and grid % 8 == 0:
        return grid // 8, ntiles // 8, 8, nkt
    return grid, ntiles, 1, nkt


SHAPES = [(8, 2048, 4, 128, 256), (64, 2048, 4, 128, 256), (4, 8192, 8, 128, 256), (64, 2048, 2, 128, 256),
          (256, 512, 4, 128, 256), (128, 1024, 4, 128, 256), (64, 2048, 8, 128, 512), (64, 2048, 2, 64, 256),
          (8, 2048, 1, 64, 256), (1, 300, 3, 128, 256), (2, 333, 5, 128, 256), (3, 1000, 4, 128, 256),
          (16, 2048, 4, 128, 256), (24, 2048, 4, 128, 256), (40, 2048, 4, 128, 256), (12, 2048, 4, 128, 256)]


@pytest.mark.parametrize("B,T,Hkv,bnk,cap", SHAPES)
def test_every_tile_once(schedule_bin, B, T, Hkv, bnk, cap):
    g8, n8, _, nkt = launch_shape(B, T, Hkv, bnk, cap)
    rows = schedule(schedule_bin, g8, n8, nkt)
    seen = [r for row in rows for r in row if r >= 0]
    assert sorted(seen) == list(range(n8))
    R = -(-n8 // g8)
    for row in rows:
        assert row[R] == -1                       # past the last round: nothing
        for i, r in enumerate(row[:R]):
            assert r == -1 or i * g8 <= r < (i + 1) * g8   # round i stays in its block of tiles


def _steps(pos, T, W, bnk):
    j0 = pos * bnk
    hi = min(T - 1, j0 + bnk - 1 + W)
    return hi // 32 - j0 // 32 + 1


@pytest.mark.parametrize("B,T,Hkv,W,bnk,worst", [(8, 2048, 4, 2048, 128, 1.001), (4, 8192, 8, 4096, 128, 1.001),
                                                 (4, 8192, 8, 8192, 128, 1.001), (64, 2048, 4, 1024, 128, 1.001),
                                                 (64, 2048, 4, 2048, 128, 1.001), (64, 2048, 2, 2048, 128, 1.001),
                                                 (64, 2048, 2, 2048, 64, 1.001), (64, 2048, 2, 1024, 64, 1.04)])
def test_balance_on_causal_bands(schedule_bin, B, T, Hkv, W, bnk, worst):
    g8, n8, _, nkt = launch_shape(B, T, Hkv, bnk, 256)
    rows = schedule(schedule_bin, g8, n8, nkt)
    work = [sum(_steps(r % nkt, T, W, bnk) for r in row if r >= 0) for row in rows]
    assert max(work) <= worst * sum(work) / len(work)
