"""Block-order maps of the HIP kernels, checked on the CPU.

The kernels reorder their linear block ids so that the work sharing one
batch row's K/V tiles (attention) or one run of GEMM output tiles stays on one
XCD's L2 (blocks are dealt round-robin over the 8 XCDs). A map that is not a
bijection would skip or repeat tiles. These tests take the maps' own source
text out of the kernel files, compile it for the host with g++, and check
every grid size the library can launch (and many more) for:
  * a bijection onto the work items;
  * the locality the comment above each map promises (one XCD per batch row,
    contiguous item runs per XCD, heavy work first).
No GPU is needed, and the test fails if a map's text can no longer be found.
"""
import ctypes
import shutil
import subprocess

import numpy as np
import pytest

from host_src import device_function


HARNESS = r"""
#define DEV static inline
%s
%s
%s
extern "C" {
void row_map(int n, int B, int per_row, int* b, int* r) {
  for (int id = 0; id < n; ++id) xcd_row_map(id, B, per_row, b[id], r[id]);
}
void level_map(int n, int B, int* b, int* level) {
  for (int id = 0; id < n; ++id) xcd_level_map(id, B, b[id], level[id]);
}
void contiguous(int nb, int* item) {
  for (int b = 0; b < nb; ++b) item[b] = xcd_contiguous(b, nb);
}
}
"""


@pytest.fixture(scope="module")
def maps(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("launch_maps")
    code = HARNESS % (device_function("attention.hip", "xcd_row_map"),
                      device_function("attention.hip", "xcd_level_map"),
                      device_function("gemm.hip", "xcd_contiguous"))
    (d / "maps.cpp").write_text(code)
    so = str(d / "maps.so")
    subprocess.run(["g++", "-O1", "-shared", "-fPIC", "-o", so, str(d / "maps.cpp")], check=True)
    lib = ctypes.CDLL(so)
    P = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
    lib.row_map.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    lib.level_map.argtypes = [ctypes.c_int, ctypes.c_int, P, P]
    lib.contiguous.argtypes = [ctypes.c_int, P]
    return lib


def xcd(ids):
    return ids & 7


def test_xcd_contiguous_is_a_bijection_with_one_run_per_xcd(maps):
    for nb in list(range(1, 600)) + [1023, 1024, 1025, 2047, 2048, 4095, 4097, 16384, 16391]:
        item = np.empty(nb, dtype=np.int32)
        maps.contiguous(nb, item)
        assert np.array_equal(np.sort(item), np.arange(nb)), nb
        blocks = np.arange(nb)
        sizes = []
        for x in range(8):
            run = item[xcd(blocks) == x]        # in dispatch order
            if run.size:
                assert np.all(np.diff(run) == 1), (nb, x)   # one contiguous run, in order
            sizes.append(run.size)
        assert max(sizes) - min(sizes) <= 1, nb


@pytest.mark.parametrize("B", list(range(1, 41)) + [48, 64, 128])
def test_xcd_row_map_covers_every_block_once(maps, B):
    for per_row in (1, 2, 3, 7, 8, 16, 20, 40, 160):
        n = B * per_row
        b = np.empty(n, dtype=np.int32)
        r = np.empty(n, dtype=np.int32)
        maps.row_map(n, B, per_row, b, r)
        assert b.min() >= 0 and b.max() < B and r.min() >= 0 and r.max() < per_row
        assert np.unique(b.astype(np.int64) * per_row + r).size == n, (B, per_row)
        ids = np.arange(n)
        for row in range(B):
            sel = b == row
            assert np.all(np.diff(r[sel]) > 0), (B, per_row, row)   # index order within a row
            if B % 8 == 0:
                assert np.unique(xcd(ids[sel])).size == 1, (B, per_row, row)


@pytest.mark.parametrize("B", list(range(1, 41)) + [48, 64, 128])
def test_xcd_level_map_covers_every_block_once_heavy_first(maps, B):
    for nkb in (1, 2, 3, 8, 16, 17, 32):
        n = B * nkb
        b = np.empty(n, dtype=np.int32)
        lv = np.empty(n, dtype=np.int32)
        maps.level_map(n, B, b, lv)
        assert b.min() >= 0 and b.max() < B and lv.min() >= 0 and lv.max() < nkb
        assert np.unique(b.astype(np.int64) * nkb + lv).size == n, (B, nkb)
        ids = np.arange(n)
        for x in range(8):
            on = xcd(ids) == x
            assert np.all(np.diff(lv[on]) >= 0), (B, nkb, x)   # each XCD: level 0 first
        if B % 8 == 0:
            for row in range(B):
                assert np.unique(xcd(ids[b == row])).size == 1, (B, nkb, row)
        else:
            assert np.all(np.diff(lv) >= 0), (B, nkb)           # level-major over all rows
