"""The value-embedding gradient's segment kernels, run on the CPU from their
own source text.

dve[v] += gate * sum over positions n with idx[n] == v of dv[n] is computed on
the GPU by two kernels over the ids sorted by value: per chunk of sorted
entries, one thread per column sums each run of equal ids, adds a run that
starts and ends in the chunk straight into dve and leaves a cut run's
partial sum in a carry slot; then the chunk in which a cut run begins finds
the chunk the run ends in (the shared run-end search) and adds the run's
partial sums in order.

Both kernels are taken out of the kernel source as text and compiled for the
host with g++. The partial kernel has no exchange between threads, so it runs
thread by thread; the fix-up runs each block as two 64-thread waves in lock
step (`__ballot` a barrier-synchronised OR per wave). The result is compared
with a brute-force float64 sum per id over: few ids, all ids equal (one run
over every chunk), Zipf ids (runs longer than a whole probe round included),
invalid ids (sorted in as id 0 with a negative position, adding nothing),
ragged and whole chunk counts, and a non-zero starting dve (accumulation).
"""
import ctypes
import shutil
import subprocess

import numpy as np
import pytest

from host_src import device_function, int_constant, kernel_function

K = int_constant("embed_bwd.hip", "kSegChunk")

HARNESS = r"""
#include <algorithm>
#include <atomic>
#include <barrier>
#include <cstdint>
#include <thread>
#include <vector>

using std::min;
constexpr int kSegChunk = %d;
#define DEV static inline
#define __global__
#define __launch_bounds__(n)
struct Idx3 { int x = 0, y = 0, z = 0; };
thread_local Idx3 blockIdx, threadIdx;

// one wave: 64 lanes in lock step; a ballot ORs every lane's bit into the
// wave's mask k %% 3 and waits at the wave's barrier; lane 0 clears the mask
// of ballot k + 2 (read in ballot k - 1, written again after barrier k + 1)
struct Wave {
  std::barrier<>* bar;
  std::atomic<uint64_t> mask[3];
};
thread_local Wave* my_wave = nullptr;
thread_local int my_lane = 0;
thread_local int my_ballots = 0;

static uint64_t __ballot(bool pred) {
  const int k = my_ballots++;
  if (pred) my_wave->mask[k %% 3].fetch_or(uint64_t(1) << my_lane);
  my_wave->bar->arrive_and_wait();
  const uint64_t m = my_wave->mask[k %% 3].load();
  if (my_lane == 0) my_wave->mask[(k + 2) %% 3].store(0);
  return m;
}

%s
%s
%s
%s

extern "C" void ve_scatter(const int32_t* keys, const int32_t* vals, const float* src, int64_t ld, int col0,
                           const float* gate, int N, float* dve, float* carry) {
  const int nseg = (N + kSegChunk - 1) / kSegChunk;
  for (int c = 0; c < nseg; ++c)
    for (int t = 0; t < 128; ++t) {
      blockIdx.x = c;
      threadIdx.x = t;
      ve_seg_partial_kernel<float>(keys, vals, src, ld, col0, gate, N, dve, carry);
    }
  for (int c = 0; c < nseg; ++c) {
    std::barrier<> b0(64), b1(64);
    Wave w[2];
    w[0].bar = &b0;
    w[1].bar = &b1;
    for (auto& wv : w)
      for (auto& m : wv.mask) m.store(0);
    std::vector<std::thread> th;
    for (int t = 0; t < 128; ++t)
      th.emplace_back([&, t] {
        blockIdx.x = c;
        threadIdx.x = t;
        my_wave = &w[t >> 6];
        my_lane = t & 63;
        my_ballots = 0;
        ve_seg_fixup_kernel<float>(keys, N, nseg, gate, carry, dve);
      });
    for (auto& x : th) x.join();
  }
}
"""


@pytest.fixture(scope="module")
def ve(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("ve_segments")
    code = HARNESS % (K, device_function("common.h", "to_f32"), device_function("embed_bwd.hip", "run_last_chunk"),
                      kernel_function("embed_bwd.hip", "ve_seg_partial_kernel"),
                      kernel_function("embed_bwd.hip", "ve_seg_fixup_kernel"))
    (d / "ve.cpp").write_text(code)
    so = str(d / "ve.so")
    subprocess.run(["g++", "-std=c++20", "-O1", "-pthread", "-shared", "-fPIC", "-w", "-o", so, str(d / "ve.cpp")],
                   check=True)
    lib = ctypes.CDLL(so)
    I = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
    F = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
    lib.ve_scatter.argtypes = [I, I, F, ctypes.c_int64, ctypes.c_int, F, ctypes.c_int, F, F]
    return lib


def cases():
    rng = np.random.default_rng(5)
    V = 4096
    for N in (K - 3, 3 * K, 999, 2048):
        yield f"few-{N}", rng.integers(0, 4, N), V
        yield f"zipf-{N}", np.minimum(rng.zipf(1.1, N) - 1, V - 1), V
    yield "equal-1200", np.full(1200, 17), V
    # one id holding more than 1,008 chunks of sorted entries (a second probe round)
    yield "long-run", np.where(rng.random(1100 * K) < 0.97, 3, rng.integers(0, V, 1100 * K)), V
    bad = rng.integers(0, 64, 777)
    bad[::9] = -5
    bad[4::13] = V + 2
    yield "invalid-ids", bad, V


@pytest.mark.parametrize("name,idx,V", list(cases()), ids=lambda x: x if isinstance(x, str) else "")
def test_value_embedding_segments_match_brute_force(ve, name, idx, V):
    rng = np.random.default_rng(len(name))
    N = idx.size
    ok = (idx >= 0) & (idx < V)
    key = np.where(ok, idx, 0).astype(np.int32)
    order = np.argsort(key, kind="stable")
    keys = np.ascontiguousarray(key[order])
    vals = np.ascontiguousarray(np.where(ok[order], order, -1 - order).astype(np.int32))
    ld, col0 = 384, 256                           # dv sits at columns 256.. of a wider row
    src = rng.standard_normal((N, ld)).astype(np.float32)
    gate = np.array([0.75], dtype=np.float32)
    dve0 = rng.standard_normal((V, 128)).astype(np.float32)
    dve = dve0.copy()
    nseg = (N + K - 1) // K
    carry = np.full(2 * nseg * 129, np.nan, dtype=np.float32)   # every slot read must have been written
    ve.ve_scatter(keys, vals, src.reshape(-1), ld, col0, gate, N, dve.reshape(-1), carry)

    want = dve0.astype(np.float64)
    np.add.at(want, idx[ok], 0.75 * src[ok, col0:col0 + 128].astype(np.float64))
    assert np.all(np.isfinite(dve))
    np.testing.assert_allclose(dve, want, rtol=1e-5, atol=1e-5 * max(1.0, np.abs(want).max()))
    untouched = np.setdiff1d(np.arange(V), idx[ok])
    assert np.array_equal(dve[untouched], dve0[untouched])    # rows of absent ids stay bit for bit
