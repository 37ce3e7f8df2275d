"""The embedding fix-up's search for the chunk a run of equal ids ends in,
checked on the CPU against brute force.

`run_last_chunk` (the embedding backward's fix-up kernel) is taken out of the
kernel source as text and compiled for the host with g++. It runs as one
64-lane wave: 64 threads execute it in lock step, each with its own lane
index, and `__ballot` is a barrier-synchronised OR of the 64 lanes' bits, as
on the GPU. Every lane must return the same chunk, and that chunk must be the
last one whose first entry still holds the run's id, for every chunk whose
last run goes on past it, over sorted ids of many shapes: a few distinct ids,
all ids equal (one run over every chunk), Zipf ids (runs of every length)
and many short runs; entry counts that fill the last chunk or leave it
ragged, up to the 65,536 tokens of the benchmarked batch.
"""
import ctypes
import shutil
import subprocess

import numpy as np
import pytest

from host_src import device_function, int_constant

K = int_constant("embed_bwd.hip", "kSegChunk")

# The ballot: every lane ORs its bit into mask[k % 3], all wait at the
# barrier, then read it; lane 0 clears mask[(k + 2) % 3] (last read in ballot
# k - 1, next written in ballot k + 2, after the barrier of ballot k + 1).
HARNESS = r"""
#include <atomic>
#include <barrier>
#include <cstdint>
#include <thread>
#include <vector>

constexpr int kSegChunk = %d;

namespace wave {
std::barrier<>* bar = nullptr;
std::atomic<uint64_t> mask[3];
thread_local int ballots = 0;
thread_local int my_lane = 0;
}

static uint64_t __ballot(bool pred) {
  const int k = wave::ballots++;
  if (pred) wave::mask[k %% 3].fetch_or(uint64_t(1) << wave::my_lane);
  wave::bar->arrive_and_wait();
  const uint64_t m = wave::mask[k %% 3].load();
  if (wave::my_lane == 0) wave::mask[(k + 2) %% 3].store(0);
  return m;
}

#define DEV static inline
%s

extern "C" int search(const int32_t* keys, int nchunks, const int32_t* cs, const int32_t* vs, int ncase,
                      int32_t* out) {
  std::barrier<> bar(64);
  wave::bar = &bar;
  for (auto& m : wave::mask) m.store(0);
  std::vector<int32_t> res((size_t)ncase * 64);
  std::vector<std::thread> lanes;
  for (int l = 0; l < 64; ++l)
    lanes.emplace_back([&, l] {
      wave::my_lane = l;
      wave::ballots = 0;
      for (int i = 0; i < ncase; ++i) res[(size_t)i * 64 + l] = run_last_chunk(keys, nchunks, cs[i], vs[i], l);
    });
  for (auto& t : lanes) t.join();
  int uniform = 1;
  for (int i = 0; i < ncase; ++i) {
    out[i] = res[(size_t)i * 64];
    for (int l = 1; l < 64; ++l) uniform &= res[(size_t)i * 64 + l] == out[i];
  }
  return uniform;
}
"""


@pytest.fixture(scope="module")
def search(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("run_search")
    code = HARNESS % (K, device_function("embed_bwd.hip", "run_last_chunk"))
    (d / "search.cpp").write_text(code)
    so = str(d / "search.so")
    subprocess.run(["g++", "-std=c++20", "-O1", "-pthread", "-shared", "-fPIC", "-o", so, str(d / "search.cpp")],
                   check=True)
    lib = ctypes.CDLL(so)
    P = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
    lib.search.argtypes = [P, ctypes.c_int, P, P, ctypes.c_int, P]
    lib.search.restype = ctypes.c_int
    return lib


def crossing_runs(keys):
    """Chunks whose last run goes on past them, with that run's id, and the
    brute-force answer: the chunk holding the run's last entry."""
    N = keys.size
    nchunks = (N + K - 1) // K
    c = np.arange(nchunks - 1)                   # the last chunk has nothing after it
    ends = (c + 1) * K
    cross = keys[ends - 1] == keys[ends]
    c = c[cross]
    v = keys[(c + 1) * K - 1]
    last_entry = np.searchsorted(keys, v, side="right") - 1
    return nchunks, c.astype(np.int32), v.astype(np.int32), (last_entry // K).astype(np.int32)


def key_sets():
    rng = np.random.default_rng(0)
    for N in (K + 1, 2 * K, 3 * K + 5, 999, 4096, 65536):
        yield f"few-{N}", np.sort(rng.integers(0, 5, N))
        yield f"equal-{N}", np.zeros(N, dtype=np.int64)
        yield f"zipf-{N}", np.sort(np.minimum(rng.zipf(1.1, N), 65535))
        yield f"short-{N}", np.sort(rng.integers(0, max(1, N // 50), N))
    # runs whose last chunk sits on every offset around the probes' stride and
    # the 63 x 16 chunks a first round covers
    for span in (15, 16, 17, 31, 32, 33, 1007, 1008, 1009, 1010, 2016, 2017):
        N = (span + 3) * K
        keys = np.full(N, 7, dtype=np.int64)
        keys[:K // 2] = 3
        keys[(span + 1) * K + 5:] = 9
        yield f"span-{span}", keys


@pytest.mark.parametrize("name,keys", list(key_sets()), ids=lambda x: x if isinstance(x, str) else "")
def test_run_last_chunk_matches_brute_force(search, name, keys):
    keys = np.ascontiguousarray(keys, dtype=np.int32)
    nchunks, cs, vs, want = crossing_runs(keys)
    if cs.size == 0:
        return
    # only the chunk in which a crossing run begins calls the search
    begins = (cs == 0) | (keys[np.maximum(cs * K - 1, 0)] != vs) | (keys[cs * K] != vs)
    cs, vs, want = cs[begins], vs[begins], want[begins]
    got = np.empty(cs.size, dtype=np.int32)
    assert search.search(keys, nchunks, cs, vs, cs.size, got) == 1, "lanes disagree"
    np.testing.assert_array_equal(got, want)
