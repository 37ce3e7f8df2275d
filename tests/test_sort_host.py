"""The embedding backward's id sort, run on the CPU from its own source text.

The kernels of the two-pass radix sort (the initial key/value pass, the
per-chunk digit histogram, the per-digit scan, the stable scatter) are taken
out of the kernel source and compiled for the host with g++. Each launch runs
its blocks in order, each block's threads as fibers on one OS thread:
`__shared__` arrays are the block's shared memory, `__syncthreads` returns to
a scheduler that resumes every live thread once per round (so each thread
reaches the barrier before any passes it), and shared-memory `atomicAdd` is a
read-modify-write that no other thread can interleave; every case runs with
the threads of each round resumed in order and in reverse. The launches follow the
launcher: the initial pass, then for each 8-bit digit histogram, scan and
scatter, ping-ponging between two buffers.

The result must be the stable sort of the ids (equal ids keep their
positions in order), with an invalid id (outside [0, V)) sorted in as id 0
carrying the position n as -1 - n; for ids of many shapes and counts: one
chunk, ragged and whole chunk counts, up to the 65,536 tokens of the
benchmarked batch, all ids equal, Zipf ids, every id distinct.
"""
import ctypes
import shutil
import subprocess

import numpy as np
import pytest

from host_src import device_function, int_constant, kernel_function

KS = int_constant("embed_bwd.hip", "kSortChunk")

HARNESS = r"""
#include <algorithm>
#include <cstdint>
#include <functional>
#include <utility>
#include <vector>
#include <ucontext.h>

using std::min;
constexpr int kSortChunk = %d;
#define DEV static inline
#define __global__
#define __launch_bounds__(n)
#define __shared__ static
struct Idx3 { int x = 0, y = 0, z = 0; };
static Idx3 blockIdx, threadIdx;

// A block's threads are fibers on one OS thread. A barrier hands control back
// to the scheduler, which resumes every live fiber once per round, in thread
// order: each fiber runs up to its next barrier (or its end) before any
// fiber passes that barrier.
namespace sim {
struct Fiber {
  ucontext_t ctx;
  bool done = false;
  std::vector<char> stack = std::vector<char>(1 << 16);
};
static ucontext_t sched;
static std::vector<Fiber> fibers;
static Fiber* cur = nullptr;
static std::function<void()> body;
static bool reverse = false;  // resume order within a round: thread order or its reverse
static void entry(int t) {
  (void)t;
  body();
  cur->done = true;  // returns to sched through uc_link
}
}  // namespace sim
static void __syncthreads() { swapcontext(&sim::cur->ctx, &sim::sched); }
static int atomicAdd(int* p, int v) {  // one OS thread: a plain read-modify-write is atomic
  const int old = *p;
  *p = old + v;
  return old;
}

%s
%s
%s
%s
%s

// one launch: the grid's blocks in order, each as `threads` fibers
template <typename F>
static void launch(int grid, int threads, F&& fn) {
  sim::body = fn;
  sim::fibers.resize(threads);
  for (int b = 0; b < grid; ++b) {
    blockIdx.x = b;
    for (int t = 0; t < threads; ++t) {
      sim::Fiber& f = sim::fibers[t];
      f.done = false;
      getcontext(&f.ctx);
      f.ctx.uc_stack.ss_sp = f.stack.data();
      f.ctx.uc_stack.ss_size = f.stack.size();
      f.ctx.uc_link = &sim::sched;
      makecontext(&f.ctx, (void (*)())sim::entry, 1, t);
    }
    for (bool live = true; live;) {
      live = false;
      for (int i = 0; i < threads; ++i) {
        const int t = sim::reverse ? threads - 1 - i : i;
        sim::Fiber& f = sim::fibers[t];
        if (f.done) continue;
        sim::cur = &f;
        threadIdx.x = t;
        swapcontext(&sim::sched, &f.ctx);
        live |= !f.done;
      }
    }
  }
}

extern "C" void sort_ids(const int32_t* idx, int N, int V, int32_t* keys_a, int32_t* vals_a, int32_t* keys_b,
                         int32_t* vals_b, int32_t* hist, int reverse) {
  sim::reverse = reverse != 0;
  launch((N + 255) / 256, 256, [&] { sort_init_kernel(idx, N, V, keys_a, vals_a); });
  const int nchunks = (N + kSortChunk - 1) / kSortChunk;
  int32_t *kin = keys_a, *vin = vals_a, *kout = keys_b, *vout = vals_b;
  for (int shift = 0; shift < 16; shift += 8) {
    int32_t* total = hist + (size_t)256 * nchunks;
    launch(nchunks, kSortChunk, [&] { radix_hist_kernel(kin, N, shift, nchunks, hist); });
    launch(256, 256, [&] { digit_scan_kernel(hist, nchunks, total); });
    launch(nchunks, kSortChunk, [&] { radix_scatter_kernel(kin, vin, N, shift, nchunks, hist, total, kout, vout); });
    std::swap(kin, kout);
    std::swap(vin, vout);
  }
}
"""


@pytest.fixture(scope="module")
def sorter(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("sort")
    code = HARNESS % (KS, kernel_function("embed_bwd.hip", "sort_init_kernel"),
                      kernel_function("embed_bwd.hip", "radix_hist_kernel"),
                      device_function("embed_bwd.hip", "block_scan256"),
                      kernel_function("embed_bwd.hip", "digit_scan_kernel"),
                      kernel_function("embed_bwd.hip", "radix_scatter_kernel"))
    (d / "sort.cpp").write_text(code)
    so = str(d / "sort.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-shared", "-fPIC", "-w", "-o", so, str(d / "sort.cpp")],
                   check=True)
    lib = ctypes.CDLL(so)
    I = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
    lib.sort_ids.argtypes = [I, ctypes.c_int, ctypes.c_int, I, I, I, I, I, ctypes.c_int]
    return lib


def cases():
    rng = np.random.default_rng(11)
    V = 65536
    yield "one-chunk-zipf", np.minimum(rng.zipf(1.1, 200) - 1, V - 1), V
    yield "ragged-uniform", rng.integers(0, V, 999), V
    yield "whole-chunks-zipf", np.minimum(rng.zipf(1.1, 4096) - 1, V - 1), V
    yield "all-equal", np.full(3000, 40000), V
    yield "distinct-descending", np.arange(5000)[::-1] * 13, V
    yield "bench-batch-zipf", np.minimum(rng.zipf(1.1, 65536) - 1, V - 1), V
    bad = rng.integers(0, 512, 1500)
    bad[::7] = -1
    bad[3::11] = 512
    yield "invalid-ids", bad, 512


@pytest.mark.parametrize("reverse", [0, 1])
@pytest.mark.parametrize("name,idx,V", list(cases()), ids=lambda x: x if isinstance(x, str) else "")
def test_radix_sort_is_the_stable_sort(sorter, name, idx, V, reverse):
    """Run with the threads of each barrier round resumed in thread order and
    in reverse: a read that a missing barrier leaves racing with a write sees
    the write in one order and not in the other."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    N = idx.size
    nchunks = (N + KS - 1) // KS
    ka, va, kb, vb = (np.full(N, -7, dtype=np.int32) for _ in range(4))
    hist = np.full(256 * nchunks + 256, -7, dtype=np.int32)
    sorter.sort_ids(idx, N, V, ka, va, kb, vb, hist, reverse)
    ok = (idx >= 0) & (idx < V)
    key = np.where(ok, idx, 0)
    order = np.argsort(key, kind="stable")
    np.testing.assert_array_equal(ka, key[order])
    np.testing.assert_array_equal(va, np.where(ok[order], order, -1 - order))
