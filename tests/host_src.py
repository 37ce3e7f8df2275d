"""Pieces of the HIP kernel sources taken out as text, for CPU tests that
compile them for the host with g++ (no GPU, no retyping of the code)."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decoder_only_transformer_gpt_amd", "csrc")


def device_function(path, name):
    """The full text of `DEV <type> name(...) { ... }` in a kernel source."""
    src = open(os.path.join(CSRC, path)).read()
    m = re.search(r"^DEV\s+\w+\s+" + name + r"\s*\(", src, flags=re.M)
    assert m, f"{name} not found in {path}"
    i = src.index("{", m.end())
    depth = 0
    for j in range(i, len(src)):
        depth += {"{": 1, "}": -1}.get(src[j], 0)
        if depth == 0:
            return src[m.start():j + 1]
    raise AssertionError(f"unbalanced braces after {name}")


def int_constant(path, name):
    """The value of `constexpr int name = <literal>;` in a kernel source."""
    src = open(os.path.join(CSRC, path)).read()
    m = re.search(r"constexpr\s+int\s+" + name + r"\s*=\s*(\d+)\s*;", src)
    assert m, f"{name} not found in {path}"
    return int(m.group(1))


def kernel_function(path, name):
    """The full text of a kernel `[template <...>] __global__ ... name(...) { ... }`."""
    src = open(os.path.join(CSRC, path)).read()
    m = re.search(r"^(template\s*<[^>]*>\s*\n)?__global__[^\n]*\b" + name + r"\s*\(", src, flags=re.M)
    assert m, f"{name} not found in {path}"
    i = src.index("{", m.end())
    depth = 0
    for j in range(i, len(src)):
        depth += {"{": 1, "}": -1}.get(src[j], 0)
        if depth == 0:
            return src[m.start():j + 1]
    raise AssertionError(f"unbalanced braces after {name}")
