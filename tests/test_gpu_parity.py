"""Parity of the HIP training step against the float64 oracle, through the C ABI.

Tolerances: fp32 model: |dloss|/loss <= 1e-5, per-tensor relative L2 of every
gradient <= 1e-4. bf16 models: |dloss|/loss <= 5e-3, per-tensor gradient
cosine >= 0.999 (W_qkv split into its q, k and v blocks)."""
import math

import numpy as np
import pytest

from decoder_only_transformer_gpt_amd import _lib
from oracle import gpt_oracle as O

import gpu_util as U

pytestmark = pytest.mark.gpu


def tiny_cfg(T=64):
    c = _lib.gpt_config_from_depth(2, _lib.GPT_F32)
    c.vocab_size = 512
    c.max_seq_len = max(T, 64)
    return c


def d4_cfg():
    c = _lib.gpt_config_from_depth(4, _lib.GPT_BF16)
    return c


def vanishing(go: dict, k: str) -> bool:
    """A gradient the mathematics makes exactly zero (e.g. W_q and W_k with
    one-token rows, where the softmax is 1 whatever q and k are): its norm is
    below 1e-12 of the whole gradient's. The GPU's value is then rounding
    residue (dP - delta cancels), checked against the whole gradient's scale."""
    total = np.sqrt(sum(float(np.sum(v * v)) for v in go.values()))
    return float(np.linalg.norm(go[k])) <= 1e-12 * total


def check_vanishing(gg, go, k, tol):
    total = np.sqrt(sum(float(np.sum(v * v)) for v in go.values()))
    assert float(np.linalg.norm(gg[k])) <= tol * total, k


def check_fp32(case, gpu, loss, G, label):
    rel = abs(gpu["loss"] - loss) / abs(loss)
    U.log(f"[{label}] loss gpu={gpu['loss']:.9f} oracle={loss:.9f} rel={rel:.2e}")
    assert rel <= 1e-5
    gg = U.split_tensors(case, gpu["grads"])
    go = U.split_tensors(case, case.flat_grads(G))
    live = [k for k in go if not vanishing(go, k)]
    worst = max((U.rel_l2(gg[k], go[k]), k) for k in live)
    U.log(f"[{label}] worst grad rel L2 {worst[0]:.2e} ({worst[1]})")
    for k in go:
        if k in live:
            assert U.rel_l2(gg[k], go[k]) <= 1e-4, k
        else:
            check_vanishing(gg, go, k, 1e-4)


def check_bf16(case, gpu, loss, G, label):
    rel = abs(gpu["loss"] - loss) / abs(loss)
    U.log(f"[{label}] loss gpu={gpu['loss']:.6f} oracle={loss:.6f} rel={rel:.2e}")
    assert rel <= 5e-3
    gg = U.split_tensors(case, gpu["grads"])
    go = U.split_tensors(case, case.flat_grads(G))
    live = [k for k in go if not vanishing(go, k)]
    worst = min((U.cosine(gg[k], go[k]), k) for k in live)
    U.log(f"[{label}] worst grad cosine {worst[0]:.6f} ({worst[1]})")
    for k in go:
        if k in live:
            assert U.cosine(gg[k], go[k]) >= 0.999, k
        else:
            check_vanishing(gg, go, k, 4.5e-2)


@pytest.mark.parametrize("tile", [0, 1, 2, 3])
def test_tiny_fp32_full_step(tile):
    U.require_gpu()
    case = U.Case(tiny_cfg(), B=2, T=64, law="uniform")
    U.log(f"case tiny fp32 B=2 T=64 V=512 seed 0/1 gemm tile {tile}")
    gpu = U.run_gpu(case, tile=tile)
    assert gpu["status"] == _lib.GPT_OK
    loss, rows, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    np.testing.assert_allclose(gpu["row_loss"], rows.reshape(-1), rtol=2e-5)
    check_fp32(case, gpu, loss, G, "tiny")


def test_tiny_fp32_ragged_and_scaled():
    """T not a multiple of any tile (ragged attention and GEMM tails), B=3,
    dloss scaling and gradient accumulation on top of a first step."""
    U.require_gpu()
    case = U.Case(tiny_cfg(T=100), B=3, T=77, law="uniform", wseed=5, tseed=6)
    U.log("case tiny fp32 ragged B=3 T=77")
    torch = U.require_gpu()
    from decoder_only_transformer_gpt_amd.model import GPT
    m = GPT(case.cfg, GPT.params_from_numpy(case.storage, case.cfg), 3, 100)
    idx, tgt = torch.from_numpy(case.idx).cuda(), torch.from_numpy(case.tgt).cuda()
    m.forward_loss(idx, tgt)
    m.backward(0.5, accumulate=False)
    m.forward_loss(idx, tgt)
    m.backward(1.5, accumulate=True)   # grads = 2.0 * dloss/dtheta
    torch.cuda.synchronize()
    loss, _, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt, dloss=2.0)
    gpu = dict(loss=float(m.loss.item()), grads=m.grads.cpu().numpy().astype(np.float64))
    check_fp32(case, gpu, loss, G, "tiny-ragged")


@pytest.mark.parametrize("tile", [0, 1, 2, 3])
def test_d4_bf16_full_step(tile):
    U.require_gpu()
    case = U.Case(d4_cfg(), B=4, T=512, law="uniform")
    U.log(f"case d4 bf16 B=4 T=512 uniform gemm tile {tile}")
    gpu = U.run_gpu(case, tile=tile)
    assert gpu["status"] == _lib.GPT_OK
    loss, rows, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    check_bf16(case, gpu, loss, G, "d4")


@pytest.mark.parametrize("tile", [0, 1, 2, 3])
def test_bf16_ragged_zipf(tile):
    """bf16, Zipf ids (heavy repeats in the embedding backward), ragged T and M
    (partial GEMM tiles in every variant)."""
    U.require_gpu()
    c = d4_cfg()
    case = U.Case(c, B=3, T=333, law="zipf", wseed=2, tseed=3)
    U.log(f"case d4 bf16 ragged B=3 T=333 zipf gemm tile {tile}")
    gpu = U.run_gpu(case, tile=tile)
    loss, rows, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    check_bf16(case, gpu, loss, G, "d4-ragged-zipf")


@pytest.mark.timeout(600)
def test_d12_bf16_one_row():
    U.require_gpu()
    c = _lib.gpt_config_from_depth(12, _lib.GPT_BF16)
    case = U.Case(c, B=1, T=2048, law="zipf")
    U.log("case d12 bf16 B=1 T=2048 zipf")
    gpu = U.run_gpu(case)
    loss, rows, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    check_bf16(case, gpu, loss, G, "d12")


@pytest.mark.timeout(900)
def test_d20_bf16_one_row():
    U.require_gpu()
    c = _lib.gpt_config_from_depth(20, _lib.GPT_BF16)
    case = U.Case(c, B=1, T=2048, law="zipf")
    U.log("case d20 bf16 B=1 T=2048 zipf")
    gpu = U.run_gpu(case)
    loss, rows, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    check_bf16(case, gpu, loss, G, "d20-B1")


@pytest.mark.timeout(900)
def test_d20_full_batch_sampled_rows():
    """The benchmarked launch (d20, B=32, T=2048): per-position losses of two
    seeded batch rows against an oracle forward of just those rows (rows are
    independent), plus the full step's gradients are finite."""
    U.require_gpu()
    c = _lib.gpt_config_from_depth(20, _lib.GPT_BF16)
    case = U.Case(c, B=32, T=2048, law="zipf")
    U.log("case d20 bf16 B=32 T=2048 zipf (bench launch)")
    gpu = U.run_gpu(case)
    assert gpu["status"] == _lib.GPT_OK
    assert np.all(np.isfinite(gpu["grads"]))
    rows_gpu = gpu["row_loss"].reshape(32, 2048)
    assert gpu["loss"] == pytest.approx(rows_gpu.mean(), rel=1e-5)
    P = case.oracle_params()
    for b in (int(np.random.default_rng(7).integers(0, 32)), 31):
        r = O.forward_rows(U.oracle_cfg(c), P, case.idx[b:b + 1], case.tgt[b:b + 1])[0]
        rel = abs(rows_gpu[b].mean() - r.mean()) / r.mean()
        err = np.abs(rows_gpu[b] - r)
        U.log(f"[d20-B32] row {b}: mean loss gpu={rows_gpu[b].mean():.5f} oracle={r.mean():.5f} rel={rel:.2e} "
              f"max abs per-position {err.max():.3e}")
        assert rel <= 5e-3
        assert np.median(err / r) <= 5e-3


# ------------------------------------------------- sliding-window layers ---

def with_windows(c, pattern: str, short: int):
    c.window_pattern = pattern.encode()
    c.window_short = short
    return c


def test_tiny_fp32_sliding_window_ragged():
    """fp32: layer 0 with a 16-token window, layer 1 (the last) full; ragged T."""
    U.require_gpu()
    c = with_windows(tiny_cfg(T=100), "S", 16)
    case = U.Case(c, B=2, T=77, law="uniform", wseed=7, tseed=8)
    U.log("case tiny fp32 B=2 T=77 window S/16")
    gpu = U.run_gpu(case)
    assert gpu["status"] == _lib.GPT_OK
    loss, rows, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    np.testing.assert_allclose(gpu["row_loss"], rows.reshape(-1), rtol=2e-5)
    check_fp32(case, gpu, loss, G, "tiny-window")


@pytest.mark.parametrize("tile", [0, 3])
def test_bf16_sssl_window_ragged(tile):
    """bf16 d4 with the SSSL pattern, a window that is not a multiple of the
    64-row tiles, ragged T and Zipf ids."""
    U.require_gpu()
    c = with_windows(d4_cfg(), "SSSL", 100)
    case = U.Case(c, B=3, T=333, law="zipf", wseed=9, tseed=10)
    U.log(f"case d4 bf16 B=3 T=333 SSSL/100 gemm tile {tile}")
    gpu = U.run_gpu(case, tile=tile)
    assert gpu["status"] == _lib.GPT_OK
    loss, rows, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    check_bf16(case, gpu, loss, G, "d4-sssl")


def test_bf16_window_changes_result_and_full_window_does_not():
    """A window as long as the sequence is the full causal prefix (bitwise); a
    shorter one changes every windowed layer's output."""
    torch = U.require_gpu()
    base = U.Case(d4_cfg(), B=2, T=256, law="uniform", wseed=11, tseed=12)
    full = U.run_gpu(base)
    longw = U.Case(with_windows(d4_cfg(), "SSSL", 256), B=2, T=256, law="uniform", wseed=11, tseed=12)
    g_long = U.run_gpu(longw)
    assert g_long["loss"] == full["loss"]
    np.testing.assert_array_equal(g_long["grads"], full["grads"])
    short = U.Case(with_windows(d4_cfg(), "SSSL", 64), B=2, T=256, law="uniform", wseed=11, tseed=12)
    g_short = U.run_gpu(short)
    assert g_short["loss"] != full["loss"]


@pytest.mark.timeout(900)
def test_d20_sssl_one_row():
    """The pages' pattern at d20: SSSL with 1,024-token short windows, T = 2048."""
    U.require_gpu()
    c = with_windows(_lib.gpt_config_from_depth(20, _lib.GPT_BF16), "SSSL", 1024)
    case = U.Case(c, B=1, T=2048, law="zipf")
    U.log("case d20 bf16 B=1 T=2048 zipf SSSL/1024")
    gpu = U.run_gpu(case)
    loss, rows, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    check_bf16(case, gpu, loss, G, "d20-sssl-B1")


# ------------------------------------------------------- degenerate sizes ---

@pytest.mark.parametrize("B,T", [(5, 1), (1, 2), (3, 65)])
def test_tiny_fp32_degenerate_lengths(B, T):
    """One-token rows (attention over the query itself only: the W_q and W_k
    gradients vanish), two tokens, and one token past a 64-row tile; the
    handle is built for a longer maximum."""
    U.require_gpu()
    case = U.Case(tiny_cfg(T=128), B=B, T=T, law="uniform", wseed=40 + T, tseed=41 + T)
    U.log(f"case tiny fp32 B={B} T={T} (max 8 x 128)")
    gpu = U.run_gpu(case, max_B=8, max_T=128)
    assert gpu["status"] == _lib.GPT_OK
    loss, rows, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    np.testing.assert_allclose(gpu["row_loss"], rows.reshape(-1), rtol=2e-5)
    check_fp32(case, gpu, loss, G, f"tiny-B{B}-T{T}")


@pytest.mark.parametrize("B,T", [(7, 1), (2, 3)])
def test_bf16_degenerate_lengths(B, T):
    """bf16 d4 with one- and three-token rows (every GEMM's M far below a tile)."""
    U.require_gpu()
    case = U.Case(d4_cfg(), B=B, T=T, law="zipf", wseed=42 + T, tseed=43 + T)
    U.log(f"case d4 bf16 B={B} T={T}")
    gpu = U.run_gpu(case, max_B=8, max_T=512)
    assert gpu["status"] == _lib.GPT_OK
    loss, rows, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    check_bf16(case, gpu, loss, G, f"d4-B{B}-T{T}")
