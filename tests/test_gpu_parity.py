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


def grad_norm(go: dict) -> float:
    """L2 norm of the whole gradient (all tensors)."""
    return float(np.sqrt(sum(float(np.dot(v.ravel(), v.ravel())) for v in go.values())))


def vanishing(go: dict, k: str, total: float) -> bool:
    """A gradient the mathematics makes exactly zero (e.g. W_q and W_k with
    one-token rows, where the softmax is 1 whatever q and k are): its norm is
    below 1e-12 of the whole gradient's (`total`). The GPU's value is then
    rounding residue (dP - delta cancels), checked against the whole
    gradient's scale."""
    return float(np.linalg.norm(go[k])) <= 1e-12 * total


def check_vanishing(gg, k, tol, total):
    assert float(np.linalg.norm(gg[k])) <= tol * total, k


def check_fp32(case, gpu, loss, G, label):
    rel = abs(gpu["loss"] - loss) / abs(loss)
    U.log(f"[{label}] loss gpu={gpu['loss']:.9f} oracle={loss:.9f} rel={rel:.2e}")
    assert rel <= 1e-5
    gg = U.split_tensors(case, gpu["grads"])
    go = U.split_tensors(case, case.flat_grads(G))
    total = grad_norm(go)
    live = [k for k in go if not vanishing(go, k, total)]
    worst = max((U.rel_l2(gg[k], go[k]), k) for k in live)
    U.log(f"[{label}] worst grad rel L2 {worst[0]:.2e} ({worst[1]})")
    for k in go:
        if k in live:
            assert U.rel_l2(gg[k], go[k]) <= 1e-4, k
        else:
            check_vanishing(gg, k, 1e-4, total)


def check_bf16(case, gpu, loss, G, label):
    rel = abs(gpu["loss"] - loss) / abs(loss)
    U.log(f"[{label}] loss gpu={gpu['loss']:.6f} oracle={loss:.6f} rel={rel:.2e}")
    assert rel <= 5e-3
    gg = U.split_tensors(case, gpu["grads"])
    go = U.split_tensors(case, case.flat_grads(G))
    total = grad_norm(go)
    live = [k for k in go if not vanishing(go, k, total)]
    worst = min((U.cosine(gg[k], go[k]), k) for k in live)
    U.log(f"[{label}] worst grad cosine {worst[0]:.6f} ({worst[1]})")
    for k in go:
        if k in live:
            assert U.cosine(gg[k], go[k]) >= 0.999, k
        else:
            check_vanishing(gg, k, 4.5e-2, total)


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


def test_d4_bf16_fp32_residual_gradient_option():
    """GPT_OPT_RESID_GRAD = 1 keeps a bf16 model's residual-stream gradient in
    fp32: the same bar against the oracle, the same loss bit for bit (the
    forward is untouched), gradients close to the default bf16-kept ones;
    values outside 0..1 are rejected."""
    U.require_gpu()
    case = U.Case(d4_cfg(), B=4, T=512, law="zipf")
    U.log("case d4 bf16 B=4 T=512 zipf, residual gradient fp32 vs bf16")
    g32 = U.run_gpu(case, resid_grad_f32=True)
    g16 = U.run_gpu(case)
    assert g32["status"] == _lib.GPT_OK and g16["status"] == _lib.GPT_OK
    loss, rows, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    check_bf16(case, g32, loss, G, "d4-resid-f32")
    assert g32["loss"] == g16["loss"]
    assert U.cosine(g32["grads"], g16["grads"]) >= 0.9999
    with pytest.raises(RuntimeError):
        _lib.gpt_set_option(g16["model"].h, _lib.GPT_OPT_RESID_GRAD, 2)


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


_ORACLE = {}


def oracle_step(key, case):
    """The oracle's step for a seeded case, computed once per test session
    (several GPU launch forms are compared with one oracle result)."""
    if key not in _ORACLE:
        _ORACLE[key] = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    return _ORACLE[key]


def replicated(case, copies):
    """The same case with its batch rows repeated `copies` times (rows
    r0, r1, ..., r0, r1, ...). Rows are independent and the loss is their
    mean, so the loss and every gradient equal those of the original batch."""
    import copy
    big = copy.copy(case)
    big.B = case.B * copies
    big.idx = np.ascontiguousarray(np.tile(case.idx, (copies, 1)))
    big.tgt = np.ascontiguousarray(np.tile(case.tgt, (copies, 1)))
    return big


@pytest.mark.parametrize("hsplit", [0, 1])
def test_d4_bf16_batch16_branches(hsplit):
    """d4 at B = 16 distinct rows (B % 8 == 0: the XCD row remap of the
    attention forward and dQ kernels), with the dK/dV kernel in both forms:
    0 picks two head halves plus the combine pass at this size, 1 forces
    one workgroup per key block storing bf16 dK/dV directly (the form the
    benchmarked d20 launch takes)."""
    U.require_gpu()
    case = U.Case(d4_cfg(), B=16, T=512, law="uniform", wseed=13, tseed=14)
    U.log(f"case d4 bf16 B=16 T=512 uniform dkv hsplit {hsplit}")
    gpu = U.run_gpu(case, hsplit=hsplit)
    assert gpu["status"] == _lib.GPT_OK
    loss, rows, G = oracle_step("d4-b16", case)
    np.testing.assert_allclose(gpu["row_loss"], rows.reshape(-1), rtol=5e-3)
    check_bf16(case, gpu, loss, G, f"d4-B16-h{hsplit}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("hsplit", [0, 1])
def test_d12_bf16_full_batch(hsplit):
    """d12 at its configured batch (B = 16, T = 2048, Zipf ids), the whole
    gradient against the oracle; dK/dV in the default form at this size
    (two head halves) and forced to one workgroup per key block."""
    U.require_gpu()
    c = _lib.gpt_config_from_depth(12, _lib.GPT_BF16)
    case = U.Case(c, B=16, T=2048, law="zipf")
    U.log(f"case d12 bf16 B=16 T=2048 zipf dkv hsplit {hsplit}")
    gpu = U.run_gpu(case, hsplit=hsplit)
    assert gpu["status"] == _lib.GPT_OK
    loss, rows, G = oracle_step("d12-b16", case)
    check_bf16(case, gpu, loss, G, f"d12-B16-h{hsplit}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("form", ["B2-h0", "B2-h1", "B32-h0", "B32-h2"])
def test_d20_bf16_gradients(form):
    """d20 against the oracle's B = 2 step (two distinct Zipf rows). B2: the
    two rows themselves, dK/dV in its default form at this size (two head
    halves) and forced to one workgroup per key block. B32: the benchmarked
    launch (B = 32, T = 2048) on 16 copies of the two rows, whose mean loss
    and gradients equal the B = 2 ones: the dK/dV form it picks by itself
    (one workgroup per key block), the remapped row order of the attention
    kernels and the weight-gradient split-K counts at K = 65,536 tokens; and
    the same launch with dK/dV forced to two head halves."""
    U.require_gpu()
    c = _lib.gpt_config_from_depth(20, _lib.GPT_BF16)
    base = U.Case(c, B=2, T=2048, law="zipf")
    B = int(form.split("-")[0][1:])
    hsplit = int(form.split("-")[1][1:])
    case = base if B == 2 else replicated(base, B // 2)
    U.log(f"case d20 bf16 B={B} T=2048 zipf dkv hsplit {hsplit}")
    gpu = U.run_gpu(case, hsplit=hsplit)
    assert gpu["status"] == _lib.GPT_OK
    loss, rows, G = oracle_step("d20-b2", base)
    got_rows = gpu["row_loss"].reshape(B, 2048)
    want_rows = np.tile(rows, (B // 2, 1))
    err = np.abs(got_rows - want_rows) / want_rows
    U.log(f"[d20-{form}] max per-position loss rel err {err.max():.2e}")
    assert err.max() <= 5e-3
    check_bf16(case, gpu, loss, G, f"d20-{form}")


@pytest.mark.timeout(900)
def test_d20_full_batch_sampled_rows():
    """The benchmarked launch (d20, B=32, T=2048) on 32 distinct rows: the
    per-position losses of three batch rows (the first two and the last)
    against the oracle on just those rows (rows are independent), every
    position within the loss tolerance, and finite gradients."""
    U.require_gpu()
    c = _lib.gpt_config_from_depth(20, _lib.GPT_BF16)
    case = U.Case(c, B=32, T=2048, law="zipf")
    U.log("case d20 bf16 B=32 T=2048 zipf (bench launch)")
    gpu = U.run_gpu(case)
    assert gpu["status"] == _lib.GPT_OK
    assert np.all(np.isfinite(gpu["grads"]))
    rows_gpu = gpu["row_loss"].reshape(32, 2048)
    assert gpu["loss"] == pytest.approx(rows_gpu.mean(), rel=1e-5)
    # rows 0 and 1 of this seeded draw are the two rows of the d20 B=2 case
    # (one [B, T+1] draw, row by row), whose oracle step the gradient tests
    # already ran; the last row gets an oracle forward of its own
    two = U.Case(c, B=2, T=2048, law="zipf")
    assert np.array_equal(two.idx, case.idx[:2]) and np.array_equal(two.tgt, case.tgt[:2])
    _, rows2, _ = oracle_step("d20-b2", two)
    P = case.oracle_params()
    for b in (0, 1, 31):
        r = rows2[b] if b < 2 else O.forward_rows(U.oracle_cfg(c), P, case.idx[b:b + 1], case.tgt[b:b + 1])[0]
        rel = abs(rows_gpu[b].mean() - r.mean()) / r.mean()
        err = np.abs(rows_gpu[b] - r) / r
        U.log(f"[d20-B32] row {b}: mean loss gpu={rows_gpu[b].mean():.5f} oracle={r.mean():.5f} rel={rel:.2e} "
              f"max per-position rel {err.max():.3e}")
        assert rel <= 5e-3
        assert err.max() <= 5e-3


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


# ------------------------------------------------- embedding gradient rows ---

def wide_one_layer_cfg(V=2048):
    """One layer at the d20 width (1280 columns: the embedding backward's
    three 512-column groups per lane, as in the benchmarked step) with a
    small vocabulary, so that Zipf ids give long runs of one id across many
    chunks of sorted entries as well as ids seen once."""
    c = _lib.gpt_config_from_depth(20, _lib.GPT_BF16)
    c.n_layer = 1
    c.vocab_size = V
    return c


def check_embedding_rows(case, gpu, G, label):
    """The embedding gradient row by row: rows of ids absent from the batch
    exactly zero, every present id's row within cosine 0.99 of the oracle
    (rows of ids seen once carry one position's contribution, so a lost,
    doubled or misplaced entry of the sorted sums fails here even where the
    whole tensor's cosine would hide it)."""
    gg = U.split_tensors(case, gpu["grads"])["wte"]
    go = U.split_tensors(case, case.flat_grads(G))["wte"]
    present = np.zeros(case.cfg.vocab_size, dtype=bool)
    present[case.idx.ravel()] = True
    assert np.all(go[~present] == 0.0)
    assert np.all(gg[~present] == 0.0), f"{label}: nonzero rows for absent ids"
    na = np.linalg.norm(gg[present], axis=1)
    nb = np.linalg.norm(go[present], axis=1)
    cos = np.einsum("ij,ij->i", gg[present], go[present]) / np.maximum(na * nb, 1e-300)
    U.log(f"[{label}] {present.sum()} present ids, worst row cosine {cos.min():.5f}")
    assert cos.min() >= 0.99


@pytest.mark.parametrize("T", [333, 512])
def test_embedding_gradient_rows_zipf(T):
    """The embedding backward at the d20 width on Zipf ids, row by row
    against the oracle: a ragged count of sorted entries (T = 333, B = 3:
    999 entries, the last chunk partly filled) and a whole number of chunks
    (T = 512); then a second step on the same model with other ids, whose
    absent rows must come back zero (nothing kept from the first step)."""
    U.require_gpu()
    import torch
    c = wide_one_layer_cfg()
    case = U.Case(c, B=3, T=T, law="zipf", wseed=21, tseed=22)
    U.log(f"case 1-layer width 1280 V=2048 bf16 B=3 T={T} zipf: embedding rows")
    gpu = U.run_gpu(case)
    assert gpu["status"] == _lib.GPT_OK
    loss, rows, G = O.step(U.oracle_cfg(c), case.oracle_params(), case.idx, case.tgt)
    check_bf16(case, gpu, loss, G, f"emb-rows-T{T}")
    check_embedding_rows(case, gpu, G, f"emb-rows-T{T}")
    # second step, same model, uniform ids over the upper half of the vocabulary
    rng = np.random.default_rng(23)
    seq = rng.integers(c.vocab_size // 2, c.vocab_size, size=(3, T + 1)).astype(np.int32)
    case.idx, case.tgt = np.ascontiguousarray(seq[:, :T]), np.ascontiguousarray(seq[:, 1:])
    m = gpu["model"]
    m.forward_loss(torch.from_numpy(case.idx).cuda(), torch.from_numpy(case.tgt).cuda(), need_grad=True)
    m.backward(1.0, False)
    torch.cuda.synchronize()
    assert m.sync_status() == _lib.GPT_OK
    gpu2 = dict(grads=m.grads.cpu().numpy().astype(np.float64))
    _, _, G2 = O.step(U.oracle_cfg(c), case.oracle_params(), case.idx, case.tgt)
    check_embedding_rows(case, gpu2, G2, f"emb-rows-T{T}-second")
