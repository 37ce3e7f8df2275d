"""FP8 (e4m3) models and the per-tensor quantiser, through the C ABI, against
the float64 oracle's FP8 reading (per-tensor current scaling, round to nearest
even with saturation, output gradients quantised, straight-through backward).

Quantiser: codes bit-exact, amax exact (both sides decide the code from the
bf16 operand in fp32). Matmul on the same codes: fp32 accumulation, checked
elementwise against the float64 product of the dequantised codes.

Whole step, against the oracle's FP8 step (O8) and, as the yardstick, the
oracle's unquantised step (O0): |dloss|/loss <= 5e-3, and for every gradient
tensor
  * rel(GPU, O8) <= rel(O0, O8): the GPU sits within the FP8 recipe's own
    quantisation distance of O8, and
  * rel(GPU, O8) < rel(GPU, O0): it is nearer the FP8 recipe than the
    unquantised model (so it does quantise, and quantises the same operands).
Why these and not a fixed bar: the GPU and the oracle feed the quantiser
slightly different values (the bf16 pipeline's own differences eps), and
e4m3's step (1/8..1/16 of the value) turns a difference eps into a code flip
with probability ~12 eps, i.e. dequantised operands apart by ~sqrt(eps/12)
RMS, against the full rounding noise of ~1/(12 sqrt 3) that separates O8
from O0; the flips also compound layer by layer through the backward, so a
fixed cosine bar that holds at depth 4 (0.996, derived from the bf16 bar's
eps of 4.5 %, checked there too) does not carry to depth 24."""
import numpy as np
import pytest

from decoder_only_transformer_gpt_amd import _lib, synthetic
from oracle import gpt_oracle as O

import gpu_util as U
pytestmark = pytest.mark.gpu

FP8_COS_D4 = 0.996


def oracle_fp8_and_unquantised(case, dloss=1.0):
    oc = U.oracle_cfg(case.cfg)
    P = case.oracle_params()
    l8, _, G8 = O.step(oc, P, case.idx, case.tgt, dloss=dloss)
    l0, _, G0 = O.step(dict(oc, fp8=False), P, case.idx, case.tgt, dloss=dloss)
    return l8, G8, G0


def check_fp8(case, gpu, loss8, G8, G0, label, cos_bar=None):
    rel = abs(gpu["loss"] - loss8) / abs(loss8)
    U.log(f"[{label}] loss gpu={gpu['loss']:.6f} oracle={loss8:.6f} rel={rel:.2e}")
    assert rel <= 5e-3
    gg = U.split_tensors(case, gpu["grads"])
    g8 = U.split_tensors(case, case.flat_grads(G8))
    g0 = U.split_tensors(case, case.flat_grads(G0))
    worst = (0.0, "")
    for k in g8:
        r_g8, r_g0, r_08 = U.rel_l2(gg[k], g8[k]), U.rel_l2(gg[k], g0[k]), U.rel_l2(g0[k], g8[k])
        worst = max(worst, (r_g8 / r_08, k))
        assert r_g8 <= r_08, (k, r_g8, r_08)
        assert r_g8 < r_g0, (k, r_g8, r_g0)
        if cos_bar is not None:
            assert U.cosine(gg[k], g8[k]) >= cos_bar, k
    U.log(f"[{label}] worst rel(GPU, O8) / rel(O0, O8) = {worst[0]:.3f} ({worst[1]})")


def fp8_cfg(depth=4):
    return _lib.gpt_config_from_depth(depth, _lib.GPT_FP8_E4M3)


def _bf16_tensor(rng, rows, cols, scale):
    bits = synthetic.f32_to_bf16_bits((rng.standard_normal((rows, cols)) * scale).astype(np.float32))
    return bits, synthetic.bf16_bits_to_f32(bits)


def _quantize_gpu(torch, bits, ldT):
    rows, cols = bits.shape
    x = torch.from_numpy(bits.view(np.int16)).cuda()
    q = torch.full((max(rows, 1), cols), 0x55, dtype=torch.uint8, device="cuda")
    qT = torch.full((cols, max(ldT, 1)), 0x55, dtype=torch.uint8, device="cuda")
    amax = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    _lib.gpt_fp8_quantize(x.data_ptr(), rows, cols, q.data_ptr(), qT.data_ptr(), ldT, amax.data_ptr(), stream)
    torch.cuda.synchronize()
    return q.cpu().numpy()[:rows], qT.cpu().numpy(), float(amax.item())


@pytest.mark.parametrize("rows,cols,scale,ldT", [(999, 1536, 1.0, 1024), (64, 16, 3e-3, 64), (1, 32, 50.0, 16),
                                                 (130, 6144, 0.02, 256), (2048, 1664, 7.0, 2048)])
def test_quantize_bit_exact(rows, cols, scale, ldT):
    torch = U.require_gpu()
    rng = np.random.default_rng(rows * 7 + cols)
    bits, vals = _bf16_tensor(rng, rows, cols, scale)
    U.log(f"case fp8 quantize rows={rows} cols={cols} scale={scale} ldT={ldT}")
    q, qT, amax = _quantize_gpu(torch, bits, ldT)
    codes, s = O.fp8_quantize(vals)
    assert amax == float(np.max(np.abs(vals)))
    np.testing.assert_array_equal(q, codes)
    np.testing.assert_array_equal(qT[:, :rows], codes.T)
    assert not qT[:, rows:ldT].any()


def test_quantize_ties_saturation_and_zero():
    """Values that land exactly on e4m3 midpoints (ties to even), the largest
    magnitude (448 after scaling), tiny values in the subnormal range, and an
    all-zero tensor (scale 1, zero codes)."""
    torch = U.require_gpu()
    grid = O.e4m3_decode(np.arange(0x7F))
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)        # exact in bf16 (<= 4 mantissa bits)
    vals = np.concatenate([mids, -mids, grid.astype(np.float32), [448.0], np.zeros(1, np.float32)])
    vals = np.resize(vals, 32 * 16).reshape(32, 16).astype(np.float32)
    vals[0, 0] = -448.0                                            # amax 448: s = 1 exactly
    bits = synthetic.f32_to_bf16_bits(vals)
    assert np.array_equal(synthetic.bf16_bits_to_f32(bits), vals)
    q, qT, amax = _quantize_gpu(torch, bits, 32)
    codes, s = O.fp8_quantize(vals)
    assert s == 1.0 and amax == 448.0
    np.testing.assert_array_equal(q, codes)
    np.testing.assert_array_equal(qT, codes.T)
    zq, zqT, zam = _quantize_gpu(torch, np.zeros((16, 32), np.uint16), 16)
    assert zam == 0.0 and not zq.any() and not zqT.any()


def _codes(torch, vals_bits, ldT=16):
    """Quantise a bf16 tensor on the GPU; returns (device codes, device amax)."""
    rows, cols = vals_bits.shape
    x = torch.from_numpy(vals_bits.view(np.int16)).cuda()
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    amax = torch.empty((1,), dtype=torch.float32, device="cuda")
    _lib.gpt_fp8_quantize(x.data_ptr(), rows, cols, q.data_ptr(), None, 0, amax.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    return q, amax


@pytest.mark.parametrize("M,N,K,out,tile,splits", [
    (999, 1536, 1024, "bf16", 0, 1), (999, 1536, 1024, "bf16", 1, 1), (999, 1536, 1024, "bf16", 2, 1),
    (999, 1536, 1024, "bf16", 3, 1), (300, 260, 384, "f32", 3, 1), (1536, 768, 4096, "f32", 1, 4),
    (640, 512, 2048, "f32", 0, 3), (33, 64, 128, "bf16", 0, 1),
    # bf16 output with N % 8 == 4: the epilogue's 4-column form (8-column
    # items would straddle the last column)
    (300, 260, 384, "bf16", 3, 1), (999, 1540, 1024, "bf16", 1, 1),
    # more 256x256 tiles than compute units, an odd K tile count
    (4500, 4224, 384, "bf16", 1, 1), (2100, 8448, 640, "f32", 1, 1)])
def test_fp8_matmul_on_identical_codes(M, N, K, out, tile, splits):
    """The e4m3 GEMM against the float64 product of the same dequantised codes
    (the oracle's codes equal the GPU's: checked bit for bit above), ragged M
    and N, every tile variant, split-K. Bound per element: the fp32
    accumulation, held to 2^-16 of sum |a b| (K-term fp32 summation could reach
    K * 2^-24 of it in the worst case; normal data stays far below), plus the
    bf16 output rounding (half an ulp: 2^-8 |ref|)."""
    torch = U.require_gpu()
    rng = np.random.default_rng(M + N + K)
    ab, av = _bf16_tensor(rng, M, K, 1.0)
    bb, bv = _bf16_tensor(rng, N, K, 0.05)
    qa, am_a = _codes(torch, ab)
    qb, am_b = _codes(torch, bb)
    odt = torch.float32 if out == "f32" else torch.bfloat16
    o = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    part = torch.empty((splits, M, N), dtype=torch.float32, device="cuda") if splits > 1 else None
    U.log(f"case fp8 matmul M={M} N={N} K={K} out={out} tile={tile} splits={splits}")
    _lib.gpt_fp8_matmul(qa.data_ptr(), K, am_a.data_ptr(), qb.data_ptr(), K, am_b.data_ptr(), M, N, K,
                        _lib.GPT_F32 if out == "f32" else _lib.GPT_BF16, o.data_ptr(), N, tile, splits,
                        None if part is None else part.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().astype(np.float64)
    ca, sa = O.fp8_quantize(av)
    cb, sb = O.fp8_quantize(bv)
    np.testing.assert_array_equal(qa.cpu().numpy(), ca)
    da, db = O.fp8_dequantize(ca, sa), O.fp8_dequantize(cb, sb)
    ref = da @ db.T
    mag = np.abs(da) @ np.abs(db).T
    bound = 2.0 ** -16 * mag + (2.0 ** -8 * np.abs(ref) if out == "bf16" else 0.0)
    err = np.abs(got - ref)
    U.log(f"[fp8-matmul] max err / sum|ab| = {np.max(err / np.maximum(mag, 1e-30)):.2e}, "
          f"max err / bound = {np.max(err / np.maximum(bound, 1e-300)):.3f}")
    assert np.all(err <= bound)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,N,K,out,splits", [
    (32768, 1792, 1536, "bf16", 1),     # d24 QKV forward (B=16 x T=2048 tokens)
    (32768, 1536, 6144, "bf16", 1),     # d24 W2 forward / W1 dX
    (6144, 1536, 32768, "f32", 4)])     # d24 W1 dW: tokens on K, split-K
def test_fp8_d24_shapes_quantise_and_matmul(M, N, K, out, splits):
    """Quantise -> e4m3 GEMM at the d24 FP8 model's own shapes, under the
    kernel-level bars: the GPU's codes of both operands equal the oracle's bit
    for bit (checked on 256 seeded rows of A and all of B), and 256 seeded
    output rows lie within the fp32-accumulation bound of the float64 product
    of the same dequantised codes (plus half a bf16 ulp for bf16 output).
    These bars hold at any depth; the whole-step d24 comparison below is a
    sanity check of the assembled step."""
    torch = U.require_gpu()
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    U.log(f"case fp8 d24 shape M={M} N={N} K={K} out={out} splits={splits}")
    ab, av = _bf16_tensor(rng, M, K, 1.0)
    bb, bv = _bf16_tensor(rng, N, K, 0.05)
    qa, am_a = _codes(torch, ab)
    qb, am_b = _codes(torch, bb)
    odt = torch.float32 if out == "f32" else torch.bfloat16
    o = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    part = torch.empty((splits, M, N), dtype=torch.float32, device="cuda") if splits > 1 else None
    _lib.gpt_fp8_matmul(qa.data_ptr(), K, am_a.data_ptr(), qb.data_ptr(), K, am_b.data_ptr(), M, N, K,
                        _lib.GPT_F32 if out == "f32" else _lib.GPT_BF16, o.data_ptr(), N, 0, splits,
                        None if part is None else part.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(M, size=256, replace=False))
    # the oracle's scale from the whole tensor's |max|, its codes on the sampled rows
    sa = np.float32(448.0) / np.float32(np.abs(av).max())
    sb = np.float32(448.0) / np.float32(np.abs(bv).max())
    assert float(am_a.item()) == float(np.abs(av).max()) and float(am_b.item()) == float(np.abs(bv).max())
    ca = O.e4m3_encode((av[rows] * sa).astype(np.float32))
    cb, sb_o = O.fp8_quantize(bv)
    assert np.float32(sb_o) == sb
    np.testing.assert_array_equal(qa.cpu().numpy()[rows], ca)
    np.testing.assert_array_equal(qb.cpu().numpy(), cb)
    da, db = O.fp8_dequantize(ca, sa), O.fp8_dequantize(cb, sb)
    ref = da @ db.T
    mag = np.abs(da) @ np.abs(db).T
    got = o.float().cpu().numpy()[rows].astype(np.float64)
    bound = 2.0 ** -16 * mag + (2.0 ** -8 * np.abs(ref) if out == "bf16" else 0.0)
    err = np.abs(got - ref)
    U.log(f"[fp8-d24] max err / bound = {np.max(err / np.maximum(bound, 1e-300)):.3f}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("tile", [0, 1, 2, 3])
def test_d4_fp8_full_step(tile):
    U.require_gpu()
    case = U.Case(fp8_cfg(), B=4, T=512, law="uniform")
    U.log(f"case d4 fp8 B=4 T=512 uniform gemm tile {tile}")
    gpu = U.run_gpu(case, tile=tile)
    assert gpu["status"] == _lib.GPT_OK
    l8, G8, G0 = oracle_fp8_and_unquantised(case)
    check_fp8(case, gpu, l8, G8, G0, "d4-fp8", cos_bar=FP8_COS_D4)


@pytest.mark.parametrize("tile", [0, 3])
def test_fp8_ragged_zipf_accumulate(tile):
    """Ragged token count (N = 999: the token-major codes are padded to 1,024),
    Zipf ids, and gradient accumulation over two identical steps."""
    torch = U.require_gpu()
    case = U.Case(fp8_cfg(), B=3, T=333, law="zipf", wseed=2, tseed=3)
    U.log(f"case d4 fp8 ragged B=3 T=333 zipf gemm tile {tile}, accumulate")
    from decoder_only_transformer_gpt_amd.model import GPT
    m = GPT(case.cfg, GPT.params_from_numpy(case.storage, case.cfg), 3, 333)
    if tile:
        m.set_gemm_tile(tile)
    idx, tgt = torch.from_numpy(case.idx).cuda(), torch.from_numpy(case.tgt).cuda()
    m.forward_loss(idx, tgt)
    m.backward(0.5, accumulate=False)
    m.forward_loss(idx, tgt)
    m.backward(1.5, accumulate=True)
    torch.cuda.synchronize()
    assert m.sync_status() == _lib.GPT_OK
    l8, G8, G0 = oracle_fp8_and_unquantised(case, dloss=2.0)
    gpu = dict(loss=float(m.loss.item()), grads=m.grads.cpu().numpy().astype(np.float64))
    check_fp8(case, gpu, l8, G8, G0, "d4-fp8-ragged", cos_bar=FP8_COS_D4)


@pytest.mark.parametrize("B,T", [(2, 256), (128, 512)])
def test_fp8_amax_slots_and_differs_from_bf16(B, T):
    """The |max| slots hold exactly the maxima of the bf16 operands: the
    activations against the debug buffers, the layer-0 gradients du and dqkv
    after the backward, and the weights against the seeded values. B = 128
    gives the dK/dV kernel one key block per block, B = 2 the head-split form
    (dV through the combine pass). At B = 2, FP8 also changes the result
    relative to the bf16 model on the same inputs."""
    torch = U.require_gpu()
    case = U.Case(fp8_cfg(), B=B, T=T, law="uniform", wseed=4, tseed=5)
    gpu = U.run_gpu(case, max_B=B, max_T=T)
    m = gpu["model"]
    C, F, N = case.cfg.model_dim, case.cfg.mlp_dim, B * T
    HD, QKV = case.cfg.n_head * 128, (case.cfg.n_head + 2) * 128
    P = case.oracle_params()
    for l in range(case.cfg.n_layer):
        am = m.debug_tensor("amax", l, (16,), torch.float32).cpu().numpy()
        for k, (nm, cols) in enumerate([("h1", C), ("o", HD), ("h2", C), ("a", F)]):
            x = m.debug_tensor(nm, l, (N, cols), torch.bfloat16).float().cpu().numpy()
            assert am[k] == np.abs(x).max(), (l, nm)
        if l == 0:  # the gradients of the last layer the backward processed
            du = m.debug_tensor("du", 0, (N, F), torch.bfloat16).float().cpu().numpy()
            dqkv = m.debug_tensor("dqkv", 0, (N, QKV), torch.bfloat16).float().cpu().numpy()
            assert am[5] == np.abs(du).max() and am[7] == np.abs(dqkv).max()
        for k, w in enumerate(["w_qkv", "w_o", "w_1", "w_2"]):
            assert am[8 + k] == np.abs(P[f"h{l}.{w}"]).max()
        assert np.all(am[:12] > 0) and np.all(np.isfinite(am))
    if B != 2:
        return
    bf = U.Case(_lib.gpt_config_from_depth(4, _lib.GPT_BF16), B=2, T=256, law="uniform", wseed=4, tseed=5)
    g_bf = U.run_gpu(bf)
    assert gpu["loss"] != g_bf["loss"] and abs(gpu["loss"] - g_bf["loss"]) / g_bf["loss"] < 1e-2


@pytest.mark.timeout(900)
def test_d24fp8_one_row():
    """The FP8 configuration's shape (d24: width 1536, 12 heads, MLP 6144), one
    2,048-token row, the whole step against the oracle."""
    U.require_gpu()
    case = U.Case(fp8_cfg(24), B=1, T=2048, law="zipf")
    U.log("case d24 fp8 B=1 T=2048 zipf")
    gpu = U.run_gpu(case)
    assert gpu["status"] == _lib.GPT_OK
    l8, G8, G0 = oracle_fp8_and_unquantised(case)
    check_fp8(case, gpu, l8, G8, G0, "d24-fp8-B1")


@pytest.mark.timeout(900)
def test_d24fp8_full_batch():
    """The FP8 configuration at its full batch (B=16, T=2048): finite loss and
    gradients, loss = mean of the per-position losses, and two sampled rows'
    mean losses within the quantisation noise (rel 1e-2) of the oracle's
    unquantised forward of just those rows (per-tensor scales couple the rows,
    so the unquantised forward is the row-local reference)."""
    U.require_gpu()
    c = fp8_cfg(24)
    case = U.Case(c, B=16, T=2048, law="zipf")
    U.log("case d24 fp8 B=16 T=2048 zipf (full batch)")
    gpu = U.run_gpu(case)
    assert gpu["status"] == _lib.GPT_OK
    assert np.isfinite(gpu["loss"]) and np.all(np.isfinite(gpu["grads"]))
    rows_gpu = gpu["row_loss"].reshape(16, 2048)
    assert gpu["loss"] == pytest.approx(rows_gpu.mean(), rel=1e-5)
    ocfg = dict(U.oracle_cfg(c), fp8=False)
    P = case.oracle_params()
    for b in (int(np.random.default_rng(8).integers(0, 16)), 15):
        r = O.forward_rows(ocfg, P, case.idx[b:b + 1], case.tgt[b:b + 1])[0]
        rel = abs(rows_gpu[b].mean() - r.mean()) / r.mean()
        U.log(f"[d24-fp8-B16] row {b}: mean loss gpu={rows_gpu[b].mean():.5f} unquantised oracle={r.mean():.5f} "
              f"rel={rel:.2e}")
        assert rel <= 1e-2


def test_d4_fp8_with_lambdas_and_value_embeds():
    """FP8 products together with the residual scalars and value embeddings
    (the lookup adds to the bf16 v after the e4m3 QKV product)."""
    U.require_gpu()
    c = fp8_cfg()
    c.x0_lambdas, c.value_embeds = 1, 1
    case = U.Case(c, B=2, T=512, law="zipf", wseed=27, tseed=28)
    U.log("case d4 fp8 B=2 T=512 lambdas + value embeddings")
    gpu = U.run_gpu(case)
    assert gpu["status"] == _lib.GPT_OK
    l8, G8, G0 = oracle_fp8_and_unquantised(case)
    check_fp8(case, gpu, l8, G8, G0, "d4-fp8-lam-ve", cos_bar=FP8_COS_D4)
