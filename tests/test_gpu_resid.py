"""Residual scalars (resid_lambdas, x0_lambdas) and value embeddings against
the float64 oracle, through the C ABI, with the tolerances of the model's
dtype (fp32: loss rel 1e-5, gradient rel-L2 1e-4; bf16: loss rel 5e-3,
gradient cosine 0.999)."""
import numpy as np
import pytest

from decoder_only_transformer_gpt_amd import _lib, synthetic
from oracle import gpt_oracle as O

import gpu_util as U
from test_gpu_parity import check_bf16, check_fp32, d4_cfg, tiny_cfg

pytestmark = pytest.mark.gpu


def with_options(c, lambdas=1, ve=1):
    c.x0_lambdas = lambdas
    c.value_embeds = ve
    return c


def test_tiny_fp32_lambdas_and_value_embeds_ragged():
    """fp32, three layers (value embeddings on layers 0 and 2), ragged T."""
    U.require_gpu()
    c = with_options(tiny_cfg(T=100))
    c.n_layer = 3
    case = U.Case(c, B=2, T=77, law="uniform", wseed=21, tseed=22)
    U.log("case tiny fp32 L3 B=2 T=77 lambdas + value embeddings")
    gpu = U.run_gpu(case)
    assert gpu["status"] == _lib.GPT_OK
    loss, rows, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    np.testing.assert_allclose(gpu["row_loss"], rows.reshape(-1), rtol=2e-5)
    check_fp32(case, gpu, loss, G, "tiny-lam-ve")


@pytest.mark.parametrize("tile", [0, 3])
def test_bf16_lambdas_and_value_embeds_zipf_ragged(tile):
    """bf16 d4 with both options, Zipf ids (repeated rows in the value-embedding
    gradient), ragged T, and gradient accumulation over two steps."""
    torch = U.require_gpu()
    c = with_options(d4_cfg())
    case = U.Case(c, B=3, T=333, law="zipf", wseed=23, tseed=24)
    U.log(f"case d4 bf16 B=3 T=333 zipf lambdas + value embeddings, tile {tile}, accumulate")
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
    loss, _, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt, dloss=2.0)
    gpu = dict(loss=float(m.loss.item()), grads=m.grads.cpu().numpy().astype(np.float64))
    check_bf16(case, gpu, loss, G, "d4-lam-ve")


def test_neutral_scalars_and_zero_gates_equal_the_plain_model():
    """resid_lambdas = 1, x0_lambdas = 0 and zero gates reproduce the plain
    model bit for bit (loss and every shared gradient), and leave the tables'
    gradients at zero. A model with the residual scalars keeps the residual
    gradient in fp32, so the plain model runs with that option too."""
    U.require_gpu()
    plain = U.Case(d4_cfg(), B=2, T=256, law="zipf", wseed=25, tseed=26)
    opt = U.Case(with_options(d4_cfg()), B=2, T=256, law="zipf", wseed=25, tseed=26)
    storage = opt.storage.copy()
    names = {n: (o, r * cc) for n, o, r, cc in _lib.gpt_param_layout(opt.cfg)}
    one, zero = synthetic.f32_to_bf16_bits(np.array([1.0, 0.0], np.float32))
    o, n = names["resid_lambdas"]; storage[o:o + n] = one
    o, n = names["x0_lambdas"]; storage[o:o + n] = zero
    o, n = names["ve_gates"]; storage[o:o + n] = zero
    # shared tensors must hold the same values in both cases
    p_names = {n: (o, r * cc) for n, o, r, cc in _lib.gpt_param_layout(plain.cfg)}
    for k, (o, n) in p_names.items():
        storage[names[k][0]:names[k][0] + n] = plain.storage[o:o + n]
    g_opt = U.run_gpu(opt, params_override=storage)
    g_plain = U.run_gpu(plain, resid_grad_f32=True)
    assert g_opt["loss"] == g_plain["loss"]
    for k, (o, n) in p_names.items():
        np.testing.assert_array_equal(g_opt["grads"][names[k][0]:names[k][0] + n], g_plain["grads"][o:o + n],
                                      err_msg=k)
    o, n = names["h0.ve"]
    assert not g_opt["grads"][o:o + n].any()


@pytest.mark.timeout(900)
def test_d20_lambdas_and_value_embeds_one_row():
    """The d20 shape with both options, one 2,048-token Zipf row."""
    U.require_gpu()
    c = with_options(_lib.gpt_config_from_depth(20, _lib.GPT_BF16))
    case = U.Case(c, B=1, T=2048, law="zipf")
    U.log("case d20 bf16 B=1 T=2048 zipf lambdas + value embeddings")
    gpu = U.run_gpu(case)
    assert gpu["status"] == _lib.GPT_OK
    loss, rows, G = O.step(U.oracle_cfg(case.cfg), case.oracle_params(), case.idx, case.tgt)
    check_bf16(case, gpu, loss, G, "d20-lam-ve-B1")
