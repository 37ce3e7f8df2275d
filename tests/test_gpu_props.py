"""Structural properties of the HIP step that hold exactly (bitwise) or in
closed form, independent of the oracle's values."""
import math

import numpy as np
import pytest

from decoder_only_transformer_gpt_amd import _lib

import gpu_util as U

pytestmark = pytest.mark.gpu


def _model(case, max_B=None, max_T=None, storage=None):
    torch = U.require_gpu()
    from decoder_only_transformer_gpt_amd.model import GPT
    return torch, GPT(case.cfg, GPT.params_from_numpy(case.storage if storage is None else storage, case.cfg),
                      max_B or case.B, max_T or case.T)


def _step(torch, m, idx, tgt, rows=True):
    rl = torch.zeros(idx.numel(), dtype=torch.float32, device="cuda")
    m.forward_loss(idx, tgt, row_loss=rl)
    m.backward(1.0)
    torch.cuda.synchronize()
    return rl.cpu().numpy(), m.grads.cpu().numpy().copy()


def d4_case(**kw):
    return U.Case(_lib.gpt_config_from_depth(4, _lib.GPT_BF16), **kw)


def test_bitwise_deterministic():
    case = d4_case(B=2, T=512, law="zipf")
    U.log("case d4 B=2 T=512 determinism")
    torch, m = _model(case)
    idx, tgt = torch.from_numpy(case.idx).cuda(), torch.from_numpy(case.tgt).cuda()
    r1, g1 = _step(torch, m, idx, tgt)
    r2, g2 = _step(torch, m, idx, tgt)
    assert np.array_equal(r1, r2)
    assert np.array_equal(g1, g2)


def test_causality_bitwise():
    case = d4_case(B=2, T=300, law="uniform")
    U.log("case d4 B=2 T=300 causality")
    torch, m = _model(case)
    idx, tgt = torch.from_numpy(case.idx).cuda(), torch.from_numpy(case.tgt).cuda()
    r1, _ = _step(torch, m, idx, tgt)
    idx2 = case.idx.copy()
    t = 170
    idx2[1, t] = (idx2[1, t] + 12345) % case.cfg.vocab_size
    r2, _ = _step(torch, m, torch.from_numpy(idx2).cuda(), tgt)
    r1, r2 = r1.reshape(2, 300), r2.reshape(2, 300)
    assert np.array_equal(r1[0], r2[0])
    assert np.array_equal(r1[1, :t], r2[1, :t])
    assert not np.array_equal(r1[1, t:], r2[1, t:])


def test_batch_rows_independent_bitwise():
    case = d4_case(B=3, T=256, law="uniform")
    U.log("case d4 B=3 T=256 row permutation")
    torch, m = _model(case)
    idx, tgt = torch.from_numpy(case.idx).cuda(), torch.from_numpy(case.tgt).cuda()
    r1, _ = _step(torch, m, idx, tgt)
    perm = [2, 0, 1]
    r2, _ = _step(torch, m, idx[perm].contiguous(), tgt[perm].contiguous())
    assert np.array_equal(r1.reshape(3, 256)[perm], r2.reshape(3, 256))


@pytest.mark.parametrize("dtype", [_lib.GPT_F32, _lib.GPT_BF16])
def test_zero_lm_head_closed_form(dtype):
    """W_lm = 0: loss = ln V, dW_lm = ((1/V - onehot)^T h_f)/N, every other gradient exactly 0."""
    c = _lib.gpt_config_from_depth(4, dtype)
    c.vocab_size = 4096
    case = U.Case(c, B=2, T=128, law="uniform")
    U.log(f"case zero lm head dtype={dtype}")
    off = [o for n, o, r, cc in _lib.gpt_param_layout(c) if n == "lm_head"][0]
    st = case.storage.copy()
    st[off:] = 0
    torch, m = _model(case, storage=st)
    idx, tgt = torch.from_numpy(case.idx).cuda(), torch.from_numpy(case.tgt).cuda()
    m.forward_loss(idx, tgt)
    m.backward(1.0)
    torch.cuda.synchronize()
    assert float(m.loss.item()) == pytest.approx(math.log(4096), rel=1e-6)
    g = m.grads.cpu().numpy()
    assert np.all(g[:off] == 0.0)
    N, V, C = 256, 4096, c.model_dim
    es = np.float32 if dtype == _lib.GPT_F32 else np.uint16
    hf = m.debug_tensor("hf", 0, (N, C), torch.float32 if dtype == _lib.GPT_F32 else torch.bfloat16)
    hf = hf.float().cpu().numpy().astype(np.float64)
    onehot = np.zeros((N, V))
    onehot[np.arange(N), case.tgt.reshape(-1)] = 1.0
    expect = (np.full((N, V), 1.0 / V) - onehot).T @ hf / N
    got = g[off:].reshape(V, C)
    assert U.rel_l2(got, expect) < (1e-5 if dtype == _lib.GPT_F32 else 1e-2)


def test_bad_token_sets_device_flag_and_nan_loss():
    case = d4_case(B=1, T=64, law="uniform")
    U.log("case bad token id")
    torch, m = _model(case)
    idx = case.idx.copy()
    idx[0, 5] = case.cfg.vocab_size + 3
    m.forward_loss(torch.from_numpy(idx).cuda(), torch.from_numpy(case.tgt).cuda())
    torch.cuda.synchronize()
    assert math.isnan(float(m.loss.item()))
    assert m.sync_status() == _lib.GPT_E_DEVICE


def test_backward_without_forward_is_a_state_error():
    case = d4_case(B=1, T=64, law="uniform")
    torch, m = _model(case)
    with pytest.raises(_lib.GptError) as e:
        m.backward(1.0)
    assert e.value.status == _lib.GPT_E_STATE
    idx, tgt = torch.from_numpy(case.idx).cuda(), torch.from_numpy(case.tgt).cuda()
    m.forward_loss(idx, tgt, need_grad=False)
    with pytest.raises(_lib.GptError):
        m.backward(1.0)
    m.forward_loss(idx, tgt, need_grad=True)
    m.backward(1.0)
    with pytest.raises(_lib.GptError):   # the stash is consumed
        m.backward(1.0)
    torch.cuda.synchronize()
    assert m.sync_status() == _lib.GPT_OK
