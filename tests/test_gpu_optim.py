"""The optimiser step (Muon for the blocks' matrices, AdamW for the rest, fp32
masters cast into the model's parameters) against the float64 oracle.

Inputs are seeded on both sides: masters, gradients (written into the
handle's gradient buffer) and a zero state; two steps with different
gradients and momenta. Tolerances: AdamW tensors and all states are fp32
elementwise arithmetic (rel-L2 1e-5); Muon updates take the model's dtype in
the Newton-Schulz products, so their update w_new - w_old is held to the
stated tolerance of that dtype (fp32: rel-L2 1e-4; bf16: cosine 0.999). The
model's parameters must equal the cast of the GPU's masters bit for bit."""
import numpy as np
import pytest

from decoder_only_transformer_gpt_amd import _lib, synthetic
from oracle import gpt_oracle as O

import gpu_util as U

pytestmark = pytest.mark.gpu


def opt_config(momentum, coeffs=(1.5, -0.5, 0.0), steps=5):
    oc = _lib.gpt_optim_config()
    oc.lr_muon, oc.lr_embed, oc.lr_unembed, oc.lr_scalar = 0.02, 0.3, 0.004, 0.5
    oc.momentum = momentum
    oc.beta1, oc.beta2, oc.eps = 0.8, 0.95, 1e-10
    oc.wd_muon, oc.wd_adamw = 0.1, 0.01
    oc.ns_steps = steps
    oc.ns_a, oc.ns_b, oc.ns_c = coeffs
    return oc


def cfg_with_options(depth, dtype):
    c = _lib.gpt_config_from_depth(depth, dtype)
    if dtype == _lib.GPT_F32:
        c.vocab_size, c.max_seq_len = 512, 64
    c.x0_lambdas, c.value_embeds = 1, 1
    return c


@pytest.mark.parametrize("which,coeffs", [("tiny-f32", (1.5, -0.5, 0.0)), ("d4-bf16", (1.5, -0.5, 0.0)),
                                          ("d4-bf16", (1.875, -1.25, 0.375)), ("d4-fp8", (1.5, -0.5, 0.0))])
def test_optimizer_two_steps_match_oracle(which, coeffs):
    torch = U.require_gpu()
    dtype = {"tiny-f32": _lib.GPT_F32, "d4-bf16": _lib.GPT_BF16, "d4-fp8": _lib.GPT_FP8_E4M3}[which]
    c = cfg_with_options(2 if which == "tiny-f32" else 4, dtype)
    layout = _lib.gpt_param_layout(c)
    shapes = [(n, r, cc) for n, _, r, cc in layout]
    U.log(f"case optimiser {which} coefficients {coeffs}")
    _, master0 = synthetic.make_weights(shapes, seed=31, dtype="f32")
    storage, _ = synthetic.make_weights(shapes, seed=31, dtype="f32" if dtype == _lib.GPT_F32 else "bf16")
    g_vals = [synthetic.make_weights(shapes, seed=s, dtype="f32", std=1e-3)[1] for s in (32, 33)]
    from decoder_only_transformer_gpt_amd.model import GPT
    m = GPT(c, GPT.params_from_numpy(storage, c), 1, 64)
    master = torch.from_numpy(master0.copy()).cuda()
    state = torch.zeros(_lib.gpt_optimizer_state_elems(c), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    oracle_w = {n: master0[o:o + r * cc].reshape(r, cc).astype(np.float64) for n, o, r, cc in layout}
    oracle_s = {}
    ocd = None
    for t, (g, mu) in enumerate(zip(g_vals, (0.85, 0.95)), start=1):
        m.grads.copy_(torch.from_numpy(g))
        oc = opt_config(mu, coeffs)
        _lib.gpt_optimizer_step(m.h, oc, master.data_ptr(), state.data_ptr(), t, stream)
        grads = {n: g[o:o + r * cc].reshape(r, cc).astype(np.float64) for n, o, r, cc in layout}
        ocd = oc.as_dict()
        prev = oracle_w
        oracle_w, oracle_s = O.optimizer_step(c.as_dict(), ocd, oracle_w, grads, oracle_s, t)
    torch.cuda.synchronize()
    got = master.cpu().numpy().astype(np.float64)
    st = state.cpu().numpy().astype(np.float64)
    soff = 0
    worst = (1.0, "")
    for n, o, r, cc in layout:
        w_gpu = got[o:o + r * cc].reshape(r, cc)
        if O.optimizer_group(n) == "muon":
            d_gpu, d_or = w_gpu - prev[n], oracle_w[n] - prev[n]
            worst = min(worst, (U.cosine(d_gpu, d_or), n))
            if dtype == _lib.GPT_F32:
                assert U.rel_l2(d_gpu, d_or) <= 1e-4, n
            else:
                assert U.cosine(d_gpu, d_or) >= 0.999, n
            assert U.rel_l2(st[soff:soff + r * cc].reshape(r, cc), oracle_s[n]["u"]) <= 1e-5, n
            soff += r * cc
        else:
            assert U.rel_l2(w_gpu, oracle_w[n]) <= 1e-5, n
            assert U.rel_l2(st[soff:soff + r * cc].reshape(r, cc), oracle_s[n]["m"]) <= 1e-5, n
            assert U.rel_l2(st[soff + r * cc:soff + 2 * r * cc].reshape(r, cc), oracle_s[n]["v"]) <= 1e-5, n
            soff += 2 * r * cc
    assert soff == st.size
    U.log(f"[optimiser {which}] worst Muon update cosine {worst[0]:.6f} ({worst[1]})")
    # the model's parameters are the cast of the masters
    p = m.params.view(torch.int16).cpu().numpy().view(np.uint16) if dtype != _lib.GPT_F32 else m.params.cpu().numpy()
    want = synthetic.f32_to_bf16_bits(got.astype(np.float32)) if dtype != _lib.GPT_F32 else got.astype(np.float32)
    np.testing.assert_array_equal(p, want)
