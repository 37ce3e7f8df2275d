"""Pins of the float64 oracle against closed forms, invariants, printed values and
library routines (CPU only). Each test names what a plausible mistake in the
oracle would break."""
import json
import math
import os

import numpy as np
import pytest

from oracle import gpt_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def _facts():
    with open(GOLDEN) as f:
        return json.load(f)


def tiny_cfg(**kw):
    cfg = dict(n_layer=2, model_dim=128, n_head=1, n_kv_head=1, head_dim=128, mlp_dim=512,
               vocab_size=512, max_seq_len=64, rope_theta=O.ROPE_THETA,
               logit_softcap=O.SOFTCAP, norm_eps=O.EPS)
    cfg.update(kw)
    return cfg


def rand_params(cfg, seed=0, std=0.02):
    rng = np.random.default_rng(seed)
    return {n: rng.standard_normal((r, c)) * std for n, r, c in O.param_shapes(cfg)}


# ---------------------------------------------------------------- shapes ---

def test_depth_dial_matches_pages():
    f = _facts()
    cfg = O.config_from_depth(20)
    assert cfg["model_dim"] == f["d20_shape"]["model_dim"]
    assert cfg["n_head"] == f["d20_shape"]["n_head"]
    assert cfg["head_dim"] == f["d20_shape"]["head_dim"]
    assert cfg["mlp_dim"] == f["mlp_expansion"]["value"] * cfg["model_dim"]
    assert cfg["vocab_size"] == f["vocab_size"]["value"]
    assert O.ROPE_THETA == f["rope_theta"]["value"]
    assert O.SOFTCAP == f["logit_softcap"]["value"]


def test_param_count_printed_values_mha():
    """With one K/V head per query head the printed d20 and d32 sizes reproduce."""
    f = _facts()
    d20 = O.config_from_depth(20)
    d20["n_kv_head"] = d20["n_head"]
    # the page prints 560.9 million: 560,988,160 truncated (not rounded) to 0.1 M
    assert math.floor(O.param_count(d20) / 1e5) / 10 == f["d20_params_mha_millions_1dp"]["value"]
    assert O.param_count(d20) == 560_988_160
    d32 = O.config_from_depth(32)
    d32["n_kv_head"] = d32["n_head"]
    assert round(O.param_count(d32) / 1e9, 2) == f["d32_params_mha_billions_2dp"]["value"]
    assert O.param_count(d32) == 1_879_048_192


def test_param_count_mqa_closed_form():
    for depth in (4, 12, 20, 24):
        cfg = O.config_from_depth(depth)
        C, H, D, V, L = cfg["model_dim"], cfg["n_head"], 128, 65536, depth
        expect = 2 * V * C + L * ((H + 2) * D * C + C * H * D + 8 * C * C)
        assert O.param_count(cfg) == expect
    assert O.param_count(O.config_from_depth(20)) == 502_005_760
    assert O.param_count(tiny_cfg()) == 524_288


# --------------------------------------------------------------- rmsnorm ---

def test_rmsnorm_output_rms_closed_form():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 256)) * np.exp(rng.uniform(-8, 2, size=(50, 1)))
    y, r = O.rmsnorm(x)
    m = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), np.sqrt(m / (m + O.EPS)), rtol=1e-13)
    np.testing.assert_allclose(r[:, 0], 1 / np.sqrt(m + O.EPS), rtol=1e-14)


def test_rmsnorm_matches_bare_torch_rms_norm_fp32():
    """Bare F.rms_norm on float32 input (no eps given) is the op the pages name;
    at weight scale 0.02 an eps other than 2**-23 would differ by >1e-3."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    x32 = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    yt = torch.nn.functional.rms_norm(torch.from_numpy(x32), (256,)).double().numpy()
    yo, _ = O.rmsnorm(x32.astype(np.float64))
    np.testing.assert_allclose(yt, yo, rtol=0, atol=4e-7)


def test_rmsnorm_bwd_euler_identity_and_fd():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 64)) * 0.01
    dy = rng.standard_normal((8, 64))
    y, r = O.rmsnorm(x)
    dx = O.rmsnorm_bwd(dy, y, r)
    m = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sum(x * dx, -1), O.EPS / (m + O.EPS) * np.sum(y * dy, -1),
                               rtol=1e-9, atol=1e-18)
    h = 1e-7
    for (i, j) in [(0, 0), (3, 17), (7, 63)]:
        xp, xm = x.copy(), x.copy()
        xp[i, j] += h
        xm[i, j] -= h
        fd = (np.sum(O.rmsnorm(xp)[0] * dy) - np.sum(O.rmsnorm(xm)[0] * dy)) / (2 * h)
        assert abs(fd - dx[i, j]) <= 1e-6 * max(1.0, abs(dx[i, j]))


# ------------------------------------------------------------------ rope ---

def test_rope_matches_complex_rotation_convention():
    """Pairs (x_i, x_{i+D/2}) as the complex number x_i + 1j x_{i+D/2}, multiplied
    by exp(1j * t * theta**(-2i/D)). Pins pairing, sign and frequencies."""
    rng = np.random.default_rng(6)
    T, D = 37, 128
    x = rng.standard_normal((2, T, 3, D))
    cos, sin = O.rope_tables(T, D)
    y = O.rope(x, cos, sin)
    zc = x[..., :D // 2] + 1j * x[..., D // 2:]
    t = np.arange(T)[None, :, None, None]
    freq = 10000.0 ** (-np.arange(0, D, 2) / D)
    rot = zc * np.exp(1j * t * freq)
    np.testing.assert_allclose(y[..., :D // 2], rot.real, atol=1e-12)
    np.testing.assert_allclose(y[..., D // 2:], rot.imag, atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(7)
    T, D = 64, 128
    cos, sin = O.rope_tables(T, D)
    x = rng.standard_normal((1, T, 2, D))
    y = O.rope(x, cos, sin)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(y[:, 0], x[:, 0])           # position 0 is the identity
    np.testing.assert_allclose(O.rope_bwd(y, cos, sin), x, atol=1e-12)   # R^T R = I
    # relative position: <R_m a, R_n b> depends only on m - n
    a, b = rng.standard_normal(D), rng.standard_normal(D)
    xa = np.broadcast_to(a, (1, T, 1, D)).copy()
    xb = np.broadcast_to(b, (1, T, 1, D)).copy()
    ra, rb = O.rope(xa, cos, sin)[0, :, 0], O.rope(xb, cos, sin)[0, :, 0]
    for (m, n, s) in [(10, 3, 20), (5, 5, 40), (0, 30, 33)]:
        assert abs(ra[m] @ rb[n] - ra[m + s] @ rb[n + s]) < 1e-10
    # adjoint
    g = rng.standard_normal(x.shape)
    assert abs(np.sum(y * g) - np.sum(x * O.rope_bwd(g, cos, sin))) < 1e-10


def test_rope_commutes_with_qk_norm():
    rng = np.random.default_rng(8)
    T, D = 16, 128
    cos, sin = O.rope_tables(T, D)
    x = rng.standard_normal((2, T, 3, D)) * 0.3
    a = O.rmsnorm(O.rope(x, cos, sin))[0]
    b = O.rope(O.rmsnorm(x)[0], cos, sin)
    np.testing.assert_allclose(a, b, atol=1e-14)


# ------------------------------------------------------------- attention ---

def _qkn(rng, B, T, H, D, scale=1.0):
    q = O.rmsnorm(rng.standard_normal((B, T, H, D)) * scale)[0]
    k = O.rmsnorm(rng.standard_normal((B, T, D)) * scale)[0]
    v = rng.standard_normal((B, T, D))
    return q, k, v


def test_attention_special_cases():
    rng = np.random.default_rng(9)
    B, T, H, D = 2, 24, 3, 128
    q, k, v = _qkn(rng, B, T, H, D)
    o, lse = O.causal_mqa_attention(q, k, v)
    # position 0 attends only to itself
    for h in range(H):
        np.testing.assert_allclose(o[:, 0, h], v[:, 0], atol=1e-14)
    # q = 0 gives uniform weights over the causal prefix
    o0, lse0 = O.causal_mqa_attention(np.zeros_like(q), k, v)
    prefix_mean = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None]
    for h in range(H):
        np.testing.assert_allclose(o0[:, :, h], prefix_mean, atol=1e-13)
    np.testing.assert_allclose(lse0[0, 0], np.log(np.arange(1, T + 1)), atol=1e-13)
    # identical query heads give identical outputs (one shared K/V head)
    q2 = np.repeat(q[:, :, :1], H, axis=2)
    o2, _ = O.causal_mqa_attention(q2, k, v)
    for h in range(1, H):
        np.testing.assert_array_equal(o2[:, :, h], o2[:, :, 0])
    # |scaled score| <= sqrt(D) for RMS-normalised q, k (Cauchy-Schwarz)
    s = np.einsum("bthd,bud->bhtu", q, k) / math.sqrt(D)
    assert np.abs(s).max() <= math.sqrt(D)


def test_attention_matches_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(10)
    B, T, H, D = 2, 33, 4, 128
    q, k, v = _qkn(rng, B, T, H, D)
    o, _ = O.causal_mqa_attention(q, k, v)
    qt = torch.tensor(q).permute(0, 2, 1, 3).requires_grad_()
    kt = torch.tensor(k)[:, None].requires_grad_()
    vt = torch.tensor(v)[:, None].requires_grad_()
    ot = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=True)
    np.testing.assert_allclose(ot.permute(0, 2, 1, 3).detach().numpy(), o, atol=1e-13)
    do = rng.standard_normal(o.shape)
    ot.backward(torch.tensor(do).permute(0, 2, 1, 3))
    dq, dk, dv = O.causal_mqa_attention_bwd(do, q, k, v)
    np.testing.assert_allclose(qt.grad.permute(0, 2, 1, 3).numpy(), dq, atol=1e-12)
    np.testing.assert_allclose(kt.grad[:, 0].numpy(), dk, atol=1e-12)
    np.testing.assert_allclose(vt.grad[:, 0].numpy(), dv, atol=1e-12)


# ------------------------------------------------------- softcap and CE ---

def test_softcap_bound_and_derivative():
    z = np.linspace(-200, 200, 4001)
    zc = O.softcap(z)
    assert np.all(np.abs(zc) <= O.SOFTCAP)
    assert np.all(np.abs(zc[np.abs(z) < 30]) < O.SOFTCAP)
    small = np.abs(z) < 0.2
    np.testing.assert_allclose(zc[small], z[small], atol=1e-4)
    h = 1e-6
    fd = (O.softcap(z + h) - O.softcap(z - h)) / (2 * h)
    np.testing.assert_allclose(O.softcap_bwd(np.ones_like(z), zc), fd, atol=1e-8)


def test_zero_head_gives_log_vocab_and_closed_form_grads():
    """W_lm = 0: every logit is 0, loss = ln V exactly, dW_lm = ((1/V - onehot)^T h_f)/N
    and every other gradient is exactly zero (dh_f = dz W_lm = 0)."""
    cfg = tiny_cfg(n_layer=1)
    P = rand_params(cfg, seed=11)
    P["lm_head"] = np.zeros_like(P["lm_head"])
    rng = np.random.default_rng(12)
    B, T, V = 2, 16, cfg["vocab_size"]
    idx = rng.integers(0, V, (B, T))
    tg = rng.integers(0, V, (B, T))
    loss, rows, cache = O.forward(cfg, P, idx, tg)
    assert loss == pytest.approx(math.log(V), abs=1e-15)
    assert math.log(512) == pytest.approx(6.238324625039508, abs=1e-15)
    G = O.backward(cfg, P, idx, tg, cache)
    for name, g in G.items():
        if name != "lm_head":
            assert np.all(g == 0.0), name
    N = B * T
    onehot = np.zeros((N, V))
    onehot[np.arange(N), tg.reshape(N)] = 1.0
    expect = (np.full((N, V), 1.0 / V) - onehot).T @ cache["hf"].reshape(N, -1) / N
    np.testing.assert_allclose(G["lm_head"], expect, atol=1e-15)


def test_cross_entropy_matches_torch_on_softcapped_logits():
    torch = pytest.importorskip("torch")
    cfg = tiny_cfg(n_layer=1)
    P = rand_params(cfg, seed=13, std=0.2)
    rng = np.random.default_rng(14)
    idx = rng.integers(0, 512, (2, 20))
    tg = rng.integers(0, 512, (2, 20))
    loss, rows, cache = O.forward(cfg, P, idx, tg)
    z = cache["hf"].reshape(40, -1) @ P["lm_head"].T
    zc = torch.tensor(15.0 * np.tanh(z / 15.0))
    ref = torch.nn.functional.cross_entropy(zc, torch.tensor(tg.reshape(-1)), reduction="none")
    np.testing.assert_allclose(rows.reshape(-1), ref.numpy(), rtol=1e-13)
    assert 0 < loss < math.log(512) + 2 * 15


# ------------------------------------------------------------ whole step ---

def test_whole_step_central_differences():
    """Analytic backward vs central differences of the float64 loss, on every tensor."""
    cfg = tiny_cfg(n_layer=2, vocab_size=64, mlp_dim=512)
    P = rand_params(cfg, seed=15, std=0.1)
    rng = np.random.default_rng(16)
    B, T = 2, 8
    idx = rng.integers(0, 64, (B, T))
    tg = rng.integers(0, 64, (B, T))
    dloss = 0.75
    loss, _, G = O.step(cfg, P, idx, tg, dloss)
    h = 1e-5
    for name, W in P.items():
        pick = [tuple(rng.integers(0, s) for s in W.shape) for _ in range(4)]
        if name == "wte":   # rows that are actually used
            pick = [(int(idx[0, 0]), 5), (int(idx[1, 3]), 100), (int(idx[0, 7]), 0)]
        for ij in pick:
            old = W[ij]
            W[ij] = old + h
            lp = O.forward(cfg, P, idx, tg)[0]
            W[ij] = old - h
            lm = O.forward(cfg, P, idx, tg)[0]
            W[ij] = old
            fd = dloss * (lp - lm) / (2 * h)
            # float64 central differences: truncation O(h^2) plus round-off ~ 1e-16 * loss / h
            assert abs(fd - G[name][ij]) <= 1e-6 * abs(fd) + 2e-10, (name, ij, fd, G[name][ij])


def _torch_step(cfg, P, idx, tg):
    """A second, independent float64 implementation with torch autograd and
    torch's own rms_norm, SDPA and cross_entropy (sliding-window layers through
    SDPA's boolean mask, built here from the window rule itself)."""
    import torch
    import torch.nn.functional as F
    eps, c, H, D = cfg["norm_eps"], cfg["logit_softcap"], cfg["n_head"], cfg["head_dim"]
    W = {k: torch.tensor(v, requires_grad=True) for k, v in P.items()}
    B, T = idx.shape
    idx_t, tg_t = torch.tensor(idx), torch.tensor(tg)
    pos = torch.arange(T, dtype=torch.float64)
    inv = cfg["rope_theta"] ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
    ang = pos[:, None] * inv[None]
    cs, sn = torch.cos(ang)[None, None], torch.sin(ang)[None, None]

    def rot(x):   # x [B, h, T, D]
        a, b = x[..., :D // 2], x[..., D // 2:]
        return torch.cat([a * cs - b * sn, a * sn + b * cs], -1)

    def norm(x):
        return F.rms_norm(x, (x.shape[-1],), eps=eps)

    def fake_quant(t):
        # per-tensor e4m3 round trip of the bf16 operand through torch's own
        # bfloat16 and float8 conversions
        t32 = t.detach().to(torch.bfloat16).to(torch.float32)
        amax = t32.abs().max()
        s = torch.tensor(448.0, dtype=torch.float32) / amax if amax > 0 else torch.tensor(1.0)
        q = (t32 * s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        return q.to(torch.float64) / s.to(torch.float64)

    class QLinear(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, w):
            xq, wq = fake_quant(x), fake_quant(w)
            ctx.save_for_backward(xq, wq)
            return xq @ wq.T

        @staticmethod
        def backward(ctx, dy):
            xq, wq = ctx.saved_tensors
            dyq = fake_quant(dy)
            return dyq @ wq, dyq.reshape(-1, dyq.shape[-1]).T @ xq.reshape(-1, xq.shape[-1])

    def lin(x, w):
        return QLinear.apply(x, w) if cfg.get("fp8", False) else x @ w.T

    x = norm(W["wte"][idx_t])
    x0 = x
    ve_l = list(range(0, cfg["n_layer"], 2)) if cfg.get("value_embeds", False) else []
    for l in range(cfg["n_layer"]):
        if cfg.get("x0_lambdas", False):
            x = W["resid_lambdas"][0, l] * x + W["x0_lambdas"][0, l] * x0
        qkv = lin(norm(x), W[f"h{l}.w_qkv"])
        q = qkv[..., :H * D].view(B, T, H, D).transpose(1, 2)
        k = qkv[..., H * D:(H + 1) * D].view(B, T, 1, D).transpose(1, 2)
        v = qkv[..., (H + 1) * D:]
        if l in ve_l:
            v = v + W["ve_gates"][0, ve_l.index(l)] * F.embedding(idx_t, W[f"h{l}.ve"])
        v = v.view(B, T, 1, D).transpose(1, 2)
        q, k = norm(rot(q)), norm(rot(k))
        pattern, short = cfg.get("window_pattern", ""), cfg.get("window_short", 0)
        if pattern and short and l != cfg["n_layer"] - 1 and pattern[l % len(pattern)] == "S":
            t_i, u_i = torch.arange(T)[:, None], torch.arange(T)[None, :]
            allowed = (u_i <= t_i) & (t_i - u_i < short)
            y = F.scaled_dot_product_attention(q, k, v, attn_mask=allowed, enable_gqa=True)
        else:
            y = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
        x = x + lin(y.transpose(1, 2).reshape(B, T, H * D), W[f"h{l}.w_o"])
        x = x + lin(F.relu(lin(norm(x), W[f"h{l}.w_1"])).square(), W[f"h{l}.w_2"])
    logits = norm(x) @ W["lm_head"].T
    logits = c * torch.tanh(logits / c)
    loss = F.cross_entropy(logits.view(B * T, -1), tg_t.view(-1))
    loss.backward()
    return loss.item(), {k: v.grad.numpy() for k, v in W.items()}


@pytest.mark.parametrize("H", [1, 3])
def test_whole_step_matches_torch_autograd_float64(H):
    pytest.importorskip("torch")
    cfg = tiny_cfg(n_layer=2, n_head=H, model_dim=128 * H, mlp_dim=512 * H, vocab_size=96)
    P = rand_params(cfg, seed=17, std=0.05)
    rng = np.random.default_rng(18)
    idx = rng.integers(0, 96, (2, 21))
    tg = rng.integers(0, 96, (2, 21))
    loss, _, G = O.step(cfg, P, idx, tg)
    tl, TG = _torch_step(cfg, P, idx, tg)
    assert loss == pytest.approx(tl, rel=1e-13)
    for k in G:
        np.testing.assert_allclose(G[k], TG[k], rtol=1e-9, atol=1e-13, err_msg=k)


def test_lm_head_row_chunks_match_torch_autograd():
    """The LM head and cross-entropy run over row chunks (to bound memory at
    d12/d20). With chunks of 5 rows over N = 42 positions (eight whole chunks
    and a ragged one), the loss and every gradient still equal the independent
    torch-autograd step's: a chunk that read another chunk's log-sum-exp,
    targets or rows would fail here."""
    pytest.importorskip("torch")
    cfg = tiny_cfg(n_layer=1, vocab_size=96)
    P = rand_params(cfg, seed=23, std=0.1)
    rng = np.random.default_rng(24)
    idx = rng.integers(0, 96, (2, 21))
    tg = rng.integers(0, 96, (2, 21))
    tl, TG = _torch_step(cfg, P, idx, tg)
    for chunk in (5, 7, 41):
        loss, _, G = O.step(cfg, P, idx, tg, row_chunk=chunk)
        assert loss == pytest.approx(tl, rel=1e-13), chunk
        for k in G:
            np.testing.assert_allclose(G[k], TG[k], rtol=1e-9, atol=1e-13, err_msg=f"{k} chunk {chunk}")


def test_causality_and_row_independence():
    cfg = tiny_cfg(n_layer=1, vocab_size=128)
    P = rand_params(cfg, seed=19, std=0.1)
    rng = np.random.default_rng(20)
    idx = rng.integers(0, 128, (3, 12))
    tg = rng.integers(0, 128, (3, 12))
    _, rows, _ = O.forward(cfg, P, idx, tg)
    idx2 = idx.copy()
    idx2[1, 7] = (idx2[1, 7] + 5) % 128
    _, rows2, _ = O.forward(cfg, P, idx2, tg)
    np.testing.assert_array_equal(rows2[1, :7], rows[1, :7])
    np.testing.assert_array_equal(rows2[0], rows[0])
    assert not np.array_equal(rows2[1, 7:], rows[1, 7:])
    perm = [2, 0, 1]
    _, rows3, _ = O.forward(cfg, P, idx[perm], tg[perm])
    np.testing.assert_allclose(rows3, rows[perm], rtol=1e-14)


# ------------------------------------------------------ sliding windows ---

def test_layer_window_pattern():
    """[P1]: "SSSL" = three short-window layers then one full-context layer,
    repeating, with the final layer always full."""
    cfg = tiny_cfg(n_layer=6, window_pattern="SSSL", window_short=4)
    assert [O.layer_window(cfg, l) for l in range(6)] == [4, 4, 4, None, 4, None]
    cfg = tiny_cfg(n_layer=4, window_pattern="SSSL", window_short=4)
    assert [O.layer_window(cfg, l) for l in range(4)] == [4, 4, 4, None]
    assert all(O.layer_window(tiny_cfg(n_layer=3), l) is None for l in range(3))
    assert all(O.layer_window(tiny_cfg(n_layer=3, window_pattern="SSSL"), l) is None for l in range(3))
    # the mask is the set {(t, u): u <= t and t - u < W}, element by element
    T, W = 9, 3
    m = O.attention_mask(T, W)
    for t in range(T):
        for u in range(T):
            assert m[t, u] == (u <= t and t - u < W)
    np.testing.assert_array_equal(O.attention_mask(T, None), np.tril(np.ones((T, T), dtype=bool)))


def test_windowed_attention_special_cases_and_brute_force():
    rng = np.random.default_rng(31)
    B, T, H, D = 2, 20, 2, 128
    q, k, v = _qkn(rng, B, T, H, D)
    full, lse_full = O.causal_mqa_attention(q, k, v)
    # a window as long as the sequence is plain causal attention
    o, lse = O.causal_mqa_attention(q, k, v, window=T)
    np.testing.assert_array_equal(o, full)
    np.testing.assert_array_equal(lse, lse_full)
    # window 1: every query sees only itself
    o1, lse1 = O.causal_mqa_attention(q, k, v, window=1)
    for h in range(H):
        np.testing.assert_allclose(o1[:, :, h], v, atol=1e-14)
        np.testing.assert_allclose(lse1[:, h], np.einsum("btd,btd->bt", q[:, :, h], k) / math.sqrt(D), atol=1e-13)
    # rows before the window fills agree with full causal attention
    W = 7
    ow, lsew = O.causal_mqa_attention(q, k, v, window=W)
    np.testing.assert_allclose(ow[:, :W], full[:, :W], atol=1e-14)
    # brute force: an explicit softmax over keys t-W+1 .. t for every row
    for b in range(B):
        for t in range(T):
            for h in range(H):
                us = range(max(0, t - W + 1), t + 1)
                sc = np.array([q[b, t, h] @ k[b, u] / math.sqrt(D) for u in us])
                w = np.exp(sc - sc.max())
                ref = sum(wi * v[b, u] for wi, u in zip(w / w.sum(), us))
                np.testing.assert_allclose(ow[b, t, h], ref, atol=1e-13)
                assert lsew[b, h, t] == pytest.approx(sc.max() + math.log(w.sum()), abs=1e-13)


def test_windowed_attention_matches_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(32)
    B, T, H, D, W = 2, 29, 3, 128, 6
    q, k, v = _qkn(rng, B, T, H, D)
    o, _ = O.causal_mqa_attention(q, k, v, window=W)
    qt = torch.tensor(q).permute(0, 2, 1, 3).requires_grad_()
    kt = torch.tensor(k)[:, None].requires_grad_()
    vt = torch.tensor(v)[:, None].requires_grad_()
    t_i, u_i = torch.arange(T)[:, None], torch.arange(T)[None, :]
    ot = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=(u_i <= t_i) & (t_i - u_i < W), enable_gqa=True)
    np.testing.assert_allclose(ot.permute(0, 2, 1, 3).detach().numpy(), o, atol=1e-13)
    do = rng.standard_normal(o.shape)
    ot.backward(torch.tensor(do).permute(0, 2, 1, 3))
    dq, dk, dv = O.causal_mqa_attention_bwd(do, q, k, v, window=W)
    np.testing.assert_allclose(qt.grad.permute(0, 2, 1, 3).numpy(), dq, atol=1e-12)
    np.testing.assert_allclose(kt.grad[:, 0].numpy(), dk, atol=1e-12)
    np.testing.assert_allclose(vt.grad[:, 0].numpy(), dv, atol=1e-12)


def test_windowed_step_matches_torch_autograd_and_fd():
    pytest.importorskip("torch")
    cfg = tiny_cfg(n_layer=3, n_head=2, model_dim=256, mlp_dim=1024, vocab_size=80, window_pattern="SL",
                   window_short=5)
    assert [O.layer_window(cfg, l) for l in range(3)] == [5, None, None]
    P = rand_params(cfg, seed=33, std=0.05)
    rng = np.random.default_rng(34)
    idx = rng.integers(0, 80, (2, 17))
    tg = rng.integers(0, 80, (2, 17))
    loss, _, G = O.step(cfg, P, idx, tg)
    tl, TG = _torch_step(cfg, P, idx, tg)
    assert loss == pytest.approx(tl, rel=1e-13)
    for name in G:
        np.testing.assert_allclose(G[name], TG[name], rtol=1e-9, atol=1e-13, err_msg=name)
    # and the window changes the result (the pattern is not ignored)
    loss_full = O.forward(tiny_cfg(n_layer=3, n_head=2, model_dim=256, mlp_dim=1024, vocab_size=80), P, idx, tg)[0]
    assert abs(loss_full - loss) > 1e-6
    # central differences on the windowed layer's attention weights
    h = 1e-5
    W = P["h0.w_qkv"]
    for ij in [(3, 7), (260, 11), (300, 200)]:
        old = W[ij]
        W[ij] = old + h
        lp = O.forward(cfg, P, idx, tg)[0]
        W[ij] = old - h
        lm = O.forward(cfg, P, idx, tg)[0]
        W[ij] = old
        fd = (lp - lm) / (2 * h)
        assert abs(fd - G["h0.w_qkv"][ij]) <= 1e-6 * abs(fd) + 2e-10


# ------------------------------------------------------------- FP8 e4m3 ---

def _torch_e4m3_values():
    import torch
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_matches_spec_points_and_torch():
    """The OCP e4m3 grid: 1.0 = 0x38, largest finite 448 = 0x7e, smallest
    subnormal 2^-9 = 0x01, smallest normal 2^-6 = 0x08, NaN at 0x7f/0xff and no
    infinities. A wrong bias, subnormal rule or sign bit breaks one of these."""
    pytest.importorskip("torch")
    v = O.e4m3_decode(np.arange(256))
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0x07] == 7 * 2.0 ** -9 and v[0xB8] == -1.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isfinite(v).sum() == 254
    assert np.all(np.diff(v[:0x7F]) > 0)
    np.testing.assert_array_equal(v, _torch_e4m3_values())


def test_e4m3_encode_is_round_to_nearest_even_like_torch():
    """Encoding agrees with torch's float8_e4m3fn conversion (round to nearest,
    ties to even) on random fp32 values over the whole range, on every exact
    midpoint between neighbouring grid values (the tie cases) and in the
    subnormal range."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(40)
    grid = O.e4m3_decode(np.arange(0x7F))
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([
        rng.uniform(-448, 448, 20000),
        np.exp2(rng.uniform(-12, 8.8, 20000)) * rng.choice([-1, 1], 20000),
        mids, -mids, grid, -grid, np.nextafter(mids, 0), np.nextafter(mids, 1000)]).astype(np.float32)
    ours = O.e4m3_encode(vals)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)
    # ties really go to the even mantissa: midpoint of 1.0 (0x38) and 1.125 (0x39)
    assert O.e4m3_encode(np.float32(1.0625)) == 0x38 and O.e4m3_encode(np.float32(1.1875)) == 0x3A


def test_e4m3_encode_saturates():
    """Magnitudes past the largest finite value clamp to +-448 (0x7e / 0xfe)
    rather than overflowing to NaN; zero keeps its sign; NaN stays NaN."""
    y = np.array([448.0, 449.0, 464.0, 465.0, 1e6, np.inf, -500.0, -np.inf, 0.0, -0.0, np.nan], np.float32)
    assert O.e4m3_encode(y).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80, 0x7F]


def test_fp8_quantize_scale_zero_tensor_and_amax_element():
    """s = 448 / amax in fp32; the largest element lands on +-448; an all-zero
    tensor keeps scale 1 and all-zero codes."""
    rng = np.random.default_rng(41)
    x = rng.standard_normal((7, 13)) * 3.0
    x[4, 5] = -9.5
    q, s = O.fp8_quantize(x)
    assert s.dtype == np.float32 and s == np.float32(448.0) / np.float32(9.5)
    assert q[4, 5] == 0xFE
    q0, s0 = O.fp8_quantize(np.zeros((3, 4)))
    assert s0 == 1.0 and not q0.any()


def test_round_bf16_matches_torch_and_ties():
    """bf16 rounding agrees with torch's float32 -> bfloat16 conversion on
    fp32 inputs (including exact ties, which go to the even mantissa)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(48)
    x = np.concatenate([rng.standard_normal(20000) * np.exp2(rng.uniform(-20, 20, 20000)),
                        [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 0.0]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(x.astype(np.float64)), ref)
    assert O.round_bf16(1 + 2.0 ** -8) == 1.0 and O.round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6


def test_fp8_round_trip_error_bound():
    """|Q(x)/s - x| <= 2^-4 |x| (three mantissa bits) or, in the subnormal
    range, half a subnormal step 2^-10 / s, plus the bf16 rounding of x
    (2^-9 |x|) and its fp32 product."""
    rng = np.random.default_rng(42)
    for scale in (1e-3, 1.0, 250.0):
        x = rng.standard_normal(50000) * scale * np.exp2(rng.uniform(-8, 0, 50000))
        r = O.fp8_round_trip(x)
        _, s = O.fp8_quantize(x)
        bound = (np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 / np.float64(s)) * (1 + 2.0 ** -8)
                 + 2.0 ** -9 * np.abs(x))
        assert np.all(np.abs(r - x) <= bound)
        assert np.max(np.abs(r - x) / np.maximum(np.abs(x), 1e-300)) > 2.0 ** -6   # it does quantise


def test_fp8_round_trip_exact_on_scaled_grid():
    """Operands that already are e4m3 values times 2^-k, with one element at
    448 * 2^-k, get scale 2^k and pass through exactly, so an FP8 matmul of
    them equals the float64 matmul (catches a dropped dequantisation or a
    scale applied the wrong way)."""
    rng = np.random.default_rng(43)
    grid = O.e4m3_decode(np.arange(0x7F))
    for k in (-3, 0, 5):
        x = rng.choice(grid, (9, 16)) * rng.choice([-1.0, 1.0], (9, 16)) * 2.0 ** -k
        x[2, 3] = 448.0 * 2.0 ** -k
        q, s = O.fp8_quantize(x)
        assert s == np.float32(2.0 ** k)
        np.testing.assert_array_equal(O.fp8_round_trip(x), x)
    cfg = dict(fp8=True)
    w = rng.choice(grid, (5, 16)) * 2.0 ** -7
    w[0, 0] = 448.0 * 2.0 ** -7
    np.testing.assert_array_equal(O.mm_operand(cfg, x) @ O.mm_operand(cfg, w).T, x @ w.T)


def test_fp8_step_matches_torch_autograd_with_float8_fake_quant():
    """The FP8 step (every QKV / O / MLP product on per-tensor e4m3 operands,
    output gradients quantised too, straight-through backward) against torch
    autograd with torch's float8 conversion as the quantiser."""
    pytest.importorskip("torch")
    cfg = tiny_cfg(n_layer=2, n_head=2, model_dim=256, mlp_dim=1024, vocab_size=96, fp8=True)
    P = rand_params(cfg, seed=44, std=0.05)
    rng = np.random.default_rng(45)
    idx = rng.integers(0, 96, (2, 19))
    tg = rng.integers(0, 96, (2, 19))
    loss, _, G = O.step(cfg, P, idx, tg)
    tl, TG = _torch_step(cfg, P, idx, tg)
    assert loss == pytest.approx(tl, rel=1e-12)
    for name in G:
        np.testing.assert_allclose(G[name], TG[name], rtol=1e-8, atol=1e-12, err_msg=name)


def test_fp8_step_close_to_unquantised_step():
    """Quantisation noise only: the FP8 step's loss and gradients stay close to
    the unquantised step's (e4m3 keeps 3 mantissa bits), and differ from it."""
    cfg = tiny_cfg(n_layer=2, n_head=2, model_dim=256, mlp_dim=1024, vocab_size=96)
    P = rand_params(cfg, seed=46, std=0.05)
    rng = np.random.default_rng(47)
    idx = rng.integers(0, 96, (2, 33))
    tg = rng.integers(0, 96, (2, 33))
    l0, _, G0 = O.step(cfg, P, idx, tg)
    l8, _, G8 = O.step(dict(cfg, fp8=True), P, idx, tg)
    assert l8 != l0 and abs(l8 - l0) / l0 < 1e-2
    for name in G0:
        a, b = G0[name].ravel(), G8[name].ravel()
        cos = a @ b / np.linalg.norm(a) / np.linalg.norm(b)
        assert cos > 0.99, name


# ------------------------------------- residual scalars, value embeddings ---

def _lam_ve_params(cfg, seed, std=0.05):
    P = rand_params(cfg, seed=seed, std=std)
    rng = np.random.default_rng(seed + 100)
    L = cfg["n_layer"]
    if cfg.get("x0_lambdas"):
        P["resid_lambdas"] = 1.0 + 0.2 * rng.standard_normal((1, L))
        P["x0_lambdas"] = 0.1 + 0.2 * rng.standard_normal((1, L))
    if cfg.get("value_embeds"):
        P["ve_gates"] = 1.0 + 0.5 * rng.standard_normal((1, len(O.ve_layers(cfg))))
        for l in O.ve_layers(cfg):
            P[f"h{l}.ve"] = P[f"h{l}.ve"] * 20   # ve rows comparable to v
    return P


def test_ve_layers_and_param_shapes():
    """Value embeddings sit on layers 0, 2, 4, ... ([V, n_kv_head*D] each),
    then the per-layer scalars; the plain config is unchanged."""
    cfg = tiny_cfg(n_layer=5, x0_lambdas=True, value_embeds=True)
    assert O.ve_layers(cfg) == [0, 2, 4]
    names = [n for n, _, _ in O.param_shapes(cfg)]
    assert names[-6:] == ["h0.ve", "h2.ve", "h4.ve", "resid_lambdas", "x0_lambdas", "ve_gates"]
    shapes = dict((n, (r, c)) for n, r, c in O.param_shapes(cfg))
    assert shapes["h2.ve"] == (512, 128) and shapes["x0_lambdas"] == (1, 5) and shapes["ve_gates"] == (1, 3)
    assert O.param_count(cfg) == O.param_count(tiny_cfg(n_layer=5)) + 3 * 512 * 128 + 2 * 5 + 3


def test_lambdas_ve_step_matches_torch_autograd():
    pytest.importorskip("torch")
    cfg = tiny_cfg(n_layer=3, n_head=2, model_dim=256, mlp_dim=1024, vocab_size=80, x0_lambdas=True,
                   value_embeds=True)
    P = _lam_ve_params(cfg, 50)
    rng = np.random.default_rng(51)
    idx = rng.integers(0, 80, (2, 17))
    tg = rng.integers(0, 80, (2, 17))
    loss, _, G = O.step(cfg, P, idx, tg)
    tl, TG = _torch_step(cfg, P, idx, tg)
    assert loss == pytest.approx(tl, rel=1e-13)
    for name in G:
        np.testing.assert_allclose(G[name], TG[name], rtol=1e-9, atol=1e-13, err_msg=name)


def test_lambdas_ve_central_differences():
    cfg = tiny_cfg(n_layer=3, n_head=1, vocab_size=64, x0_lambdas=True, value_embeds=True)
    P = _lam_ve_params(cfg, 52)
    rng = np.random.default_rng(53)
    idx = rng.integers(0, 64, (2, 9))
    tg = rng.integers(0, 64, (2, 9))
    _, _, G = O.step(cfg, P, idx, tg)
    h = 1e-6
    tok = int(idx[1, 3])
    for name, ij in [("resid_lambdas", (0, 1)), ("x0_lambdas", (0, 0)), ("x0_lambdas", (0, 2)),
                     ("ve_gates", (0, 1)), ("h2.ve", (tok, 5)), ("h0.ve", (tok, 77)), ("wte", (tok, 3))]:
        Wt = P[name]
        old = Wt[ij]
        Wt[ij] = old + h
        lp = O.forward(cfg, P, idx, tg)[0]
        Wt[ij] = old - h
        lm = O.forward(cfg, P, idx, tg)[0]
        Wt[ij] = old
        fd = (lp - lm) / (2 * h)
        assert abs(fd - G[name][ij]) <= 1e-6 * abs(fd) + 1e-9, (name, fd, G[name][ij])
    # rows of a value-embedding table that no token reads get no gradient
    unused = np.setdiff1d(np.arange(64), idx)
    assert not G["h0.ve"][unused].any()


def test_neutral_scalars_and_zero_gate_reduce_to_the_plain_model():
    """resid_lambdas = 1, x0_lambdas = 0 and zero gates leave the plain model:
    the same loss and the same gradients for every shared tensor, bit for bit."""
    base = tiny_cfg(n_layer=2, vocab_size=64)
    cfg = dict(base, x0_lambdas=True, value_embeds=True)
    P = _lam_ve_params(cfg, 54)
    P["resid_lambdas"][:] = 1.0
    P["x0_lambdas"][:] = 0.0
    P["ve_gates"][:] = 0.0
    rng = np.random.default_rng(55)
    idx = rng.integers(0, 64, (2, 11))
    tg = rng.integers(0, 64, (2, 11))
    l1, _, G1 = O.step(cfg, P, idx, tg)
    l0, _, G0 = O.step(base, {k: v for k, v in P.items() if k in dict((n, 0) for n, _, _ in O.param_shapes(base))},
                       idx, tg)
    assert l1 == l0
    for k in G0:
        np.testing.assert_array_equal(G1[k], G0[k], err_msg=k)
    assert not G1["h0.ve"].any() and G1["ve_gates"][0, 0] != 0.0


# ------------------------------------------------------------- optimiser ---

def test_optimizer_groups():
    cfg = tiny_cfg(n_layer=2, x0_lambdas=True, value_embeds=True)
    groups = {n: O.optimizer_group(n) for n, _, _ in O.param_shapes(cfg)}
    assert groups["h1.w_qkv"] == groups["h0.w_2"] == "muon"
    assert groups["wte"] == groups["h0.ve"] == "embed" and groups["lm_head"] == "unembed"
    assert groups["resid_lambdas"] == groups["x0_lambdas"] == groups["ve_gates"] == "scalar"


def test_adamw_matches_torch():
    """Three AdamW steps against torch.optim.AdamW (decoupled weight decay,
    bias correction)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(60)
    w0 = rng.standard_normal((7, 5))
    gs = [rng.standard_normal((7, 5)) for _ in range(3)]
    p = torch.tensor(w0, requires_grad=True)
    opt = torch.optim.AdamW([p], lr=0.01, betas=(0.8, 0.95), eps=1e-10, weight_decay=0.1)
    w, m, v = w0, np.zeros_like(w0), np.zeros_like(w0)
    for t, g in enumerate(gs, start=1):
        p.grad = torch.tensor(g)
        opt.step()
        w, m, v = O.adamw_update(w, g, m, v, t, 0.01, 0.8, 0.95, 1e-10, 0.1)
    np.testing.assert_allclose(w, p.detach().numpy(), rtol=1e-13, atol=1e-15)


def test_newton_schulz_reaches_the_polar_factor():
    """Enough cubic Newton-Schulz steps give U V^T of the SVD (the orthogonal
    polar factor) for both orientations; the result is invariant to scaling
    and commutes with transposition; rows of the wide result are orthonormal."""
    rng = np.random.default_rng(61)
    U_, _ = np.linalg.qr(rng.standard_normal((12, 12)))
    V_, _ = np.linalg.qr(rng.standard_normal((40, 12)))
    M = U_ @ np.diag(np.linspace(1.0, 3.0, 12)) @ V_.T          # 12 x 40, condition number 3
    P = U_ @ V_.T
    X = O.newton_schulz(M, 60)
    np.testing.assert_allclose(X, P, atol=1e-10)
    np.testing.assert_allclose(O.newton_schulz(M.T, 60), P.T, atol=1e-10)
    np.testing.assert_allclose(O.newton_schulz(7.5 * M, 60), X, atol=1e-10)
    np.testing.assert_allclose(X @ X.T, np.eye(12), atol=1e-10)
    # a few steps only approach it, monotonically in the singular values
    s5 = np.linalg.svd(O.newton_schulz(M, 5), compute_uv=False)
    assert np.all(s5 < 1.0 + 1e-12) and np.all(s5 > 0.2)


def _with_singular_values(rng, rows, cols, s):
    """A rows x cols matrix U diag(s) V^T with random orthonormal U, V."""
    r = min(rows, cols)
    U_, _ = np.linalg.qr(rng.standard_normal((rows, r)))
    V_, _ = np.linalg.qr(rng.standard_normal((cols, r)))
    return U_, V_, U_ @ np.diag(s) @ V_.T


def test_newton_schulz_one_step_closed_form_and_quintic_convergence():
    """One step X <- a X + (b A + c A^2) X with A = X X^T keeps the singular
    vectors of X0 = M / (||M||_F + 1e-7) and maps each singular value s to
    a s + b s^3 + c s^5 (A has eigenvalues s^2, A^2 has s^4), in both
    orientations: a wrong power in the c term or a dropped term fails here.
    The quintic coefficients (1.875, -1.25, 0.375) (p(1) = 1, p'(1) = p''(1) = 0)
    also converge to the polar factor U V^T of the SVD."""
    rng = np.random.default_rng(63)
    s = np.linspace(0.5, 4.0, 9)
    U_, V_, M = _with_singular_values(rng, 9, 25, s)
    s0 = s / (np.linalg.norm(M) + 1e-7)
    for a, b, c in [(1.875, -1.25, 0.375), (2.0, -1.5, 0.5), (0.0, 0.0, 1.0), (0.0, 1.0, 0.0)]:
        want = U_ @ np.diag(a * s0 + b * s0 ** 3 + c * s0 ** 5) @ V_.T
        np.testing.assert_allclose(O.newton_schulz(M, 1, a, b, c), want, atol=1e-14)
        np.testing.assert_allclose(O.newton_schulz(M.T, 1, a, b, c), want.T, atol=1e-14)
    # two steps compose the scalar map
    p = lambda x: 1.875 * x - 1.25 * x ** 3 + 0.375 * x ** 5  # noqa: E731
    np.testing.assert_allclose(O.newton_schulz(M, 2, 1.875, -1.25, 0.375), U_ @ np.diag(p(p(s0))) @ V_.T,
                               atol=1e-14)
    X = O.newton_schulz(M, 40, 1.875, -1.25, 0.375)
    np.testing.assert_allclose(X, U_ @ V_.T, atol=1e-10)


def test_optimizer_step_gives_each_group_its_own_learning_rate():
    """A first step with four distinct learning rates: every AdamW-group tensor
    equals torch.optim.AdamW run with its own group's rate (embeddings incl.
    value-embedding tables, unembedding, scalars), and every block matrix the
    converged Muon step w (1 - lr wd) - lr sqrt(max(1, rows/cols)) U V^T of its
    gradient (the momentum buffer is the gradient on the first step). Swapping
    any two groups' rates, or sending a tensor to the wrong group, fails here."""
    torch = pytest.importorskip("torch")
    cfg = tiny_cfg(n_layer=2, vocab_size=64, x0_lambdas=True, value_embeds=True)
    oc = dict(lr_embed=0.3, lr_unembed=0.004, lr_scalar=0.05, lr_muon=0.02, momentum=0.9,
              beta1=0.8, beta2=0.95, eps=1e-10, wd_muon=0.1, wd_adamw=0.01, ns_steps=60)
    rng = np.random.default_rng(64)
    master = {n: rng.standard_normal((r, c)) * 0.02 for n, r, c in O.param_shapes(cfg)}
    grads, polar = {}, {}
    for n, r, c in O.param_shapes(cfg):
        if O.optimizer_group(n) == "muon":
            U_, V_, grads[n] = _with_singular_values(rng, r, c, np.linspace(1.0, 3.0, min(r, c)))
            polar[n] = U_ @ V_.T
        else:
            grads[n] = rng.standard_normal((r, c))
    new_w, new_s = O.optimizer_step(cfg, oc, master, grads, {}, 1)
    lr = dict(embed=oc["lr_embed"], unembed=oc["lr_unembed"], scalar=oc["lr_scalar"])
    seen = set()
    for n, w in master.items():
        grp = O.optimizer_group(n)
        seen.add(grp)
        if grp == "muon":
            scale = math.sqrt(max(1.0, w.shape[0] / w.shape[1]))
            want = w * (1 - oc["lr_muon"] * oc["wd_muon"]) - oc["lr_muon"] * scale * polar[n]
            np.testing.assert_allclose(new_w[n], want, rtol=0, atol=1e-11, err_msg=n)
            np.testing.assert_array_equal(new_s[n]["u"], grads[n])
        else:
            p = torch.tensor(w, requires_grad=True)
            opt = torch.optim.AdamW([p], lr=lr[grp], betas=(oc["beta1"], oc["beta2"]), eps=oc["eps"],
                                    weight_decay=oc["wd_adamw"])
            p.grad = torch.tensor(grads[n])
            opt.step()
            np.testing.assert_allclose(new_w[n], p.detach().numpy(), rtol=1e-13, atol=1e-15, err_msg=n)
    assert seen == {"muon", "embed", "unembed", "scalar"}


def test_muon_step_momentum_and_scale():
    """u accumulates mu u + g; a converged update moves w by exactly lr *
    sqrt(max(1, rows/cols)) in spectral norm; weight decay scales w first."""
    rng = np.random.default_rng(62)
    w = rng.standard_normal((30, 10))
    g1, g2 = rng.standard_normal((30, 10)), rng.standard_normal((30, 10))
    w1, u1 = O.muon_update(w, g1, np.zeros_like(w), 0.02, 0.9, 0.0, 60, (1.5, -0.5, 0.0))
    w2, u2 = O.muon_update(w1, g2, u1, 0.02, 0.9, 0.0, 60, (1.5, -0.5, 0.0))
    np.testing.assert_allclose(u2, 0.9 * g1 + g2, rtol=1e-14)
    step = np.linalg.svd(w2 - w1, compute_uv=False)
    np.testing.assert_allclose(step, 0.02 * math.sqrt(3.0), rtol=1e-8)
    w3, _ = O.muon_update(w, g1, np.zeros_like(w), 0.02, 0.9, 0.5, 60, (1.5, -0.5, 0.0))
    np.testing.assert_allclose(w3 - w1, -0.02 * 0.5 * w, rtol=1e-12, atol=1e-15)
