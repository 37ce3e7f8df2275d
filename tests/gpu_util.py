"""Shared helpers for the GPU tests: build seeded inputs, run the HIP library
through its C ABI, run the float64 oracle on the same values, compare."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from decoder_only_transformer_gpt_amd import _lib, synthetic
from oracle import gpt_oracle as O


def require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()  # a missing library on a GPU machine is an error, not a skip
    return torch


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_cfg(c: _lib.gpt_config) -> dict:
    d = c.as_dict()
    d["rope_theta"] = float(np.float32(d["rope_theta"]))
    d["logit_softcap"] = float(np.float32(d["logit_softcap"]))
    d["norm_eps"] = float(np.float32(d["norm_eps"]))
    d["fp8"] = c.dtype == _lib.GPT_FP8_E4M3
    return d


_WEIGHTS: dict = {}


def seeded_weights(shapes, seed: int, dtype: str):
    """synthetic.make_weights, kept for the next test that asks for the same
    draw (the d20 draw takes seconds). The arrays are shared: callers copy
    before changing them."""
    key = (tuple(shapes), seed, dtype)
    if key not in _WEIGHTS:
        while len(_WEIGHTS) >= 2:
            _WEIGHTS.pop(next(iter(_WEIGHTS)))
        _WEIGHTS[key] = synthetic.make_weights(shapes, seed=seed, dtype=dtype)
    return _WEIGHTS[key]


class Case:
    """One configuration with seeded weights and tokens."""

    def __init__(self, cfg: _lib.gpt_config, B: int, T: int, law: str, wseed: int = 0, tseed: int = 1):
        self.cfg, self.B, self.T, self.law = cfg, B, T, law
        self.shapes = [(n, r, c) for n, _, r, c in _lib.gpt_param_layout(cfg)]
        dt = "f32" if cfg.dtype == _lib.GPT_F32 else "bf16"  # FP8 models keep bf16 parameters
        self.storage, self.values = seeded_weights(self.shapes, wseed, dt)
        self.idx, self.tgt = synthetic.make_tokens(B, T, cfg.vocab_size, law, seed=tseed)

    def oracle_params(self) -> dict:
        out, off = {}, 0
        for n, r, c in self.shapes:
            out[n] = self.values[off:off + r * c].reshape(r, c).astype(np.float64)
            off += r * c
        return out

    def flat_grads(self, G: dict) -> np.ndarray:
        return np.concatenate([G[n].reshape(-1) for n, _, _ in self.shapes])


def run_gpu(case: Case, dloss: float = 1.0, accumulate: bool = False, row_loss: bool = True, backward: bool = True,
            max_B: int | None = None, max_T: int | None = None, params_override=None, tile: int = 0,
            hsplit: int = 0, resid_grad_f32: bool = False):
    torch = require_gpu()
    from decoder_only_transformer_gpt_amd.model import GPT
    params = GPT.params_from_numpy(case.storage if params_override is None else params_override, case.cfg)
    m = GPT(case.cfg, params, max_B or case.B, max_T or case.T)
    if tile:
        m.set_gemm_tile(tile)
    if hsplit:
        m.set_dkv_hsplit(hsplit)
    if resid_grad_f32:
        m.set_resid_grad_f32(True)
    idx = torch.from_numpy(case.idx).cuda()
    tgt = torch.from_numpy(case.tgt).cuda()
    rl = torch.zeros(case.B * case.T, dtype=torch.float32, device="cuda") if row_loss else None
    loss = m.forward_loss(idx, tgt, need_grad=backward, row_loss=rl)
    if backward:
        m.backward(dloss, accumulate)
    torch.cuda.synchronize()
    st = m.sync_status()
    out = dict(loss=float(loss.item()), status=st, model=m,
               row_loss=None if rl is None else rl.cpu().numpy().astype(np.float64),
               grads=m.grads.cpu().numpy().astype(np.float64) if backward else None)
    return out


def rel_l2(a, b) -> float:
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def cosine(a, b) -> float:
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(np.dot(a.ravel(), b.ravel()) / (na * nb))


def split_tensors(case: Case, flat: np.ndarray) -> dict:
    """Per-tensor views, with W_qkv split into W_q, W_k, W_v."""
    H, D = case.cfg.n_head, 128
    out, off = {}, 0
    for n, r, c in case.shapes:
        t = flat[off:off + r * c].reshape(r, c)
        off += r * c
        if n.endswith("w_qkv"):
            out[n + ".q"] = t[:H * D]
            out[n + ".k"] = t[H * D:(H + 1) * D]
            out[n + ".v"] = t[(H + 1) * D:]
        else:
            out[n] = t
    return out
