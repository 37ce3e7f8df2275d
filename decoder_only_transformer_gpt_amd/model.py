"""Thin torch-facing wrapper over the C ABI: owns the device tensors the
library computes into (parameters, fp32 gradients, workspace) and passes their
pointers and the current stream through. No arithmetic happens here."""
from __future__ import annotations

import numpy as np
import torch

from . import _lib


class GPT:
    def __init__(self, cfg: _lib.gpt_config, params: torch.Tensor, max_B: int, max_T: int, device="cuda"):
        self.cfg = cfg
        self.layout = _lib.gpt_param_layout(cfg)
        n = _lib.gpt_param_count(cfg)
        dt = torch.float32 if cfg.dtype == _lib.GPT_F32 else torch.bfloat16  # FP8 models keep bf16 parameters
        if params.dtype != dt or params.numel() != n or not params.is_cuda:
            raise ValueError(f"params must be a cuda {dt} tensor of {n} elements")
        self.params = params.contiguous()
        self.grads = torch.zeros(n, dtype=torch.float32, device=device)
        self.ws_bytes = _lib.gpt_workspace_bytes(cfg, max_B, max_T)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        self._stream = torch.cuda.current_stream().cuda_stream
        self.h = _lib.gpt_init(cfg, self.params.data_ptr(), self.grads.data_ptr(), self.ws.data_ptr(),
                               self.ws_bytes, max_B, max_T, self._stream)
        self._inputs = None

    @staticmethod
    def params_from_numpy(storage: np.ndarray, cfg: _lib.gpt_config, device="cuda") -> torch.Tensor:
        if cfg.dtype != _lib.GPT_F32:
            return torch.from_numpy(storage.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(storage).to(device)

    def stream(self) -> int:
        return torch.cuda.current_stream().cuda_stream

    def forward_loss(self, idx: torch.Tensor, targets: torch.Tensor, need_grad: bool = True,
                     row_loss: torch.Tensor | None = None) -> torch.Tensor:
        B, T = idx.shape
        assert idx.dtype == torch.int32 and targets.dtype == torch.int32 and idx.is_contiguous()
        self._inputs = (idx, targets)  # the library reads them again in backward
        _lib.gpt_forward_loss(self.h, idx.data_ptr(), targets.data_ptr(), B, T, int(need_grad),
                              self.loss.data_ptr(), None if row_loss is None else row_loss.data_ptr(),
                              self.stream())
        return self.loss

    def backward(self, dloss: float = 1.0, accumulate: bool = False):
        _lib.gpt_backward(self.h, float(dloss), int(accumulate), self.stream())

    def sync_status(self) -> int:
        return _lib.gpt_sync_status(self.h, self.stream())

    def grad_tensors(self) -> dict:
        return {name: self.grads[off:off + r * c].view(r, c) for name, off, r, c in self.layout}

    def debug_tensor(self, name: str, layer: int, shape, dtype) -> torch.Tensor:
        """A torch view of a stashed activation (copy it before the next call)."""
        ptr, nbytes = _lib.gpt_debug_buffer(self.h, name, layer)
        base = self.ws.data_ptr()
        off = ptr - base
        return self.ws[off:off + nbytes].view(dtype).view(*shape)

    def set_gemm_tile(self, tile: int):
        _lib.gpt_set_option(self.h, _lib.GPT_OPT_GEMM_TILE, tile)

    def set_dkv_hsplit(self, hsplit: int):
        _lib.gpt_set_option(self.h, _lib.GPT_OPT_DKV_HSPLIT, hsplit)

    def set_resid_grad_f32(self, on: bool):
        _lib.gpt_set_option(self.h, _lib.GPT_OPT_RESID_GRAD, 1 if on else 0)

    def close(self):
        if self.h is not None:
            _lib.gpt_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
