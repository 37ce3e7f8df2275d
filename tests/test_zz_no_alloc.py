"""The no-allocation variant of the e4m3 matmul (split-K partials in the
library's fixed device array) against the entry point that takes a caller
buffer: same codes, same kernels, so the outputs must be equal bit for bit.
Two calls in a row, the second smaller (the fixed array keeps the first
call's partials, which the second must not read), then a size past the
array's limit is rejected before any work is queued."""
import numpy as np
import pytest

from decoder_only_transformer_gpt_amd import _lib, synthetic

import gpu_util as U

pytestmark = pytest.mark.gpu

SCRATCH_FLOATS = 4 << 20


def _codes(torch, rng, rows, cols, std):
    vals = (rng.standard_normal((rows, cols)) * std).astype(np.float32)
    bits = synthetic.f32_to_bf16_bits(vals)
    x = torch.from_numpy(bits.view(np.int16)).cuda()
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    amax = torch.empty((1,), dtype=torch.float32, device="cuda")
    _lib.gpt_fp8_quantize(x.data_ptr(), rows, cols, q.data_ptr(), None, 0, amax.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    return q, amax


def _both(torch, M, N, K, splits, seed):
    rng = np.random.default_rng(seed)
    qa, am_a = _codes(torch, rng, M, K, 1.0)
    qb, am_b = _codes(torch, rng, N, K, 0.05)
    stream = torch.cuda.current_stream().cuda_stream
    ref = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    part = torch.empty((splits, M, N), dtype=torch.float32, device="cuda")
    _lib.gpt_fp8_matmul(qa.data_ptr(), K, am_a.data_ptr(), qb.data_ptr(), K, am_b.data_ptr(), M, N, K,
                        _lib.GPT_F32, ref.data_ptr(), N, 0, splits, part.data_ptr(), stream)
    got = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    _lib.gpt_fp8_matmul_noalloc(qa.data_ptr(), K, am_a.data_ptr(), qb.data_ptr(), K, am_b.data_ptr(), M, N, K,
                                _lib.GPT_F32, got.data_ptr(), N, 0, splits, stream)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_noalloc_matmul_equals_buffered_two_calls():
    torch = U.require_gpu()
    for M, N, K, splits, seed in [(640, 512, 2048, 8, 1), (300, 260, 1024, 3, 2)]:
        U.log(f"case fp8 matmul noalloc M={M} N={N} K={K} splits={splits}")
        ref, got = _both(torch, M, N, K, splits, seed)
        assert np.all(np.isfinite(ref))
        np.testing.assert_array_equal(got, ref)


def test_noalloc_matmul_without_split_and_size_limit():
    torch = U.require_gpu()
    U.log("case fp8 matmul noalloc splits=1 and the size limit")
    ref, got = _both(torch, 96, 128, 256, 1, 3)
    np.testing.assert_array_equal(got, ref)
    # splits * M * N just past the fixed array: rejected before any launch
    # (the buffers are real and large enough, so nothing depends on the check's order)
    M, N, K = 1024, 1024, 256
    splits = SCRATCH_FLOATS // (M * N) + 1
    rng = np.random.default_rng(4)
    qa, am_a = _codes(torch, rng, M, K, 1.0)
    qb, am_b = _codes(torch, rng, N, K, 1.0)
    out = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    with pytest.raises(_lib.GptError, match="exceeds"):
        _lib.gpt_fp8_matmul_noalloc(qa.data_ptr(), K, am_a.data_ptr(), qb.data_ptr(), K, am_b.data_ptr(), M, N, K,
                                    _lib.GPT_F32, out.data_ptr(), N, 0, splits, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert not out.any()
