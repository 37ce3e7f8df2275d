"""Host logic behind the reported figures, no GPU needed: bench.py's
algorithmic FLOP and byte counts and profsum's traffic-report checks, pinned
to closed forms, brute-force counts and invariants that tie the per-launch
figures to the whole step."""
import os

import pytest

import bench
from decoder_only_transformer_gpt_amd import _lib, profsum
from decoder_only_transformer_gpt_amd.workloads import WORKLOADS

D = 128

# call sites per step: layer products once per layer, the LM head once
LAYER_GEMMS = ("gemm_qkv", "gemm_o", "gemm_w1_relu2", "gemm_w2", "gemm_w2_dw", "gemm_w2_dx", "gemm_w1_dw",
               "gemm_w1_dx_relu2bwd", "gemm_o_dw", "gemm_o_dx", "gemm_qkv_dw", "gemm_qkv_dx")
HEAD_GEMMS = ("gemm_lm_head_softcap", "gemm_lm_head_dw", "gemm_lm_head_dx")


def brute_pairs(T, W):
    """(query, key) pairs with key <= query and, for W > 0, query - key < W."""
    return sum(1 for q in range(T) for k in range(q + 1) if W <= 0 or q - k < W)


@pytest.mark.parametrize("T,W", [(1, 0), (7, 0), (64, 0), (9, 3), (20, 20), (20, 25), (33, 1), (50, 16)])
def test_attn_pairs_brute_force(T, W):
    assert bench.attn_pairs(T, W) == brute_pairs(T, W)


def n_matmul(cfg):
    C, H, F, V, L = cfg.model_dim, cfg.n_head, cfg.mlp_dim, cfg.vocab_size, cfg.n_layer
    return L * ((H + 2) * D * C + C * H * D + 2 * F * C) + V * C


@pytest.mark.parametrize("wl", ["d4", "d12", "d20", "d20-sssl", "d24fp8"])
def test_gemm_call_sites_add_up_to_six_flops_per_weight(wl):
    """Forward 2 N P, backward dX + dW 4 N P: the per-launch GEMM figures over
    one step's launches sum to 6 N P (P = matmul weights, N = B T tokens)."""
    w = WORKLOADS[wl]
    cfg = w.config()
    B, T = w.batch, w.seq_len
    tot = sum(cfg.n_layer * bench.kernel_flops_per_launch(t, cfg, B, T) for t in LAYER_GEMMS)
    tot += sum(bench.kernel_flops_per_launch(t, cfg, B, T) for t in HEAD_GEMMS)
    assert tot == pytest.approx(6.0 * B * T * n_matmul(cfg), rel=1e-12)


@pytest.mark.parametrize("wl", ["d20", "d20-sssl"])
def test_attention_launches_add_up_to_the_step_term(wl):
    """Forward, dQ and dK/dV launches (4 D per needed pair each, one per layer)
    give the step's attention term 12 H D x pairs; a windowed layer counts only
    the pairs inside its band."""
    w = WORKLOADS[wl]
    cfg = w.config()
    B, T, H, L = w.batch, w.seq_len, cfg.n_head, cfg.n_layer
    per_launch = sum(bench.kernel_flops_per_launch(t, cfg, B, T)
                     for t in ("attn_fwd", "attn_bwd_dq", "attn_bwd_dkv"))
    step_attn = bench.step_flops(cfg, T)["total"] - 6.0 * n_matmul(cfg)
    assert per_launch * L == pytest.approx(step_attn * B * T, rel=1e-12)
    if wl == "d20":
        assert step_attn == pytest.approx(12.0 * L * H * D * (T + 1) / 2, rel=1e-12)
    else:
        assert step_attn < 12.0 * L * H * D * (T + 1) / 2


def test_d20_flops_per_token_and_peak():
    """2.8234 GFLOP per d20 token (6 P + 6 L H D (T + 1)); the bf16 peak is
    256 CUs x 4096 FLOP/clk x 2.4 GHz."""
    cfg = WORKLOADS["d20"].config()
    f = bench.step_flops(cfg, 2048)
    assert f["total"] == pytest.approx(6 * 418_119_680 + 6 * 20 * 10 * 128 * 2049, rel=1e-12)
    assert round(f["total"] / 1e9, 4) == 2.8234
    assert f["palm"] == pytest.approx(6 * 418_119_680 + 12 * 20 * 10 * 128 * 2048, rel=1e-12)
    assert bench.PEAK_BF16_TFLOPS == pytest.approx(256 * 4096 * 2.4e9 / 1e12, rel=1e-4)


def test_layer_windows_follow_the_pattern_and_keep_the_last_layer_full():
    cfg = WORKLOADS["d20-sssl"].config()
    ws = bench.layer_windows(cfg)
    assert len(ws) == cfg.n_layer and ws[-1] == 0
    pat = cfg.window_pattern.decode()
    for l, w in enumerate(ws[:-1]):
        assert w == (cfg.window_short if pat[l % len(pat)] == "S" else 0)
    assert all(w == 0 for w in bench.layer_windows(WORKLOADS["d20"].config()))


def test_row_kernel_bytes_per_token():
    """The algorithmic bytes of the row kernels per token, bf16 activations
    (a = 2 bytes), fp32 statistics."""
    cfg = WORKLOADS["d20"].config()
    C, H = cfg.model_dim, cfg.n_head
    per = {t: bench.kernel_bytes_per_launch(t, cfg, 1, 1, 2) for t in
           ("rmsnorm", "rmsnorm_bwd", "embed_rmsnorm", "rope_qknorm", "rope_qknorm_bwd", "attn_fwd_transpose")}
    assert per["rmsnorm"] == 4 * C + 4
    assert per["rmsnorm_bwd"] == 8 * C + 4    # the residual gradient kept in bf16
    assert per["embed_rmsnorm"] == 4 + 4 * C + 4
    assert per["rope_qknorm"] == 4 * (H + 1) * D + 4 * (H + 1)
    assert per["rope_qknorm_bwd"] == 6 * (H + 1) * D + 4 * (H + 1)
    assert per["attn_fwd_transpose"] == 4 * D
    # embedding backward: per token the bf16 gradient row and 12 bytes, every
    # dwte row once (fp32), one embedding row per distinct id
    V = cfg.vocab_size
    assert bench.kernel_bytes_per_launch("embed_bwd", cfg, 2, 3, 2, distinct=5) == 6 * (2 * C + 12) + V * C * 4 + 5 * C * 2
    # ...for the whole step: the zeroing of dwte and the segment sums are two
    # launches of that tag, counted once between them
    assert bench.STEP_BYTE_TAGS == {"embed_bwd"}
    assert bench.kernel_bytes_per_launch("gemm_qkv", cfg, 2, 3, 2) is None


def test_traffic_report_is_read_only_while_its_sources_match(tmp_path):
    tag = "gemm_w2_dx"
    good = tmp_path / "ok.txt"
    good.write_text(f"tag: {tag}\ntraffic_bytes_per_launch: 123456\nsource_sha256: {profsum.source_digest(tag)}\n")
    assert profsum.read_traffic(str(good), tag) == 123456.0
    stale = tmp_path / "stale.txt"
    stale.write_text(f"tag: {tag}\ntraffic_bytes_per_launch: 123456\nsource_sha256: {'0' * 64}\n")
    assert profsum.read_traffic(str(stale), tag) is None
    assert profsum.read_traffic(str(good), "attn_bwd_dkv") is None      # another kernel's report
    assert profsum.read_traffic(str(tmp_path / "missing.txt"), tag) is None


def test_committed_traffic_reports_match_the_sources():
    """The reports under profiles/ were taken from the kernels as they are."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for tag in ("gemm_w2_dx", "attn_bwd_dkv"):
        v = profsum.read_traffic(os.path.join(root, "profiles", f"{tag}_d20_traffic.txt"), tag)
        assert v is not None and v > 0, tag


def test_every_kernel_tag_has_sources():
    """Every tag the library times maps to the source files of its kernels."""
    csrc = os.path.join(os.path.dirname(profsum.__file__), "csrc")
    for t in _lib.gpt_kernel_tag_names():
        files = profsum.sources_for_tag(t)
        assert files and all(os.path.exists(os.path.join(csrc, f)) for f in files), t
