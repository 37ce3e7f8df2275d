"""Training-step throughput of the HIP library on one MI355X.

A step is gpt_forward_loss(need_grad=1) + gpt_backward on one stream, over one
synthetic batch already resident in HBM: the whole forward and backward pass
of nanochat's GPT (no optimiser, no data loading). Default workload: d20
(depth 20, width 1280, 10 query heads / 1 K/V head, MLP 5120, vocab 65,536),
batch 32 x 2048 Zipf(1.1) tokens, bf16 weights/activations with fp32
accumulation and fp32 gradients.

Prints one JSON line: tokens/s, bf16 MFU, the roofline of the kernel with the
largest share of step time (timed with HIP events on the library's stream
inside the timed region) and the float64 oracle's throughput on a bounded
sample on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CUs x 4096 FLOP/clk x 2.4 GHz ("2.5 PFLOP/s")
PEAK_FP32_TFLOPS = 157.3
PEAK_FP8_TFLOPS = 5033.2    # dense fp8 (e4m3) MFMA, twice the bf16 rate
# call sites whose operands are e4m3 codes in FP8 models
FP8_TAGS = ("gemm_qkv", "gemm_o", "gemm_w1_relu2", "gemm_w2", "gemm_w2_dw", "gemm_w2_dx", "gemm_w1_dw",
            "gemm_w1_dx_relu2bwd", "gemm_o_dw", "gemm_o_dx", "gemm_qkv_dw", "gemm_qkv_dx")
PEAK_HBM_GBS = 8000.0
METRIC = "train tokens/sec + bf16 MFU, d20 fwd+bwd, seq 2048, 1 MI355X"


def layer_windows(cfg) -> list:
    """Sliding window of every layer (0 = full causal prefix): the pattern
    repeats over the layers, 'S' selects window_short, the last layer is full."""
    pat = cfg.window_pattern.decode() if isinstance(cfg.window_pattern, bytes) else cfg.window_pattern
    out = []
    for l in range(cfg.n_layer):
        w = 0
        if pat and cfg.window_short > 0 and l != cfg.n_layer - 1 and pat[l % len(pat)] == "S":
            w = cfg.window_short
        out.append(w)
    return out


def attn_pairs(T: int, W: int) -> int:
    """(query, key) pairs a layer needs per sequence: causal, within W if W > 0."""
    if W <= 0 or W >= T:
        return T * (T + 1) // 2
    return W * (W + 1) // 2 + (T - W) * W


def step_flops(cfg, T: int) -> dict:
    """Algorithmic FLOPs per token (fwd+bwd): 6 x matmul weights + attention over
    the needed (query, key) pairs only (T(T+1)/2 per sequence for a causal
    layer, fewer for a sliding-window one); the embedding gather counts zero."""
    C, H, D, F, V, L = cfg.model_dim, cfg.n_head, 128, cfg.mlp_dim, cfg.vocab_size, cfg.n_layer
    n_mm = L * ((H + 2) * D * C + C * H * D + 2 * F * C) + V * C
    attn = sum(12.0 * H * D * attn_pairs(T, w) / T for w in layer_windows(cfg))
    return {"total": 6.0 * n_mm + attn, "palm": 6.0 * n_mm + 12.0 * L * H * D * T}


def kernel_flops_per_launch(tag: str, cfg, B: int, T: int) -> float | None:
    """Algorithmic FLOPs of one launch of a GEMM / attention call site."""
    N, C, H, F, V, D = B * T, cfg.model_dim, cfg.n_head, cfg.mlp_dim, cfg.vocab_size, 128
    QKV, HD = (H + 2) * D, H * D
    g = {"gemm_qkv": (N, QKV, C), "gemm_o": (N, C, HD), "gemm_w1_relu2": (N, F, C), "gemm_w2": (N, C, F),
         "gemm_lm_head_softcap": (N, V, C), "gemm_lm_head_dw": (V, C, N), "gemm_lm_head_dx": (N, C, V),
         "gemm_w2_dw": (C, F, N), "gemm_w2_dx": (N, F, C), "gemm_w1_dw": (F, C, N), "gemm_w1_dx_relu2bwd": (N, C, F),
         "gemm_o_dw": (C, HD, N), "gemm_o_dx": (N, HD, C), "gemm_qkv_dw": (QKV, C, N), "gemm_qkv_dx": (N, C, QKV)}
    if tag in g:
        m, n, k = g[tag]
        return 2.0 * m * n * k
    # causal attention counts only the T(T+1)/2 needed (query, key) pairs; per
    # pair the forward's S and PV contractions are 2D FLOPs each. The backward's
    # four contractions (dP, dQ, dK, dV; 2D each) are split between its two
    # kernels: dP and dQ to the dQ kernel, dK and dV to the dK/dV kernel. The
    # recomputation of S (both kernels) and of dP (the dK/dV kernel) is not
    # algorithmic work and is not counted.
    # per-launch pairs: the mean over the layers (one launch per layer)
    ws = layer_windows(cfg)
    pairs = B * H * sum(attn_pairs(T, w) for w in ws) / len(ws)
    if tag == "attn_fwd":
        return 4.0 * D * pairs
    if tag in ("attn_bwd_dq", "attn_bwd_dkv"):
        return 4.0 * D * pairs
    return None


# tags whose byte figure below covers all of the tag's launches in a step
STEP_BYTE_TAGS = {"embed_bwd"}


def kernel_bytes_per_launch(tag: str, cfg, B: int, T: int, es: int, distinct: int = 0,
                            fp8: bool = False) -> float | None:
    """Algorithmic HBM bytes of one launch of a memory-bound kernel (distinct:
    the number of distinct token ids in the batch; fp8: an FP8 model, whose
    layer weights get e4m3 copies instead of bf16 transposes)."""
    N, C, H, V, F = B * T, cfg.model_dim, cfg.n_head, cfg.vocab_size, cfg.mlp_dim
    L, QKV = cfg.n_layer, (H + 2) * 128
    # FP8 operand passes: per layer the forward quantises h1, o, h2, a and the
    # backward dy (twice), du, dqkv -- 8 tensors, N (4C + 2F + (H+2)128)
    # elements in all; per launch the mean. amax reads each element (bf16),
    # the quantiser reads it and writes two codes.
    q_elems = N * (4 * C + 2 * F + (H + 2) * 128) / 8
    b = {"fp8_amax": 2 * q_elems, "fp8_quantize": 4 * q_elems,
         "embed_rmsnorm": N * (4 + 2 * C * es + 4), "rmsnorm": N * (2 * C * es + 4),
         "rope_qknorm": N * (2 * (H + 1) * 128 * es + 4 * (H + 1)),
         "ce_bwd": N * (2 * C * es + 16 + es),  # lse, z'_t, target, r; the target entry; h in, r*h out
         # dy and y in, the residual-stream gradient in and out (kept in the
         # activation dtype by default), rstd
         "rmsnorm_bwd": N * (4 * C * es + 4),
         "rope_qknorm_bwd": N * (3 * (H + 1) * 128 * es + 4 * (H + 1)),
         # transposed copies: read and write each (V; then Q, K, dO) once, plus delta's
         # read of O and dO and its fp32 write
         "attn_fwd_transpose": N * 128 * es * 2,
         "attn_bwd_prep": N * (2 * (2 * H + 1) * 128 * es + 2 * H * 128 * es + 4 * H),
         # per row: the V/64 fp32 exp partials and z'_t in, lse and the row loss out, the mean's read
         "ce_loss": N * (V // 64 * 4 + 16),
         # the residual-gradient rows (activation dtype), rstd and the sorted (id, position)
         # pairs in; every dwte row written once (zeros included); one embedding row per
         # distinct id (for the step: the zeroing and the segment sums together)
         "embed_bwd": N * (C * es + 12) + V * C * 4 + distinct * C * es,
         # two radix passes over (id, position) pairs plus the initial pairs
         "embed_sort": N * (4 + 8 + 2 * 16),
         # every weight the dX products read transposed (FP8 models: the LM head only):
         # read and written once
         "weight_transpose": 2 * es * ((0 if fp8 else L * (QKV * C + C * H * 128 + 2 * F * C)) + V * C)}
    return b.get(tag)


def environment(torch) -> dict:
    """GPU name and architecture, HIP/ROCm versions, engine clock, measured
    device copy bandwidth and the host CPU model."""
    import glob
    import subprocess
    props = torch.cuda.get_device_properties(0)
    env = {"gpu": props.name, "arch": getattr(props, "gcnArchName", ""), "cus": props.multi_processor_count,
           "hbm_gib": round(props.total_memory / 2**30, 1), "hip": torch.version.hip, "torch": torch.__version__}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    sclk = None
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                lines = f.read().split("\n")
            sclk = next((ln.split(":", 1)[1].replace("*", "").strip() for ln in lines if ln.endswith("*")), None)
            if sclk:
                break
        except OSError:
            pass
    # rocm-smi is a Python script started through env: under a profiler whose
    # library is preloaded into every child, that hop is an exec after GPU
    # initialisation, so it is only asked when nothing is preloaded.
    if sclk is None and "rocprof" not in os.environ.get("LD_PRELOAD", ""):
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
            d = json.loads(r.stdout[r.stdout.index("{"):]) if "{" in r.stdout else {}
            for card in d.values():
                if isinstance(card, dict):
                    sclk = next((v for k, v in card.items() if "sclk" in k.lower()), None)
                if sclk:
                    break
        except Exception:
            pass
    env["sclk"] = sclk
    # device copy bandwidth: 1 GiB read + 1 GiB written, best of 6 copies, HIP events
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    best = float("inf")
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    env["copy_gbs"] = round(2 * 4 * n / (best * 1e-3) / 1e9, 1)
    del src, dst
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    env["cpu"] = cpu
    env["host_cores"] = len(os.sched_getaffinity(0))
    return env


def cpu_baseline(cfg_lib, seconds_hint: float = 20.0) -> dict:
    """The float64 oracle, as it stands, on a bounded sample of the workload."""
    import numpy as np

    from decoder_only_transformer_gpt_amd import _lib, synthetic
    from oracle import gpt_oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    B, T = 1, 2048
    shapes = [(n, r, c) for n, _, r, c in _lib.gpt_param_layout(cfg_lib)]
    _, vals = synthetic.make_weights(shapes, seed=0, dtype="f32" if cfg_lib.dtype == _lib.GPT_F32 else "bf16")
    idx, tgt = synthetic.make_tokens(B, T, cfg_lib.vocab_size, "zipf", seed=1)
    P, off = {}, 0
    for n, r, c in shapes:
        P[n] = vals[off:off + r * c].reshape(r, c).astype(np.float64)
        off += r * c
    oc = cfg_lib.as_dict()
    oc["norm_eps"] = float(np.float32(oc["norm_eps"]))
    oc["fp8"] = cfg_lib.dtype == _lib.GPT_FP8_E4M3
    t0 = time.perf_counter()
    O.step(oc, P, idx, tgt)
    dt = time.perf_counter() - t0
    return {"value": round(B * T / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 NumPy oracle, one fwd+bwd of the same model on 1 x {T} Zipf tokens "
                      f"({dt:.1f} s, {len(os.sched_getaffinity(0))} host cores visible)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="d20", choices=["tiny", "d4", "d12", "d20", "d20-sssl", "d24fp8", "d20-ve"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--optimizer", action="store_true",
                    help="also time the optimiser step (Muon + AdamW) after the timed region; reported apart")
    ap.add_argument("--gemm-tile", type=int, default=0, choices=[0, 1, 2, 3],
                    help="force one GEMM tile variant (0 = by shape)")
    ap.add_argument("--resid-grad-f32", action="store_true",
                    help="keep the residual-stream gradient in fp32 (default for bf16 models: bf16)")
    ap.add_argument("--kernel-table", action="store_true", help="print per-tag timings to stderr")
    ap.add_argument("--dominant", default=None,
                    help="kernel tag to report in the roofline (skips the one-step-per-tag scan)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one torch.neg over a buffer of this many MiB (reference kernel for "
                         "the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from decoder_only_transformer_gpt_amd import _lib, synthetic
    from decoder_only_transformer_gpt_amd.model import GPT
    from decoder_only_transformer_gpt_amd.workloads import WORKLOADS

    wl = WORKLOADS[args.workload]
    cfg = wl.config()
    B, T = wl.batch, wl.seq_len
    torch.cuda.set_device(0)
    shapes = [(n, r, c) for n, _, r, c in _lib.gpt_param_layout(cfg)]
    storage, _ = synthetic.make_weights(shapes, seed=0, dtype="f32" if wl.dtype == "f32" else "bf16")
    idx_np, tgt_np = synthetic.make_tokens(B, T, cfg.vocab_size, wl.tokens, seed=1)
    m = GPT(cfg, GPT.params_from_numpy(storage, cfg), B, T)
    if args.gemm_tile:
        m.set_gemm_tile(args.gemm_tile)
    if args.resid_grad_f32:
        m.set_resid_grad_f32(True)
    idx = torch.from_numpy(idx_np).cuda()
    tgt = torch.from_numpy(tgt_np).cuda()
    print(f"[bench] workload {wl.name}: B={B} T={T} params={_lib.gpt_param_count(cfg)} "
          f"workspace={m.ws_bytes / 2**30:.1f} GiB", file=sys.stderr, flush=True)

    def step():
        m.forward_loss(idx, tgt, need_grad=True)
        m.backward(1.0, accumulate=False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if m.sync_status() != _lib.GPT_OK:
        raise RuntimeError("device flag raised during warmup")

    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # one profiled step (every launch timed) to find the kernel with the largest share of time
    tags = _lib.gpt_kernel_tag_names()
    per_tag = {}
    if args.dominant is None or args.kernel_table:
        for t_i, t in enumerate(tags):
            _lib.gpt_profile_begin(m.h, t_i)
            step()
            ms, n = _lib.gpt_profile_end(m.h)
            if n:
                per_tag[t] = (ms, n)
    dominant = args.dominant or max(per_tag, key=lambda t: per_tag[t][0])
    if args.kernel_table:
        tot = sum(v[0] for v in per_tag.values())
        distinct = int(np.unique(idx_np).size)
        for t, (ms, n) in sorted(per_tag.items(), key=lambda kv: -kv[1][0]):
            f = kernel_flops_per_launch(t, cfg, B, T)
            kb = kernel_bytes_per_launch(t, cfg, B, T, 4 if wl.dtype == "f32" else 2, distinct, wl.dtype == "fp8")
            # the embedding backward's bytes are the step's: its zeroing of dwte
            # and its segment sums are two launches of the one tag
            nb = 1 if t in STEP_BYTE_TAGS else n
            rate = f"{f * n / ms / 1e9:8.1f} TFLOP/s" if f else (f"{kb * nb / ms / 1e6:8.1f} GB/s" if kb else "")
            print(f"[bench] {t:24s} {ms:9.3f} ms {n:4d} launches {100 * ms / tot:5.1f}% {rate}",
                  file=sys.stderr, flush=True)

    # timed region: K steps, the dominant kernel's launches timed with HIP events
    # on its stream, and every step bracketed by HIP events on the same stream
    dom_tag = tags.index(dominant)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _lib.gpt_profile_begin(m.h, dom_tag)
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dom_ms, dom_n = _lib.gpt_profile_end(m.h)
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    if m.sync_status() != _lib.GPT_OK:
        raise RuntimeError("device flag raised")
    loss = float(m.loss.item())

    elapsed = t1 - t0
    tokens = B * T * args.steps
    tok_s = tokens / elapsed
    fl = step_flops(cfg, T)
    mfu = fl["total"] * tok_s / (PEAK_BF16_TFLOPS * 1e12)
    avg_ms = dom_ms / max(dom_n, 1)
    es = 4 if wl.dtype == "f32" else 2
    kf = kernel_flops_per_launch(dominant, cfg, B, T)
    if kf is not None:
        peak = PEAK_FP32_TFLOPS if wl.dtype == "f32" else PEAK_BF16_TFLOPS
        if wl.dtype == "fp8" and dominant in FP8_TAGS:
            peak = PEAK_FP8_TFLOPS
        achieved = kf / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None}
    else:
        kb = kernel_bytes_per_launch(dominant, cfg, B, T, es) or 0.0
        achieved = kb / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    from decoder_only_transformer_gpt_amd import profsum
    tr = profsum.read_traffic(os.path.join(ROOT, "profiles", f"{dominant}_{wl.name}_traffic.txt"), dominant)
    roof["traffic"] = None if tr is None else round(tr)
    roof.update({"kernel": dominant, "launches": dom_n, "avg_ms": round(avg_ms, 4)})

    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(1e3 * elapsed / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3 (QKV/O/MLP) + bf16" if wl.dtype == "fp8" else wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: depth {cfg.n_layer}, width {cfg.model_dim}, {cfg.n_head} query heads / "
                               f"1 kv head, head_dim 128, MLP {cfg.mlp_dim}, vocab {cfg.vocab_size}"
                               + (f", windows {wl.window_pattern} (short {wl.window_short})" if wl.window_pattern
                                  else "")
                               + (", resid/x0 lambdas" if wl.x0_lambdas else "")
                               + (", value embeddings on even layers" if wl.value_embeds else ""),
                   "global_batch": B, "seq_len": T, "tokens": wl.tokens, "parallelism": "single GPU"},
        "mfu_bf16": round(mfu, 4), "mfu_palm_convention": round(fl["palm"] * tok_s / (PEAK_BF16_TFLOPS * 1e12), 4),
        "loss": round(loss, 5), "roofline": roof,
        "step_ms_events": {"median": round(float(np.median(step_ms)), 3), "mean": round(float(np.mean(step_ms)), 3),
                           "min": round(min(step_ms), 3), "max": round(max(step_ms), 3)},
        "env": environment(torch),
    }
    if args.optimizer:
        oc = _lib.gpt_optim_config()
        oc.lr_muon, oc.lr_embed, oc.lr_unembed, oc.lr_scalar = 0.02, 0.3, 0.004, 0.5
        oc.momentum, oc.beta1, oc.beta2, oc.eps = 0.95, 0.8, 0.95, 1e-10
        oc.wd_muon, oc.wd_adamw, oc.ns_steps = 0.0, 0.0, 5
        oc.ns_a, oc.ns_b, oc.ns_c = 1.5, -0.5, 0.0
        master = m.params.float()
        state = torch.zeros(_lib.gpt_optimizer_state_elems(cfg), dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        _lib.gpt_optimizer_step(m.h, oc, master.data_ptr(), state.data_ptr(), 1, stream)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for t in range(2, 2 + args.steps):
            _lib.gpt_optimizer_step(m.h, oc, master.data_ptr(), state.data_ptr(), t, stream)
        torch.cuda.synchronize()
        out["optimizer_ms_per_step"] = round(1e3 * (time.perf_counter() - t2) / args.steps, 3)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
