"""Mutation sweep over the oracle (CPU only; not collected by pytest).

Each entry plants one plausible mistake in a temporary copy of
oracle/gpt_oracle.py (a dropped term, a flipped sign, an off-by-one window, a
transposed operand, a swapped learning rate ...) and runs the CPU suite
(`pytest -m "not gpu"`) against that copy. Every mutant must fail some test,
except those listed in EQUIVALENT, which compute the same function.

    python tests/mutate_oracle.py            # all mutants, 4 at a time
    python tests/mutate_oracle.py rope_sign  # named ones

Exit status 0 when every non-equivalent mutant is caught.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY = ("oracle", "tests", "decoder_only_transformer_gpt_amd", "include", "profiles")

MUTS = [
 ("rms_eps", "np.mean(x * x, axis=-1, keepdims=True) + eps)", "np.mean(x * x, axis=-1, keepdims=True))"),
 ("rms_sum", "np.mean(x * x, axis=-1, keepdims=True) + eps)", "np.sum(x * x, axis=-1, keepdims=True) + eps)"),
 ("rmsb_sign", "return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))", "return r * (dy + y * np.mean(dy * y, axis=-1, keepdims=True))"),
 ("rmsb_drop", "return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))", "return r * dy"),
 ("rope_freq", "inv_freq = theta ** (-2.0 * i / D)", "inv_freq = theta ** (-1.0 * i / D)"),
 ("rope_sign", "return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)", "return np.concatenate([x1 * c + x2 * s, -x1 * s + x2 * c], axis=-1)"),
 ("ropeb_sign", "return np.concatenate([d1 * c + d2 * s, -d1 * s + d2 * c], axis=-1)", "return np.concatenate([d1 * c - d2 * s, d1 * s + d2 * c], axis=-1)"),
 ("win_off1", "m &= (t - u) < window", "m &= (t - u) <= window"),
 ("win_last", "if not pattern or short <= 0 or layer == cfg[\"n_layer\"] - 1:", "if not pattern or short <= 0:"),
 ("win_patidx", "pattern[layer % len(pattern)] == \"S\"", "pattern[(layer + 1) % len(pattern)] == \"S\""),
 ("causal_strict", "m = u <= t\n", "m = u < t\n    m[0, 0] = True\n"),
 ("attn_scale", "s = (q[b, :, h, :] @ k[b].T) * scale               # [T(query), T(key)]", "s = (q[b, :, h, :] @ k[b].T)"),
 ("attn_lse", "lse[b, h] = (m + np.log(z))[:, 0]", "lse[b, h] = (np.log(z))[:, 0]"),
 ("attnb_ds", "ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))", "ds = p * dp"),
 ("attnb_dq_scale", "dq[b, :, h, :] = (ds @ k[b]) * scale", "dq[b, :, h, :] = (ds @ k[b])"),
 ("attnb_dk_scale", "return dq, dk_h.sum(axis=1) * scale, dv_h.sum(axis=1)", "return dq, dk_h.sum(axis=1), dv_h.sum(axis=1)"),
 ("attnb_dv", "dv_h[b, h] = p.T @ doh", "dv_h[b, h] = ds.T @ doh"),
 ("softcapb", "return dzc * (1.0 - (zc / c) ** 2)", "return dzc * (1.0 - (zc / c))"),
 ("e4m3_sub", "mag = np.where(e == 0, m / 8.0 * 2.0 ** -6,", "mag = np.where(e == 0, m / 8.0 * 2.0 ** -7,"),
 ("e4m3_enc_rint", "v = np.rint(a / step) * step", "v = np.floor(a / step + 0.5) * step"),
 ("e4m3_enc_sat", "a = np.minimum(np.abs(y), np.float32(E4M3_MAX))", "a = np.minimum(np.abs(y), np.float32(480.0))"),
 ("bf16_trunc", "return np.ldexp(np.rint(m * 256.0), e - 8)", "return np.ldexp(np.trunc(m * 256.0), e - 8)"),
 ("bf16_half", "return np.ldexp(np.rint(m * 256.0), e - 8)", "return np.ldexp(np.floor(m * 256.0 + 0.5), e - 8)"),
 ("fp8_scale", "s = np.float32(E4M3_MAX) / amax if amax > 0 else np.float32(1.0)", "s = np.float32(E4M3_MAX) / amax if amax > 0 else np.float32(0.0)"),
 ("fp8_nobf16", "x32 = round_bf16(x).astype(np.float32)", "x32 = np.asarray(x, dtype=np.float32)"),
 ("fwd_relu", "a = np.maximum(u, 0.0) ** 2", "a = np.maximum(u, 0.0)"),
 ("fwd_qknorm_order", "qr, kr = rope(q, cos, sin), rope(k, cos, sin)\n        qn, rq = rmsnorm(qr, eps)", "qr, kr = rope(q, cos, sin), rope(k, cos, sin)\n        qn, rq = rmsnorm(q, eps)"),
 ("fwd_ve_gate", "v = v + W[\"ve_gates\"][0, vel.index(l)] * W[f\"h{l}.ve\"][idx][:, :, None, :]", "v = v + W[f\"h{l}.ve\"][idx][:, :, None, :]"),
 ("fwd_x0mix", "x = W[\"resid_lambdas\"][0, l] * x + W[\"x0_lambdas\"][0, l] * x0", "x = W[\"resid_lambdas\"][0, l] * x + W[\"x0_lambdas\"][0, l] * xprev"),
 ("ns_c_term", "X = a * X + (b * A + c * (A @ A)) @ X", "X = a * X + (b * A + c * A) @ X"),
 ("bwd_lse_chunk", 'p = np.exp(zc - cache["lse_rows"][s0:s1, None])', 'p = np.exp(zc - cache["lse_rows"][0:s1 - s0, None])'),
 ("lr_swap", 'lrs = dict(embed=oc["lr_embed"], unembed=oc["lr_unembed"]', 'lrs = dict(embed=oc["lr_unembed"], unembed=oc["lr_embed"]'),
 ("fwd_lse_chunk", "row_loss[s0:s1] = lse_rows[s0:s1] - zc[np.arange(s1 - s0), tg[s0:s1]]", "row_loss[s0:s1] = lse_rows[0:s1 - s0] - zc[np.arange(s1 - s0), tg[s0:s1]]"),
 ("fwd_tgt", "row_loss[s0:s1] = lse_rows[s0:s1] - zc[np.arange(s1 - s0), tg[s0:s1]]", "row_loss[s0:s1] = lse_rows[s0:s1] - zc[np.arange(s1 - s0), tg[s0]]"),
 ("bwd_relu2", "du = da * 2.0 * np.maximum(L[\"u\"], 0.0)", "du = da * np.maximum(L[\"u\"], 0.0)"),
 ("bwd_w2_unq", "G[f\"h{l}.w_2\"] += dy.reshape(N, C).T @ L[\"am\"].reshape(N, -1)", "G[f\"h{l}.w_2\"] += dy.reshape(N, C).T @ L[\"a\"].reshape(N, -1)"),
 ("bwd_w1_unq", "G[f\"h{l}.w_1\"] += duq.reshape(N, -1).T @ L[\"h2m\"].reshape(N, C)", "G[f\"h{l}.w_1\"] += du.reshape(N, -1).T @ L[\"h2m\"].reshape(N, C)"),
 ("bwd_ve_gate", "np.add.at(G[f\"h{l}.ve\"], idx.reshape(N), W[\"ve_gates\"][0, j] * dv.reshape(N, D))", "np.add.at(G[f\"h{l}.ve\"], idx.reshape(N), dv.reshape(N, D))"),
 ("bwd_x0", "dx0 = dx0 + W[\"x0_lambdas\"][0, l] * dx", "dx0 = dx0 + dx"),
 ("bwd_resid_l", "G[\"resid_lambdas\"][0, l] += np.sum(dx * L[\"xprev\"])", "G[\"resid_lambdas\"][0, l] += np.sum(dx * cache[\"x0\"])"),
 ("bwd_embed_x0", "de = rmsnorm_bwd(dx + dx0, y0, cache[\"r0\"])", "de = rmsnorm_bwd(dx, y0, cache[\"r0\"])"),
 ("bwd_dloss", "dz = softcap_bwd(p * (dloss / N), zc, c)", "dz = softcap_bwd(p * (1.0 / N), zc, c)"),
 ("bwd_qkv_q", "dqkv = mm_operand(cfg, dqkv)", "pass"),
 ("adam_bc", "w = w - (lr / bc1) * m / (np.sqrt(v) / math.sqrt(bc2) + eps)", "w = w - lr * m / (np.sqrt(v) + eps)"),
 ("adam_wd_order", "w = w * (1.0 - lr * wd)\n    m = beta1", "w = w * (1.0 - wd)\n    m = beta1"),
 ("muon_mom", "u = mu * u + g\n", "u = mu * u + (1.0 - mu) * g\n"),
 ("muon_scale", "scale = math.sqrt(max(1.0, w.shape[0] / w.shape[1]))", "scale = math.sqrt(max(1.0, w.shape[1] / w.shape[0]))"),
 ("muon_wd", "return w * (1.0 - lr * wd) - lr * scale * X, u", "return w - lr * scale * X, u"),
 ("ns_norm", "X = u / (np.linalg.norm(u) + 1e-7)", "X = u / (np.abs(u).max() + 1e-7)"),
 ("grp_ve", "if name == \"wte\" or name.endswith(\".ve\"):", "if name == \"wte\":"),
 ("grp_lmhead", "if name == \"lm_head\":\n        return \"unembed\"", "if name == \"lm_head\":\n        return \"embed\""),
 ("cfg_heads", "n_head=C // D, n_kv_head=n_kv_head,", "n_head=C // 64, n_kv_head=n_kv_head,"),
 ("cfg_mlp", "mlp_dim=4 * C,", "mlp_dim=8 * C // 3,"),
 ("shapes_qkv", "(f\"h{l}.w_qkv\", (H + 2 * Hkv) * D, C)", "(f\"h{l}.w_qkv\", (H + 2) * D, C)"),
 ("theta", "ROPE_THETA = 10000.0", "ROPE_THETA = 100000.0"),
 ("softcap_c", "SOFTCAP = 15.0 ", "SOFTCAP = 30.0 "),
 ("eps", "EPS = 2.0 ** -23 ", "EPS = 1e-6 "),
]

# no pin can tell this one apart: (X X^T) X = X (X^T X), so the orientation
# of the Newton-Schulz iteration changes its cost, not its result
EQUIVALENT = {"ns_orient"}

MUTS += [
 ("split_kv", "k = qkv[..., H * D:(H + Hkv) * D].reshape(B, T, Hkv, D)\n    v = qkv[..., (H + Hkv) * D:].reshape(B, T, Hkv, D)", "v = qkv[..., H * D:(H + Hkv) * D].reshape(B, T, Hkv, D)\n    k = qkv[..., (H + Hkv) * D:].reshape(B, T, Hkv, D)"),
 ("lse_nom", "return (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))[..., 0]", "return (np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))[..., 0]"),
 ("unflat_T", "out[name] = flat[off:off + r * c].reshape(r, c)", "out[name] = flat[off:off + r * c].reshape(c, r).T"),
 ("e4m3_nan", "mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)", "pass"),
 ("e4m3_enc_nan", "code = np.where(np.isnan(y), 0x7F, code)", "pass"),
 ("deq_mul", "return e4m3_decode(codes) / np.float64(s)", "return e4m3_decode(codes) * np.float64(s)"),
 ("adam_beta", "v = beta2 * v + (1.0 - beta2) * g * g", "v = beta1 * v + (1.0 - beta1) * g * g"),
 ("adam_eps", "m / (np.sqrt(v) / math.sqrt(bc2) + eps)", "m / (np.sqrt(v / bc2 + eps))"),
 ("ns_orient", "tr = X.shape[0] > X.shape[1]", "tr = X.shape[0] < X.shape[1]"),
 ("ns_coeff", "X = a * X + (b * A + c * (A @ A)) @ X", "X = a * X + X @ (b * A + c * (A @ A))"),
 ("cos_sin", "return np.cos(ang), np.sin(ang)", "return np.sin(ang), np.cos(ang)"),
 ("pos_restart", "ang = np.arange(T, dtype=np.float64)[:, None] * inv_freq[None, :]", "ang = np.arange(1, T + 1, dtype=np.float64)[:, None] * inv_freq[None, :]"),
 ("ve_layers_odd", "return list(range(0, cfg[\"n_layer\"], 2)) if cfg.get(\"value_embeds\", False) else []", "return list(range(1, cfg[\"n_layer\"], 2)) if cfg.get(\"value_embeds\", False) else []"),
 ("kn_norm_axis", "kn, rk = rmsnorm(kr, eps)", "kn, rk = kr, np.ones(kr.shape[:-1] + (1,))"),
 ("attn_o_resid", "x = x + o2m @ Wm[f\"h{l}.w_o\"].T", "x = o2m @ Wm[f\"h{l}.w_o\"].T"),
 ("final_norm", "hf, rf = rmsnorm(x, eps)\n", "hf, rf = x, np.ones(x.shape[:-1] + (1,))\n"),
 ("loss_sum", "loss = float(row_loss.mean())", "loss = float(row_loss.sum())"),
 ("bwd_ve_gate_grad", "G[\"ve_gates\"][0, j] += np.sum(dv * W[f\"h{l}.ve\"][idx])", "G[\"ve_gates\"][0, j] += np.sum(dv)"),
 ("bwd_x0_grad", "G[\"x0_lambdas\"][0, l] += np.sum(dx * cache[\"x0\"])", "G[\"x0_lambdas\"][0, l] += np.sum(dx * L[\"xprev\"])"),
 ("bwd_kr", "dkr = rmsnorm_bwd(dkn[:, :, None, :], L[\"kn\"], L[\"rk\"])", "dkr = dkn[:, :, None, :] * L[\"rk\"]"),
 ("fp8_amax_empty", "amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)", "amax = np.float32(np.max(x32)) if x32.size else np.float32(0.0)"),
]


def run(mut):
    name, old, new = mut
    with tempfile.TemporaryDirectory(prefix=f"oracle_mut_{name}_") as d:
        for sub in COPY:
            shutil.copytree(os.path.join(ROOT, sub), os.path.join(d, sub),
                            ignore=shutil.ignore_patterns("__pycache__"))
        for f in ("bench.py", "__graft_entry__.py"):
            shutil.copy(os.path.join(ROOT, f), d)
        p = os.path.join(d, "oracle", "gpt_oracle.py")
        s = open(p).read()
        if s.count(old) != 1:
            return name, "STALE", f"pattern found {s.count(old)} times"
        open(p, "w").write(s.replace(old, new))
        r = subprocess.run([sys.executable, "-m", "pytest", "tests/", "-x", "-q", "-m", "not gpu",
                            "-p", "no:cacheprovider"], cwd=d, capture_output=True, text=True,
                           timeout=1200, env=dict(os.environ, OMP_NUM_THREADS="2"))
    out = r.stdout.splitlines()
    first = next((l for l in out if l.startswith(("FAILED", "ERROR"))), out[-1] if out else "")
    return name, "caught" if r.returncode != 0 else "SURVIVED", first


def main(names):
    muts = [m for m in MUTS if not names or m[0] in names]
    bad = 0
    with ThreadPoolExecutor(4) as ex:
        for name, st, info in ex.map(run, muts):
            if name in EQUIVALENT and st == "SURVIVED":
                st = "equivalent"
            bad += st in ("SURVIVED", "STALE")
            print(f"{st:10s} {name:18s} {info[:140]}", flush=True)
    print(f"{len(muts)} mutants, {bad} not caught")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
