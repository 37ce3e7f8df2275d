"""Float64 CPU oracle for one pretraining step (forward + backward) of nanochat's GPT.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module. The product path (the HIP library
and its Python binding) never calls it and shares no code with it.

Every function below is the plain definition of what it computes, in float64,
with no blocking or fusion beyond chunking the LM head over rows to bound
memory. It takes the exact values the GPU holds (fp32 or bf16 widened to
float64) and rounds nothing in between.

Citation keys (page, then section on that page):

* [P1] aethryn.com, "Nanochat: full-stack LLM training in 8,000 lines for $72";
  sections "One dial controls everything" and "A Llama-class transformer with
  ten modern departures".
* [P2] aimarketly.com model card "nanochat-train" with the nanochat README;
  section "Precision / dtype".
* [P4] atlas.blal.pro wiki "nanochat — full-stack ChatGPT in ~8k lines";
  section "How it works", item "0. The model".
* [P5] energyai.berlin, "nanochat vs GPT-OSS"; section "Architectural
  decisions" (subsections RoPE, RMSNorm, MQA, Squared ReLU, QK normalization,
  Logit softcap) and section "Model scale and parameters".

Readings where the pages are silent (each also fixed in the HIP path):

* RMSNorm has no gain and eps = 2**-23 everywhere (the pages give no formula).
* Attention scale is 1/sqrt(D) (SDPA's default; the pages name SDPA as the
  fallback path).
* RoPE pairs element i with i + D/2 ("split halves"), rotates by +angle with
  angle = t * theta**(-2i/D), positions restart at 0 in every batch row.
* QK-norm is a per-(token, head) RMSNorm over D, applied after RoPE.
* Plain causal mask over the whole row; no document masking.
* Sliding windows ([P1] "A Llama-class transformer...": the "SSSL" pattern of
  three short-window layers then one full-context layer, the final layer
  always full; [P4] item 0: a per-layer window pattern) are optional and off
  by default. A short window W admits key u for query t iff 0 <= t - u < W
  (the query itself and the W-1 tokens before it); the pages do not say
  whether the window counts the query token.
* Loss is the mean over all B*T positions; targets are given explicitly.
* FP8 matmuls (optional, cfg["fp8"]): readings listed with the e4m3
  functions below. Quantisation decisions are taken in fp32, as the kernels
  take them; everything else stays float64.
* Residual scalars (optional, cfg["x0_lambdas"]; [P1] "A Llama-class
  transformer...": per-layer resid_lambdas and x0_lambdas, initialised to 1.0
  and 0.1, mixing each layer's residual stream with the normalised
  embedding; [P4] item 0): before layer l's block the stream becomes
  x <- resid_lambdas[l] * x + x0_lambdas[l] * x0, x0 = rmsnorm(wte[idx]).
* Value embeddings (optional, cfg["value_embeds"]; [P1] same section: at
  alternating layers a gated embedding lookup adds to V; [P4] item 0:
  ve_gate): layers 0, 2, 4, ... hold a table ve_l [V, n_kv_head * D]; after
  the QKV projection v <- v + ve_gates[j] * ve_l[idx] (j-th such layer),
  before attention. Which layers "alternate" and the gate's form (here one
  learned scalar per layer, i.e. per K/V head under MQA) are readings.

Parity pins: every function here is pinned by a test in ``tests/`` against a
closed form, an invariant, a library routine or finite differences; none is
"parity unpinned".
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

EPS = 2.0 ** -23          # RMSNorm epsilon (reading: float32 machine epsilon)
ROPE_THETA = 10000.0      # [P1] "A Llama-class transformer..."; RoPE base
SOFTCAP = 15.0            # [P1] same section; logits = 15 * tanh(z / 15)
_WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))  # threads for independent attention heads


# ---------------------------------------------------------------------------
# Shapes: the depth dial
# ---------------------------------------------------------------------------

def config_from_depth(depth: int, vocab: int = 65536, seq_len: int = 2048, n_kv_head: int = 1) -> dict:
    """[P1] "One dial controls everything": width = 64 * depth, heads = width / 128.

    [P4] item "0. The model": head dim 128; [P5] "Squared ReLU": MLP 4x wide;
    MQA ([P5] "Multi-Query Attention") by default, so one K/V head.
    """
    C = 64 * depth
    D = 128
    return dict(n_layer=depth, model_dim=C, n_head=C // D, n_kv_head=n_kv_head,
                head_dim=D, mlp_dim=4 * C, vocab_size=vocab, max_seq_len=seq_len,
                rope_theta=ROPE_THETA, logit_softcap=SOFTCAP, norm_eps=EPS)


def param_shapes(cfg: dict):
    """Canonical parameter order and shapes (rows, cols) of every weight.

    Untied embedding and LM head ([P1] "untied"; [P5] "Embedding strategy"),
    bias-free linears ([P4] item 0: bias=False). W_qkv stacks the query heads,
    then the K head(s), then the V head(s).
    """
    C, H, Hkv, D = cfg["model_dim"], cfg["n_head"], cfg["n_kv_head"], cfg["head_dim"]
    F, V = cfg["mlp_dim"], cfg["vocab_size"]
    shapes = [("wte", V, C)]
    for l in range(cfg["n_layer"]):
        shapes += [(f"h{l}.w_qkv", (H + 2 * Hkv) * D, C), (f"h{l}.w_o", C, H * D),
                   (f"h{l}.w_1", F, C), (f"h{l}.w_2", C, F)]
    shapes.append(("lm_head", V, C))
    for l in ve_layers(cfg):
        shapes.append((f"h{l}.ve", V, Hkv * D))
    if cfg.get("x0_lambdas", False):
        shapes += [("resid_lambdas", 1, cfg["n_layer"]), ("x0_lambdas", 1, cfg["n_layer"])]
    if ve_layers(cfg):
        shapes.append(("ve_gates", 1, len(ve_layers(cfg))))
    return shapes


def ve_layers(cfg: dict) -> list:
    """Layers with a value embedding: every other layer from layer 0."""
    return list(range(0, cfg["n_layer"], 2)) if cfg.get("value_embeds", False) else []


def param_count(cfg: dict) -> int:
    return sum(r * c for _, r, c in param_shapes(cfg))


def unflatten(cfg: dict, flat: np.ndarray) -> dict:
    out, off = {}, 0
    for name, r, c in param_shapes(cfg):
        out[name] = flat[off:off + r * c].reshape(r, c)
        off += r * c
    assert off == flat.size
    return out


# ---------------------------------------------------------------------------
# Building blocks
# ---------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, eps: float = EPS):
    """Parameter-free RMSNorm over the last axis ([P1] "A Llama-class
    transformer..."; [P5] "RMSNorm without learnable parameters").

    y = x / sqrt(mean(x**2) + eps). Returns (y, r) with r = 1/sqrt(mean + eps).
    """
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r, r


def rmsnorm_bwd(dy: np.ndarray, y: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Gradient of y = x*r(x): dx = r * (dy - y * mean(dy*y))."""
    return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def rope_tables(T: int, D: int, theta: float = ROPE_THETA):
    """cos/sin of angle[t, i] = t * theta**(-2i/D), i < D/2 ([P1]; [P5] "RoPE")."""
    i = np.arange(D // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / D)
    ang = np.arange(T, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate pairs (x_i, x_{i+D/2}) by +angle. x is [B, T, heads, D]."""
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_bwd(dy: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Transpose of the rotation (the inverse rotation, by -angle)."""
    h = dy.shape[-1] // 2
    d1, d2 = dy[..., :h], dy[..., h:]
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    return np.concatenate([d1 * c + d2 * s, -d1 * s + d2 * c], axis=-1)


def attention_mask(T: int, window: int | None = None) -> np.ndarray:
    """[T, T] boolean mask over (query t, key u): u <= t, and t - u < window
    when a sliding window is given ([P1] "A Llama-class transformer...")."""
    t = np.arange(T)[:, None]
    u = np.arange(T)[None, :]
    m = u <= t
    if window is not None:
        m &= (t - u) < window
    return m


def layer_window(cfg: dict, layer: int) -> int | None:
    """Window of a layer under the config's pattern ([P1]: "SSSL" = three
    short-window layers then one full-context layer, repeating; the final layer
    always full). None means full causal context."""
    pattern = cfg.get("window_pattern", "") or ""
    short = int(cfg.get("window_short", 0) or 0)
    if not pattern or short <= 0 or layer == cfg["n_layer"] - 1:
        return None
    return short if pattern[layer % len(pattern)] == "S" else None


def _each(fn, items):
    """Runs fn on every item. The items (batch rows and heads of attention) are
    independent and each writes only its own output slice, so they run on a
    thread pool: NumPy's elementwise kernels release the GIL, and the softmax
    work of different heads proceeds side by side. Nothing about the result
    depends on the order."""
    items = list(items)
    if len(items) <= 1 or _WORKERS <= 1:
        for it in items:
            fn(it)
        return
    with ThreadPoolExecutor(min(len(items), _WORKERS)) as ex:
        list(ex.map(fn, items))


def causal_mqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, window: int | None = None):
    """Causal attention where all query heads share one K/V head
    ([P5] "Multi-Query Attention"; [P1] causal decoder).

    q [B, T, H, D]; k, v [B, T, D]. Scores s = q.k / sqrt(D), key u <= query t
    (and t - u < window for a sliding-window layer).
    Returns o [B, T, H, D] and the log-sum-exp of the scaled scores [B, H, T].
    """
    B, T, H, D = q.shape
    scale = 1.0 / math.sqrt(D)
    mask = attention_mask(T, window)
    o = np.empty_like(q)
    lse = np.empty((B, H, T))

    def one(bh):
        b, h = bh
        s = (q[b, :, h, :] @ k[b].T) * scale               # [T(query), T(key)]
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=-1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=-1, keepdims=True)
        o[b, :, h, :] = (e / z) @ v[b]
        lse[b, h] = (m + np.log(z))[:, 0]

    _each(one, [(b, h) for b in range(B) for h in range(H)])
    return o, lse


def causal_mqa_attention_bwd(do, q, k, v, window: int | None = None):
    """Backward of ``causal_mqa_attention`` through the softmax Jacobian.

    dP = do.v ; dS = P * (dP - sum_u P dP) ; dq = dS.k/sqrt(D) ;
    dk = sum over heads and queries of dS^T q / sqrt(D) ; dv = sum of P^T do.
    """
    B, T, H, D = q.shape
    scale = 1.0 / math.sqrt(D)
    mask = attention_mask(T, window)
    dq = np.empty_like(q)
    dk_h = np.empty((B, H, T, D))     # per-head terms of dk and dv, summed over heads below
    dv_h = np.empty((B, H, T, D))

    def one(bh):
        b, h = bh
        qh, doh = q[b, :, h, :], do[b, :, h, :]            # [T, D]
        s = (qh @ k[b].T) * scale
        s = np.where(mask, s, -np.inf)
        e = np.exp(s - s.max(axis=-1, keepdims=True))
        p = e / e.sum(axis=-1, keepdims=True)
        dp = doh @ v[b].T
        ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
        dq[b, :, h, :] = (ds @ k[b]) * scale
        dk_h[b, h] = ds.T @ qh
        dv_h[b, h] = p.T @ doh

    _each(one, [(b, h) for b in range(B) for h in range(H)])
    return dq, dk_h.sum(axis=1) * scale, dv_h.sum(axis=1)


def softcap(z: np.ndarray, c: float = SOFTCAP) -> np.ndarray:
    """[P1]: logits are squashed to c * tanh(z / c) with c = 15, in fp32 or wider."""
    return c * np.tanh(z / c)


def softcap_bwd(dzc: np.ndarray, zc: np.ndarray, c: float = SOFTCAP) -> np.ndarray:
    """d/dz [c tanh(z/c)] = 1 - tanh^2 = 1 - (zc/c)^2."""
    return dzc * (1.0 - (zc / c) ** 2)


def logsumexp(z: np.ndarray) -> np.ndarray:
    m = z.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))[..., 0]


# ---------------------------------------------------------------------------
# FP8 (OCP e4m3) matmuls
# ---------------------------------------------------------------------------
# [P3] repo-explainer.com, section "The Engine Room: Muon and FP8": training
# with a small FP8 implementation; [P4] item "2. Pretrain": FP8 matmuls are
# optional. The pages give no recipe, so these readings are fixed here:
# * format e4m3 in the OCP form (no infinities, NaN = 0x7f/0xff, largest
#   finite 448, subnormals down to 2**-9) for both operands of every
#   QKV / O / MLP matmul, in the forward pass and in both backward products
#   (the output gradient is quantised too);
# * one scale per tensor from its current absolute maximum,
#   s = 448 / amax (s = 1 for an all-zero tensor);
# * code = round-to-nearest-even of x * s to the e4m3 grid, saturating at
#   +-448. The operand is quantised as the bf16 compute dtype holds it ([P2]
#   "Precision / dtype": bf16 compute), so x is first rounded to bf16 (as
#   every bf16 activation and gradient is stored); amax, the scale and the
#   product are then taken in fp32, the precision in which the code is decided;
# * the matmul of two quantised tensors is the exact product of the
#   dequantised values q / s (float64 here); the LM head and attention stay
#   unquantised;
# * the backward treats quantisation as the identity (straight through):
#   dX = Q(dY) Q(W), dW = Q(dY)^T Q(X), with Q(X), Q(W) the forward's codes.

E4M3_MAX = 448.0


def _e4m3_value(c: np.ndarray) -> np.ndarray:
    """Value of each e4m3 byte: sign bit 7, exponent bits 6..3 with bias 7,
    mantissa bits 2..0; exponent 0 is subnormal (m/8 * 2**-6); 0x7f and 0xff
    are NaN."""
    c = np.asarray(c, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


_E4M3_TABLE = _e4m3_value(np.arange(256))


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each e4m3 byte (the definition above, looked up per code)."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code of each fp32 value (ties to the even code, i.e. the
    even mantissa), after clamping the magnitude to 448. NaN maps to 0x7f.

    In the binade [2**E, 2**(E+1)) (E >= -6; the subnormals share the spacing
    of E = -6) the grid has spacing 2**(E-3), so the nearest grid value is
    rint(a / spacing) * spacing, rint rounding halves to even; an even
    multiple of the spacing is an even mantissa (and an even code)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y), np.float32(E4M3_MAX))
    a = np.where(np.isnan(a), np.float32(0.0), a)
    _, e = np.frexp(a)                              # a = f * 2**e, 0.5 <= f < 1
    E = np.maximum(e - 1, -6)
    step = np.ldexp(np.float32(1.0), E - 3)
    v = np.rint(a / step) * step                    # exact in fp32 (power-of-two scaling)
    _, e2 = np.frexp(v)
    E2 = e2 - 1
    code = np.where(E2 < -6, v * np.float32(2.0 ** 9), (E2 + 7) * 8 + (np.ldexp(v, -E2) - 1) * 8)
    code = np.where(v == 0, 0, code).astype(np.int64)
    code = code | np.where(np.signbit(y), 0x80, 0)
    code = np.where(np.isnan(y), 0x7F, code)
    return code.astype(np.uint8)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """x rounded to bf16 (8 significant bits), round to nearest, ties to even,
    straight from float64: x = m * 2**e with 0.5 <= |m| < 1, keep rint(m * 2**8)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def fp8_quantize(x: np.ndarray):
    """Per-tensor current scaling of the bf16 operand: returns (codes, s) with
    s = 448 / max|bf16(x)| in fp32 and codes = e4m3(bf16(x) * s)."""
    x32 = round_bf16(x).astype(np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    s = np.float32(E4M3_MAX) / amax if amax > 0 else np.float32(1.0)
    return e4m3_encode(x32 * s), s


def fp8_dequantize(codes: np.ndarray, s) -> np.ndarray:
    return e4m3_decode(codes) / np.float64(s)


def fp8_round_trip(x: np.ndarray) -> np.ndarray:
    """The value a quantised matmul operand stands for: Q(x) / s."""
    return fp8_dequantize(*fp8_quantize(x))


def mm_operand(cfg: dict, t: np.ndarray) -> np.ndarray:
    """A QKV / O / MLP matmul operand as the config's precision sees it: the
    tensor itself, or its e4m3 round trip when cfg["fp8"] is set."""
    return fp8_round_trip(t) if cfg.get("fp8", False) else t


# ---------------------------------------------------------------------------
# The step
# ---------------------------------------------------------------------------

def _split_qkv(qkv, H, Hkv, D):
    B, T, _ = qkv.shape
    q = qkv[..., :H * D].reshape(B, T, H, D)
    k = qkv[..., H * D:(H + Hkv) * D].reshape(B, T, Hkv, D)
    v = qkv[..., (H + Hkv) * D:].reshape(B, T, Hkv, D)
    return q, k, v


def forward(cfg: dict, params: dict, idx: np.ndarray, targets: np.ndarray, row_chunk: int = 4096):
    """Forward pass and mean cross-entropy loss. Returns (loss, row_loss[B,T], cache).

    Block order ([P1] "A Llama-class transformer..."; [P4] item 0; [P5]):
    x = rmsnorm(wte[idx]); per layer x += attn(rmsnorm(x)), x += mlp(rmsnorm(x));
    logits = softcap(rmsnorm(x) W_lm^T); loss = mean(lse(logits) - logits[target]).
    """
    assert cfg["n_kv_head"] == 1, "the oracle's attention is multi-query (one K/V head)"
    B, T = idx.shape
    C, H, D = cfg["model_dim"], cfg["n_head"], cfg["head_dim"]
    eps, c = cfg["norm_eps"], cfg["logit_softcap"]
    cos, sin = rope_tables(T, D, cfg["rope_theta"])
    W = {k: np.asarray(v, dtype=np.float64) for k, v in params.items()}

    # matmul operands as the config's precision sees them (the e4m3 round trip
    # for FP8 models, else the tensors themselves); the backward reuses them
    Wm = {k: mm_operand(cfg, v) for k, v in W.items() if k.startswith("h") and not k.endswith(".ve")}
    x, r0 = rmsnorm(W["wte"][idx], eps)
    x0 = x
    lam = cfg.get("x0_lambdas", False)
    vel = ve_layers(cfg)
    cache = dict(r0=r0, layers=[], cos=cos, sin=sin, Wm=Wm, x0=x0)
    for l in range(cfg["n_layer"]):
        xprev = x
        if lam:
            x = W["resid_lambdas"][0, l] * x + W["x0_lambdas"][0, l] * x0
        h1, r1 = rmsnorm(x, eps)
        h1m = mm_operand(cfg, h1)
        qkv = h1m @ Wm[f"h{l}.w_qkv"].T
        q, k, v = _split_qkv(qkv, H, 1, D)
        if l in vel:
            v = v + W["ve_gates"][0, vel.index(l)] * W[f"h{l}.ve"][idx][:, :, None, :]
        qr, kr = rope(q, cos, sin), rope(k, cos, sin)
        qn, rq = rmsnorm(qr, eps)
        kn, rk = rmsnorm(kr, eps)
        o, lse = causal_mqa_attention(qn, kn[:, :, 0], v[:, :, 0], layer_window(cfg, l))
        o2 = o.reshape(B, T, H * D)
        o2m = mm_operand(cfg, o2)
        x = x + o2m @ Wm[f"h{l}.w_o"].T
        h2, r2 = rmsnorm(x, eps)
        h2m = mm_operand(cfg, h2)
        u = h2m @ Wm[f"h{l}.w_1"].T
        a = np.maximum(u, 0.0) ** 2
        am = mm_operand(cfg, a)
        x = x + am @ Wm[f"h{l}.w_2"].T
        cache["layers"].append(dict(h1=h1, r1=r1, qn=qn, rq=rq, kn=kn, rk=rk, v=v,
                                    o=o, lse=lse, h2=h2, r2=r2, u=u, a=a,
                                    h1m=h1m, o2m=o2m, h2m=h2m, am=am, xprev=xprev))
    hf, rf = rmsnorm(x, eps)
    cache.update(hf=hf, rf=rf)

    N = B * T
    hf2 = hf.reshape(N, C)
    tg = targets.reshape(N)
    row_loss = np.empty(N)
    lse_rows = np.empty(N)
    for s0 in range(0, N, row_chunk):
        s1 = min(N, s0 + row_chunk)
        zc = softcap(hf2[s0:s1] @ W["lm_head"].T, c)
        lse_rows[s0:s1] = logsumexp(zc)
        row_loss[s0:s1] = lse_rows[s0:s1] - zc[np.arange(s1 - s0), tg[s0:s1]]
    cache["lse_rows"] = lse_rows
    loss = float(row_loss.mean())
    return loss, row_loss.reshape(B, T), cache


def backward(cfg: dict, params: dict, idx: np.ndarray, targets: np.ndarray, cache: dict,
             dloss: float = 1.0, row_chunk: int = 4096) -> dict:
    """Analytic gradients of dloss * loss with respect to every weight."""
    B, T = idx.shape
    N = B * T
    C, H, D = cfg["model_dim"], cfg["n_head"], cfg["head_dim"]
    c = cfg["logit_softcap"]
    cos, sin = cache["cos"], cache["sin"]
    W = {k: np.asarray(v, dtype=np.float64) for k, v in params.items()}
    G = {k: np.zeros_like(v) for k, v in W.items()}

    # LM head + softcap + cross-entropy
    hf2 = cache["hf"].reshape(N, C)
    tg = targets.reshape(N)
    dhf = np.empty((N, C))
    for s0 in range(0, N, row_chunk):
        s1 = min(N, s0 + row_chunk)
        zc = softcap(hf2[s0:s1] @ W["lm_head"].T, c)
        p = np.exp(zc - cache["lse_rows"][s0:s1, None])
        p[np.arange(s1 - s0), tg[s0:s1]] -= 1.0
        dz = softcap_bwd(p * (dloss / N), zc, c)
        G["lm_head"] += dz.T @ hf2[s0:s1]
        dhf[s0:s1] = dz @ W["lm_head"]
    dx = rmsnorm_bwd(dhf.reshape(B, T, C), cache["hf"], cache["rf"])
    lam = cfg.get("x0_lambdas", False)
    vel = ve_layers(cfg)
    dx0 = np.zeros_like(dx)  # gradient reaching x0 through the x0_lambdas mixes

    Wm = cache["Wm"]
    for l in reversed(range(cfg["n_layer"])):
        L = cache["layers"][l]
        # MLP: x_out = x_mid + relu(u)^2 W2^T, u = rmsnorm(x_mid) W1^T
        # (for FP8 models every product takes the e4m3 round trips of its
        # operands; the quantisation itself is passed straight through)
        dy = mm_operand(cfg, dx)
        G[f"h{l}.w_2"] += dy.reshape(N, C).T @ L["am"].reshape(N, -1)
        da = dy @ Wm[f"h{l}.w_2"]
        du = da * 2.0 * np.maximum(L["u"], 0.0)
        duq = mm_operand(cfg, du)
        G[f"h{l}.w_1"] += duq.reshape(N, -1).T @ L["h2m"].reshape(N, C)
        dh2 = duq @ Wm[f"h{l}.w_1"]
        dx = dx + rmsnorm_bwd(dh2, L["h2"], L["r2"])
        # attention: x_mid = x_in + o W_o^T
        o2 = L["o"].reshape(B, T, H * D)
        dy = mm_operand(cfg, dx)
        G[f"h{l}.w_o"] += dy.reshape(N, C).T @ L["o2m"].reshape(N, -1)
        do = (dy @ Wm[f"h{l}.w_o"]).reshape(B, T, H, D)
        dqn, dkn, dv = causal_mqa_attention_bwd(do, L["qn"], L["kn"][:, :, 0], L["v"][:, :, 0],
                                                layer_window(cfg, l))
        dqr = rmsnorm_bwd(dqn, L["qn"], L["rq"])
        dkr = rmsnorm_bwd(dkn[:, :, None, :], L["kn"], L["rk"])
        dq = rope_bwd(dqr, cos, sin)
        dk = rope_bwd(dkr, cos, sin)
        if l in vel:
            j = vel.index(l)
            G["ve_gates"][0, j] += np.sum(dv * W[f"h{l}.ve"][idx])
            np.add.at(G[f"h{l}.ve"], idx.reshape(N), W["ve_gates"][0, j] * dv.reshape(N, D))
        dqkv = np.concatenate([dq.reshape(B, T, H * D), dk.reshape(B, T, D),
                               dv.reshape(B, T, D)], axis=-1)
        dqkv = mm_operand(cfg, dqkv)
        G[f"h{l}.w_qkv"] += dqkv.reshape(N, -1).T @ L["h1m"].reshape(N, C)
        dh1 = dqkv @ Wm[f"h{l}.w_qkv"]
        dx = dx + rmsnorm_bwd(dh1, L["h1"], L["r1"])
        if lam:  # x_in = resid_lambdas[l] * xprev + x0_lambdas[l] * x0
            G["resid_lambdas"][0, l] += np.sum(dx * L["xprev"])
            G["x0_lambdas"][0, l] += np.sum(dx * cache["x0"])
            dx0 = dx0 + W["x0_lambdas"][0, l] * dx
            dx = W["resid_lambdas"][0, l] * dx

    # embedding: x0 = rmsnorm(wte[idx]); dwte[v] = sum over positions with idx == v
    e = W["wte"][idx]
    y0 = e * cache["r0"]
    de = rmsnorm_bwd(dx + dx0, y0, cache["r0"])
    np.add.at(G["wte"], idx.reshape(N), de.reshape(N, C))
    return G


def step(cfg: dict, params: dict, idx: np.ndarray, targets: np.ndarray, dloss: float = 1.0,
         row_chunk: int = 4096):
    """One forward + backward. Returns (loss, row_loss [B, T], grads dict).
    `row_chunk` bounds the rows of the LM head and cross-entropy held at once;
    it changes memory use only, not what is computed."""
    loss, row_loss, cache = forward(cfg, params, idx, targets, row_chunk)
    grads = backward(cfg, params, idx, targets, cache, dloss, row_chunk)
    return loss, row_loss, grads


def forward_rows(cfg: dict, params: dict, idx: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """Per-position losses only (no cache kept beyond one layer's use)."""
    _, row_loss, _ = forward(cfg, params, idx, targets)
    return row_loss


# ---------------------------------------------------------------------------
# The optimiser step that follows the backward
# ---------------------------------------------------------------------------
# [P4] item "2. Pretrain": the transformer's matrix weights go to Muon, the
# embeddings, the unembedding and the scalars to AdamW; Muon's momentum
# follows a schedule (0.85 -> 0.97 -> 0.90); fp32 master weights, bf16
# compute. [P1] "A Llama-class transformer...": input and output embeddings
# have different learning rates; Muon handles all weight matrices, AdamW the
# embeddings and scalars. [P3] "The Engine Room: Muon and FP8" and [P5]
# "Muon optimizer": Muon post-processes the update into an orthogonalisation.
# Readings (the pages give no formulas):
# * AdamW is the standard algorithm with decoupled weight decay and bias
#   correction (w <- w (1 - lr wd); m, v moments; w <- w - (lr / (1 - b1^t))
#   m / (sqrt(v) / sqrt(1 - b2^t) + eps)), one learning rate per group
#   (embeddings incl. value-embedding tables, unembedding, scalars);
# * Muon: momentum buffer u <- mu u + g (mu given per step by the caller's
#   schedule); the update direction is the orthogonal polar factor of u,
#   approximated by k steps of the Newton-Schulz iteration
#   X <- a X + (b A + c A^2) X, A = X X^T, from X_0 = u / (||u||_F + 1e-7),
#   on the orientation with fewer rows; w <- w (1 - lr wd) - lr *
#   sqrt(max(1, rows / cols)) * X. The default coefficients (1.5, -0.5, 0)
#   are the cubic Newton-Schulz iteration for the polar factor; the pages'
#   "Polar Express" coefficients and variance reduction are not given.

MUON_SUFFIXES = (".w_qkv", ".w_o", ".w_1", ".w_2")


def optimizer_group(name: str) -> str:
    """'muon' for the blocks' matrix weights, else the AdamW group."""
    if name.startswith("h") and name.endswith(MUON_SUFFIXES):
        return "muon"
    if name == "lm_head":
        return "unembed"
    if name == "wte" or name.endswith(".ve"):
        return "embed"
    return "scalar"


def adamw_update(w, g, m, v, t, lr, beta1, beta2, eps, wd):
    """One AdamW step (decoupled weight decay, bias-corrected moments).
    Returns (w, m, v)."""
    w = w * (1.0 - lr * wd)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    bc1, bc2 = 1.0 - beta1 ** t, 1.0 - beta2 ** t
    w = w - (lr / bc1) * m / (np.sqrt(v) / math.sqrt(bc2) + eps)
    return w, m, v


def newton_schulz(u, steps: int, a: float = 1.5, b: float = -0.5, c: float = 0.0):
    """k Newton-Schulz steps towards the orthogonal polar factor of u."""
    X = u / (np.linalg.norm(u) + 1e-7)
    tr = X.shape[0] > X.shape[1]
    if tr:
        X = X.T
    for _ in range(steps):
        A = X @ X.T
        X = a * X + (b * A + c * (A @ A)) @ X
    return X.T if tr else X


def muon_update(w, g, u, lr, mu, wd, steps, coeffs):
    """One Muon step. Returns (w, u)."""
    u = mu * u + g
    X = newton_schulz(u, steps, *coeffs)
    scale = math.sqrt(max(1.0, w.shape[0] / w.shape[1]))
    return w * (1.0 - lr * wd) - lr * scale * X, u


def optimizer_step(cfg: dict, oc: dict, master: dict, grads: dict, state: dict, t: int):
    """Updates every parameter from its gradient: Muon for the matrix
    weights, AdamW for the rest. `state` maps a name to its buffers ("u", or
    "m" and "v"), zeros on the first step (t = 1). Returns (master, state)."""
    lrs = dict(embed=oc["lr_embed"], unembed=oc["lr_unembed"], scalar=oc["lr_scalar"])
    coeffs = (oc.get("ns_a", 1.5), oc.get("ns_b", -0.5), oc.get("ns_c", 0.0))
    new_w, new_s = {}, {}
    for name, w in master.items():
        g = grads[name]
        grp = optimizer_group(name)
        if grp == "muon":
            u = state.get(name, {}).get("u", np.zeros_like(w))
            new_w[name], u = muon_update(w, g, u, oc["lr_muon"], oc["momentum"], oc["wd_muon"],
                                         oc["ns_steps"], coeffs)
            new_s[name] = dict(u=u)
        else:
            s = state.get(name, {})
            m, v = s.get("m", np.zeros_like(w)), s.get("v", np.zeros_like(w))
            new_w[name], m, v = adamw_update(w, g, m, v, t, lrs[grp], oc["beta1"], oc["beta2"], oc["eps"],
                                             oc["wd_adamw"])
            new_s[name] = dict(m=m, v=v)
    return new_w, new_s
