"""Float64 CPU oracle for the Gemma-4 E-series decoder-layer forward.

TEST INFRASTRUCTURE. Only the tests, the package entry's smoke check and the benchmark's CPU-baseline
leg may import this module. The product path never calls it and shares no code with it.

It is the plain definition of what the layer computes, written from the pages in their order:
  * cortiq-engine `g4e.rs` (page 1): module doc (PLE, shared KV), `G4eGlobals` (inverse frequencies,
    window "tokens, current included"), `rms`, `rms_plain`, `gelu_tanh`, `extend_embedding`,
    `g4e_forward` (the layer body).
  * ferrox-models `gemma4_engine.rs` (page 2): `Gemma4Hparams` (`is_swa`, `head_dim`, `has_kv`,
    `rope_theta_for`), `project_per_layer_inputs`, `forward_token_on_worker` (embedding scale,
    attention scale 1.0, V norm without weight, shared-KV head-dim assert).
  * taconite-embeddinggemma2 `model.rs` (page 4): `rope_half` (NeoX half-split rotation), `rms_row`,
    `text_attention` (GQA head map `kh = hh / group`).
  * turbospark-runtime `gemma4/attn.rs` (page 5): `rotated_pairs = full_head_dim * partial_rotary / 2`,
    sliding `kv_start = seq_len - sliding_window`.
  * the output head after the stack (page 2 `forward_token_on_worker`, page 1 module doc): final RMSNorm,
    output projection, final-logit softcap.

Readings where the pages are silent or disagree (each also listed in the design notes):
  * Proportional RoPE: pair j of a full layer rotates by pos * theta^(-2j/hd_full) for j < R and is the
    identity for R <= j < hd_full/2 (the "zero tail" of `G4eGlobals::inv_freq_global`).
  * Shared-KV source: the last non-shared layer of the same attention type (page 1 module doc). A
    shared layer with no such layer keeps its own K/V.
  * Window: query at position i sees keys i-W < j <= i. The encoder (page 4 `text_attention`) is not
    causal: it sees the call's keys with |i - j| <= W on sliding layers and all of them on full layers.
  * Out-of-range token ids give a zero embedding row and a zero PLE table term.
  * Variants: full layers may have their own KV head count; per-layer FFN widths follow the weight
    shapes (page 2 `ffn_dim`); with K=V a full layer's V is the K projection output before the K norm
    and RoPE, normed without scale (page 5 `forward_layer`). Page 2 instead clones the normed, rotated
    K when a layer has no V projection; the page-5 reading is the one taken here.

All arithmetic is numpy float64 on the given inputs (bf16 inputs are converted exactly).
"""
import math

import numpy as np

try:  # inputs may arrive as torch tensors (bf16 has no numpy dtype)
    import torch
except ImportError:  # pragma: no cover
    torch = None


def f64(x):
    """Exact float64 copy of an array or tensor (bf16/f32 values are representable in f64)."""
    if x is None:
        return None
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _ints(x):
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.int64).numpy()
    return np.asarray(x, dtype=np.int64)


# --------------------------------------------------------------------------------------------
# Primitives (page 1 `rms`, `rms_plain`, `gelu_tanh`; page 4 `rms_row`, `rope_half`)
# --------------------------------------------------------------------------------------------

def rms_norm(x, w=None, eps=1e-6):
    """Plain x-hat times w over the last axis: x * (mean(x^2) + eps)^-1/2 * w.

    eps sits inside the mean and the weight multiplies as is (no 1 + w) -- page 1, `rms` and the module
    note that every norm is plain x-hat times w. With w None this is the scale-less norm of V (page 1,
    `rms_plain`; page 2 applies a ones weight to V).
    """
    x = f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x * (ms + eps) ** -0.5
    if w is not None:
        y = y * f64(w)
    return y


def gelu_tanh(x):
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) -- page 1, `gelu_tanh`."""
    x = f64(x)
    return 0.5 * x * (1.0 + np.tanh(0.7978845608028654 * (x + 0.044715 * x * x * x)))


def rotated_pairs(cfg, sliding):
    """Pairs that rotate: all hd/2 on sliding layers; floor(hd_full * p / 2) on full layers (page 5)."""
    if sliding:
        return cfg["head_dim_swa"] // 2
    return int(cfg["head_dim_full"] * cfg["partial_rotary"] / 2.0)


def inv_freq(hd, theta, n_rot):
    """Inverse frequencies of the hd/2 NeoX pairs: theta^(-2j/hd) for j < n_rot, 0 beyond.

    The zero tail makes those pairs the identity (page 1, `G4eGlobals` inverse-frequency note).
    """
    j = np.arange(hd // 2, dtype=np.float64)
    inv = float(theta) ** (-2.0 * j / hd)
    inv[n_rot:] = 0.0
    return inv


def rope(x, pos, inv):
    """NeoX half-split rotation of the last axis (page 4, `rope_half`).

    For pair j < hd/2: (x_j, x_{j+hd/2}) -> (x_j c - x_{j+hd/2} s, x_{j+hd/2} c + x_j s) with
    (c, s) = (cos, sin)(pos * inv_j). `pos` broadcasts against x's leading axes.
    """
    x = f64(x)
    h = x.shape[-1] // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# --------------------------------------------------------------------------------------------
# Routing (page 1 module doc; page 2 `Gemma4Hparams`)
# --------------------------------------------------------------------------------------------

def kv_sources(layer_types, n_shared):
    """Layer whose KV cache each layer attends over.

    The first L - n_shared layers own their cache. A later (shared) layer reads the last non-shared
    layer of its own attention type (page 1 module doc). If there is none, the layer keeps its own
    cache (reading; the pages do not cover that case).
    """
    L = len(layer_types)
    first_shared = L - n_shared
    src = []
    for l in range(L):
        if l < first_shared:
            src.append(l)
            continue
        cands = [j for j in range(first_shared) if layer_types[j] == layer_types[l]]
        src.append(cands[-1] if cands else l)
    return src


def kv_sources_shortcut(layer_types, n_shared):
    """The index shortcut of page 2 (`kv_reuse_layer`): sliding -> first_shared-2, full -> first_shared-1.

    Kept only to pin the page's own fixture; it equals `kv_sources` only when the last two non-shared
    layers are [sliding, full].
    """
    L = len(layer_types)
    first_shared = L - n_shared
    return [l if l < first_shared else first_shared - (2 if layer_types[l] == "S" else 1)
            for l in range(L)]


def layer_geometry(cfg, layer):
    """(sliding, head_dim, theta, rotated pairs) of a layer (page 2 `head_dim`, `rope_theta_for`)."""
    sliding = cfg["layer_types"][layer] == "S"
    hd = cfg["head_dim_swa"] if sliding else cfg["head_dim_full"]
    theta = cfg["theta_swa"] if sliding else cfg["theta_full"]
    return sliding, hd, theta, rotated_pairs(cfg, sliding)


def kv_heads(cfg, layer):
    """KV head count of a layer (page 5 `forward_layer`: full layers take `num_full_kv_heads`, sliding
    layers `num_kv_heads`). A config without a separate full-layer count uses one count for both."""
    if cfg["layer_types"][layer] == "S":
        return cfg["n_kv_heads"]
    return cfg.get("n_kv_heads_full") or cfg["n_kv_heads"]


def value_weight(cfg, lw, layer):
    """Weight whose projection gives V (page 5 `forward_layer`: a full layer of a model flagged
    `attention_k_eq_v` projects V with the K projection's weight; V is then normed without scale and
    never rotated, like any other V)."""
    if cfg.get("k_eq_v") and cfg["layer_types"][layer] != "S":
        return lw["wk"]
    return lw["wv"]


# --------------------------------------------------------------------------------------------
# Attention (page 1 `attend_all_heads(..., 1.0, window, ...)`; page 4 `text_attention`)
# --------------------------------------------------------------------------------------------

def attention(q, K, V, qpos, window=None, scale=1.0, chunk=256):
    """Causal GQA softmax attention of one sequence against its cache.

    q [T, nh, hd]; K, V [nkv, cap, hd]; qpos [T] absolute positions. Head h reads kv head
    h // (nh / nkv). Query at position i sees keys j with lo <= j <= i, lo = 0 (full) or
    i - W + 1 (sliding, W keys including itself). Score scale 1.0, no softcap.
    """
    q, K, V = f64(q), f64(K), f64(V)
    qpos = _ints(qpos)
    T, nh, hd = q.shape
    nkv = K.shape[0]
    grp = nh // nkv
    out = np.zeros((T, nh, V.shape[-1]))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        p = qpos[t0:t1]
        lo = 0 if window is None else max(0, int(p.min()) - window + 1)
        hi = int(p.max()) + 1
        j = np.arange(lo, hi)
        vis = j[None, :] <= p[:, None]
        if window is not None:
            vis &= j[None, :] > p[:, None] - window
        for h in range(nh):
            g = h // grp
            s = scale * (q[t0:t1, h, :] @ K[g, lo:hi, :].T)
            s = np.where(vis, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            out[t0:t1, h, :] = (e / e.sum(axis=1, keepdims=True)) @ V[g, lo:hi, :]
    return out


def attention_bidirectional(q, K, V, qpos, k0, k1, window=None, scale=1.0, chunk=256):
    """Non-causal GQA softmax attention of one sequence over its own keys (page 4 `text_attention`).

    q [T, nh, hd]; K, V [nkv, cap, hd]; qpos [T] absolute positions; the sequence's keys are the cache
    rows k0 <= j < k1. A query at position i sees all of them on a full layer, and on a sliding layer
    those with |i - j| <= W (up to W keys on either side of it, itself included). Score scale 1.0.
    """
    q, K, V = f64(q), f64(K), f64(V)
    qpos = _ints(qpos)
    T, nh, hd = q.shape
    nkv = K.shape[0]
    grp = nh // nkv
    out = np.zeros((T, nh, V.shape[-1]))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        p = qpos[t0:t1]
        lo = k0 if window is None else max(k0, int(p.min()) - window)
        hi = k1 if window is None else min(k1, int(p.max()) + window + 1)
        j = np.arange(lo, hi)
        vis = np.ones((t1 - t0, hi - lo), dtype=bool)
        if window is not None:
            vis &= np.abs(j[None, :] - p[:, None]) <= window
        for h in range(nh):
            g = h // grp
            s = scale * (q[t0:t1, h, :] @ K[g, lo:hi, :].T)
            s = np.where(vis, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            out[t0:t1, h, :] = (e / e.sum(axis=1, keepdims=True)) @ V[g, lo:hi, :]
    return out


# --------------------------------------------------------------------------------------------
# Entry: embedding and per-layer inputs (page 1 `extend_embedding`; page 2 `project_per_layer_inputs`)
# --------------------------------------------------------------------------------------------

def _gather_rows(table, ids, n_rows):
    """Rows of `table` for ids in [0, n_rows); out-of-range ids give zero rows."""
    ids = _ints(ids)
    ok = (ids >= 0) & (ids < n_rows)
    safe = np.where(ok, ids, 0)
    if torch is not None and isinstance(table, torch.Tensor):
        rows = f64(table[torch.from_numpy(safe.reshape(-1))])
    else:
        rows = f64(table)[safe.reshape(-1)]
    rows = rows.reshape(ids.shape + (rows.shape[-1],))
    return rows * ok[..., None]


def embed(ids, E, cfg):
    """e = E[id] * sqrt(H) (page 2, token embedding times `(hidden as f32).sqrt()`)."""
    return _gather_rows(E, ids, cfg["vocab"]) * math.sqrt(cfg["hidden"])


def ple_inputs(ids, e, W_pm, ple_norm, Tab, cfg):
    """Per-layer inputs [.., L, d] from the scaled embedding e and the token ids.

    P = (W_pm e) * H^-1/2; chunk l of P is RMS-normed with ple_norm; the table row chunk times sqrt(d)
    is added (zero when id >= ple_vocab); the sum is multiplied by 1/sqrt(2)
    (page 1 `extend_embedding`, page 2 `project_per_layer_inputs`).
    """
    H, L, d, eps = cfg["hidden"], cfg["n_layers"], cfg["ple_dim"], cfg["eps"]
    e = f64(e)
    P = (e @ f64(W_pm).T) * (H ** -0.5)
    P = P.reshape(e.shape[:-1] + (L, d))
    pn = rms_norm(P, ple_norm, eps)
    tab = _gather_rows(Tab, ids, cfg["ple_vocab"]).reshape(e.shape[:-1] + (L, d)) * math.sqrt(d)
    return (pn + tab) * (1.0 / math.sqrt(2.0))


# --------------------------------------------------------------------------------------------
# One decoder layer (page 1 `g4e_forward` body; page 2 `forward_token_on_worker`)
# --------------------------------------------------------------------------------------------

def layer_forward(cfg, lw, layer, src, h, ple_l, pos, caches, trace=None, bidirectional=False):
    """One layer over all tokens of a batch.

    h [B, T, H] residual (f64, updated copy returned); ple_l [B, T, d] this layer's per-layer input;
    pos [B, T] absolute positions; caches {layer: (K, V)} with K, V [B, nkv, cap, hd] float64 arrays,
    modified in place when the layer owns its cache (src == layer). `trace`, if a dict, receives the
    intermediates. `bidirectional`: the encoder's attention (page 4 `text_attention`) over the call's
    own keys, positions pos[b, 0] .. pos[b, 0] + T - 1, instead of the causal one.
    """
    eps = cfg["eps"]
    nh, nkv = cfg["n_heads"], kv_heads(cfg, layer)
    sliding, hd, theta, n_rot = layer_geometry(cfg, layer)
    inv = inv_freq(hd, theta, n_rot)
    h = f64(h).copy()
    B, T, H = h.shape
    pos = _ints(pos)

    # attention block
    xn = rms_norm(h, lw["input_norm"], eps)
    q = (xn @ f64(lw["wq"]).T).reshape(B, T, nh, hd)
    q = rope(rms_norm(q, lw["q_norm"], eps), pos[:, :, None], inv)
    if src == layer:
        k = (xn @ f64(lw["wk"]).T).reshape(B, T, nkv, hd)
        k = rope(rms_norm(k, lw["k_norm"], eps), pos[:, :, None], inv)
        v = rms_norm((xn @ f64(value_weight(cfg, lw, layer)).T).reshape(B, T, nkv, hd), None, eps)
        K, V = caches[layer]
        for b in range(B):
            for t in range(T):
                K[b, :, pos[b, t], :] = k[b, t]
                V[b, :, pos[b, t], :] = v[b, t]
    K, V = caches[src]
    if K.shape[-1] != hd:
        raise ValueError(f"layer {layer}: source cache head_dim {K.shape[-1]} != {hd}")
    window = cfg["window"] if sliding else None
    if bidirectional:
        o = np.stack([attention_bidirectional(q[b], K[b], V[b], pos[b], int(pos[b, 0]), int(pos[b, 0]) + T, window)
                      for b in range(B)])
    else:
        o = np.stack([attention(q[b], K[b], V[b], pos[b], window) for b in range(B)])
    a = o.reshape(B, T, nh * hd) @ f64(lw["wo"]).T
    h = h + rms_norm(a, lw["post_attn_norm"], eps)

    # gelu-tanh gated FFN
    xn2 = rms_norm(h, lw["pre_ffn_norm"], eps)
    act = gelu_tanh(xn2 @ f64(lw["w_gate"]).T) * (xn2 @ f64(lw["w_up"]).T)
    ffn = act @ f64(lw["w_down"]).T
    h = h + rms_norm(ffn, lw["post_ffn_norm"], eps)

    # per-layer input injection: the gate reads the raw residual
    g = gelu_tanh(h @ f64(lw["ple_gate"]).T) * f64(ple_l)
    p = g @ f64(lw["ple_proj"]).T
    h = h + rms_norm(p, lw["post_ple_norm"], eps)

    h = h * float(lw.get("layer_scalar", 1.0))
    if trace is not None:
        trace.update(xn=xn, q=q, o=o, a=a, xn2=xn2, act=act, ffn=ffn, g=g, h=h)
    return h


def layer_forward_rows(cfg, lw, layer, h, ple_l, pos0, rows, bidirectional=False):
    """Selected output rows of one cache-owning layer over a prefill of one sequence.

    h [T, H] is the layer's input for tokens at positions pos0 .. pos0+T-1 (nothing cached before pos0),
    ple_l [T, d]. Only the K/V rows the selected queries can see are formed, so a long sequence can be
    checked at a few rows. Same formulas as `layer_forward`, restricted to rows (`bidirectional` as there).
    """
    eps = cfg["eps"]
    nh, nkv = cfg["n_heads"], kv_heads(cfg, layer)
    sliding, hd, theta, n_rot = layer_geometry(cfg, layer)
    inv = inv_freq(hd, theta, n_rot)
    h = f64(h)
    rows = np.asarray(sorted(set(int(r) for r in rows)))
    W = cfg["window"]
    T = h.shape[0]
    need = set()
    for r in rows:
        if bidirectional:
            need.update(range(max(0, r - W), min(T, r + W + 1)) if sliding else range(T))
        else:
            need.update(range(max(0, r - W + 1) if sliding else 0, r + 1))
    need = np.asarray(sorted(need))
    xk = rms_norm(h[need], lw["input_norm"], eps)
    pk = (pos0 + need)[:, None]
    k = rope(rms_norm((xk @ f64(lw["wk"]).T).reshape(len(need), nkv, hd), lw["k_norm"], eps), pk, inv)
    v = rms_norm((xk @ f64(value_weight(cfg, lw, layer)).T).reshape(len(need), nkv, hd), None, eps)
    cap = pos0 + int(need.max()) + 1
    K, V = np.zeros((nkv, cap, hd)), np.zeros((nkv, cap, hd))
    K[:, pos0 + need, :] = k.transpose(1, 0, 2)
    V[:, pos0 + need, :] = v.transpose(1, 0, 2)
    hr = h[rows]
    xn = rms_norm(hr, lw["input_norm"], eps)
    q = rope(rms_norm((xn @ f64(lw["wq"]).T).reshape(len(rows), nh, hd), lw["q_norm"], eps), (pos0 + rows)[:, None], inv)
    if bidirectional:
        o = attention_bidirectional(q, K, V, pos0 + rows, pos0, pos0 + T, W if sliding else None)
    else:
        o = attention(q, K, V, pos0 + rows, W if sliding else None)
    hr = hr + rms_norm(o.reshape(len(rows), nh * hd) @ f64(lw["wo"]).T, lw["post_attn_norm"], eps)
    xn2 = rms_norm(hr, lw["pre_ffn_norm"], eps)
    act = gelu_tanh(xn2 @ f64(lw["w_gate"]).T) * (xn2 @ f64(lw["w_up"]).T)
    hr = hr + rms_norm(act @ f64(lw["w_down"]).T, lw["post_ffn_norm"], eps)
    g = gelu_tanh(hr @ f64(lw["ple_gate"]).T) * f64(ple_l)[rows]
    hr = hr + rms_norm(g @ f64(lw["ple_proj"]).T, lw["post_ple_norm"], eps)
    return rows, hr * float(lw.get("layer_scalar", 1.0))


# --------------------------------------------------------------------------------------------
# Stack
# --------------------------------------------------------------------------------------------

def new_caches(cfg, B, cap, srcs=None):
    """Zeroed float64 caches for every layer that owns one."""
    srcs = srcs if srcs is not None else kv_sources(cfg["layer_types"], cfg["n_shared"])
    out = {}
    for l, s in enumerate(srcs):
        if s == l:
            _, hd, _, _ = layer_geometry(cfg, l)
            nkv = kv_heads(cfg, l)
            out[l] = (np.zeros((B, nkv, cap, hd)), np.zeros((B, nkv, cap, hd)))
    return out


def entry(cfg, glob, ids):
    """(h0, ple_in) from token ids: the scaled embedding and the per-layer inputs."""
    e = embed(ids, glob["embed"], cfg)
    ple = ple_inputs(ids, e, glob["ple_model_proj"], glob["ple_norm"], glob["ple_embed"], cfg)
    return e, ple


def forward(cfg, layers, h0, ple_in, pos, caches, srcs=None, layer_range=None, per_layer=None, bidirectional=False):
    """Run layers over h0 [B, T, H] with per-layer inputs ple_in [B, T, L, d] at positions pos [B, T].

    Returns the hidden state before the final norm (page 1: the caller applies the final norm, lm_head
    and softcap). `layers` is a list (or a callable layer -> weights dict, for lazy loading).
    `bidirectional`: every layer attends like page 4's encoder (see `layer_forward`).
    """
    srcs = srcs if srcs is not None else kv_sources(cfg["layer_types"], cfg["n_shared"])
    h = f64(h0)
    ple_in = f64(ple_in)
    rng = layer_range if layer_range is not None else range(cfg["n_layers"])
    for l in rng:
        lw = layers(l) if callable(layers) else layers[l]
        h = layer_forward(cfg, lw, l, srcs[l], h, ple_in[:, :, l, :], pos, caches, bidirectional=bidirectional)
        if per_layer is not None:
            per_layer.append(h)
    return h


def prefill_positions(pos0, T):
    pos0 = _ints(pos0)
    return pos0[:, None] + np.arange(T)[None, :]


# --------------------------------------------------------------------------------------------
# Output head (ferrox-models `forward_token_on_worker` tail; page 1 module doc: final norm + lm_head +
# final-logit softcap)
# --------------------------------------------------------------------------------------------

def softcap(x, cap):
    """cap * tanh(x / cap); cap <= 0 leaves x unchanged (no softcap configured)."""
    x = f64(x)
    if cap is None or cap <= 0:
        return x
    return cap * np.tanh(x / cap)


def logits(h, out_norm, w_out, cap, eps=1e-6):
    """Logits of hidden rows h [M, H]: W_out rms(h) * out_norm (W_out [vocab, H]), then the softcap."""
    return softcap(rms_norm(h, out_norm, eps) @ f64(w_out).T, cap)

