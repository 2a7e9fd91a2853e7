"""The oracle's layer with the bf16 path's roundings applied: the error floor of a bf16 implementation.

TEST INFRASTRUCTURE, like the oracle it is built from. The bf16 path takes its weights in bf16 and stores
a fixed set of intermediates in bf16, everything else (the residual stream, accumulations, norm
statistics, RoPE angles, softmax sums) in float32 or wider. This module replays one layer in float64
with exactly those intermediates rounded to the nearest bf16 (through float32, as a kernel rounds its
float32 value). The relative L2 distance of its output from the oracle's is the deviation that storing
those values in bf16 causes by itself; the GPU parity tests hold the HIP path's per-layer deviation to a
small multiple of it.

Rounding points (names used by `MODES`):
  act   the normed GEMM inputs (pre-attention and pre-FFN norms), the attention output, the gated FFN
        product gelu(gate) * up, the residual copy the PLE gate reads, the PLE gate product
  qkv   the raw q/k/v projections (a prefill stores them before the per-head norms; the few-row path
        used for decode sums float32 partials inside the head-norm kernel instead)
  q     the normed, rotated queries
  kv    the K/V cache rows
  p     the attention probabilities fed to the P V product (prefill: they are a bf16 MFMA operand;
        the normaliser sums the unrounded values; decode keeps them in float32)

The layer follows the oracle's `layer_forward` step by step (page 1 `g4e_forward`), reusing its
primitives; only the rounding calls are added.
"""
import numpy as np

import oracle as O


def to_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def to_bf16(x):
    """Nearest-even bf16 of the float32 rounding of x (finite inputs)."""
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


MODES = {
    "bf16_prefill": {"act", "qkv", "q", "kv", "p"},
    "bf16_few_rows": {"act", "q", "kv", "p"},  # a prefill of at most 64 token rows (float32 q/k/v partials)
    "bf16_decode": {"act", "q", "kv"},
    "kv_only": {"kv"},
    "none": set(),
}


class Rounder:
    """r(point, x): x rounded to bf16 if `point` is in the mode's set (to float32 with f32=True)."""

    def __init__(self, mode, f32=False):
        self.points = MODES[mode] if not f32 else MODES["bf16_prefill"]
        self.fn = to_f32 if f32 else to_bf16

    def __call__(self, point, x):
        return self.fn(x) if point in self.points else O.f64(x)


def attention_rounded(q, K, V, qpos, window, r, chunk=256):
    """The oracle's causal GQA attention (scale 1) with the P V operand rounded at point `p`; the
    normaliser sums the unrounded probabilities."""
    q, K, V = O.f64(q), O.f64(K), O.f64(V)
    qpos = np.asarray(qpos, dtype=np.int64)
    T, nh, hd = q.shape
    grp = nh // K.shape[0]
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
            s = np.where(vis, q[t0:t1, h, :] @ K[g, lo:hi, :].T, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            out[t0:t1, h, :] = (r("p", e) @ V[g, lo:hi, :]) / e.sum(axis=1, keepdims=True)
    return out


def layer_rounded(cfg, lw, layer, src, h, ple_l, pos, caches, r):
    """`oracle.layer_forward` (causal) with the rounding points of `r`. Caches are float64 arrays
    [B, nkv, cap, hd], written in place (rounded at point `kv`) when the layer owns its cache."""
    eps = cfg["eps"]
    nh, nkv = cfg["n_heads"], O.kv_heads(cfg, layer)
    sliding, hd, theta, n_rot = O.layer_geometry(cfg, layer)
    inv = O.inv_freq(hd, theta, n_rot)
    h = O.f64(h).copy()
    B, T, H = h.shape
    pos = np.asarray(pos, dtype=np.int64)
    w = {k: (O.f64(v) if k != "layer_scalar" else v) for k, v in lw.items()}

    xn = r("act", O.rms_norm(h, w["input_norm"], eps))
    q = r("qkv", xn @ w["wq"].T).reshape(B, T, nh, hd)
    q = r("q", O.rope(O.rms_norm(q, w["q_norm"], eps), pos[:, :, None], inv))
    if src == layer:
        k = r("qkv", xn @ w["wk"].T).reshape(B, T, nkv, hd)
        k = r("kv", O.rope(O.rms_norm(k, w["k_norm"], eps), pos[:, :, None], inv))
        v = r("qkv", xn @ O.f64(O.value_weight(cfg, lw, layer)).T).reshape(B, T, nkv, hd)
        v = r("kv", O.rms_norm(v, None, eps))
        K, V = caches[layer]
        for b in range(B):
            for t in range(T):
                K[b, :, pos[b, t], :] = k[b, t]
                V[b, :, pos[b, t], :] = v[b, t]
    K, V = caches[src]
    window = cfg["window"] if sliding else None
    o = np.stack([attention_rounded(q[b], K[b], V[b], pos[b], window, r) for b in range(B)])
    a = r("act", o.reshape(B, T, nh * hd)) @ w["wo"].T
    h = h + O.rms_norm(a, w["post_attn_norm"], eps)

    xn2 = r("act", O.rms_norm(h, w["pre_ffn_norm"], eps))
    act = r("act", O.gelu_tanh(xn2 @ w["w_gate"].T) * (xn2 @ w["w_up"].T))
    h = h + O.rms_norm(act @ w["w_down"].T, w["post_ffn_norm"], eps)

    hb = r("act", h)
    g = r("act", O.gelu_tanh(hb @ w["ple_gate"].T) * O.f64(ple_l))
    h = h + O.rms_norm(g @ w["ple_proj"].T, w["post_ple_norm"], eps)
    return h * float(lw.get("layer_scalar", 1.0))


def rel_l2(a, b):
    a, b = O.f64(a), O.f64(b)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def layer_floors(cfg, layers, hs, ple, pos, caches, mode, rows=None):
    """Per-layer floors: layer l replayed with `mode`'s roundings from the oracle's input hs[l], over
    caches written by the replayed layers themselves (as the GPU per-layer tests run), against the
    oracle's output hs[l+1]. `caches` (float64, modified) start as the call's initial caches; `layers`
    is a list or a callable layer -> weights. `rows`: sequences to compare (decode samples)."""
    r = Rounder(mode)
    srcs = O.kv_sources(cfg["layer_types"], cfg["n_shared"])
    out = []
    ple = O.f64(ple)
    for l in range(cfg["n_layers"]):
        lw = layers(l) if callable(layers) else layers[l]
        hl = layer_rounded(cfg, lw, l, srcs[l], hs[l], ple[:, :, l, :], pos, caches, r)
        sel = slice(None) if rows is None else rows
        out.append(rel_l2(hl[sel], hs[l + 1][sel]))
    return out


def stack_rounded(cfg, layers, h0, ple, pos, caches, mode, f32=False):
    """The whole stack replayed with `mode`'s roundings (to float32 instead with f32=True)."""
    r = Rounder(mode, f32=f32)
    srcs = O.kv_sources(cfg["layer_types"], cfg["n_shared"])
    h = O.f64(h0)
    ple = O.f64(ple)
    for l in range(cfg["n_layers"]):
        lw = layers(l) if callable(layers) else layers[l]
        h = layer_rounded(cfg, lw, l, srcs[l], h, ple[:, :, l, :], pos, caches, r)
    return h
