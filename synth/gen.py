"""Seeded synthetic inputs shared by the HIP path's tests/bench and by the oracle.

Every tensor is drawn from its own torch generator seeded from (config seed, tensor name), so any
tensor can be regenerated alone and in any order. Draws happen on the requested device: the CPU for
small cases, the GPU for E4B-sized tables (a host Mersenne/Philox stream of ~7e9 normals would take
minutes). A tensor drawn on the GPU is copied to the host before the oracle sees it.

Distributions (one recipe for every config):
  * projection and embedding weights ~ N(0, 0.02)
  * every norm weight (input/post-attn/pre-ffn/post-ffn/post-ple, q_norm, k_norm, ple_norm) ~ 1 + N(0, 0.1)
  * hidden states and per-layer inputs given directly ~ N(0, 1) (f32)
  * token ids ~ U[0, vocab)
  * decode KV caches: rows [0, ctx-1) ~ N(0, 1), the row of the new token is zero
This module holds no step of the method: K/V weights are drawn for every layer, whether or not the
routing later gives that layer its own cache (a full layer of a K=V model has no V weight to draw).
"""
import zlib

import torch

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def seed_of(cfg):
    return 1000 + int(cfg.get("id", 0)) if cfg.get("mode") != "decode" else 4000 + int(cfg["B"])


def _gen(seed, name, device):
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + zlib.crc32(name.encode())) & ((1 << 63) - 1))
    return g


def normal(shape, std, mean, seed, name, device="cpu", dtype=torch.float32, chunk_rows=None):
    """N(mean, std) of `shape`, rounded to `dtype` (rounding happens once, after scaling)."""
    device = torch.device(device)
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0] if len(shape) > 0 else 1
    step = chunk_rows or max(1, (1 << 27) // max(1, out[0].numel() if out.dim() > 0 else 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        g = _gen(seed, f"{name}#{r0}", device)
        sub = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
        sub.mul_(std).add_(mean)
        out[r0:r1] = sub.to(dtype)
    return out


def uniform_ids(n_shape, high, seed, name, device="cpu"):
    g = _gen(seed, name, torch.device(device))
    return torch.randint(0, high, n_shape, generator=g, device=device, dtype=torch.int64).to(torch.int32)


def head_dim(cfg, layer):
    return cfg["head_dim_swa"] if cfg["layer_types"][layer] == "S" else cfg["head_dim_full"]


def kv_heads(cfg, layer):
    """Shape data: KV head count of a layer (full layers may carry their own, `n_kv_heads_full`)."""
    if cfg["layer_types"][layer] == "S":
        return cfg["n_kv_heads"]
    return cfg.get("n_kv_heads_full") or cfg["n_kv_heads"]


def ffn_dim(cfg, layer):
    """Shape data: FFN width of a layer (`ffn_dims` lists one per layer, else every layer has `ffn`)."""
    dims = cfg.get("ffn_dims")
    return int(dims[layer]) if dims else cfg["ffn"]


def has_v_proj(cfg, layer):
    """Weight inventory: a full layer of a K=V model carries no V projection weight."""
    return not (cfg.get("k_eq_v") and cfg["layer_types"][layer] != "S")


def model_globals(cfg, device="cpu"):
    """Embedding table, PLE table, PLE model projection and PLE norm (configs built from token ids)."""
    s, dt = seed_of_model(cfg), TORCH_DTYPES[cfg["dtype"]]
    H, L, d = cfg["hidden"], cfg["n_layers"], cfg["ple_dim"]
    return dict(
        embed=normal((cfg["vocab"], H), 0.02, 0.0, s, "embed", device, dt),
        ple_embed=normal((cfg["ple_vocab"], L * d), 0.02, 0.0, s, "ple_embed", device, dt),
        ple_model_proj=normal((L * d, H), 0.02, 0.0, s, "ple_model_proj", device, dt),
        ple_norm=normal((d,), 0.1, 1.0, s, "ple_norm", device, dt),
    )


def seed_of_model(cfg):
    """Weights of the decode config equal those of the 42-layer prefill config (same model)."""
    return 1000 + (3 if cfg.get("id") == 4 else int(cfg.get("id", 0)))


def layer_weights(cfg, layer, device="cpu"):
    s, dt = seed_of_model(cfg), TORCH_DTYPES[cfg["dtype"]]
    H, nh, d = cfg["hidden"], cfg["n_heads"], cfg["ple_dim"]
    nkv, F, hd = kv_heads(cfg, layer), ffn_dim(cfg, layer), head_dim(cfg, layer)
    p = f"L{layer}."
    w = lambda shape, name: normal(shape, 0.02, 0.0, s, p + name, device, dt)  # noqa: E731
    n = lambda size, name: normal((size,), 0.1, 1.0, s, p + name, device, dt)  # noqa: E731
    out = dict(
        input_norm=n(H, "input_norm"),
        wq=w((nh * hd, H), "wq"),
        wk=w((nkv * hd, H), "wk"),
        wo=w((H, nh * hd), "wo"),
        q_norm=n(hd, "q_norm"),
        k_norm=n(hd, "k_norm"),
        post_attn_norm=n(H, "post_attn_norm"),
        pre_ffn_norm=n(H, "pre_ffn_norm"),
        w_gate=w((F, H), "w_gate"),
        w_up=w((F, H), "w_up"),
        w_down=w((H, F), "w_down"),
        post_ffn_norm=n(H, "post_ffn_norm"),
        ple_gate=w((d, H), "ple_gate"),
        ple_proj=w((H, d), "ple_proj"),
        post_ple_norm=n(H, "post_ple_norm"),
        layer_scalar=1.0,
    )
    if has_v_proj(cfg, layer):
        out["wv"] = w((nkv * hd, H), "wv")
    return out


def activations(cfg, device="cpu"):
    """Inputs of one forward: token ids (embedding configs) or h0 and ple_in, plus positions."""
    s = seed_of(cfg)
    B, T = cfg["B"], cfg["T"]
    out = {}
    if cfg["embed"]:
        out["ids"] = uniform_ids((B, T), cfg["vocab"], s, "ids", device)
    else:
        H, L, d = cfg["hidden"], cfg["n_layers"], cfg["ple_dim"]
        out["h0"] = normal((B, T, H), 1.0, 0.0, s, "h0", device, torch.float32)
        out["ple_in"] = normal((B, T, L, d), 1.0, 0.0, s, "ple_in", device, torch.float32)
    if cfg["mode"] == "decode":
        out["pos"] = torch.full((B,), cfg["ctx"] - 1, dtype=torch.int32, device=device)
    else:
        out["pos"] = torch.zeros((B,), dtype=torch.int32, device=device)
    return out


def decode_cache(cfg, layer, device="cpu"):
    """K and V of one layer, [B, nkv, ctx, hd]: rows before the new token ~ N(0,1), its row zero."""
    s, dt = seed_of(cfg), TORCH_DTYPES[cfg["dtype"]]
    B, nkv, ctx = cfg["B"], kv_heads(cfg, layer), cfg["ctx"]
    hd = head_dim(cfg, layer)
    kv = []
    for nm in ("k", "v"):
        t = normal((B * nkv, ctx, hd), 1.0, 0.0, s, f"cache{layer}.{nm}", device, dt, chunk_rows=1)
        t[:, ctx - 1, :] = 0
        kv.append(t.view(B, nkv, ctx, hd))
    return kv[0], kv[1]
