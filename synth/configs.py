"""Workload descriptions: the Gemma-4 E-series shapes this repository is tested and timed on.

Plain data only (sizes, dtypes, the layer-type pattern, how many tail layers share KV). Nothing here
computes any step of the method; the routing of shared layers, head widths per type, frequencies and so
on are derived independently by the HIP path's host code and by the oracle.

Shapes follow the pages' E-series description (cortiq-engine `g4e.rs`, module doc and `G4eGlobals`;
ferrox-models `gemma4_engine.rs`, `Gemma4Hparams`): sliding layers at `head_dim` with a local RoPE base,
full layers at `global_head_dim` with the model base and a proportional partial-rotary prefix.
"""

E4B = dict(
    hidden=2560, n_heads=8, n_kv_heads=2, head_dim_swa=256, head_dim_full=512, window=512,
    theta_swa=1.0e4, theta_full=1.0e6, partial_rotary=0.25, ffn=10240, ple_dim=256, eps=1e-6,
    vocab=262144, ple_vocab=262144,
)

CONFIGS = {
    # Tiny fp32 stack: correctness config, small enough for pure-Python pins.
    1: dict(
        name="tiny-fp32-4L", dtype="f32", mode="prefill", B=1, T=64,
        hidden=256, n_heads=4, n_kv_heads=1, head_dim_swa=64, head_dim_full=128, window=32,
        theta_swa=1.0e4, theta_full=1.0e6, partial_rotary=0.25, ffn=1024, ple_dim=32, eps=1e-6,
        vocab=512, ple_vocab=512, layer_types="SSSF", n_shared=2, embed=True,
    ),
    # One E4B-shaped sliding layer followed by one full layer, both owning their KV.
    2: dict(E4B, name="e4b-layer-pair", dtype="bf16", mode="prefill", B=1, T=2048,
            layer_types="SF", n_shared=0, embed=False),
    # The 42-layer E4B-like stack from token ids (embedding + PLE inputs included).
    3: dict(E4B, name="e4b-42L-prefill", dtype="bf16", mode="prefill", B=1, T=4096,
            layer_types="SSSSSF" * 7, n_shared=18, embed=True),
    # Decode over an 8192-token context, one new token per sequence.
    4: dict(E4B, name="e4b-42L-decode", dtype="bf16", mode="decode", B=1, T=1, ctx=8192,
            batches=(1, 8, 32, 64), layer_types="SSSSSF" * 7, n_shared=18, embed=True),
    # Long-context, attention-heavy 12-layer slice.
    5: dict(E4B, name="e4b-12L-T32k", dtype="bf16", mode="prefill", B=1, T=32768,
            layer_types="SSSSSF" * 2, n_shared=4, embed=False),
    # The variants at E4B widths: full layers with their own KV head count and V taken from the K
    # projection (turbospark-runtime gemma4 `forward_layer`), and one FFN width per layer (ferrox-models
    # `Gemma4Hparams::ffn_dim`). The two tail layers share KV, so the last full layer reads a K=V cache.
    6: dict(E4B, name="e4b-variants-6L", dtype="bf16", mode="prefill", B=1, T=2048, layer_types="SSFSSF",
            n_shared=2, embed=False, n_kv_heads_full=4, k_eq_v=True,
            ffn_dims=[10240, 6144, 8192, 10240, 4096, 8192]),
    # The encoder at E4B widths (taconite-embeddinggemma2 `text`/`text_attention`): the same layers with
    # the non-causal mask, every layer computing its own K/V (no shared tail), given h0 and ple_in.
    7: dict(E4B, name="e4b-encoder-6L", dtype="bf16", mode="encode", B=1, T=2048, layer_types="SSSSSF",
            n_shared=0, embed=False),
}


def get(cid, **overrides):
    """A copy of config `cid` with fields overridden (e.g. a shorter T for a parity case)."""
    c = dict(CONFIGS[cid])
    c["id"] = cid
    c.update(overrides)
    c["n_layers"] = len(c["layer_types"])
    return c


def tiny(**overrides):
    """A very small bf16/f32 model for pure-Python brute force and fast parity cases."""
    c = dict(
        id=0, name="micro", dtype="f32", mode="prefill", B=1, T=8,
        hidden=32, n_heads=4, n_kv_heads=2, head_dim_swa=8, head_dim_full=16, window=3,
        theta_swa=1.0e4, theta_full=1.0e6, partial_rotary=0.25, ffn=48, ple_dim=8, eps=1e-6,
        vocab=40, ple_vocab=32, layer_types="SSF", n_shared=0, embed=True,
    )
    c.update(overrides)
    c["n_layers"] = len(c["layer_types"])
    return c
