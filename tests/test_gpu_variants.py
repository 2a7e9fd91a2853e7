"""The variants on the GPU against the float64 oracle: full layers with their own KV head count, K=V full
layers (V from the K projection, normed without scale, not rotated) and one FFN width per layer.

Same bars as the base workloads: float32 end to end within max relative error 1e-3; bf16 layer by layer
within relative L2 2e-2 (each GPU layer starts from the oracle's input for that layer); decode on
cached contexts per layer; the caches the GPU writes checked against the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gemma_decoder_forward_amd import binding as bd
from synth import configs, gen
from tests.gpu_util import TOL_BF16_RELL2, assert_close, build_model, host_layer, log, max_rel, rel_l2
from tests.test_gpu_stack import _oracle_entry

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).cuda()


def _per_layer(model, hs, ple, pos, table, cap, mode, rows=None):
    ple_d = _dev(ple)
    errs = []
    for l in range(model.L):
        h = _dev(hs[l])
        model.forward(h, ple_d, pos, table, cap, mode, layer=l)
        torch.cuda.synchronize()
        sel = slice(None) if rows is None else rows
        errs.append(rel_l2(h[sel], hs[l + 1][sel]))
    return errs


# kv heads of the full layer (4 query heads): 2 per kv head, 1 per kv head, all 4 on one
@pytest.mark.parametrize("nkv_full,k_eq_v", [(2, True), (4, False), (1, True)])
def test_fp32_variant_stack_end_to_end(nkv_full, k_eq_v):
    """Config-1 shapes with the variants, float32, whole stack from token ids, caches included."""
    cfg = configs.get(1, T=72, n_heads=4, n_kv_heads_full=nkv_full, k_eq_v=k_eq_v, ffn_dims=[1024, 768, 512, 640])
    model, layers, glob = build_model(cfg)
    assert "wv" not in layers[3] if k_eq_v else "wv" in layers[3]
    acts = gen.activations(cfg, "cuda")
    h, ple = model.embed(acts["ids"])
    caches, table = model.new_caches(1, cfg["T"])
    model.forward(h, ple, acts["pos"], table, cfg["T"], bd.G4_PREFILL)
    torch.cuda.synchronize()
    rc = O.new_caches(cfg, 1, cfg["T"])
    h0, ple0 = _oracle_entry(cfg, glob, acts["ids"])
    ref = O.forward(cfg, host_layer(layers), h0, ple0, O.prefill_positions([0], cfg["T"]), rc)
    e = assert_close(h, ref, "f32", "final hidden")
    log(f"fp32 variants nkv_full={nkv_full} k_eq_v={k_eq_v}: max rel {e:.2e}")
    for l, (k, v) in caches.items():
        assert k.shape[1] == (nkv_full if cfg["layer_types"][l] == "F" else cfg["n_kv_heads"])
        assert_close(k, rc[l][0], "f32", f"K cache {l}")
        assert_close(v, rc[l][1], "f32", f"V cache {l}")


@pytest.mark.parametrize("T,nkv_full", [(1100, 4), (24, 4), (300, 1)])
def test_bf16_variant_stack_per_layer(T, nkv_full):
    """E4B widths with the variants (bf16): T = 1100 takes the tiled path (ragged last tile), T = 24 the
    few-row path, whose K=V full layers form V from the K partial sums; one kv head for all eight query
    heads of a full layer is a group size outside the matrix-core attention kernels (generic kernel)."""
    cfg = configs.get(6, T=T, n_kv_heads_full=nkv_full)
    model, layers, glob = build_model(cfg)
    acts = gen.activations(cfg, "cuda")
    h = acts["h0"].clone()
    caches, table = model.new_caches(1, T)
    model.forward(h, acts["ple_in"], acts["pos"], table, T, bd.G4_PREFILL)
    torch.cuda.synchronize()
    assert torch.isfinite(h).all()
    h0, ple = O.f64(acts["h0"]), O.f64(acts["ple_in"])
    hs = [h0]
    rc = O.new_caches(cfg, 1, T)
    O.forward(cfg, host_layer(layers), h0, ple, O.prefill_positions([0], T), rc, per_layer=hs)
    log(f"variants T={T}: end-to-end bf16 deviation rel L2 {rel_l2(h, hs[-1]):.3e}")
    caches, table = model.new_caches(1, T)
    errs = _per_layer(model, hs, ple, acts["pos"], table, T, bd.G4_PREFILL)
    log(f"variants T={T} per-layer rel L2: " + " ".join(f"{e:.1e}" for e in errs))
    assert max(errs) <= TOL_BF16_RELL2, f"layer {int(np.argmax(errs))}: {max(errs):.3e}"
    # the K=V full layer's cache, written from the oracle's layer input
    k, v = caches[2]
    assert k.shape[1] == cfg["n_kv_heads_full"] and v.shape == k.shape
    assert rel_l2(k, rc[2][0]) <= TOL_BF16_RELL2 and rel_l2(v, rc[2][1]) <= TOL_BF16_RELL2


@pytest.mark.parametrize("B", [1, 5])
def test_bf16_variant_decode_per_layer(B):
    """Decode at E4B widths with the variants over a 1000-token cached context, layer by layer."""
    cfg = configs.get(6, mode="decode", B=B, T=1, ctx=1000)
    model, layers, glob = build_model(cfg)
    acts = gen.activations(cfg, "cuda")
    ctx = cfg["ctx"]
    fills = {l: gen.decode_cache(cfg, l, "cuda") for l in range(cfg["n_layers"]) if model.kv_src[l] == l}
    assert fills[2][0].shape[1] == cfg["n_kv_heads_full"]
    caches, table = model.new_caches(B, ctx, fill=lambda l: fills[l])
    ocache = {l: (O.f64(k), O.f64(v)) for l, (k, v) in fills.items()}
    h0, ple = O.f64(acts["h0"]), O.f64(acts["ple_in"])
    hs = [h0]
    O.forward(cfg, host_layer(layers), h0, ple, np.full((B, 1), ctx - 1), ocache, per_layer=hs)
    errs = _per_layer(model, hs, ple, acts["pos"], table, ctx, bd.G4_DECODE)
    log(f"variants decode B={B} per-layer rel L2: " + " ".join(f"{e:.1e}" for e in errs))
    assert max(errs) <= TOL_BF16_RELL2, f"layer {int(np.argmax(errs))}: {max(errs):.3e}"
    # the new token's K=V row landed in the full layer's cache like the oracle's
    k, v = caches[2]
    assert rel_l2(v[:, :, ctx - 1], ocache[2][1][:, :, ctx - 1]) <= TOL_BF16_RELL2


def test_variant_equals_base_when_the_variants_are_neutral():
    """With n_kv_heads_full equal to n_kv_heads, no K=V and every FFN width equal to ffn, the variant
    descriptor fields change nothing: bit-identical output to the base model (same weights)."""
    base = configs.get(2, T=300)
    model, layers, _ = build_model(base)
    neutral = dict(base, n_kv_heads_full=base["n_kv_heads"], k_eq_v=False, ffn_dims=[base["ffn"]] * 2)
    from gemma_decoder_forward_amd.model import G4Model
    m2 = G4Model(neutral, layers)
    acts = gen.activations(base, "cuda")
    outs = []
    for m in (model, m2):
        h = acts["h0"].clone()
        caches, table = m.new_caches(1, 300)
        m.forward(h, acts["ple_in"], acts["pos"], table, 300, bd.G4_PREFILL)
        torch.cuda.synchronize()
        outs.append(h)
    assert torch.equal(outs[0], outs[1])
    assert max_rel(outs[0], outs[1]) == 0.0
