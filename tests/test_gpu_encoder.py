"""The encoder's non-causal attention on the GPU (taconite-embeddinggemma2 `text_attention`): the call's
own keys, all of them on full layers and those with |i - j| <= W on sliding layers.

Kernel level through g4_attn_encode against the oracle's `attention_bidirectional`, with cache rows
outside the call holding values that must never be read; a bit-exact mask probe; then the encoder
workload (E4B widths) layer by layer through g4_stack_forward / g4_layer_forward in G4_ENCODE mode.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gemma_decoder_forward_amd import binding as bd
from synth import configs, gen
from tests.gpu_util import DT, TOL_BF16_RELL2, assert_close, build_model, host_layer, log, randn, rel_l2, stream

pytestmark = pytest.mark.gpu


def _kv_table(entries):
    t = (bd.KvEntry * len(entries))()
    for i, (k, v, sliding) in enumerate(entries):
        t[i] = bd.KvEntry(k=k.data_ptr(), v=v.data_ptr(), cap=k.shape[2], hd=k.shape[3], sliding=sliding)
    return t


def _encode(q, K, V, sliding, window, pos0, B, T, nh, nkv, hd, gdt):
    out = torch.empty((B * T, nh * hd), dtype=q.dtype, device="cuda")
    t = _kv_table([(K, V, sliding)])
    bd.g4_attn_encode(q.data_ptr(), nh * hd, t, 1, 0, 0, sliding, window, pos0.data_ptr(), B, T, nh, nkv, hd, 1.0,
                      out.data_ptr(), nh * hd, None, 0, gdt, stream())
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("hd,sliding,window,nh,nkv", [(64, 1, 32, 4, 1), (128, 0, 0, 4, 1), (256, 1, 512, 8, 2),
                                                      (512, 0, 0, 8, 2), (256, 1, 7, 4, 2), (128, 1, 40, 2, 2),
                                                      (512, 1, 100, 4, 2)])
def test_attention_encode_vs_oracle(dt, hd, sliding, window, nh, nkv):
    """Two sequences of 77 tokens at cache rows 0.. and 600..: every other row of the 700-row cache holds
    values scaled by 30 that would dominate any softmax they leaked into."""
    log(f"attn_encode {dt} hd={hd} sliding={sliding} W={window}")
    gdt, tdt = DT[dt]
    B, T, cap = 2, 77, 700
    pos0_l = [0, 600]
    pos0 = torch.tensor(pos0_l, dtype=torch.int32, device="cuda")
    q = randn((B * T, nh * hd), 130 + hd, tdt)
    K = randn((B, nkv, cap, hd), 131, tdt, 30.0)
    V = randn((B, nkv, cap, hd), 132, tdt, 30.0)
    for b, p0 in enumerate(pos0_l):  # the call's own rows at the usual scale
        K[b, :, p0:p0 + T] = randn((nkv, T, hd), 133 + b, tdt)
        V[b, :, p0:p0 + T] = randn((nkv, T, hd), 135 + b, tdt)
    out = _encode(q, K, V, sliding, window, pos0, B, T, nh, nkv, hd, gdt)
    qv = O.f64(q).reshape(B, T, nh, hd)
    pos = O.prefill_positions(pos0_l, T)
    for b, p0 in enumerate(pos0_l):
        ref = O.attention_bidirectional(qv[b], O.f64(K[b]), O.f64(V[b]), pos[b], p0, p0 + T,
                                        window if sliding else None)
        assert_close(out.reshape(B, T, nh, hd)[b], ref, dt, f"seq {b}")


@pytest.mark.parametrize("hd,sliding,window,p0", [(64, 1, 7, 0), (64, 0, 0, 9), (256, 1, 33, 0), (128, 0, 0, 0),
                                                  (512, 1, 21, 5), (256, 1, 40, 3)])
def test_attention_encode_mask_probe_bit_exact(hd, sliding, window, p0):
    """q = 0 gives uniform weights over the visible keys; V_j = onehot(j mod hd) for the call's rows and a
    large value elsewhere, so round(o * n) is exactly the row of the mask |i - j| <= W within the call."""
    T, nh, nkv = 64, 4, 1
    cap = p0 + T + 6
    q = torch.zeros((T, nh * hd), dtype=torch.bfloat16, device="cuda")
    K = randn((1, nkv, cap, hd), 140, torch.bfloat16)
    Vh = torch.full((1, nkv, cap, hd), 64.0)
    for j in range(T):
        Vh[0, :, p0 + j] = 0.0
        Vh[0, :, p0 + j, j % hd] = 1.0
    V = Vh.to(torch.bfloat16).cuda()
    pos0 = torch.tensor([p0], dtype=torch.int32, device="cuda")
    out = _encode(q, K, V, sliding, window, pos0, 1, T, nh, nkv, hd, bd.G4_BF16)
    o = O.f64(out).reshape(T, nh, hd)
    for i in range(T):
        vis = [j for j in range(T) if not sliding or abs(i - j) <= window]
        want = np.zeros(hd)
        for j in vis:
            want[j % hd] += 1
        for h in range(nh):
            assert np.array_equal(np.rint(o[i, h] * len(vis)), want), (i, h)


@pytest.mark.parametrize("hd,sliding,W", [(256, 1, 512), (512, 0, 0)])
def test_attention_encode_e4b_shapes(hd, sliding, W):
    """E4B heads (8 q / 2 kv) over T = 2048: the encoder workload's attention call, whole output."""
    log(f"attn_encode long hd={hd}")
    B, T, nh, nkv = 1, 2048, 8, 2
    q = randn((T, nh * hd), 145 + hd, torch.bfloat16)
    K = randn((1, nkv, T, hd), 146, torch.bfloat16)
    V = randn((1, nkv, T, hd), 147, torch.bfloat16)
    pos0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = _encode(q, K, V, sliding, W, pos0, B, T, nh, nkv, hd, bd.G4_BF16)
    ref = O.attention_bidirectional(O.f64(q).reshape(T, nh, hd), O.f64(K[0]), O.f64(V[0]), np.arange(T), 0, T,
                                    W if sliding else None)
    e = assert_close(out.reshape(T, nh, hd), ref, "bf16", "encoder attention")
    log(f"encoder attention hd={hd} T=2048: rel L2 {e:.2e}")


# ------------------------------------------------------------------------------- encoder stacks
def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).cuda()


def test_fp32_encoder_stack_end_to_end():
    """Config-1 shapes as an encoder (float32), the whole stack including its shared layers, end to end."""
    cfg = configs.get(1, T=72, mode="encode", embed=False)
    model, layers, _ = build_model(cfg)
    acts = gen.activations(cfg, "cuda")
    h = acts["h0"].clone()
    caches, table = model.new_caches(1, cfg["T"])
    model.forward(h, acts["ple_in"], acts["pos"], table, cfg["T"], bd.G4_ENCODE)
    torch.cuda.synchronize()
    ref = O.forward(cfg, host_layer(layers), O.f64(acts["h0"]), O.f64(acts["ple_in"]), O.prefill_positions([0], 72),
                    O.new_caches(cfg, 1, 72), bidirectional=True)
    e = assert_close(h, ref, "f32", "encoder final hidden")
    log(f"fp32 encoder stack: max rel {e:.2e}")
    causal = O.forward(cfg, host_layer(layers), O.f64(acts["h0"]), O.f64(acts["ple_in"]), O.prefill_positions([0], 72),
                       O.new_caches(cfg, 1, 72))
    assert rel_l2(h, causal) > 1e-2  # the mask matters: the causal stack is far from the encoder's


@pytest.mark.parametrize("T", [1100, 24])
def test_bf16_encoder_per_layer(T):
    """The encoder workload (E4B widths, bf16), layer by layer: T = 1100 on the tiled path with a ragged
    last tile, T = 24 on the few-row path."""
    cfg = configs.get(7, T=T)
    model, layers, _ = build_model(cfg)
    acts = gen.activations(cfg, "cuda")
    h = acts["h0"].clone()
    caches, table = model.new_caches(1, T)
    model.forward(h, acts["ple_in"], acts["pos"], table, T, bd.G4_ENCODE)
    torch.cuda.synchronize()
    assert torch.isfinite(h).all()
    h0, ple = O.f64(acts["h0"]), O.f64(acts["ple_in"])
    hs = [h0]
    O.forward(cfg, host_layer(layers), h0, ple, O.prefill_positions([0], T), O.new_caches(cfg, 1, T), per_layer=hs,
              bidirectional=True)
    log(f"encoder T={T}: end-to-end bf16 deviation rel L2 {rel_l2(h, hs[-1]):.3e}")
    ple_d = _dev(ple)
    caches, table = model.new_caches(1, T)
    errs = []
    for l in range(model.L):
        x = _dev(hs[l])
        model.forward(x, ple_d, acts["pos"], table, T, bd.G4_ENCODE, layer=l)
        torch.cuda.synchronize()
        errs.append(rel_l2(x, hs[l + 1]))
    log(f"encoder T={T} per-layer rel L2: " + " ".join(f"{e:.1e}" for e in errs))
    assert max(errs) <= TOL_BF16_RELL2, f"layer {int(np.argmax(errs))}: {max(errs):.3e}"


@pytest.mark.parametrize("layer", [0, 5])
def test_encoder_full_size_layer_sampled_rows(layer):
    """A sliding (0) and the full (5) layer of the encoder workload at its full size, T = 2048, in the
    launch configuration the benchmark times; rows checked one by one against the oracle."""
    cfg = configs.get(7)
    T = cfg["T"]
    model, layers, _ = build_model(cfg)
    acts = gen.activations(cfg, "cuda")
    rows = list(range(16)) + [600, 1023, 1500] + list(range(T - 16, T))
    lw = host_layer(layers)(layer)
    h0, ple = O.f64(acts["h0"]), O.f64(acts["ple_in"])
    rr, ref = O.layer_forward_rows(cfg, lw, layer, h0[0], ple[0, :, layer, :], 0, rows, bidirectional=True)
    caches, table = model.new_caches(1, T)
    h = _dev(h0)
    model.forward(h, _dev(ple), acts["pos"], table, T, bd.G4_ENCODE, layer=layer)
    torch.cuda.synchronize()
    e = rel_l2(h[0, rr], ref)
    log(f"encoder layer {layer} T={T}: sampled rows rel L2 {e:.3e}")
    assert e <= TOL_BF16_RELL2


def test_bf16_encoder_batch_at_offsets_ignores_earlier_rows():
    """Two sequences encoded at cache offsets 0 and 37 of a 160-row cache whose other rows hold junk
    (x 50): every layer, from the oracle's input, matches the oracle's encoder over each call's own keys."""
    cfg = configs.get(7, T=100, B=2, layer_types="SSF")
    T, cap, offs = 100, 160, [0, 37]
    model, layers, _ = build_model(cfg)
    acts = gen.activations(cfg, "cuda")
    pos = torch.tensor(offs, dtype=torch.int32, device="cuda")
    caches, table = model.new_caches(2, cap)
    for l, (k, v) in caches.items():
        k.copy_(randn(k.shape, 150 + l, k.dtype, 50.0))
        v.copy_(randn(v.shape, 160 + l, v.dtype, 50.0))
    h0, ple = O.f64(acts["h0"]), O.f64(acts["ple_in"])
    hs = [h0]
    O.forward(cfg, host_layer(layers), h0, ple, O.prefill_positions(offs, T), O.new_caches(cfg, 2, cap),
              per_layer=hs, bidirectional=True)
    ple_d = _dev(ple)
    errs = []
    for l in range(model.L):
        x = _dev(hs[l])
        model.forward(x, ple_d, pos, table, cap, bd.G4_ENCODE, layer=l)
        torch.cuda.synchronize()
        errs.append(max(rel_l2(x[b], hs[l + 1][b]) for b in range(2)))
    log("encoder at offsets, per-layer rel L2 (worst sequence): " + " ".join(f"{e:.1e}" for e in errs))
    assert max(errs) <= TOL_BF16_RELL2
