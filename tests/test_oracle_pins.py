"""Pins of the float64 oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something other than itself: a closed form, an invariant, a
special case, a library routine the oracle does not call (torch CPU), a value the pages print
(tests/golden), or pure-Python brute force on tiny inputs (tests/bruteforce.py).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from synth import configs, gen
from tests import bruteforce as bf

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(7)


# ---------------------------------------------------------------- RMSNorm
def test_rms_unit_rms_before_weight():
    x = rng.normal(size=(5, 96)) * 3.0
    y = O.rms_norm(x, None, 1e-6)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), np.sqrt(ms / (ms + 1e-6)), rtol=1e-14)


def test_rms_constant_vector_closed_form():
    for c in (0.5, -2.0, 1e-4):
        x = np.full(64, c)
        w = rng.normal(size=64)
        np.testing.assert_allclose(O.rms_norm(x, w, 1e-6), c / math.sqrt(c * c + 1e-6) * w, rtol=1e-14)


def test_rms_matches_torch_rms_norm():
    x = rng.normal(size=(7, 128))
    w = 1 + 0.1 * rng.normal(size=128)
    ref = F.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, w, 1e-6), ref, rtol=1e-13, atol=1e-15)


def test_rms_of_zero_is_zero():
    assert np.all(O.rms_norm(np.zeros((2, 16)), np.ones(16), 1e-6) == 0.0)


def test_rms_eps_inside_mean_not_plus_one_weight():
    # a tiny vector where eps dominates: x / sqrt(x^2 + eps), weight applied as is
    x = np.full(8, 1e-4)
    w = np.full(8, 0.5)
    np.testing.assert_allclose(O.rms_norm(x, w, 1e-6), 0.5 * 1e-4 / math.sqrt(1e-8 + 1e-6), rtol=1e-14)


# ---------------------------------------------------------------- gelu-tanh
def test_gelu_constants_are_the_pages():
    g = json.load(open(os.path.join(GOLD, "constants.json")))
    assert abs(g["gelu_tanh_inner_scale"] - math.sqrt(2 / math.pi)) < 1e-16
    x = np.array([0.3, -1.7, 2.5])
    manual = 0.5 * x * (1 + np.tanh(g["gelu_tanh_inner_scale"] * (x + g["gelu_tanh_cubic"] * x ** 3)))
    np.testing.assert_allclose(O.gelu_tanh(x), manual, rtol=1e-15)


def test_gelu_matches_torch_tanh_approximation():
    x = rng.normal(size=1000) * 4
    ref = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(x), ref, rtol=1e-12, atol=1e-15)


def test_gelu_odd_part_identity():
    x = rng.normal(size=100) * 3
    np.testing.assert_allclose(O.gelu_tanh(x) - O.gelu_tanh(-x), x, rtol=1e-13, atol=1e-14)
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0


# ---------------------------------------------------------------- RoPE
@pytest.mark.parametrize("hd,theta,n_rot", [(64, 1e4, 32), (128, 1e6, 16), (512, 1e6, 64), (256, 1e4, 128)])
def test_rope_matches_complex_rotation(hd, theta, n_rot):
    x = rng.normal(size=hd)
    for pos in (0, 1, 17, 4095, 32767):
        got = O.rope(x, pos, O.inv_freq(hd, theta, n_rot))
        ref = bf.rope_complex(list(x), pos, theta, n_rot)
        np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9)


def test_rope_preserves_pair_norms_and_identity_at_zero():
    hd = 128
    inv = O.inv_freq(hd, 1e6, 16)
    x = rng.normal(size=(3, hd))
    y = O.rope(x, np.array([5, 99, 1234]), inv)
    h = hd // 2
    np.testing.assert_allclose(x[:, :h] ** 2 + x[:, h:] ** 2, y[:, :h] ** 2 + y[:, h:] ** 2, rtol=1e-12)
    assert np.array_equal(O.rope(x, 0, inv), x)


def test_rope_zero_frequency_tail_is_bit_exact_identity():
    hd, n_rot = 512, 64
    inv = O.inv_freq(hd, 1e6, n_rot)
    x = rng.normal(size=hd)
    y = O.rope(x, 31234, inv)
    h = hd // 2
    assert np.array_equal(y[n_rot:h], x[n_rot:h]) and np.array_equal(y[h + n_rot:], x[h + n_rot:])
    assert not np.allclose(y[:n_rot], x[:n_rot])


def test_rope_relative_position_and_composition():
    hd = 256
    inv = O.inv_freq(hd, 1e4, hd // 2)
    q, k = rng.normal(size=hd), rng.normal(size=hd)
    d1 = np.dot(O.rope(q, 40, inv), O.rope(k, 13, inv))
    d2 = np.dot(O.rope(q, 40 + 777, inv), O.rope(k, 13 + 777, inv))
    assert abs(d1 - d2) < 1e-9 * (1 + abs(d1))
    np.testing.assert_allclose(O.rope(O.rope(q, 11, inv), 30, inv), O.rope(q, 41, inv), rtol=1e-10, atol=1e-12)


def test_rotated_pairs_formula():
    g = json.load(open(os.path.join(GOLD, "constants.json")))
    for ex in g["rotated_pairs_examples"]:
        cfg = dict(head_dim_full=ex["full_head_dim"], partial_rotary=ex["partial_rotary_factor"], head_dim_swa=8)
        assert O.rotated_pairs(cfg, sliding=False) == ex["rotated_pairs"]
    assert O.rotated_pairs(dict(head_dim_swa=256), sliding=True) == 128
    inv = O.inv_freq(512, 1e6, 64)
    assert inv[0] == 1.0 and np.all(inv[64:] == 0) and np.all(inv[:64] > 0)


# ---------------------------------------------------------------- attention
def _rand_qkv(T, nh, nkv, hd, cap=None):
    cap = cap or T
    return rng.normal(size=(T, nh, hd)), rng.normal(size=(nkv, cap, hd)), rng.normal(size=(nkv, cap, hd))


@pytest.mark.parametrize("window", [None, 1, 3, 8])
def test_attention_brute_force(window):
    T, nh, nkv, hd = 7, 4, 2, 8
    q, K, V = _rand_qkv(T, nh, nkv, hd)
    pos = np.arange(T)
    got = O.attention(q, K, V, pos, window)
    for t in range(T):
        lo = 0 if window is None else max(0, t - window + 1)
        for h in range(nh):
            g = h // (nh // nkv)
            ref = bf.attend(list(q[t, h]), [list(K[g, j]) for j in range(lo, t + 1)],
                            [list(V[g, j]) for j in range(lo, t + 1)])
            np.testing.assert_allclose(got[t, h], ref, rtol=1e-12, atol=1e-12)


def test_attention_matches_torch_sdpa_with_mask_and_repeated_kv():
    T, nh, nkv, hd, W = 33, 8, 2, 16, 5
    q, K, V = _rand_qkv(T, nh, nkv, hd)
    for window in (None, W):
        got = O.attention(q, K, V, np.arange(T), window, chunk=8)
        i, j = np.arange(T)[:, None], np.arange(T)[None, :]
        mask = (j <= i) if window is None else ((j <= i) & (j > i - window))
        Kr = torch.from_numpy(K).repeat_interleave(nh // nkv, dim=0)
        Vr = torch.from_numpy(V).repeat_interleave(nh // nkv, dim=0)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q).transpose(0, 1), Kr, Vr,
                                             attn_mask=torch.from_numpy(mask), scale=1.0)
        np.testing.assert_allclose(got, ref.transpose(0, 1).numpy(), rtol=1e-11, atol=1e-12)


def test_bidirectional_attention_matches_torch_sdpa():
    """Page 4 `text_attention`: no causal mask; sliding keys within |i - j| <= W (a band of 2W + 1);
    the call's keys only (rows outside [k0, k1) of the cache hold junk that must not be seen)."""
    T, nh, nkv, hd, W = 29, 8, 2, 16, 4
    q, K, V = _rand_qkv(T, nh, nkv, hd)
    k0 = 3  # the sequence occupies cache rows 3 .. 3 + T - 1 of a longer cache
    Kc = np.concatenate([rng.normal(size=(nkv, 3, hd)) * 50, K, rng.normal(size=(nkv, 4, hd)) * 50], axis=1)
    Vc = np.concatenate([rng.normal(size=(nkv, 3, hd)) * 50, V, rng.normal(size=(nkv, 4, hd)) * 50], axis=1)
    for window in (None, W):
        got = O.attention_bidirectional(q, Kc, Vc, k0 + np.arange(T), k0, k0 + T, window, chunk=8)
        i, j = np.arange(T)[:, None], np.arange(T)[None, :]
        mask = np.ones((T, T), bool) if window is None else (np.abs(i - j) <= window)
        Kr = torch.from_numpy(K).repeat_interleave(nh // nkv, dim=0)
        Vr = torch.from_numpy(V).repeat_interleave(nh // nkv, dim=0)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q).transpose(0, 1), Kr, Vr,
                                             attn_mask=torch.from_numpy(mask), scale=1.0)
        np.testing.assert_allclose(got, ref.transpose(0, 1).numpy(), rtol=1e-11, atol=1e-12)
    # band edges: the first query sees keys 0..W, a middle one 2W + 1 keys; a window of T - 1 is full
    full = O.attention_bidirectional(q, K, V, np.arange(T), 0, T, None)
    np.testing.assert_allclose(O.attention_bidirectional(q, K, V, np.arange(T), 0, T, T - 1), full, rtol=1e-13)
    assert not np.allclose(O.attention_bidirectional(q, K, V, np.arange(T), 0, T, T - 2), full)
    # the last query of a full layer sees every key either way: causal and bidirectional rows agree
    causal = O.attention(q, K, V, np.arange(T), None)
    np.testing.assert_allclose(full[-1], causal[-1], rtol=1e-12)
    assert not np.allclose(full[0], causal[0])


def test_attention_special_cases():
    T, nh, nkv, hd = 9, 4, 1, 8
    q, K, V = _rand_qkv(T, nh, nkv, hd)
    # T = 1: the only key is itself
    np.testing.assert_allclose(O.attention(q[:1], K, V, [0]), np.broadcast_to(V[0, 0], (1, nh, hd)), rtol=1e-15)
    # q = 0: uniform weights, the mean of V over the visible keys
    z = O.attention(np.zeros_like(q), K, V, np.arange(T), 3)
    for t in range(T):
        lo = max(0, t - 2)
        np.testing.assert_allclose(z[t, 0], V[0, lo:t + 1].mean(axis=0), rtol=1e-13)
    # a window at least T equals full attention
    np.testing.assert_allclose(O.attention(q, K, V, np.arange(T), T), O.attention(q, K, V, np.arange(T)), rtol=1e-15)
    # V = 1 everywhere: softmax rows sum to one
    np.testing.assert_allclose(O.attention(q, K, np.ones_like(V), np.arange(T), 4), 1.0, rtol=1e-14)


def test_attention_gqa_heads_are_consecutive_groups():
    nh, nkv, hd = 8, 2, 4
    K = rng.normal(size=(nkv, 3, hd))
    V = np.stack([np.full((3, hd), 10.0 * g) for g in range(nkv)])
    o = O.attention(np.zeros((1, nh, hd)), K, V, [2])
    assert [o[0, h, 0] for h in range(nh)] == [10.0 * (h // 4) for h in range(nh)]


# ---------------------------------------------------------------- routing
def test_routing_page_fixture():
    fx = json.load(open(os.path.join(GOLD, "routing_fixture.json")))
    types = "".join("F" if (i + 1) % 5 == 0 else "S" for i in range(fx["n_layer"]))
    n_shared = fx["n_layer"] - fx["n_layer_kv_from_start"]
    short = O.kv_sources_shortcut(types, n_shared)
    for l, s in fx["page_asserts"]["kv_reuse_layer_shortcut"].items():
        assert short[int(l)] == s
    sem = O.kv_sources(types, n_shared)
    for l, s in fx["semantic_rule_expected"]["kv_source"].items():
        assert sem[int(l)] == s
    for l in range(6):
        assert sem[l] == l


def test_routing_configs_closed_form():
    c1, c3, c5 = configs.get(1), configs.get(3), configs.get(5)
    assert O.kv_sources(c1["layer_types"], c1["n_shared"]) == [0, 1, 1, 3]
    s3 = O.kv_sources(c3["layer_types"], c3["n_shared"])
    assert s3[:24] == list(range(24))
    assert all(s3[l] == (23 if c3["layer_types"][l] == "F" else 22) for l in range(24, 42))
    assert O.kv_sources(c5["layer_types"], c5["n_shared"]) == [0, 1, 2, 3, 4, 5, 6, 7, 7, 7, 7, 5]
    # the shortcut agrees only where the last two owners are [S, F]
    assert O.kv_sources_shortcut(c3["layer_types"], 18) == s3
    assert O.kv_sources_shortcut(c5["layer_types"], 4)[11] == 7  # would read a sliding cache


# ---------------------------------------------------------------- entry (embedding + PLE)
def _tiny_model(cfg, seed_shift=0):
    cfg = dict(cfg, id=cfg["id"] + seed_shift)
    glob = gen.model_globals(cfg)
    layers = [gen.layer_weights(cfg, l) for l in range(cfg["n_layers"])]
    return glob, layers


def test_ple_and_embedding_brute_force_and_special_cases():
    cfg = configs.tiny()
    glob, _ = _tiny_model(cfg)
    ids = np.array([[0, 5, 31, 33, 39, 45]])  # 33..39 are beyond ple_vocab; 45 beyond vocab
    e, ple = O.entry(cfg, glob, ids)
    for t, tok in enumerate(ids[0]):
        be, brows = bf.ple_row(cfg, int(tok), f64l(glob["embed"]), f64l(glob["ple_embed"]),
                               f64l(glob["ple_model_proj"]), f64l(glob["ple_norm"]))
        np.testing.assert_allclose(e[0, t], be, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ple[0, t], np.array(brows), rtol=1e-11, atol=1e-13)
    # id beyond vocab: zero embedding and zero table term -> the whole input is 0
    assert np.all(e[0, 5] == 0) and np.all(ple[0, 5] == 0)
    # W_pm = 0: the norm branch vanishes and ple_in = sqrt(d) row / sqrt(2)
    g0 = dict(glob, ple_model_proj=torch.zeros_like(glob["ple_model_proj"]))
    _, p0 = O.entry(cfg, g0, ids[:, :3])
    tab = O.f64(glob["ple_embed"])[ids[0, :3]].reshape(3, cfg["n_layers"], cfg["ple_dim"])
    np.testing.assert_allclose(p0[0], tab * math.sqrt(cfg["ple_dim"]) / math.sqrt(2), rtol=1e-14)


def f64l(t):
    return O.f64(t).tolist()


# ---------------------------------------------------------------- layer and stack
def _run_oracle_stack(cfg, layers, h0, ple, pos, srcs, cap):
    caches = O.new_caches(cfg, h0.shape[0], cap, srcs)
    return O.forward(cfg, layers, h0, ple, pos, caches, srcs), caches


VARIANT = dict(n_kv_heads_full=4, k_eq_v=True, ffn_dims=[48, 40, 56, 32, 24])


@pytest.mark.parametrize("types,n_shared,extra,bidir", [("SSF", 0, {}, False), ("SFSSF", 2, {}, False),
                                                        ("SFSSF", 2, VARIANT, False),
                                                        ("SFSFF", 0, dict(VARIANT, n_kv_heads_full=1), False),
                                                        ("SFSSF", 0, {}, True), ("SSFSF", 2, {"window": 2}, True)])
def test_stack_brute_force(types, n_shared, extra, bidir):
    cfg = configs.tiny(layer_types=types, n_shared=n_shared, T=6, **extra)
    glob, layers = _tiny_model(cfg)
    for lw in layers:
        lw["layer_scalar"] = 0.9
    ids = np.array([[1, 7, 3, 30, 2, 11]])
    h0, ple = O.entry(cfg, glob, ids)
    srcs = O.kv_sources(types, n_shared)
    pos = O.prefill_positions([0], cfg["T"])
    caches = O.new_caches(cfg, 1, cfg["T"], srcs)
    got = O.forward(cfg, layers, h0, ple, pos, caches, srcs, bidirectional=bidir)
    rows = h0[0].tolist()
    bcache = {}
    for l in range(cfg["n_layers"]):
        hd = cfg["head_dim_swa"] if types[l] == "S" else cfg["head_dim_full"]
        if srcs[l] == l:
            nkv = layers[l]["wk"].shape[0] // hd
            bcache[l] = {"k": [[None] * cfg["T"] for _ in range(nkv)],
                         "v": [[None] * cfg["T"] for _ in range(nkv)]}
        lw = {k: (f64l(v) if isinstance(v, torch.Tensor) else v) for k, v in layers[l].items()}
        rows = bf.layer(cfg, lw, l, srcs[l] == l, rows, ple[0, :, l, :].tolist(), list(range(cfg["T"])),
                        bcache[srcs[l]], bidirectional=bidir)
        assert len(rows[0]) == cfg["hidden"] and hd > 0
    np.testing.assert_allclose(got[0], np.array(rows), rtol=1e-10, atol=1e-11)


def test_k_eq_v_full_layer_is_base_layer_with_v_weight_from_k():
    """K=V (page 5 `forward_layer`): a full layer projects V with the K weight; sliding layers keep theirs."""
    base = configs.tiny(layer_types="SF")
    var = dict(base, k_eq_v=True)
    _, lb = _tiny_model(base)
    _, lv = _tiny_model(var)
    assert "wv" not in lv[1] and "wv" in lv[0]
    h = rng.normal(size=(1, 5, base["hidden"]))
    ple = rng.normal(size=(1, 5, base["ple_dim"]))
    pos = O.prefill_positions([0], 5)
    got = O.layer_forward(var, lv[1], 1, 1, h, ple, pos, O.new_caches(var, 1, 5))
    want = O.layer_forward(base, dict(lb[1], wv=lb[1]["wk"]), 1, 1, h, ple, pos, O.new_caches(base, 1, 5))
    assert np.array_equal(got, want)
    got = O.layer_forward(var, lv[0], 0, 0, h, ple, pos, O.new_caches(var, 1, 5))
    want = O.layer_forward(base, lb[0], 0, 0, h, ple, pos, O.new_caches(base, 1, 5))
    assert np.array_equal(got, want)
    # V is not the normed, rotated K: with the same projection, the cached V rows differ from K rows
    caches = O.new_caches(var, 1, 5)
    O.layer_forward(var, lv[1], 1, 1, h, ple, pos, caches)
    K, V = caches[1]
    raw = (O.rms_norm(h, lv[1]["input_norm"], var["eps"]) @ O.f64(lv[1]["wk"]).T).reshape(1, 5, 2, 16)
    np.testing.assert_allclose(V[0].transpose(1, 0, 2), raw[0] / np.sqrt((raw[0] ** 2).mean(-1, keepdims=True) + 1e-6),
                               rtol=1e-12)
    assert not np.allclose(K, V)


def test_full_layer_kv_heads_repeated_equal_fewer_heads():
    """A full layer with its own KV head count: 4 KV heads that repeat in pairs equal 2 KV heads (each of the
    4 query heads then reads its own copy, page 4 `text_attention` head map)."""
    base = configs.tiny(layer_types="SF")
    var = dict(base, n_kv_heads_full=4)
    _, lb = _tiny_model(base)
    hd = base["head_dim_full"]
    rep = lambda w: w.reshape(2, hd, -1).repeat_interleave(2, dim=0).reshape(4 * hd, -1)  # noqa: E731
    lv = dict(lb[1], wk=rep(lb[1]["wk"]), wv=rep(lb[1]["wv"]))
    h = rng.normal(size=(1, 5, base["hidden"]))
    ple = rng.normal(size=(1, 5, base["ple_dim"]))
    pos = O.prefill_positions([0], 5)
    cv = O.new_caches(var, 1, 5)
    got = O.layer_forward(var, lv, 1, 1, h, ple, pos, cv)
    want = O.layer_forward(base, lb[1], 1, 1, h, ple, pos, O.new_caches(base, 1, 5))
    assert cv[1][0].shape == (1, 4, 5, hd)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
    # sliding layers keep the shared count
    assert O.new_caches(var, 1, 5)[0][0].shape[1] == base["n_kv_heads"]


def test_ffn_width_zero_padding_is_invisible():
    """Per-layer FFN width (page 2 `ffn_dim`): extra units with zero gate/up rows and zero down columns add
    gelu(0) * 0 = 0, so a wider layer built that way equals the narrower one."""
    cfg = configs.tiny(layer_types="SF")
    _, layers = _tiny_model(cfg)
    lw = layers[0]
    F, H = lw["w_gate"].shape
    z = torch.zeros((16, H), dtype=lw["w_gate"].dtype)
    wide = dict(lw, w_gate=torch.cat([lw["w_gate"], z]), w_up=torch.cat([lw["w_up"], z]),
                w_down=torch.cat([lw["w_down"], z.T], dim=1))
    h = rng.normal(size=(1, 5, cfg["hidden"]))
    ple = rng.normal(size=(1, 5, cfg["ple_dim"]))
    pos = O.prefill_positions([0], 5)
    a = O.layer_forward(cfg, lw, 0, 0, h, ple, pos, O.new_caches(cfg, 1, 5))
    b = O.layer_forward(cfg, wide, 0, 0, h, ple, pos, O.new_caches(cfg, 1, 5))
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def test_layer_zero_branches_leave_h_scaled_exactly():
    cfg = configs.tiny()
    _, layers = _tiny_model(cfg)
    lw = dict(layers[0], wo=torch.zeros_like(layers[0]["wo"]), w_down=torch.zeros_like(layers[0]["w_down"]),
              ple_proj=torch.zeros_like(layers[0]["ple_proj"]), layer_scalar=0.75)
    h = rng.normal(size=(1, 5, cfg["hidden"]))
    caches = O.new_caches(cfg, 1, 5)
    out = O.layer_forward(cfg, lw, 0, 0, h, rng.normal(size=(1, 5, cfg["ple_dim"])), O.prefill_positions([0], 5), caches)
    assert np.array_equal(out, h * 0.75)


def test_layer_zero_ple_input_equals_no_ple_branch():
    cfg = configs.tiny()
    _, layers = _tiny_model(cfg)
    h = rng.normal(size=(1, 5, cfg["hidden"]))
    pos = O.prefill_positions([0], 5)
    a = O.layer_forward(cfg, layers[1], 1, 1, h, np.zeros((1, 5, cfg["ple_dim"])), pos, O.new_caches(cfg, 1, 5))
    lw = dict(layers[1], ple_proj=torch.zeros_like(layers[1]["ple_proj"]))
    b = O.layer_forward(cfg, lw, 1, 1, h, rng.normal(size=(1, 5, cfg["ple_dim"])), pos, O.new_caches(cfg, 1, 5))
    assert np.array_equal(a, b)


def test_prefill_equals_sequential_decode():
    cfg = configs.tiny(layer_types="SFSF", n_shared=2, T=7)
    glob, layers = _tiny_model(cfg)
    ids = np.array([[3, 1, 4, 1, 5, 9, 2], [6, 5, 3, 5, 8, 9, 7]])
    h0, ple = O.entry(cfg, glob, ids)
    srcs = O.kv_sources(cfg["layer_types"], 2)
    full, _ = _run_oracle_stack(cfg, layers, h0, ple, O.prefill_positions([0, 0], 7), srcs, 7)
    caches = O.new_caches(cfg, 2, 7, srcs)
    for t in range(7):
        step = O.forward(cfg, layers, h0[:, t:t + 1], ple[:, t:t + 1], np.array([[t], [t]]), caches, srcs)
        np.testing.assert_allclose(step[:, 0], full[:, t], rtol=1e-12, atol=1e-12)


def test_shared_layer_attends_over_source_cache():
    cfg = configs.tiny(layer_types="SFS", n_shared=1, T=6)
    _, layers = _tiny_model(cfg)
    srcs = O.kv_sources("SFS", 1)
    assert srcs == [0, 1, 0]
    h = rng.normal(size=(1, 6, cfg["hidden"]))
    pos = O.prefill_positions([0], 6)
    caches = O.new_caches(cfg, 1, 6, srcs)
    for l in range(2):
        h = O.layer_forward(cfg, layers[l], l, srcs[l], h, np.zeros((1, 6, cfg["ple_dim"])), pos, caches)
    tr = {}
    O.layer_forward(cfg, layers[2], 2, 0, h, np.zeros((1, 6, cfg["ple_dim"])), pos, caches, trace=tr)
    K, V = caches[0]
    direct = O.attention(tr["q"][0], K[0], V[0], pos[0], cfg["window"])
    assert np.array_equal(direct, tr["o"][0])


def test_batch_rows_are_independent():
    cfg = configs.tiny(T=5)
    glob, layers = _tiny_model(cfg)
    ids = np.array([[1, 2, 3, 4, 5], [9, 8, 7, 6, 5], [1, 2, 3, 4, 5]])
    h0, ple = O.entry(cfg, glob, ids)
    srcs = O.kv_sources(cfg["layer_types"], 0)
    out, _ = _run_oracle_stack(cfg, layers, h0, ple, O.prefill_positions([0, 0, 0], 5), srcs, 5)
    assert np.array_equal(out[0], out[2])
    one, _ = _run_oracle_stack(cfg, layers, h0[1:2], ple[1:2], O.prefill_positions([0], 5), srcs, 5)
    np.testing.assert_allclose(one[0], out[1], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("types,bidir", [("SSF", False), ("FSS", False), ("SSF", True), ("FSS", True)])
def test_layer_rows_equal_whole_layer_rows(types, bidir):
    cfg = configs.tiny(layer_types=types, T=13, window=4)
    _, layers = _tiny_model(cfg)
    h = rng.normal(size=(1, 13, cfg["hidden"]))
    ple = rng.normal(size=(1, 13, cfg["ple_dim"]))
    whole = O.layer_forward(cfg, layers[0], 0, 0, h, ple, O.prefill_positions([3], 13), O.new_caches(cfg, 1, 16),
                            bidirectional=bidir)
    rows, part = O.layer_forward_rows(cfg, layers[0], 0, h[0], ple[0], 3, [12, 0, 5, 9], bidirectional=bidir)
    np.testing.assert_allclose(part, whole[0, rows], rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- output head
def test_softcap_bounds_taylor_and_identity():
    """Pins of cap * tanh(x / cap): odd, strictly inside (-cap, cap), slope 1 at 0, third-order Taylor
    term -x^3 / (3 cap^2), saturation at +-cap, and no cap -> identity."""
    cap = json.load(open(os.path.join(GOLD, "constants.json")))["final_logit_softcap"]
    x = rng.normal(size=2000) * 50
    y = O.softcap(x, cap)
    assert np.all(np.abs(y) < cap) and np.allclose(O.softcap(-x, cap), -y, rtol=0, atol=0)
    small = np.array([1e-3, 0.05, 0.3])
    np.testing.assert_allclose(O.softcap(small, cap), small - small ** 3 / (3 * cap ** 2), rtol=0, atol=1e-8)
    assert abs(O.softcap(np.array([1e4]), cap)[0] - cap) < 1e-12
    np.testing.assert_array_equal(O.softcap(x, 0.0), x)


def test_logits_brute_force():
    """Final norm + output projection + softcap against pure-Python loops on tiny sizes."""
    M, H, V, cap = 3, 8, 11, 30.0
    h = rng.normal(size=(M, H)) * 3
    wn = 1 + 0.1 * rng.normal(size=H)
    W = rng.normal(size=(V, H)) * 2
    got = O.logits(h, wn, W, cap)
    for m in range(M):
        ms = sum(float(v) * float(v) for v in h[m]) / H
        inv = 1.0 / math.sqrt(ms + 1e-6)
        xn = [float(h[m][k]) * inv * float(wn[k]) for k in range(H)]
        for v in range(V):
            z = sum(xn[k] * float(W[v][k]) for k in range(H))
            assert abs(got[m, v] - cap * math.tanh(z / cap)) < 1e-12

