"""How far a bf16 implementation must land from the float64 oracle: the bf16 error floor (CPU only).

`tests/bf16_floor.py` replays the oracle's layer with the bf16 path's stored intermediates rounded to bf16
(weights are bf16 inputs in every workload). These tests pin that replay to the oracle and record what it
shows:

  * with no rounding it is the oracle (to float64 rounding), and its rounding is nearest-even bf16;
  * one layer's floor is about 1e-2 relative L2 on the first layer of a random-weight stack (where
    h0 ~ N(0, 1) dominates the branches) and a few 1e-3 on later layers;
  * end to end the stack is chaotic: the same roundings grow to a large fraction of the signal over 12
    layers, while float32 roundings at the same points stay near 1e-4, so no bf16 implementation can meet
    a 2e-2 end-to-end bound on these stacks. The GPU parity tests therefore bound each layer, run from
    the oracle's input, by a small multiple of this floor.

The opt-in full run (G4_FLOORS=1) prints the per-layer floors of the benchmark workloads at the sizes the
GPU parity tests use.
"""
import os

import numpy as np
import pytest
import torch

import oracle as O
from synth import configs, gen
from tests import bf16_floor as F


def _prefill_case(cid, T, **kw):
    cfg = configs.get(cid, T=T, **kw)
    layers = [gen.layer_weights(cfg, l, "cpu") for l in range(cfg["n_layers"])]
    acts = gen.activations(cfg, "cpu")
    h0, ple = O.f64(acts["h0"]), O.f64(acts["ple_in"])
    pos = O.prefill_positions([0], T)
    hs = [h0]
    O.forward(cfg, layers, h0, ple, pos, O.new_caches(cfg, 1, T), per_layer=hs)
    return cfg, layers, h0, ple, pos, hs


def test_rounding_is_nearest_even_bf16():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        [0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 65504.0, -3.0 - 2 ** -7]])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.to_bf16(x), want)
    assert F.to_bf16(np.array([1.0 + 2 ** -8]))[0] == 1.0            # a tie goes to the even neighbour
    assert F.to_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6


@pytest.mark.parametrize("cid,T", [(2, 96), (5, 40)])
def test_replay_without_rounding_is_the_oracle(cid, T):
    """Every layer, shared ones included, replayed with no rounding point equals the oracle's layer."""
    cfg, layers, h0, ple, pos, hs = _prefill_case(cid, T)
    errs = F.layer_floors(cfg, layers, hs, ple, pos, O.new_caches(cfg, 1, T), "none")
    assert max(errs) < 1e-13, errs


def test_replay_follows_the_decode_positions():
    """Decode (one token per sequence at its own position over filled caches), no rounding: the oracle."""
    cfg = configs.get(2, T=1, B=3, mode="prefill")
    layers = [gen.layer_weights(cfg, l, "cpu") for l in range(cfg["n_layers"])]
    rng = np.random.default_rng(5)
    caches = O.new_caches(cfg, 3, 700)
    for k, v in caches.values():
        k[...] = rng.standard_normal(k.shape)
        v[...] = rng.standard_normal(v.shape)
    pos = np.array([[0], [512], [699]])
    h0 = rng.standard_normal((3, 1, cfg["hidden"]))
    ple = rng.standard_normal((3, 1, 2, cfg["ple_dim"]))
    c1 = {l: (k.copy(), v.copy()) for l, (k, v) in caches.items()}
    hs = [h0]
    O.forward(cfg, layers, h0, ple, pos, c1, per_layer=hs)
    errs = F.layer_floors(cfg, layers, hs, ple, pos, caches, "none")
    assert max(errs) < 1e-13


def test_bf16_floor_per_layer_and_the_chaotic_stack():
    """The 12-layer E4B slice (config 5's pattern and widths) at T = 128: per-layer bf16 floors are
    1e-3 .. 2e-2, while end to end the bf16 roundings grow past 2e-2 by an order of magnitude (only the KV
    cache rounded: still past it) and float32 roundings at the same points stay small."""
    T = 128
    cfg, layers, h0, ple, pos, hs = _prefill_case(5, T)
    fl = F.layer_floors(cfg, layers, hs, ple, pos, O.new_caches(cfg, 1, T), "bf16_prefill")
    print("per-layer bf16 floors: " + " ".join(f"{e:.1e}" for e in fl))
    assert 5e-3 < fl[0] < 2e-2 and all(1e-3 < e < 2e-2 for e in fl)
    e2e = {}
    for name, mode, f32 in (("bf16", "bf16_prefill", False), ("kv only", "kv_only", False), ("f32", "bf16_prefill", True)):
        e2e[name] = F.rel_l2(F.stack_rounded(cfg, layers, h0, ple, pos, O.new_caches(cfg, 1, T), mode, f32), hs[-1])
    print("end to end after 12 layers: " + ", ".join(f"{k} {v:.3e}" for k, v in e2e.items()))
    assert e2e["bf16"] > 0.2 and e2e["kv only"] > 0.1 and e2e["f32"] < 1e-3


@pytest.mark.skipif(os.environ.get("G4_FLOORS") != "1", reason="opt-in (G4_FLOORS=1): minutes of float64 work")
@pytest.mark.parametrize("case", ["2:T2048", "5:T1100", "3:T520", "4:B1", "4:B64"])
def test_print_floors_of_the_workloads(case):
    """Per-layer floors of the benchmark workloads at the GPU parity tests' sizes (host-generated weights:
    the GPU tests compute their own floors on their own weights)."""
    cid, size = case.split(":")
    cid = int(cid)
    if cid in (2, 5):
        T = int(size[1:])
        cfg, layers, h0, ple, pos, hs = _prefill_case(cid, T)
        fl = F.layer_floors(cfg, layers, hs, ple, pos, O.new_caches(cfg, 1, T), "bf16_prefill")
    elif cid == 3:
        T = int(size[1:])
        cfg = configs.get(3, T=T)
        glob = gen.model_globals(cfg, "cpu")
        layers = lambda l: gen.layer_weights(cfg, l, "cpu")  # noqa: E731
        ids = gen.activations(cfg, "cpu")["ids"].numpy()
        h0, ple = O.entry(cfg, glob, ids)
        pos = O.prefill_positions([0], T)
        hs = [h0]
        O.forward(cfg, layers, h0, ple, pos, O.new_caches(cfg, 1, T), per_layer=hs)
        fl = F.layer_floors(cfg, layers, hs, ple, pos, O.new_caches(cfg, 1, T), "bf16_prefill")
    else:
        B = int(size[1:])
        cfg = configs.get(4, B=B)
        sample = sorted({0, B - 1})
        sub = dict(cfg, B=len(sample))
        glob = gen.model_globals(cfg, "cpu")
        layers = lambda l: gen.layer_weights(cfg, l, "cpu")  # noqa: E731
        ids = gen.activations(cfg, "cpu")["ids"].numpy()[sample]
        h0, ple = O.entry(sub, glob, ids)
        srcs = O.kv_sources(cfg["layer_types"], cfg["n_shared"])
        caches = {}
        for l in range(cfg["n_layers"]):
            if srcs[l] == l:
                k, v = gen.decode_cache(cfg, l, "cpu")
                caches[l] = (O.f64(k[sample]), O.f64(v[sample]))
        pos = np.full((len(sample), 1), cfg["ctx"] - 1)
        c0 = {l: (k.copy(), v.copy()) for l, (k, v) in caches.items()}
        hs = [h0]
        O.forward(sub, layers, h0, ple, pos, caches, per_layer=hs)
        fl = F.layer_floors(sub, layers, hs, ple, pos, c0, "bf16_decode")
    print(f"config {case}: per-layer bf16 floors " + " ".join(f"{e:.1e}" for e in fl))
    assert all(e < 2e-2 for e in fl)
