"""Sliding-window ring caches on the GPU: chunked prefill, then decode, against the float64 oracle.

A ring of R rows keeps position p of a sliding layer in row p mod R (R >= window), so a sliding layer's
cache is bounded by the window instead of the context. The layer's result must not depend on where its
keys live, so a schedule of prefill chunks followed by decode steps over rings must
  (a) equal the same schedule over linear caches bit for bit (only addresses differ), and
  (b) match the oracle's single full-length prefill of the whole sequence.
The ring sizes are not multiples of the attention key tile, so tiles straddle the wrap.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gemma_decoder_forward_amd import binding as bd
from synth import configs, gen
from tests.gpu_util import TOL_BF16_RELL2, build_model, host_layer, log, max_rel, rel_l2

pytestmark = pytest.mark.gpu


def _schedule(chunks, n_decode):
    """[(start, tokens, mode)]: prefill chunks back to back, then single-token decode steps."""
    s, out = 0, []
    for c in chunks:
        out.append((s, c, bd.G4_PREFILL))
        s += c
    for _ in range(n_decode):
        out.append((s, 1, bd.G4_DECODE))
        s += 1
    return out


def _pos(B, s):
    return torch.full((B,), s, dtype=torch.int32, device="cuda")


def _run_stack(model, h0, ple, sched, table, cap):
    """The whole stack over the schedule; returns the hidden states of every position, in order."""
    B = h0.shape[0]
    outs = []
    for s, n, mode in sched:
        h = h0[:, s:s + n].clone()
        model.forward(h, ple[:, s:s + n].contiguous(), _pos(B, s), table, cap, mode)
        outs.append(h)
    torch.cuda.synchronize()
    return torch.cat(outs, 1)


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).cuda()


def _ring_rows(T, R):
    """Position held by each ring row after positions 0..T-1 were written (the latest with p mod R == row)."""
    return [r + R * ((T - 1 - r) // R) for r in range(R)]


def test_ring_fp32_chunked_prefill_then_decode():
    cfg = configs.get(1, T=100, B=2)  # window 32; layer 2 shares layer 1's sliding cache
    R, T = 45, 100
    sched = _schedule([14, 14, 14, 14, 14, 10], 20)  # a chunk may hold R - window + 1 = 14 tokens
    assert sched[-1][0] + 1 == T
    model, layers, glob = build_model(cfg)
    acts = gen.activations(cfg, "cuda")
    h0, ple = model.embed(acts["ids"])
    ring_caches, ring_table = model.new_caches(2, T, ring=R)
    lin_caches, lin_table = model.new_caches(2, T)
    hr = _run_stack(model, h0, ple, sched, ring_table, T)
    hl = _run_stack(model, h0, ple, sched, lin_table, T)
    assert torch.equal(hr, hl), "ring and linear caches give different results"
    # the oracle: one prefill of all 100 tokens
    uniq, inv = np.unique(acts["ids"].cpu().numpy(), return_inverse=True)
    idx = torch.from_numpy(uniq).cuda()
    sub = dict(cfg, vocab=len(uniq), ple_vocab=len(uniq))
    g_host = dict(embed=glob["embed"][idx].cpu(), ple_embed=glob["ple_embed"][idx].cpu(),
                  ple_model_proj=glob["ple_model_proj"].cpu(), ple_norm=glob["ple_norm"].cpu())
    oh0, ople = O.entry(sub, g_host, inv.reshape(acts["ids"].shape))
    rc = O.new_caches(cfg, 2, T)
    ref = O.forward(cfg, host_layer(layers), oh0, ople, O.prefill_positions([0, 0], T), rc)
    e = max_rel(hr, ref)
    log(f"ring fp32 chunks+decode: max rel {e:.2e}")
    assert e <= 1e-3
    # every ring row holds the latest position that maps to it
    rows = _ring_rows(T, R)
    for l, (k, v) in ring_caches.items():
        if model.sliding[l]:
            assert k.shape[2] == R
            assert max_rel(k, rc[l][0][:, :, rows]) <= 1e-3, f"K ring {l}"
            assert max_rel(v, rc[l][1][:, :, rows]) <= 1e-3, f"V ring {l}"
        else:
            assert k.shape[2] == T


def test_ring_bf16_e4b_layer_pair_chunked_per_layer():
    """E4B layer pair (window 512) with a 1000-row sliding ring: chunks of 489 tokens (the most a call may
    hold), a 72-token chunk, a few-row 61-token chunk and 6 decode steps; each layer from the oracle's input
    for that layer, chunk-major, at the bf16 bound."""
    T, R = 1606, 1000
    cfg = configs.get(2, T=T)
    sched = _schedule([489, 489, 489, 72, 61], 6)
    assert sched[-1][0] + 1 == T
    model, layers, glob = build_model(cfg)
    acts = gen.activations(cfg, "cuda")
    # bit-equality of the GPU's own chained run, ring against linear
    ring_caches, ring_table = model.new_caches(1, T, ring=R)
    lin_caches, lin_table = model.new_caches(1, T)
    hr = _run_stack(model, acts["h0"], acts["ple_in"], sched, ring_table, T)
    hl = _run_stack(model, acts["h0"], acts["ple_in"], sched, lin_table, T)
    assert torch.isfinite(hr).all()
    assert torch.equal(hr, hl), "ring and linear caches give different results"
    log("oracle layer pair")
    h0, ple = O.f64(acts["h0"]), O.f64(acts["ple_in"])
    hs = [h0]
    O.forward(cfg, host_layer(layers), h0, ple, O.prefill_positions([0], T), O.new_caches(cfg, 1, T), per_layer=hs)
    log(f"end-to-end bf16 deviation: rel L2 {rel_l2(hr, hs[-1]):.3e}")
    caches, table = model.new_caches(1, T, ring=R)
    outs = [[] for _ in range(model.L)]
    for s, n, mode in sched:
        for l in range(model.L):
            x = _dev(hs[l][:, s:s + n])
            model.forward(x, _dev(ple[:, s:s + n]), _pos(1, s), table, T, mode, layer=l)
            outs[l].append(x)
    torch.cuda.synchronize()
    # the bound is on a tensor: each prefill chunk, and the decode steps' rows taken together (one row of
    # 2560 values alone scatters around the same mean with a wider spread)
    nd = sum(1 for _, _, m in sched if m == bd.G4_DECODE)
    for l in range(model.L):
        ref = hs[l + 1]
        errs = [rel_l2(x, ref[:, s:s + n]) for x, (s, n, m) in zip(outs[l], sched) if m == bd.G4_PREFILL]
        dec = rel_l2(torch.cat(outs[l][-nd:], 1), ref[:, T - nd:])
        log(f"layer {l}: prefill chunks rel L2 " + " ".join(f"{e:.1e}" for e in errs) + f"; decode rows {dec:.1e}")
        assert max(errs) <= TOL_BF16_RELL2 and dec <= TOL_BF16_RELL2, f"layer {l}"
