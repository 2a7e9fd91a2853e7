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


def _seq_view(table, b, caches, L):
    """A kv table over sequence b's slabs only (its [nkv, rows, hd] block of every cache), for B = 1 calls."""
    t = (bd.KvEntry * L)()
    for l, (k, v) in caches.items():
        e = table[l]
        off = b * k.shape[1] * k.shape[2] * k.shape[3] * k.element_size()
        t[l] = bd.KvEntry(k=e.k + off, v=e.v + off, cap=e.cap, hd=e.hd, sliding=e.sliding, ring=e.ring)
    return t


def _per_sequence_schedule(model, h0, ple, prompts, n_decode, caches, table, cap, chunk):
    """Each sequence's prompt prefilled alone (B = 1 over its own cache slabs, chunks of at most `chunk`),
    then n_decode joint steps in which sequence b sits at position prompts[b] + i. Returns each sequence's
    hidden states of the decode steps [B, n_decode, H]."""
    B = len(prompts)
    for b, P in enumerate(prompts):
        view = _seq_view(table, b, caches, model.L)
        for s in range(0, P, chunk):
            n = min(chunk, P - s)
            h = h0[b:b + 1, s:s + n].clone()
            model.forward(h, ple[b:b + 1, s:s + n].contiguous(), _pos(1, s), view, cap, bd.G4_PREFILL)
    outs = []
    for i in range(n_decode):
        pos = torch.tensor([P + i for P in prompts], dtype=torch.int32, device="cuda")
        h = torch.stack([h0[b, P + i] for b, P in enumerate(prompts)])[:, None].contiguous()
        p = torch.stack([ple[b, P + i] for b, P in enumerate(prompts)])[:, None].contiguous()
        model.forward(h, p, pos, table, cap, bd.G4_DECODE)
        outs.append(h)
    torch.cuda.synchronize()
    return torch.cat(outs, 1)


def test_ring_fp32_per_sequence_positions():
    """Three sequences with prompts of 20, 50 and 33 tokens over 45-row sliding rings (window 32), then 25
    joint decode steps: every step's batch holds three different positions, and the sequences wrap their
    rings at different steps. The result equals the same schedule over linear caches bit for bit, and
    each sequence's decode rows match the oracle's one-shot prefill of that sequence within 1e-3."""
    prompts, n_dec, R = [20, 50, 33], 25, 45
    Tmax = max(prompts) + n_dec
    cfg = configs.get(1, T=Tmax, B=3)
    model, layers, glob = build_model(cfg)
    acts = gen.activations(cfg, "cuda")
    h0, ple = model.embed(acts["ids"])
    ring_caches, ring_table = model.new_caches(3, Tmax, ring=R)
    lin_caches, lin_table = model.new_caches(3, Tmax)
    hr = _per_sequence_schedule(model, h0, ple, prompts, n_dec, ring_caches, ring_table, Tmax, R - 32 + 1)
    hl = _per_sequence_schedule(model, h0, ple, prompts, n_dec, lin_caches, lin_table, Tmax, R - 32 + 1)
    assert torch.equal(hr, hl), "ring and linear caches give different results"
    worst = 0.0
    for b, P in enumerate(prompts):
        n = P + n_dec
        ids = acts["ids"][b:b + 1, :n].cpu().numpy()
        uniq, inv = np.unique(ids, return_inverse=True)
        idx = torch.from_numpy(uniq).cuda()
        sub = dict(cfg, B=1, T=n, vocab=len(uniq), ple_vocab=len(uniq))
        g_host = dict(embed=glob["embed"][idx].cpu(), ple_embed=glob["ple_embed"][idx].cpu(),
                      ple_model_proj=glob["ple_model_proj"].cpu(), ple_norm=glob["ple_norm"].cpu())
        oh0, ople = O.entry(sub, g_host, inv.reshape(ids.shape))
        ref = O.forward(sub, host_layer(layers), oh0, ople, O.prefill_positions([0], n), O.new_caches(sub, 1, n))
        e = max_rel(hr[b], ref[0, P:])
        worst = max(worst, e)
        assert e <= 1e-3, f"sequence {b}: max rel {e:.2e}"
    log(f"ring fp32, per-sequence positions {prompts} + {n_dec} decode steps: max rel {worst:.2e}")


def test_ring_bf16_e4b_per_sequence_positions_bit_equal_to_linear():
    """The E4B layer pair (window 512) over 700-row sliding rings: prompts of 100, 530 and 777 tokens
    (chunks of at most 189), then 6 joint decode steps at three different positions, bit-identical to the
    same schedule over linear caches (the ring changes only where rows live)."""
    prompts, n_dec, R = [100, 530, 777], 6, 700
    Tmax = max(prompts) + n_dec
    cfg = configs.get(2, T=Tmax, B=3)
    model, layers, glob = build_model(cfg)
    acts = gen.activations(cfg, "cuda")
    ring_caches, ring_table = model.new_caches(3, Tmax, ring=R)
    lin_caches, lin_table = model.new_caches(3, Tmax)
    args = (acts["h0"], acts["ple_in"], prompts, n_dec)
    hr = _per_sequence_schedule(model, *args, ring_caches, ring_table, Tmax, R - 512 + 1)
    hl = _per_sequence_schedule(model, *args, lin_caches, lin_table, Tmax, R - 512 + 1)
    assert torch.isfinite(hr).all()
    assert torch.equal(hr, hl), "ring and linear caches give different results"
    log(f"ring bf16 E4B pair, per-sequence positions {prompts} + {n_dec} decode steps: bit-equal to linear")
