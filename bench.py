#!/usr/bin/env python3
"""Throughput of the Gemma-4 E-series decoder forward on one MI355X.

Default workload: the full E4B-like 42-layer stack (5 sliding + 1 full layer, repeated; the last 18
layers share KV), bf16 weights, prefill of T = 4096 tokens of batch 1 from token ids: the embedding and
per-layer inputs, then every layer. A step is one pass of that whole forward over the batch, inputs
resident in HBM. In the same process, on the same weights, `extra.decode` times one decode step at
context 8192 for batch 1 and 64 (the 42-layer model, caches filled to position 8190), `extra.logits`
the output head (final norm, projection onto the 262144-token vocabulary, softcap) on 1 and 64 rows,
and `extra.long` the 12-layer T = 32768 slice. Other workloads (--workload 2/4/5/6/7): the E4B layer
pair at T = 2048, decode alone (--batch B), the 12-layer slice alone, a 6-layer E4B-width model with
the variants (own full-layer KV heads, K=V, per-layer FFN widths) at T = 2048, and the 6-layer
E4B-width bidirectional encoder at T = 2048.

Prints one JSON line. The dominant kernel's launches are timed inside the timed region with HIP events
recorded by the library on its launch stream (g4_timer_*); `roofline` divides its algorithmic work per
launch by that average duration. `cpu_baseline` times the float64 oracle on a bounded sample of the same
workload on the host cores.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def workload(cid, batch):
    from synth import configs
    if cid == 4:
        return configs.get(4, B=batch)
    return configs.get(cid)


def layer_shape(cfg, l):
    """(head dim, kv heads, FFN width, has a V projection) of layer l."""
    from synth import gen
    return gen.head_dim(cfg, l), gen.kv_heads(cfg, l), gen.ffn_dim(cfg, l), gen.has_v_proj(cfg, l)


def gemm_flops(cfg, M):
    """Algorithmic GEMM flops of one layer-stack pass (2MNK), by kernel class."""
    H, nh, d = cfg["hidden"], cfg["n_heads"], cfg["ple_dim"]
    from gemma_decoder_forward_amd import binding as bd
    srcs = bd.g4_kv_sources([1 if t == "S" else 0 for t in cfg["layer_types"]], cfg["n_shared"])
    out = dict(qkv=0, o=0, gate_up=0, down=0, ple=0)
    for l in range(cfg["n_layers"]):
        hd, nkv, F, has_v = layer_shape(cfg, l)
        nq = nh * hd + ((2 if has_v else 1) * nkv * hd if srcs[l] == l else 0)
        out["qkv"] += 2 * M * nq * H
        out["o"] += 2 * M * H * nh * hd
        out["gate_up"] += 2 * M * 2 * F * H
        out["down"] += 2 * M * H * F
        out["ple"] += 2 * M * d * H * 2
    return out


def attn_flops(cfg, T):
    """4 * nh * hd * (visible query-key pairs) over all layers of a prefill from position 0 (the
    encoder: every pair on full layers, |i - j| <= W on sliding layers)."""
    tot = 0
    W = cfg["window"]
    enc = cfg["mode"] == "encode"
    for t in cfg["layer_types"]:
        hd = cfg["head_dim_swa"] if t == "S" else cfg["head_dim_full"]
        if enc:
            pairs = T * T if t == "F" else sum(min(i + W, T - 1) - max(i - W, 0) + 1 for i in range(T))
        else:
            pairs = T * (T + 1) // 2 if t == "F" else sum(min(i + 1, W) for i in range(T))
        tot += 4 * cfg["n_heads"] * hd * pairs * cfg["B"]
    return tot


def class_rates(cfg, M, decode, per_ms):
    """Achieved rate of each timed kernel class from its per-step time, against its own bound.

    Prefill GEMMs and attention: algorithmic TFLOP/s against bf16 dense MFMA. Decode GEMMs: weight bytes
    streamed, attention: K and V bytes read (shared layers re-read their source), both against HBM.
    Row tails and head norms (elementwise, HBM): bytes each step needs at the layer's dtypes, with the
    float32 projection outputs counted once (split-K slices are an implementation choice, not counted).
    """
    H, nh = cfg["hidden"], cfg["n_heads"]
    E = 2 if cfg["dtype"] == "bf16" else 4
    from gemma_decoder_forward_amd import binding as bd
    srcs = bd.g4_kv_sources([1 if t == "S" else 0 for t in cfg["layer_types"]], cfg["n_shared"])
    L = cfg["n_layers"]
    out = {}
    gf = gemm_flops(cfg, M)
    keyname = dict(qkv="qkv_gemm", o="o_gemm", gate_up="gate_up_gemm", down="down_gemm", ple="ple_gemm")
    for k, f in gf.items():
        ms = per_ms.get(keyname[k], 0)
        if ms <= 0:
            continue
        if decode:
            gb = f / (2 * M) * E / (ms / 1e3) / 1e9  # weight bytes = flops / (2M) elements
            out[keyname[k]] = dict(GB_s=round(gb, 1), frac_hbm=round(gb / PEAK_HBM_GBS, 3))
        else:
            tf = f / (ms / 1e3) / 1e12
            out[keyname[k]] = dict(TFLOP_s=round(tf, 1), frac_mfma=round(tf / PEAK_BF16_TFLOPS, 3))
    ms = per_ms.get("attention", 0)
    if ms > 0:
        if decode:
            kv = 0
            for l, t in enumerate(cfg["layer_types"]):
                hd, nkv, _, _ = layer_shape(cfg, l)
                keys = min(cfg["ctx"], cfg["window"]) if t == "S" else cfg["ctx"]
                kv += 2 * nkv * keys * hd * E * M
            gb = kv / (ms / 1e3) / 1e9
            out["attention"] = dict(GB_s=round(gb, 1), frac_hbm=round(gb / PEAK_HBM_GBS, 3))
        else:
            tf = attn_flops(cfg, cfg["T"]) / (ms / 1e3) / 1e12
            out["attention"] = dict(TFLOP_s=round(tf, 1), frac_mfma=round(tf / PEAK_BF16_TFLOPS, 3))
    # per token per layer: three residual tails (read f32 projection + h, write h + one dtype row) and the
    # pre-attention norm of the first layer; head norms read and write q (and k, v when the layer owns them)
    tail = L * 3 * (4 * H + 4 * H + 4 * H + E * H) + (4 * H + E * H)
    qk = 0
    for l in range(L):
        hd, nkv, _, _ = layer_shape(cfg, l)
        # reads q (and k, v: a K=V layer reads its k columns twice) and writes q, k, v rows
        qk += 2 * (nh + (2 * nkv if srcs[l] == l else 0)) * hd * E
    for name, per_tok in (("row_tail", tail), ("qk_norm_rope", qk)):
        ms = per_ms.get(name, 0)
        if ms > 0:
            gb = per_tok * M / (ms / 1e3) / 1e9
            out[name] = dict(GB_s=round(gb, 1), frac_hbm=round(gb / PEAK_HBM_GBS, 3))
    return out


def mean_ffn(cfg):
    """FFN width averaged over the layers (the gate/up kernel runs once per layer)."""
    return sum(layer_shape(cfg, l)[2] for l in range(cfg["n_layers"])) / cfg["n_layers"]


def gate_up_weight_bytes(cfg):
    return 2 * mean_ffn(cfg) * cfg["hidden"] * 2


def decode_step_bytes(cfg):
    """Algorithmic HBM bytes of one decode step of B sequences: every weight the step reads once (the layer
    projections and norms by routing, the PLE model projection), the embedding and PLE table rows of the B
    tokens, each attention layer's K and V over its visible keys (shared layers count their re-read of the
    source cache), and the new K/V rows the owning layers write."""
    E = 2 if cfg["dtype"] == "bf16" else 4
    H, nh, d, L, B = cfg["hidden"], cfg["n_heads"], cfg["ple_dim"], cfg["n_layers"], cfg["B"]
    from gemma_decoder_forward_amd import binding as bd
    srcs = bd.g4_kv_sources([1 if t == "S" else 0 for t in cfg["layer_types"]], cfg["n_shared"])
    w = 0
    kv = 0
    for l, t in enumerate(cfg["layer_types"]):
        hd, nkv, F, has_v = layer_shape(cfg, l)
        own = srcs[l] == l
        w += (nh * hd * H + (nkv * hd * H * (2 if has_v else 1) if own else 0) + H * nh * hd + 3 * F * H
              + 2 * d * H) * E
        w += (5 * H + hd * (2 if own else 1)) * E  # norm weights
        keys = min(cfg["ctx"], cfg["window"]) if t == "S" else cfg["ctx"]
        kv += B * 2 * nkv * keys * hd * E
        if own:
            kv += B * 2 * nkv * hd * E
    w += (L * d * H + d) * E  # PLE model projection and its norm
    gathers = B * (H + L * d) * E
    return dict(weights=w, kv=kv, gathers=gathers, total=w + kv + gathers)


def build_weights(cfg):
    """Device weights of a workload (layers, and the embedding/PLE tables for configs built from ids)."""
    from synth import gen
    layers = [gen.layer_weights(cfg, l, "cuda") for l in range(cfg["n_layers"])]
    glob = gen.model_globals(cfg, "cuda") if cfg["embed"] else None
    return layers, glob


def run_gpu(cfg, layers, glob, steps, warmup, breakdown, use_graph=True):
    import torch
    from gemma_decoder_forward_amd import binding as bd
    from gemma_decoder_forward_amd.model import G4Model
    from synth import gen

    torch.cuda.set_device(0)
    B, T = cfg["B"], cfg["T"]
    model = G4Model(cfg, layers, glob)
    acts = gen.activations(cfg, "cuda")
    decode = cfg["mode"] == "decode"
    if decode:
        cap = cfg["ctx"]
        fills = {l: gen.decode_cache(cfg, l, "cuda") for l in range(cfg["n_layers"]) if model.kv_src[l] == l}
        _, table = model.new_caches(B, cap, fill=lambda l: fills[l])
        mode = bd.G4_DECODE
    else:
        cap = T
        _, table = model.new_caches(B, cap)
        mode = bd.G4_ENCODE if cfg["mode"] == "encode" else bd.G4_PREFILL
    H = cfg["hidden"]
    h = torch.empty((B, T, H), dtype=torch.float32, device="cuda")
    if cfg["embed"]:
        ple = torch.empty((B, T, cfg["n_layers"], cfg["ple_dim"]), dtype=torch.float32, device="cuda")
    else:
        ple = acts["ple_in"]
    model.workspace(B, T, cap, mode)

    def step():
        if cfg["embed"]:
            model.embed(acts["ids"], h, ple)  # the entry writes h0 and the per-layer inputs in place
        else:
            h.copy_(acts["h0"])
        model.forward(h, ple, acts["pos"], table, cap, mode)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    dom = "gate_up_gemm"
    run = step
    if decode and use_graph:
        # A decode step is hundreds of short kernels: it is captured once as a HIP graph and replayed.
        # The gate/up launch time comes from capture()'s warm-up step, whose launches are eager (on a side
        # stream, an event pair around each of its first min(2*steps, layers) gate/up launches),
        # so it includes each launch's dispatch gap; the replayed graph records no events.
        from gemma_decoder_forward_amd.model import capture
        # at most one step's gate/up launches, so that the warm-up step fills the timer and no event is
        # recorded into the graph
        bd.g4_timer_enable(bd.KC[dom], min(2 * steps, cfg["n_layers"]))
        graph = capture(step)
        run = graph.replay
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
    else:
        # Only the first 2*steps gate/up launches of the timed region are timed (all launches of the
        # class have one shape): each event pair adds a dispatch gap, about 0.24 ms per 42-layer
        # T=4096 step with a pair around every launch (37.13 against 36.89 ms).
        bd.g4_timer_enable(bd.KC[dom], 2 * steps)
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms, dom_n = bd.g4_timer_read()
    res = dict(ms_per_step=wall * 1e3 / steps, dom_ms=dom_ms, dom_n=dom_n, graph=run is not step)
    if breakdown:
        per = {}
        for name, cls in bd.KC.items():
            bd.g4_timer_enable(cls, 4 * cfg["n_layers"] * 3 + 8)
            for _ in range(2):
                step()
            torch.cuda.synchronize()
            ms, n = bd.g4_timer_read()
            per[name] = round(ms / 2, 4)
        res["breakdown_ms_per_step"] = per
    assert torch.isfinite(h).all().item(), "non-finite output"
    del model, table, h, acts
    if decode:
        del fills
    torch.cuda.empty_cache()
    return res


def run_logits(cfg, glob, rows, steps, warmup):
    """The output head on `rows` rows of the model's width: final RMS norm, the projection onto the vocabulary
    (the embedding table, [vocab, hidden] bf16, serves as its weights: same shape) and the softcap of 30.
    Times `steps` calls between two events on the library's stream; returns the summary with the HBM rate of
    its algorithmic bytes (weights once, the rows in, the float32 logits out)."""
    import torch
    from gemma_decoder_forward_amd import binding as bd
    from synth import gen
    H, V = cfg["hidden"], cfg["vocab"]
    s = 7000 + rows
    h = gen.normal((rows, H), 1.0, 0.0, s, "head_rows", "cuda", torch.float32)
    wn = gen.normal((H,), 0.1, 1.0, s, "final_norm", "cuda", torch.bfloat16)
    w = glob["embed"]
    out = torch.empty((rows, V), dtype=torch.float32, device="cuda")
    wsb = bd.g4_logits_ws(rows, H, V, bd.G4_BF16)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream()

    def call():
        bd.g4_logits(h.data_ptr(), rows, H, wn.data_ptr(), w.data_ptr(), V, cfg["eps"], 30.0, out.data_ptr(),
                     ws.data_ptr(), wsb, bd.G4_BF16, st.cuda_stream)

    for _ in range(warmup):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        call()
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    assert torch.isfinite(out).all().item() and float(out.abs().max()) <= 30.0, "output head: bad logits"
    nbytes = 2 * V * H + 2 * H + 4 * rows * H + 4 * rows * V
    gbs = nbytes / (ms / 1e3) / 1e9
    del h, out, ws
    return dict(workload=f"e4b output head (final norm, vocabulary projection, softcap 30): rows={rows} vocab={V}",
                rows_per_s=round(rows / (ms / 1e3), 2), ms_per_call=round(ms, 4), bytes_per_call=nbytes,
                GB_s=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4))


WORKLOAD_NAMES = {2:"e4b-layer-pair prefill", 3: "e4b-42-layer prefill from token ids", 4: "e4b-42-layer decode",
                  5: "e4b-12-layer long-context prefill",
                  6: "e4b-width 6-layer prefill with the variants (full-layer kv heads, K=V, per-layer FFN widths)",
                  7: "e4b-width 6-layer bidirectional encoder"}


def workload_name(cfg):
    decode = cfg["mode"] == "decode"
    return f"{WORKLOAD_NAMES[cfg['id']]}: B={cfg['B']} T={cfg['T']}" + (f" ctx={cfg['ctx']}" if decode else "")


def summarize(cfg, r):
    """Throughput, the dominant kernel's roofline and (decode) the step's HBM fraction of one GPU run."""
    B, T = cfg["B"], cfg["T"]
    tokens = B * T
    ms = r["ms_per_step"]
    decode = cfg["mode"] == "decode"
    dom_avg_s = r["dom_ms"] / max(r["dom_n"], 1) / 1e3
    out = dict(workload=workload_name(cfg), tokens_per_s=round(tokens / (ms / 1e3), 2), ms_per_step=round(ms, 4),
               hip_graph=r["graph"])
    if decode:
        per_launch = gate_up_weight_bytes(cfg) + 2 * B * cfg["hidden"] + 2 * B * mean_ffn(cfg)
        achieved = per_launch / dom_avg_s / 1e9
        out["roofline"] = dict(bound="hbm", kernel="gate_up_gemm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS,
                               unit="GB/s", frac=round(achieved / PEAK_HBM_GBS, 4), bytes_per_launch=per_launch,
                               avg_launch_us=round(dom_avg_s * 1e6, 2))
        sb = decode_step_bytes(cfg)
        gbs = sb["total"] / (ms / 1e3) / 1e9
        out["step_bytes"] = sb
        out["step_GB_s"] = round(gbs, 1)
        out["frac_hbm"] = round(gbs / PEAK_HBM_GBS, 4)
    else:
        per_launch = 2 * tokens * 2 * mean_ffn(cfg) * cfg["hidden"]
        achieved = per_launch / dom_avg_s / 1e12
        out["roofline"] = dict(bound="mfma", kernel="gate_up_gemm", achieved=round(achieved, 2),
                               peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", frac=round(achieved / PEAK_BF16_TFLOPS, 4),
                               flops_per_launch=per_launch, avg_launch_us=round(dom_avg_s * 1e6, 2))
        gf = gemm_flops(cfg, tokens)
        af = attn_flops(cfg, T)
        out["gemm_tflop_per_step"] = round(sum(gf.values()) / 1e12, 4)
        out["attn_tflop_per_step"] = round(af / 1e12, 4)
        out["model_tflops"] = round((sum(gf.values()) + af) / (ms / 1e3) / 1e12, 2)
        out["frac_mfma"] = round(out["model_tflops"] / PEAK_BF16_TFLOPS, 4)
    if "breakdown_ms_per_step" in r:
        out["breakdown_ms_per_step"] = r["breakdown_ms_per_step"]
        out["class_rates"] = class_rates(cfg, tokens, decode, r["breakdown_ms_per_step"])
    return out


def host_cores():
    """Threads the oracle's BLAS may use: the CPUs this process may run on, capped by the cgroup CPU quota
    when one is set (a container's share can be smaller than its affinity mask)."""
    aff = len(os.sched_getaffinity(0))
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, per = f.read().split()[:2]
        if q != "max":
            quota = max(1, -(-int(q) // int(per)))
    except (OSError, ValueError):
        pass
    return (min(aff, quota) if quota else aff), aff, quota


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, layers_dev, glob_dev, budget_s):
    """The float64 oracle, as it stands, on a bounded sample of the workload (host cores, BLAS threads
    pinned to the cores this process may use). Only the oracle's forward is timed; each layer's weights
    are copied to the host and widened to float64 before its timed call, one layer at a time."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle as O
    from synth import gen

    cores, aff, quota = host_cores()
    L = cfg["n_layers"]
    acts = gen.activations(cfg, "cuda")
    srcs = O.kv_sources(cfg["layer_types"], cfg["n_shared"])

    def host_layer(l):
        return {k: (O.f64(v) if isinstance(v, torch.Tensor) else v) for k, v in layers_dev[l].items()}

    def run(Tp, nseq):
        """Seconds of oracle compute for a prefill of Tp tokens (or one decode step of nseq sequences)."""
        if cfg["mode"] == "decode":
            sub = dict(cfg, B=nseq)
            ids = acts["ids"][:nseq].cpu().numpy()
            caches = {}
            for l in range(L):
                if srcs[l] == l:
                    k, v = gen.decode_cache(sub, l, "cuda")
                    caches[l] = (O.f64(k), O.f64(v))
            pos = np.full((nseq, 1), cfg["ctx"] - 1)
        else:
            sub = dict(cfg, T=Tp)
            ids = acts["ids"][:, :Tp].cpu().numpy() if cfg["embed"] else None
            caches = O.new_caches(cfg, 1, Tp, srcs)
            pos = O.prefill_positions([0], Tp)
        t = 0.0
        if cfg["embed"]:
            uniq, inv = np.unique(ids, return_inverse=True)
            idx = torch.from_numpy(uniq).cuda()
            gh = dict(embed=glob_dev["embed"][idx].cpu(), ple_embed=glob_dev["ple_embed"][idx].cpu(),
                      ple_model_proj=O.f64(glob_dev["ple_model_proj"]), ple_norm=glob_dev["ple_norm"].cpu())
            sub2 = dict(sub, vocab=len(uniq), ple_vocab=len(uniq))
            t0 = time.perf_counter()
            h, ple = O.entry(sub2, gh, inv.reshape(ids.shape))
            t += time.perf_counter() - t0
        else:
            h = O.f64(acts["h0"][:, :Tp])
            ple = O.f64(acts["ple_in"][:, :Tp])
        for l in range(L):
            lw = host_layer(l)
            t0 = time.perf_counter()
            h = O.forward(sub, {l: lw}, h, ple, pos, caches, srcs, layer_range=[l],
                          bidirectional=cfg["mode"] == "encode")
            t += time.perf_counter() - t0
        return t

    with threadpool_limits(limits=cores, user_api="blas"):
        if cfg["mode"] == "decode":
            n = 1
            t = run(0, n)
            tokens, sample = n, f"decode step of {n} sequence at context {cfg['ctx']} through all {L} layers"
        else:
            Tp = 64
            t = run(Tp, 1)
            target = int(Tp * budget_s / max(t, 1e-3)) // 64 * 64
            target = min(cfg["T"], target)
            if target > Tp:
                Tp = target
                t = run(Tp, 1)
            reps = 1
            # a sample shorter than the budget (the whole workload fits) is repeated until about 2/3 of it
            # is spent, so that the rate is not one short run's
            while t < budget_s * 2 / 3:
                t += run(Tp, 1)
                reps += 1
            tokens = Tp * reps
            sample = (f"prefill of the first {Tp} of {cfg['T']} tokens (batch 1) through all {L} layers"
                      + (" from token ids (embedding and per-layer inputs included)" if cfg["embed"] else "")
                      + (f", {reps} runs" if reps > 1 else ""))
    return dict(value=round(tokens / t, 3), unit="tokens/s", cores=cores, kind="oracle", sample=sample,
                seconds=round(t, 2), cpu_model=cpu_model(), affinity_cpus=aff, cgroup_cpu_quota=quota,
                blas_threads=cores)


def counted_traffic(workload_name, kernel_class):
    """HBM bytes per launch of the roofline kernel from the committed rocprofv3 counter summary.

    The figure is used only while the kernel's sources still hash to what was profiled; otherwise None.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            entries = json.load(f)["entries"]
    except (OSError, ValueError, KeyError):
        return None
    for e in entries:
        if e["workload"] != workload_name or e["kernel_class"] != kernel_class:
            continue
        h = hashlib.sha256()
        try:
            for src in e["sources"]:
                with open(os.path.join(ROOT, src), "rb") as f:
                    h.update(f.read())
        except OSError:
            return None
        return e["traffic_bytes_per_launch"] if h.hexdigest() == e["source_sha256"] else None
    return None


def copy_calibration(mib):
    """A plain streaming kernel of known traffic (read N floats, write N floats), to scale HBM counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps(dict(copy_calibration=True, read_bytes=4 * n, write_bytes=4 * n, launches=3)), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, choices=[2, 3, 4, 5, 6, 7])
    ap.add_argument("--batch", type=int, default=64, help="decode batch (workload 4)")
    ap.add_argument("--no-extra", action="store_true",
                    help="workload 3: skip the decode (B=1, 64), output head and T=32768 lines of `extra`")
    ap.add_argument("--only-logits", action="store_true",
                    help="only the output head lines of `extra` (1 and 64 rows on the E4B vocabulary), as one JSON line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-graph", action="store_true", help="decode: launch every kernel eagerly (no HIP graph)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (scale for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): the library "
              "implements the single-GPU forward; sharding across GPUs is described, not implemented.", file=sys.stderr)
        sys.exit(2)
    from synth import configs
    if args.only_logits:
        from synth import gen
        c3 = configs.get(3)
        print("[bench] output head: building the embedding table", file=sys.stderr, flush=True)
        g3 = gen.model_globals(c3, "cuda")
        lines = {f"rows{rows}": run_logits(c3, g3, rows, args.steps, args.warmup) for rows in (1, 64)}
        print(json.dumps(dict(logits=lines, steps=args.steps, warmup=args.warmup)), flush=True)
        return
    cfg = workload(args.workload, args.batch)
    breakdown = not args.no_breakdown
    print(f"[bench] {workload_name(cfg)}: building weights", file=sys.stderr, flush=True)
    layers, glob = build_weights(cfg)
    r = run_gpu(cfg, layers, glob, args.steps, args.warmup, breakdown, not args.no_graph)
    main_sum = summarize(cfg, r)
    print(f"[bench] {main_sum['workload']}: {main_sum['tokens_per_s']} tokens/s", file=sys.stderr, flush=True)
    decode = cfg["mode"] == "decode"
    wname = main_sum["workload"]
    roof = dict(main_sum["roofline"], traffic=counted_traffic(wname, "gate_up_gemm"))
    extra = {k: v for k, v in main_sum.items() if k not in ("workload", "tokens_per_s", "ms_per_step", "roofline")}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, layers, glob, args.cpu_seconds)
        print(f"[bench] oracle on the host: {cpu['value']} tokens/s", file=sys.stderr, flush=True)
    if args.workload == 3 and not args.no_extra:
        # decode on the same model (config 4's weights are config 3's), then the long-context slice
        extra["decode"] = {}
        for B in (1, 64):
            c4 = configs.get(4, B=B)
            r4 = run_gpu(c4, layers, glob, args.steps, args.warmup, breakdown, not args.no_graph)
            extra["decode"][f"B{B}"] = summarize(c4, r4)
            print(f"[bench] {extra['decode'][f'B{B}']['workload']}: {extra['decode'][f'B{B}']['tokens_per_s']} "
                  "tokens/s", file=sys.stderr, flush=True)
        # the output head after the stack: one row per sequence (decode batches 1 and 64)
        extra["logits"] = {}
        for rows in (1, 64):
            extra["logits"][f"rows{rows}"] = lg = run_logits(cfg, glob, rows, args.steps, args.warmup)
            print(f"[bench] {lg['workload']}: {lg['ms_per_call']} ms per call, {lg['GB_s']} GB/s", file=sys.stderr,
                  flush=True)
        del layers, glob
        import torch
        torch.cuda.empty_cache()
        c5 = configs.get(5)
        l5, _ = build_weights(c5)
        r5 = run_gpu(c5, l5, None, args.steps, args.warmup, breakdown)
        extra["long"] = summarize(c5, r5)
        print(f"[bench] {extra['long']['workload']}: {extra['long']['tokens_per_s']} tokens/s", file=sys.stderr,
              flush=True)
        del l5
    B, T = cfg["B"], cfg["T"]
    line = dict(
        metric="decode tokens/s" if decode else ("encoder tokens/s" if cfg["mode"] == "encode" else "prefill tokens/s"),
        value=main_sum["tokens_per_s"], unit="tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=main_sum["ms_per_step"], higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
        data="synthetic (seeded N(0,0.02) weights, N(0,1) activations / uniform token ids)",
        config=dict(workload=wname,
                    layers=cfg["n_layers"], layer_types=cfg["layer_types"], hidden=cfg["hidden"],
                    ffn=cfg.get("ffn_dims") or cfg["ffn"],
                    heads=f"{cfg['n_heads']}/{cfg['n_kv_heads']}"
                    + (f" (full layers /{cfg['n_kv_heads_full']})" if cfg.get("n_kv_heads_full") else ""),
                    k_eq_v=bool(cfg.get("k_eq_v")),
                    head_dim=f"{cfg['head_dim_swa']}/{cfg['head_dim_full']}", window=cfg["window"],
                    global_batch=B, seq_len=T, parallelism="none (1 GPU)"),
        roofline=roof, extra=extra,
    )
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
