"""Helpers shared by the GPU parity tests: device inputs, tolerance checks, model construction."""
import numpy as np
import torch

import oracle as O
from gemma_decoder_forward_amd import binding as bd
from gemma_decoder_forward_amd.model import G4Model
from synth import gen

DT = {"f32": (bd.G4_F32, torch.float32), "bf16": (bd.G4_BF16, torch.bfloat16)}

# Tolerances from the workload statement: float32 kernels, max relative error 1e-3 (max |g - o| over
# max |o|); the bf16 path, relative L2 2e-2 over its output.
TOL_F32_MAXREL = 1e-3
TOL_BF16_RELL2 = 2e-2


def stream():
    return torch.cuda.current_stream().cuda_stream


def g(seed):
    return torch.Generator(device="cuda").manual_seed(seed)


def randn(shape, seed, dtype=torch.float32, std=1.0, mean=0.0):
    x = torch.randn(shape, generator=g(seed), device="cuda", dtype=torch.float32) * std + mean
    return x.to(dtype)


def rel_l2(gpu, ref):
    gpu, ref = O.f64(gpu), O.f64(ref)
    return float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300))


def max_rel(gpu, ref):
    gpu, ref = O.f64(gpu), O.f64(ref)
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-300))


def assert_close(gpu, ref, path, what=""):
    """path 'f32': max relative error <= 1e-3; 'bf16': relative L2 <= 2e-2."""
    if path == "f32":
        e = max_rel(gpu, ref)
        assert e <= TOL_F32_MAXREL, f"{what}: max rel err {e:.3e} > {TOL_F32_MAXREL}"
    else:
        e = rel_l2(gpu, ref)
        assert e <= TOL_BF16_RELL2, f"{what}: rel L2 err {e:.3e} > {TOL_BF16_RELL2}"
    return e


def build_model(cfg, device="cuda", with_glob=None):
    layers = [gen.layer_weights(cfg, l, device) for l in range(cfg["n_layers"])]
    glob = gen.model_globals(cfg, device) if (cfg["embed"] if with_glob is None else with_glob) else None
    return G4Model(cfg, layers, glob), layers, glob


def host_layer(layers):
    """Lazy host copies of device layer weights, for the oracle."""
    def get(l):
        return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in layers[l].items()}
    return get


def log(msg):
    print(msg, flush=True)


def assert_layers_within_floor(errs, floors, what=""):
    """Each layer's relative L2 from the oracle within max(1.5 x its bf16 floor, 5e-3), and within the
    2e-2 outer bar. The floor (tests/bf16_floor.py) is what storing the bf16 path's intermediates in bf16
    costs by itself on the same inputs; a kernel adding error of its own would exceed it."""
    assert len(errs) == len(floors)
    log(f"{what} per-layer rel L2 / floor: " + " ".join(f"{e:.1e}/{f:.1e}" for e, f in zip(errs, floors)))
    for l, (e, f) in enumerate(zip(errs, floors)):
        bound = min(TOL_BF16_RELL2, max(1.5 * f, 5e-3))
        assert e <= bound, f"{what} layer {l}: rel L2 {e:.3e} > {bound:.3e} (floor {f:.3e})"
