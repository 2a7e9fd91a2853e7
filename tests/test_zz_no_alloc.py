"""g4_stack_forward_noalloc (static device scratch, no workspace argument) against g4_stack_forward.

Both entry points run the same kernels over the same plan, so their outputs (hidden state and every K/V
cache row written) must agree bit for bit. The workspace-taking reference gets a workspace filled with
NaN bit patterns, so a kernel that read scratch it had not written in the same call would show up as a
difference. Each case makes two no-alloc calls in a row, the second with a smaller input, so the second
runs over the first call's leftovers in the shared static buffer.
"""
import pytest
import torch

from gemma_decoder_forward_amd import binding as bd
from synth import configs, gen
from tests.gpu_util import build_model, log, randn, stream

pytestmark = pytest.mark.gpu


def _caches(model, B, cap, seed):
    """Random bf16/f32 caches (rows the calls do not write stay as drawn) and a copy of them."""
    def fill(l):
        shape = (B, model.kv_heads(l), cap, model.head_dim(l))
        return randn(shape, seed + 2 * l, model.torch_dtype), randn(shape, seed + 2 * l + 1, model.torch_dtype)
    return model.new_caches(B, cap, fill=fill)


def _run_pair(model, h0, ple, pos, B, T, cap, mode, seed):
    """(h, caches) from g4_stack_forward (NaN-filled workspace) and from g4_stack_forward_noalloc."""
    out = []
    for noalloc in (False, True):
        caches, table = _caches(model, B, cap, seed)
        h = h0.clone()
        if noalloc:
            bd.g4_stack_forward_noalloc(model.desc, model.descs, h.data_ptr(), ple.data_ptr(), table, model.L,
                                        pos.data_ptr(), B, T, mode, stream())
        else:
            need = bd.g4_workspace_size(model.desc, B, T, cap, mode)
            assert 0 < need <= bd.NOALLOC_SCRATCH_BYTES
            ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
            bd.g4_stack_forward(model.desc, model.descs, h.data_ptr(), ple.data_ptr(), table, model.L,
                                pos.data_ptr(), B, T, mode, ws.data_ptr(), need, stream())
        torch.cuda.synchronize()
        out.append((h, caches))
    return out


def _assert_same(a, b, what):
    (ha, ca), (hb, cb) = a, b
    assert torch.isfinite(ha).all(), what
    assert torch.equal(ha, hb), f"{what}: hidden state differs (max |d| {float((ha - hb).abs().max()):.3e})"
    assert sorted(ca) == sorted(cb)
    for l in ca:
        assert torch.equal(ca[l][0], cb[l][0]) and torch.equal(ca[l][1], cb[l][1]), f"{what}: cache {l} differs"


@pytest.mark.parametrize("cid", [1, 2])
def test_noalloc_prefill_matches_workspace_entry(cid):
    cfg = configs.get(cid)
    model, _, _ = build_model(cfg, with_glob=False)
    H, L, d = cfg["hidden"], model.L, cfg["ple_dim"]
    for call, (B, T) in enumerate(((2, 300), (1, 40))):  # the second call is smaller (and few-row for bf16)
        h0 = randn((B, T, H), 700 + call)
        ple = randn((B, T, L, d), 710 + call)
        pos = torch.tensor([0, 37][:B], dtype=torch.int32, device="cuda")
        cap = T + 40
        ref, got = _run_pair(model, h0, ple, pos, B, T, cap, bd.G4_PREFILL, 720 + 10 * call)
        _assert_same(ref, got, f"{cfg['name']} prefill B={B} T={T}")
        log(f"noalloc {cfg['name']} prefill B={B} T={T}: bit-identical to g4_stack_forward")


def test_noalloc_decode_matches_workspace_entry():
    """The E4B layer pair in decode over 1024-row caches: batch 6, then batch 2 at other positions."""
    cfg = configs.get(2)
    model, _, _ = build_model(cfg, with_glob=False)
    H, L, d = cfg["hidden"], model.L, cfg["ple_dim"]
    cap = 1024
    for call, (B, positions) in enumerate(((6, [0, 5, 511, 512, 900, 1023]), (2, [700, 3]))):
        h0 = randn((B, 1, H), 800 + call)
        ple = randn((B, 1, L, d), 810 + call)
        pos = torch.tensor(positions, dtype=torch.int32, device="cuda")
        ref, got = _run_pair(model, h0, ple, pos, B, 1, cap, bd.G4_DECODE, 820 + 10 * call)
        _assert_same(ref, got, f"decode B={B}")
        log(f"noalloc decode B={B}: bit-identical to g4_stack_forward")


def test_noalloc_refuses_a_call_beyond_its_scratch():
    """A prefill whose plan exceeds the static buffer is refused with G4_ERANGE and nothing is launched:
    h is left as it was."""
    cfg = configs.get(2)
    model, _, _ = build_model(cfg, with_glob=False)
    B, T = 1, 4096
    assert bd.g4_workspace_size(model.desc, B, T, T, bd.G4_PREFILL) > bd.NOALLOC_SCRATCH_BYTES
    h = randn((B, T, cfg["hidden"]), 900)
    h_before = h.clone()
    ple = randn((B, T, model.L, cfg["ple_dim"]), 901)
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    caches, table = model.new_caches(B, T)
    with pytest.raises(bd.G4Error) as e:
        bd.g4_stack_forward_noalloc(model.desc, model.descs, h.data_ptr(), ple.data_ptr(), table, model.L,
                                    pos.data_ptr(), B, T, bd.G4_PREFILL, stream())
    assert e.value.status == bd.G4_ERANGE
    torch.cuda.synchronize()
    assert torch.equal(h, h_before)
