"""C-ABI boundary on the host (no GPU): the library loads, exports every declared symbol, routes
shared-KV layers exactly like the oracle, and rejects bad arguments before launching anything."""
import ctypes as C
import os
import random
import re

import pytest

import oracle as O
from gemma_decoder_forward_amd import binding as bd
from synth import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "g4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(g4_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_bound():
    L = bd.lib()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), f"{n} declared in g4.h but not exported"
    assert set(names) == set(bd.exported_names())


def test_version_and_status_strings():
    assert bd.lib().g4_version() >= 300
    assert bd.lib().g4_status_str(bd.G4_EGEOM) == b"G4_EGEOM"


@pytest.mark.parametrize("cid", [1, 3, 5])
def test_routing_matches_oracle_on_configs(cid):
    c = configs.get(cid)
    sliding = [1 if t == "S" else 0 for t in c["layer_types"]]
    assert bd.g4_kv_sources(sliding, c["n_shared"]) == O.kv_sources(c["layer_types"], c["n_shared"])


def test_routing_matches_oracle_on_random_patterns():
    rnd = random.Random(3)
    for _ in range(300):
        L = rnd.randint(1, 24)
        types = "".join(rnd.choice("SF") for _ in range(L))
        ns = rnd.randint(0, L)
        assert bd.g4_kv_sources([1 if t == "S" else 0 for t in types], ns) == O.kv_sources(types, ns)


def _model(**kw):
    c = dict(configs.get(2), **kw)
    return bd.ModelDesc(hidden=c["hidden"], n_heads=c["n_heads"], n_kv_heads=c["n_kv_heads"],
                        head_dim_swa=c["head_dim_swa"], head_dim_full=c["head_dim_full"], ffn=c["ffn"],
                        ple_dim=c["ple_dim"], n_layers=2, window=c["window"], vocab=c["vocab"],
                        ple_vocab=c["ple_vocab"], eps=c["eps"], theta_swa=c["theta_swa"],
                        theta_full=c["theta_full"], partial_rotary=c["partial_rotary"], dtype=bd.G4_BF16)


FAKE = 0x1000  # never dereferenced: every call below fails validation on the host


def _table(entries):
    t = (bd.KvEntry * len(entries))()
    for i, e in enumerate(entries):
        if e is not None:
            t[i] = bd.KvEntry(k=FAKE, v=FAKE, cap=e[0], hd=e[1], sliding=e[2], ring=e[3] if len(e) > 3 else 0)
    return t


def _attn(table, layer, kv_src, sliding, hd, T=8, window=512, nh=8, nkv=2, q=FAKE, ws=None, ws_bytes=0):
    return bd.lib().g4_attn_prefill(q, nh * hd, table, len(table), layer, kv_src, sliding, window, FAKE, 1, T, nh,
                                    nkv, hd, 1.0, FAKE, nh * hd, ws, ws_bytes, bd.G4_BF16, None)


def test_attention_validation_errors():
    t = _table([(64, 256, 1), (64, 512, 0), None])
    assert _attn(t, 2, 3, 1, 256) == bd.G4_EGEOM      # kv_src after the layer
    assert _attn(t, 2, 2, 1, 256) == bd.G4_EGEOM      # source is a hole (shared layer)
    assert _attn(t, 2, 1, 1, 512) == bd.G4_EGEOM      # sliding layer reading a full cache
    assert _attn(t, 2, 0, 1, 512) == bd.G4_EGEOM      # head-dim mismatch
    assert _attn(t, 2, 0, 1, 256, T=65) == bd.G4_ERANGE  # T beyond capacity
    assert _attn(t, 2, 0, 1, 256, window=0) == bd.G4_ERANGE
    assert _attn(t, 2, 0, 1, 256, nh=6, nkv=4) == bd.G4_EGEOM
    assert _attn(t, 2, 0, 1, 256, q=None) == bd.G4_EINVAL
    assert _attn(t, 7, 0, 1, 256) == bd.G4_EINVAL     # layer outside the table
    need = bd.g4_attn_prefill_ws(1, 8, 8, 2, 256)
    assert need > 0                                   # a short prefill splits its keys when given scratch
    assert _attn(t, 2, 0, 1, 256, ws=FAKE, ws_bytes=need - 1) == bd.G4_EINVAL  # scratch too small
    assert b"workspace" in bd.lib().g4_last_error()
    assert _attn(t, 2, 0, 1, 256, ws=FAKE + 8, ws_bytes=need) == bd.G4_EINVAL  # misaligned scratch
    assert b"head_dim" in bd.lib().g4_last_error() or bd.lib().g4_last_error()


def test_encode_validation_errors():
    """The encoder's attention takes the prefill checks, and a ring cache is refused (its call's keys could
    have been overwritten); the layer forward accepts G4_ENCODE and refuses unknown modes."""
    t = _table([(640, 256, 1, 1), (64, 256, 1)])
    L = bd.lib()

    def enc(table, layer, kv_src, T=8, window=512):
        return L.g4_attn_encode(FAKE, 8 * 256, table, len(table), layer, kv_src, 1, window, FAKE, 1, T, 8, 2, 256, 1.0,
                                FAKE, 8 * 256, None, 0, bd.G4_BF16, None)

    assert enc(t, 0, 0) == bd.G4_EINVAL and b"linear" in L.g4_last_error()
    assert enc(t, 1, 1, T=65) == bd.G4_ERANGE
    assert enc(t, 1, 1, window=0) == bd.G4_ERANGE
    m = _model()
    ld = bd.LayerDesc(sliding=1, kv_src=0, layer_scalar=1.0)
    for n in bd.LAYER_PTRS:
        setattr(ld, n, FAKE)
    lt = _table([(64, 256, 1), (64, 512, 0)])
    for mode, want in ((3, bd.G4_EINVAL), (bd.G4_ENCODE, bd.G4_EINVAL)):
        # mode 3 is unknown; G4_ENCODE passes validation and stops at the (too small) workspace
        assert L.g4_layer_forward(C.byref(m), C.byref(ld), 0, FAKE, FAKE, lt, 2, FAKE, 1, 8, mode, FAKE, 1,
                                  None) == want
    assert b"workspace" in L.g4_last_error()


def test_ring_cache_validation_errors():
    """A ring cache: sliding layers only, at least a window of rows, and at most rows - window + 1 tokens a call."""
    t = _table([(640, 256, 1, 1), (640, 512, 0, 1), (512, 256, 1, 1), (640, 256, 1, 2)])
    L = bd.lib()
    # every case fails on the host before any launch
    assert _attn(t, 1, 1, 0, 512, T=8) == bd.G4_EGEOM      # full-attention cache marked as a ring
    assert _attn(t, 2, 2, 1, 256, T=8, window=600) == bd.G4_ERANGE  # ring shorter than the window
    assert _attn(t, 0, 0, 1, 256, T=130) == bd.G4_ERANGE   # 130 > 640 - 512 + 1
    assert _attn(t, 3, 3, 1, 256, T=8) == bd.G4_EINVAL     # ring flag neither 0 nor 1
    assert b"ring" in L.g4_last_error()


def test_layer_validation_errors():
    m = _model()
    ld = bd.LayerDesc(sliding=1, kv_src=0, layer_scalar=1.0)
    for n in bd.LAYER_PTRS:
        setattr(ld, n, FAKE)
    t = _table([(64, 256, 1), (64, 512, 0)])
    L = bd.lib()

    def call(layer=0, T=8, B=1, mode=bd.G4_PREFILL, ws_bytes=1 << 40, model=m, desc=ld, table=t):
        return L.g4_layer_forward(C.byref(model), C.byref(desc), layer, FAKE, FAKE, table, len(table), FAKE, B, T,
                                  mode, FAKE, ws_bytes, None)

    assert call(ws_bytes=10) == bd.G4_EINVAL          # workspace too small
    assert call(T=2, mode=bd.G4_DECODE) == bd.G4_EINVAL
    assert call(T=100) == bd.G4_ERANGE
    bad = bd.LayerDesc.from_buffer_copy(ld)
    bad.wk = None
    assert call(desc=bad) == bd.G4_EINVAL             # owning layer without wk
    bad2 = bd.LayerDesc.from_buffer_copy(ld)
    bad2.kv_src = 1
    assert call(desc=bad2) == bd.G4_EGEOM             # later layer as source
    m2 = _model(n_kv_heads=3)
    assert call(model=m2) == bd.G4_EGEOM
    m3 = _model()
    m3.dtype = 7
    assert call(model=m3) == bd.G4_EINVAL
    assert bd.g4_workspace_size(m, 1, 2048, 2048, bd.G4_PREFILL) > 0
    assert bd.g4_workspace_size(m3, 1, 2048, 2048, bd.G4_PREFILL) == 0


def test_variant_validation_errors():
    """Per-type KV heads, per-layer FFN widths and K=V are checked on the host before any launch."""
    ld = bd.LayerDesc(sliding=0, kv_src=1, layer_scalar=1.0)
    for n in bd.LAYER_PTRS:
        setattr(ld, n, FAKE)
    t = _table([(64, 256, 1), (64, 512, 0)])
    L = bd.lib()

    def call(model, desc, ws_bytes=1 << 40):
        return L.g4_layer_forward(C.byref(model), C.byref(desc), 1, FAKE, FAKE, t, len(t), FAKE, 1, 8,
                                  bd.G4_PREFILL, FAKE, ws_bytes, None)

    m = _model()
    m.n_kv_heads_full = 3
    assert call(m, ld) == bd.G4_EGEOM                 # 8 query heads do not split into 3 kv groups
    assert b"n_kv_heads_full" in L.g4_last_error()
    m = _model()
    m.k_eq_v = 2
    assert call(m, ld) == bd.G4_EINVAL
    no_v = bd.LayerDesc.from_buffer_copy(ld)
    no_v.wv = None
    assert call(_model(), no_v) == bd.G4_EINVAL       # a full layer needs wv unless the model is K=V
    wide = bd.LayerDesc.from_buffer_copy(ld)
    wide.ffn = _model().ffn + 64
    assert call(_model(), wide) == bd.G4_ERANGE       # wider than the model's (workspace) width
    wide.ffn = -1
    assert call(_model(), wide) == bd.G4_ERANGE
    # K=V model: the full layer may omit wv; the descriptor passes every check up to the (too small)
    # workspace, so nothing is launched
    m = _model()
    m.k_eq_v = 1
    m.n_kv_heads_full = 1
    assert call(m, no_v, ws_bytes=1) == bd.G4_EINVAL
    assert b"workspace" in L.g4_last_error()
    # workspace grows with the larger of the two kv head counts
    a = bd.g4_workspace_size(_model(), 1, 256, 256, bd.G4_PREFILL)
    m = _model()
    m.n_kv_heads_full = 8
    assert bd.g4_workspace_size(m, 1, 256, 256, bd.G4_PREFILL) > a


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes structs agree with the C compiler's layout of include/g4.h (size and every offset)."""
    structs = {"g4_model_desc": bd.ModelDesc, "g4_layer_desc": bd.LayerDesc, "g4_kv_entry": bd.KvEntry}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "g4.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for ln in out:
        if ln:
            a, b, c = ln.split()
            got[(a, b)] = int(c)
    for cname, py in structs.items():
        assert got[(cname, "size")] == C.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_row_op_validation_errors():
    L = bd.lib()
    assert L.g4_rmsnorm(None, 0, 1, None, FAKE, None, 1.0, None, None, 4, 16, 1e-6, 0, None) == bd.G4_EINVAL
    assert L.g4_rmsnorm(FAKE, 0, 1, None, FAKE, None, 1.0, None, FAKE, 4, 16, 1e-6, 0, None) == bd.G4_EINVAL
    assert L.g4_rmsnorm(FAKE, 0, 1, None, FAKE, None, 1.0, None, None, 4, 20000, 1e-6, 0, None) == bd.G4_ERANGE
    assert L.g4_qk_norm_rope(FAKE, 256, None, FAKE, 256, 0, FAKE, 1, 4, 1, 257, 1e4, 0, 1e-6, 0, None) == bd.G4_EGEOM
    assert L.g4_qk_norm_rope(FAKE, 256, None, FAKE, 256, 0, FAKE, 1, 4, 1, 256, 1e4, 129, 1e-6, 0, None) == bd.G4_ERANGE
    assert L.g4_qk_norm_rope(FAKE, 256, None, FAKE, 256, 0, None, 1, 4, 1, 256, 1e4, 64, 1e-6, 0, None) == bd.G4_EINVAL
    assert L.g4_qk_norm_rope(FAKE, 256, None, FAKE, 0, 3, FAKE, 1, 4, 1, 256, 1e4, 64, 1e-6, 0, None) == bd.G4_ERANGE
    assert L.g4_linear(FAKE, FAKE, FAKE, 4, 0, 8, 0, 0, None, 0, None) == bd.G4_EINVAL
    assert L.g4_linear(FAKE, FAKE, FAKE, 4, 8, 8, 1, 0, None, 0, None) == bd.G4_EINVAL
    assert L.g4_ffn_geglu(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 8, FAKE, 1, 1, None) == bd.G4_EINVAL
    assert L.g4_kv_sources(None, 3, 1, None) == bd.G4_EINVAL


def test_logits_validation_errors():
    L = bd.lib()
    ws = bd.g4_logits_ws(4, 64, 128, bd.G4_BF16)
    assert ws > 0 and bd.g4_logits_ws(0, 64, 128, bd.G4_BF16) == 0
    assert L.g4_logits(None, 0, 64, None, None, 128, 1e-6, 30.0, None, None, 0, 1, None) == bd.G4_OK  # empty
    assert L.g4_logits(FAKE, 4, 64, FAKE, FAKE, 128, 1e-6, -1.0, FAKE, FAKE, ws, 1, None) == bd.G4_EINVAL
    assert L.g4_logits(FAKE, 4, 64, FAKE, FAKE, 128, 1e-6, 30.0, FAKE, FAKE, ws - 1, 1, None) == bd.G4_EINVAL
    assert L.g4_logits(FAKE, 4, 64, None, FAKE, 128, 1e-6, 30.0, FAKE, FAKE, ws, 1, None) == bd.G4_EINVAL
    assert L.g4_logits(FAKE, 4, 64, FAKE, FAKE, 0, 1e-6, 30.0, FAKE, FAKE, ws, 1, None) == bd.G4_EINVAL
    assert L.g4_logits(FAKE, 4, 64, FAKE, FAKE, 128, 1e-6, 30.0, FAKE, FAKE, ws, 5, None) == bd.G4_EINVAL


def _stack_descs(pattern, n_shared):
    """Layer descriptors of a stack with fake weight pointers and the library's own routing."""
    srcs = bd.g4_kv_sources([1 if t == "S" else 0 for t in pattern], n_shared)
    descs = (bd.LayerDesc * len(pattern))()
    for l, t in enumerate(pattern):
        descs[l].sliding = 1 if t == "S" else 0
        descs[l].kv_src = srcs[l]
        descs[l].layer_scalar = 1.0
        for n in bd.LAYER_PTRS:
            setattr(descs[l], n, FAKE)
    return descs, srcs


def test_stack_workspace_checked_once_for_the_largest_cache():
    """Mixed ring (sliding) and linear (full) caches: a workspace sized for the ring's capacity is too small
    for the full layers' decode partials. The stack call must refuse it before the first layer launches
    (the message names the workspace), and accept the size planned for the largest capacity."""
    pattern = "SSSSSF"
    m = _model(n_layers=len(pattern))
    m.n_layers = len(pattern)
    descs, srcs = _stack_descs(pattern, 0)
    t = _table([(1024, 256, 1, 1) if c == "S" else (8192, 512, 0, 0) for c in pattern])
    L = bd.lib()
    B = 4
    small = bd.g4_workspace_size(m, B, 1, 1024, bd.G4_DECODE)
    big = bd.g4_workspace_size(m, B, 1, 8192, bd.G4_DECODE)
    assert 0 < small < big

    def stack(ws_bytes, model=m):
        return L.g4_stack_forward(C.byref(model), descs, FAKE, FAKE, t, len(t), FAKE, B, 1, bd.G4_DECODE, FAKE,
                                  ws_bytes, None)

    assert stack(small) == bd.G4_EINVAL and b"workspace" in L.g4_last_error()
    assert stack(big - 1) == bd.G4_EINVAL
    assert L.g4_stack_forward(C.byref(m), descs, FAKE, FAKE, t, len(t), FAKE, B, 1, bd.G4_DECODE, FAKE + 16, big,
                              None) == bd.G4_EINVAL
    assert b"aligned" in L.g4_last_error()


def test_stack_unsupported_decode_group_refused_before_launch():
    """Decode attention groups at most 8 query heads per kv head: 16 query heads over one kv head is
    refused by the layer checks (G4_EUNSUP), with nothing launched and the workspace never consulted."""
    pattern = "SF"
    m = _model(n_layers=2, n_heads=16, n_kv_heads=1)
    descs, _ = _stack_descs(pattern, 0)
    t = _table([(64, 256, 1), (64, 512, 0)])
    L = bd.lib()
    st = L.g4_stack_forward(C.byref(m), descs, FAKE, FAKE, t, 2, FAKE, 1, 1, bd.G4_DECODE, FAKE, 1 << 40, None)
    assert st == bd.G4_EUNSUP and b"8 query heads" in L.g4_last_error()
    # the same model prefills (the prefill kernels take any group size)
    st = L.g4_stack_forward(C.byref(m), descs, FAKE, FAKE, t, 2, FAKE, 1, 8, bd.G4_PREFILL, FAKE, 1, None)
    assert st == bd.G4_EINVAL and b"workspace" in L.g4_last_error()


def test_noalloc_stack_validation_on_the_host():
    """g4_stack_forward_noalloc takes g4_stack_forward's checks, and refuses a call whose workspace plan
    exceeds its static buffer (G4_ERANGE) before resolving the buffer or launching anything."""
    pattern = "SF"
    m = _model(n_layers=2)
    descs, _ = _stack_descs(pattern, 0)
    L = bd.lib()
    t = _table([(8192, 256, 1), (8192, 512, 0)])
    assert bd.g4_workspace_size(m, 1, 4096, 8192, bd.G4_PREFILL) > bd.NOALLOC_SCRATCH_BYTES
    assert L.g4_stack_forward_noalloc(C.byref(m), descs, FAKE, FAKE, t, 2, FAKE, 1, 4096, bd.G4_PREFILL,
                                      None) == bd.G4_ERANGE
    assert b"static buffer" in L.g4_last_error()
    assert bd.g4_workspace_size(m, 64, 1, 8192, bd.G4_DECODE) <= bd.NOALLOC_SCRATCH_BYTES
    assert L.g4_stack_forward_noalloc(C.byref(m), descs, FAKE, FAKE, t, 2, FAKE, 1, 9000, bd.G4_PREFILL,
                                      None) == bd.G4_ERANGE  # T beyond the caches
    assert L.g4_stack_forward_noalloc(C.byref(m), descs, None, FAKE, t, 2, FAKE, 1, 8, bd.G4_PREFILL,
                                      None) == bd.G4_EINVAL
    assert L.g4_stack_forward_noalloc(C.byref(m), descs, FAKE, FAKE, t, 2, FAKE, 1, 8, 5, None) == bd.G4_EINVAL


def test_noalloc_limit_matches_the_header():
    src = open(os.path.join(ROOT, "include", "g4.h")).read()
    m = re.search(r"#define G4_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == bd.NOALLOC_SCRATCH_BYTES
