"""Per-export parity on the GPU: each g4_* entry point through the C ABI against the float64 oracle
fed the same seeded inputs (bf16 inputs are compared as the exact bf16 values)."""
import numpy as np
import pytest
import torch

import oracle as O
from gemma_decoder_forward_amd import binding as bd
from tests.gpu_util import DT, assert_close, log, max_rel, randn, rel_l2, stream

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------------------- rmsnorm
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("rows,dim,parts", [(37, 2560, 3), (5, 300, 1), (1, 64, 2), (0, 64, 1),
                                            (1030, 2560, 3), (1025, 4096, 1), (1500, 300, 2)])
def test_rmsnorm_fused_tail(dt, rows, dim, parts):
    log(f"rmsnorm {dt} rows={rows} dim={dim} parts={parts}")
    gdt, tdt = DT[dt]
    x = randn((parts, rows, dim), 1 + dim)
    w = randn((dim,), 2, tdt, 0.1, 1.0)
    wn = randn((dim,), 3, tdt, 0.1, 1.0)
    res = randn((rows, dim), 4)
    res0 = res.clone()
    y = torch.empty((rows, dim), dtype=tdt, device="cuda")
    yn = torch.empty_like(y)
    bd.g4_rmsnorm(x.data_ptr(), bd.G4_F32, parts, w.data_ptr(), y.data_ptr(), res.data_ptr(), 0.75, wn.data_ptr(),
                  yn.data_ptr(), rows, dim, 1e-6, gdt, stream())
    torch.cuda.synchronize()
    if rows == 0:  # empty input: a valid call that launches nothing, whatever the pointers
        bd.g4_rmsnorm(None, bd.G4_F32, 1, None, None, None, 1.0, None, None, 0, dim, 1e-6, gdt, stream())
        bd.g4_linear(None, None, None, 0, 8, 8, gdt, gdt, None, 0, stream())
        return
    n = O.rms_norm(O.f64(x).sum(0), w, 1e-6)
    r = (O.f64(res0) + n) * 0.75
    assert_close(y, n, dt, "y")
    assert max_rel(res, r) <= 1e-5
    assert_close(yn, O.rms_norm(r, wn, 1e-6), dt, "y_next")
    # scale-less norm, copy-out of the residual
    y2 = torch.empty((rows, dim), dtype=tdt, device="cuda")
    res2 = res0.clone()
    bd.g4_rmsnorm(x.data_ptr(), bd.G4_F32, parts, None, None, res2.data_ptr(), 1.0, None, y2.data_ptr(), rows, dim,
                  1e-6, gdt, stream())
    torch.cuda.synchronize()
    r2 = O.f64(res0) + O.rms_norm(O.f64(x).sum(0), None, 1e-6)
    assert max_rel(res2, r2) <= 1e-5
    assert_close(y2, r2, dt, "copy")


# ------------------------------------------------------------------------------- qk norm + rope
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("hd,theta,nrot", [(64, 1e4, 32), (128, 1e6, 16), (256, 1e4, 128), (512, 1e6, 64)])
def test_qk_norm_rope_token_major_and_cache(dt, hd, theta, nrot):
    log(f"qk_norm_rope {dt} hd={hd}")
    gdt, tdt = DT[dt]
    B, T, heads, cap = 2, 9, 3, 40
    pos0 = torch.tensor([5, 23], dtype=torch.int32, device="cuda")
    x = randn((B * T, heads * hd + 7), 10 + hd, tdt)  # padded leading dimension
    ld = heads * hd + 7
    w = randn((hd,), 11, tdt, 0.1, 1.0)
    y = torch.empty((B * T, heads * hd), dtype=tdt, device="cuda")
    bd.g4_qk_norm_rope(x.data_ptr(), ld, w.data_ptr(), y.data_ptr(), heads * hd, 0, pos0.data_ptr(), B, T, heads, hd,
                       theta, nrot, 1e-6, gdt, stream())
    sentinel = randn((B, heads, cap, hd), 12, tdt)
    cache = sentinel.clone()
    bd.g4_qk_norm_rope(x.data_ptr(), ld, w.data_ptr(), cache.data_ptr(), 0, cap, pos0.data_ptr(), B, T, heads, hd,
                       theta, nrot, 1e-6, gdt, stream())
    torch.cuda.synchronize()
    xv = O.f64(x)[:, :heads * hd].reshape(B, T, heads, hd)
    pos = O.prefill_positions([5, 23], T)
    ref = O.rope(O.rms_norm(xv, w, 1e-6), pos[:, :, None], O.inv_freq(hd, theta, nrot))
    assert_close(y.reshape(B, T, heads, hd), ref, dt, "token-major")
    c = cache.cpu()
    s = sentinel.cpu()
    for b in range(B):
        p0 = int(pos[b, 0])
        written = c[b, :, p0:p0 + T, :]
        assert_close(written.permute(1, 0, 2), ref[b], dt, "cache rows")
        # every other row is bit-exactly untouched
        assert torch.equal(c[b, :, :p0, :], s[b, :, :p0, :])
        assert torch.equal(c[b, :, p0 + T:, :], s[b, :, p0 + T:, :])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("hd,theta,nrot", [(256, 1e4, 128), (512, 1e6, 64)])
def test_qk_norm_rope_long_prefill_rows(dt, hd, theta, nrot):
    """A long prefill's rows (2 x 1027): against the oracle, bit for bit against one call per sequence,
    and the cache rows bit for bit against the token-major output (every other cache row untouched)."""
    log(f"qk_norm_rope long {dt} hd={hd}")
    gdt, tdt = DT[dt]
    B, T, heads, cap = 2, 1027, 2, 1100
    pos_l = [5, 23]
    pos0 = torch.tensor(pos_l, dtype=torch.int32, device="cuda")
    x = randn((B * T, heads * hd), 13 + hd, tdt)
    w = randn((hd,), 14, tdt, 0.1, 1.0)
    y = torch.empty((B * T, heads * hd), dtype=tdt, device="cuda")
    bd.g4_qk_norm_rope(x.data_ptr(), heads * hd, w.data_ptr(), y.data_ptr(), heads * hd, 0, pos0.data_ptr(), B, T,
                       heads, hd, theta, nrot, 1e-6, gdt, stream())
    y1 = torch.empty_like(y)
    cache = torch.zeros((B, heads, cap, hd), dtype=tdt, device="cuda")
    bd.g4_qk_norm_rope(x.data_ptr(), heads * hd, w.data_ptr(), cache.data_ptr(), 0, cap, pos0.data_ptr(), B, T,
                       heads, hd, theta, nrot, 1e-6, gdt, stream())
    for b in range(B):
        xb, yb = x[b * T:(b + 1) * T], y1[b * T:(b + 1) * T]
        bd.g4_qk_norm_rope(xb.data_ptr(), heads * hd, w.data_ptr(), yb.data_ptr(), heads * hd, 0,
                           pos0[b:b + 1].data_ptr(), 1, T, heads, hd, theta, nrot, 1e-6, gdt, stream())
    torch.cuda.synchronize()
    assert torch.equal(y, y1)
    xv = O.f64(x).reshape(B, T, heads, hd)
    pos = O.prefill_positions(pos_l, T)
    ref = O.rope(O.rms_norm(xv, w, 1e-6), pos[:, :, None], O.inv_freq(hd, theta, nrot))
    assert_close(y.reshape(B, T, heads, hd), ref, dt, "token-major")
    c = cache.cpu()
    for b in range(B):
        assert torch.equal(c[b, :, pos_l[b]:pos_l[b] + T, :], y.cpu()[b * T:(b + 1) * T].reshape(T, heads, hd).permute(1, 0, 2))
        assert not c[b, :, :pos_l[b], :].any() and not c[b, :, pos_l[b] + T:, :].any()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rope_zero_frequency_tail_is_exact_identity(dt):
    gdt, tdt = DT[dt]
    hd, nrot, heads, T = 512, 64, 8, 33
    pos0 = torch.tensor([31000], dtype=torch.int32, device="cuda")
    x = randn((T, heads * hd), 20, tdt)
    w = randn((hd,), 21, tdt, 0.1, 1.0)
    a = torch.empty_like(x)
    b = torch.empty_like(x)
    bd.g4_qk_norm_rope(x.data_ptr(), heads * hd, w.data_ptr(), a.data_ptr(), heads * hd, 0, pos0.data_ptr(), 1, T,
                       heads, hd, 1e6, nrot, 1e-6, gdt, stream())
    bd.g4_qk_norm_rope(x.data_ptr(), heads * hd, w.data_ptr(), b.data_ptr(), heads * hd, 0, pos0.data_ptr(), 1, T,
                       heads, hd, 1e6, 0, 1e-6, gdt, stream())
    torch.cuda.synchronize()
    a, b = a.view(T, heads, hd), b.view(T, heads, hd)
    h = hd // 2
    assert torch.equal(a[..., nrot:h], b[..., nrot:h]) and torch.equal(a[..., h + nrot:], b[..., h + nrot:])
    assert not torch.equal(a[..., :nrot], b[..., :nrot])


# ------------------------------------------------------------------------------- attention
def _kv_table(entries):
    t = (bd.KvEntry * len(entries))()
    for i, e in enumerate(entries):
        if e is not None:
            k, v, sliding = e
            t[i] = bd.KvEntry(k=k.data_ptr(), v=v.data_ptr(), cap=k.shape[2], hd=k.shape[3], sliding=sliding)
    return t


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("hd,sliding,window,nh,nkv", [(64, 1, 32, 4, 1), (128, 0, 0, 4, 1), (256, 1, 512, 8, 2),
                                                      (512, 0, 0, 8, 2), (256, 1, 7, 4, 2), (128, 1, 40, 2, 2),
                                                      (512, 1, 100, 4, 2), (512, 0, 0, 8, 1), (256, 1, 100, 8, 1),
                                                      (128, 0, 0, 8, 1)])
def test_attention_prefill_vs_oracle(dt, hd, sliding, window, nh, nkv):
    log(f"attn_prefill {dt} hd={hd} sliding={sliding} W={window}")
    gdt, tdt = DT[dt]
    B, T, cap = 2, 77, 700
    pos0_l = [0, 600]
    pos0 = torch.tensor(pos0_l, dtype=torch.int32, device="cuda")
    q = randn((B * T, nh * hd), 30 + hd, tdt)
    K = randn((B, nkv, cap, hd), 31, tdt)
    V = randn((B, nkv, cap, hd), 32, tdt)
    out = torch.empty((B * T, nh * hd), dtype=tdt, device="cuda")
    t = _kv_table([(K, V, sliding)])
    bd.g4_attn_prefill(q.data_ptr(), nh * hd, t, 1, 0, 0, sliding, window, pos0.data_ptr(), B, T, nh, nkv, hd, 1.0,
                       out.data_ptr(), nh * hd, None, 0, gdt, stream())
    torch.cuda.synchronize()
    qv = O.f64(q).reshape(B, T, nh, hd)
    pos = O.prefill_positions(pos0_l, T)
    for b in range(B):
        ref = O.attention(qv[b], O.f64(K[b]), O.f64(V[b]), pos[b], window if sliding else None)
        assert_close(out.reshape(B, T, nh, hd)[b], ref, dt, f"seq {b}")


@pytest.mark.parametrize("scale", [0.0625, 0.0, -0.5])
@pytest.mark.parametrize("hd,sliding,window,nh,nkv", [(256, 1, 100, 8, 2), (512, 0, 0, 8, 2)])
def test_attention_prefill_score_scale(hd, sliding, window, nh, nkv, scale):
    """g4_attn_prefill with a score scale other than the layers' 1.0: the matrix-core kernels fold a
    positive scale into the exponential (the maximum is taken over the unscaled scores); zero and negative
    scales go to the generic kernel. Against the oracle with the same scale."""
    log(f"attn_prefill scale={scale} hd={hd}")
    B, T, cap = 2, 77, 700
    pos0_l = [0, 600]
    pos0 = torch.tensor(pos0_l, dtype=torch.int32, device="cuda")
    q = randn((B * T, nh * hd), 70 + hd, torch.bfloat16)
    K = randn((B, nkv, cap, hd), 71, torch.bfloat16)
    V = randn((B, nkv, cap, hd), 72, torch.bfloat16)
    out = torch.empty((B * T, nh * hd), dtype=torch.bfloat16, device="cuda")
    t = _kv_table([(K, V, sliding)])
    bd.g4_attn_prefill(q.data_ptr(), nh * hd, t, 1, 0, 0, sliding, window, pos0.data_ptr(), B, T, nh, nkv, hd, scale,
                       out.data_ptr(), nh * hd, None, 0, bd.G4_BF16, stream())
    torch.cuda.synchronize()
    qv = O.f64(q).reshape(B, T, nh, hd)
    pos = O.prefill_positions(pos0_l, T)
    for b in range(B):
        ref = O.attention(qv[b], O.f64(K[b]), O.f64(V[b]), pos[b], window if sliding else None, scale=scale)
        assert_close(out.reshape(B, T, nh, hd)[b], ref, "bf16", f"seq {b}")


@pytest.mark.parametrize("hd,sliding,window", [(64, 1, 7), (64, 0, 0), (256, 1, 33), (128, 0, 0), (512, 1, 21)])
def test_attention_mask_probe_bit_exact(hd, sliding, window):
    """q = 0 gives uniform weights; V_j = onehot(j mod hd) makes round(o * n) the mask row."""
    T, nh, nkv = 64, 4, 1
    q = torch.zeros((T, nh * hd), dtype=torch.bfloat16, device="cuda")
    K = randn((1, nkv, T, hd), 40, torch.bfloat16)
    Vh = torch.zeros((1, nkv, T, hd))
    for j in range(T):
        Vh[0, :, j, j % hd] = 1.0
    V = Vh.to(torch.bfloat16).cuda()
    pos0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    t = _kv_table([(K, V, sliding)])
    bd.g4_attn_prefill(q.data_ptr(), nh * hd, t, 1, 0, 0, sliding, window, pos0.data_ptr(), 1, T, nh, nkv, hd, 1.0,
                       out.data_ptr(), nh * hd, None, 0, bd.G4_BF16, stream())
    torch.cuda.synchronize()
    o = O.f64(out).reshape(T, nh, hd)
    for i in range(T):
        lo = max(0, i - window + 1) if sliding else 0
        n = i - lo + 1
        want = np.zeros(hd)
        for j in range(lo, i + 1):
            want[j % hd] += 1
        for h in range(nh):
            assert np.array_equal(np.rint(o[i, h] * n), want), (i, h)


def test_attention_reads_kv_src_cache_without_copy():
    """Caches filled with the constant layer+1: the output is exactly kv_src+1."""
    hd, T, nh, nkv = 128, 16, 4, 1
    caches = []
    for l in range(4):
        k = randn((1, nkv, 32, hd), 50 + l, torch.bfloat16)
        v = torch.full((1, nkv, 32, hd), float(l + 1), dtype=torch.bfloat16, device="cuda")
        caches.append((k, v, 0))
    caches[2] = None  # a shared layer: a hole in the table
    t = _kv_table(caches)
    q = randn((T, nh * hd), 55, torch.bfloat16)
    pos0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    for src in (0, 1, 3):
        out = torch.empty_like(q)
        bd.g4_attn_prefill(q.data_ptr(), nh * hd, t, 4, 3, src, 0, 0, pos0.data_ptr(), 1, T, nh, nkv, hd, 1.0,
                           out.data_ptr(), nh * hd, None, 0, bd.G4_BF16, stream())
        torch.cuda.synchronize()
        assert torch.all(out == float(src + 1))


@pytest.mark.parametrize("with_ws", [False, True])
@pytest.mark.parametrize("hd,sliding,W,nkv", [(256, 1, 512, 2), (512, 0, 0, 2), (512, 0, 0, 1), (256, 1, 512, 1)])
def test_attention_prefill_long_e4b_shapes(hd, sliding, W, nkv, with_ws):
    """E4B heads (8 q / 2 kv, or the variant's full layer with one kv head) over T = 2048 from position
    0, the layer pair's attention call. With a workspace the export takes the key split (128 query blocks
    for 256 compute units), without one it does not; both must match the oracle. With 8 query heads per
    kv head a block covers half of a 32-token run's heads, so a split threshold can fall inside a run."""
    log(f"attn_prefill long hd={hd} nkv={nkv} ws={with_ws}")
    B, T, nh = 1, 2048, 8
    q = randn((T, nh * hd), 35 + hd, torch.bfloat16)
    K = randn((1, nkv, T, hd), 36, torch.bfloat16)
    V = randn((1, nkv, T, hd), 37, torch.bfloat16)
    out = torch.empty_like(q)
    pos0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    t = _kv_table([(K, V, sliding)])
    nws = bd.g4_attn_prefill_ws(B, T, nh, nkv, hd)
    assert nws > 0  # this shape splits its keys when given scratch
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if with_ws else None
    bd.g4_attn_prefill(q.data_ptr(), nh * hd, t, 1, 0, 0, sliding, W, pos0.data_ptr(), B, T, nh, nkv, hd, 1.0,
                       out.data_ptr(), nh * hd, None if ws is None else ws.data_ptr(), nws if with_ws else 0,
                       bd.G4_BF16, stream())
    torch.cuda.synchronize()
    ref = O.attention(O.f64(q).reshape(T, nh, hd), O.f64(K[0]), O.f64(V[0]), np.arange(T), W if sliding else None)
    assert_close(out.reshape(T, nh, hd), ref, "bf16", "long")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("hd,sliding,window,nh,nkv", [(64, 1, 32, 4, 1), (512, 0, 0, 8, 2), (256, 1, 512, 8, 2),
                                                      (128, 0, 0, 4, 2), (512, 0, 0, 8, 1)])
def test_attention_decode_vs_oracle(dt, hd, sliding, window, nh, nkv):
    log(f"attn_decode {dt} hd={hd} sliding={sliding}")
    gdt, tdt = DT[dt]
    B, cap = 3, 1500
    pos_l = [0, 700, 1499]
    pos = torch.tensor(pos_l, dtype=torch.int32, device="cuda")
    q = randn((B, nh * hd), 60 + hd, tdt)
    K = randn((B, nkv, cap, hd), 61, tdt)
    V = randn((B, nkv, cap, hd), 62, tdt)
    out = torch.empty((B, nh * hd), dtype=tdt, device="cuda")
    wsb = bd.g4_attn_decode_ws(B, nh, hd, cap)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    t = _kv_table([(K, V, sliding)])
    bd.g4_attn_decode(q.data_ptr(), nh * hd, t, 1, 0, 0, sliding, window, pos.data_ptr(), B, nh, nkv, hd, 1.0,
                      out.data_ptr(), nh * hd, ws.data_ptr(), wsb, gdt, stream())
    torch.cuda.synchronize()
    qv = O.f64(q).reshape(B, 1, nh, hd)
    for b in range(B):
        ref = O.attention(qv[b], O.f64(K[b]), O.f64(V[b]), [pos_l[b]], window if sliding else None)
        assert_close(out.reshape(B, 1, nh, hd)[b], ref, dt, f"seq {b}")


@pytest.mark.parametrize("hd,sliding,window,nh,nkv", [(256, 1, 512, 2, 2), (512, 0, 0, 8, 2), (128, 1, 100, 8, 2)])
def test_attention_decode_many_sequences_long_chunks(hd, sliding, window, nh, nkv):
    """64 sequences: the key chunks grow to 256 keys (several 16-key steps per wave), ragged ends."""
    log(f"attn_decode bf16 B=64 hd={hd} sliding={sliding} G={nh // nkv}")
    gdt, tdt = DT["bf16"]
    B, cap = 64, 1500
    g = torch.Generator().manual_seed(70 + hd)
    pos_l = torch.randint(0, cap, (B,), generator=g).tolist()
    pos_l[0], pos_l[1], pos_l[2] = 0, cap - 1, 255
    pos = torch.tensor(pos_l, dtype=torch.int32, device="cuda")
    q = randn((B, nh * hd), 71 + hd, tdt)
    K = randn((B, nkv, cap, hd), 72, tdt)
    V = randn((B, nkv, cap, hd), 73, tdt)
    out = torch.empty((B, nh * hd), dtype=tdt, device="cuda")
    wsb = bd.g4_attn_decode_ws(B, nh, hd, cap)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    t = _kv_table([(K, V, sliding)])
    bd.g4_attn_decode(q.data_ptr(), nh * hd, t, 1, 0, 0, sliding, window, pos.data_ptr(), B, nh, nkv, hd, 0.5,
                      out.data_ptr(), nh * hd, ws.data_ptr(), wsb, gdt, stream())
    torch.cuda.synchronize()
    qv = O.f64(q).reshape(B, 1, nh, hd)
    Kc, Vc, oc = K.cpu(), V.cpu(), out.reshape(B, 1, nh, hd)
    for b in range(B):
        ref = O.attention(qv[b], O.f64(Kc[b]), O.f64(Vc[b]), [pos_l[b]], window if sliding else None, scale=0.5)
        assert_close(oc[b], ref, "bf16", f"seq {b} pos {pos_l[b]}")


# ------------------------------------------------------------------------------- projections
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(77, 130, 200), (256, 512, 2560), (1, 256, 64), (300, 2560, 256)])
def test_linear_vs_oracle(dt, M, N, K):
    log(f"linear {dt} {M}x{N}x{K}")
    gdt, tdt = DT[dt]
    A = randn((M, K), 70, tdt)
    W = randn((N, K), 71, tdt, 0.02)
    C32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    Cd = torch.empty((M, N), dtype=tdt, device="cuda")
    bd.g4_linear(A.data_ptr(), W.data_ptr(), C32.data_ptr(), M, N, K, bd.G4_F32, gdt, None, 0, stream())
    bd.g4_linear(A.data_ptr(), W.data_ptr(), Cd.data_ptr(), M, N, K, gdt, gdt, None, 0, stream())
    torch.cuda.synchronize()
    ref = O.f64(A) @ O.f64(W).T
    assert max_rel(C32, ref) <= 1e-3
    assert_close(Cd, ref, dt, "C in dtype")


@pytest.mark.parametrize("M,N,K", [(1000, 12288, 576), (520, 24576, 128), (600, 24576, 64), (300, 24576, 2560),
                                   (1024, 16384, 576), (4096, 2048, 1024), (7168, 2560, 256)])
def test_linear_large_tiles_pipeline_depths(M, N, K):
    """The 256-row-tile MFMA paths (at least 192 tiles): ragged M, and K steps fewer than, equal to and
    more than the LDS stages (K = 64, 128, 576, 2560 in steps of 64). On 256 CUs the tile widths are
    192 (the first four shapes: the segmented loader over one matrix), 256 (1024 x 16384), 128
    (4096 x 2048: more loads than MFMAs per k-slice) and 320 (7168 x 2560). Large outputs are checked
    on every 7th row and the last rows."""
    log(f"linear large tiles {M}x{N}x{K}")
    A = randn((M, K), 74, torch.bfloat16)
    W = randn((N, K), 75, torch.bfloat16, 0.02)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    bd.g4_linear(A.data_ptr(), W.data_ptr(), C.data_ptr(), M, N, K, bd.G4_F32, bd.G4_BF16, None, 0, stream())
    torch.cuda.synchronize()
    rows = np.arange(M) if M * N <= 24576 * 1000 else np.unique(np.r_[np.arange(0, M, 7), np.arange(M - 300, M)])
    ref = O.f64(A)[rows] @ O.f64(W).T
    assert max_rel(C[torch.as_tensor(rows, device="cuda")], ref) <= 1e-3


@pytest.mark.parametrize("M,N,K", [(1, 256, 2560), (8, 3072, 2560), (33, 512, 10240), (64, 2560, 10240),
                                   (17, 20480, 2560),
                                   # the vector-ALU path (M <= 4): several 512-k chunk groups per row, a part-filled
                                   # last chunk, every token-row bound (1, 2, 4) and odd M; then M = 5, 7 either side
                                   (1, 16384, 4096), (2, 16384, 6400), (3, 640, 384), (4, 128, 256), (3, 16384, 5248),
                                   (5, 2560, 10240), (7, 2048, 2688)])
def test_linear_few_rows_weight_streaming(M, N, K):
    """Decode-shaped projections (M = batch): the weight-streaming split-K path, given a workspace."""
    log(f"linear few rows {M}x{N}x{K}")
    A = randn((M, K), 72, torch.bfloat16)
    W = randn((N, K), 73, torch.bfloat16, 0.02)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    bd.g4_linear(A.data_ptr(), W.data_ptr(), C.data_ptr(), M, N, K, bd.G4_F32, bd.G4_BF16, ws.data_ptr(), ws.numel(),
                 stream())
    Cb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    bd.g4_linear(A.data_ptr(), W.data_ptr(), Cb.data_ptr(), M, N, K, bd.G4_BF16, bd.G4_BF16, ws.data_ptr(),
                 ws.numel(), stream())
    torch.cuda.synchronize()
    ref = O.f64(A) @ O.f64(W).T
    assert max_rel(C, ref) <= 1e-3
    assert_close(Cb, ref, "bf16", "bf16 out")


@pytest.mark.parametrize("M,N,K", [(17, 16384, 2560), (64, 20480, 640), (48, 16512, 512)])
def test_linear_rows64_tiles(M, N, K):
    """17 to 64 token rows on wide, short weights (at least 16384 rows, K <= 4096): one 64-row MFMA tile
    over all token rows, 64 output columns per tile (16512 = 258 x 64 is not a whole number of wider
    tiles); float32 and bf16 outputs."""
    log(f"linear 64-row tiles {M}x{N}x{K}")
    A = randn((M, K), 88, torch.bfloat16)
    W = randn((N, K), 89, torch.bfloat16, 0.02)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    Cb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    bd.g4_linear(A.data_ptr(), W.data_ptr(), C.data_ptr(), M, N, K, bd.G4_F32, bd.G4_BF16, None, 0, stream())
    bd.g4_linear(A.data_ptr(), W.data_ptr(), Cb.data_ptr(), M, N, K, bd.G4_BF16, bd.G4_BF16, None, 0, stream())
    torch.cuda.synchronize()
    ref = O.f64(A) @ O.f64(W).T
    assert max_rel(C, ref) <= 1e-3
    assert_close(Cb, ref, "bf16", "bf16 out")


@pytest.mark.parametrize("M,H,F", [(40, 2560, 10240), (23, 256, 8224)])
def test_ffn_geglu_rows64(M, H, F):
    """17 to 64 token rows: the gate/up product on 64-row tiles with the gated epilogue, 64 outputs per
    tile (E4B widths: 160 tiles), or 32 when F is not a multiple of 64 (8224 = 257 x 32); then the down
    projection."""
    log(f"ffn geglu {M} rows H={H} F={F}")
    x = randn((M, H), 90, torch.bfloat16)
    wg, wu = randn((F, H), 91, torch.bfloat16, 0.02), randn((F, H), 92, torch.bfloat16, 0.02)
    wd = randn((H, F), 93, torch.bfloat16, 0.02)
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    wsb = bd.g4_ffn_geglu_ws(M, H, F, bd.G4_BF16)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    bd.g4_ffn_geglu(x.data_ptr(), wg.data_ptr(), wu.data_ptr(), wd.data_ptr(), out.data_ptr(), M, H, F, ws.data_ptr(),
                    wsb, bd.G4_BF16, stream())
    torch.cuda.synchronize()
    xv = O.f64(x)
    ref = (O.gelu_tanh(xv @ O.f64(wg).T) * (xv @ O.f64(wu).T)) @ O.f64(wd).T
    assert_close(out, ref, "bf16", f"ffn {M} rows")


def _sample_rows(M):
    return sorted(set(list(range(24)) + list(range(M // 2 - 8, M // 2 + 8)) + list(range(M - 24, M))))


def test_linear_bf16_e4b_gate_up_shape():
    """M = 2048, N = 20480 (the E4B gate and up rows at T = 2048) with bf16 output: 640 big tiles, a
    persistent grid walking several tiles per block; sampled rows over every column block."""
    M, N, K = 2048, 20480, 256
    log(f"linear bf16 {M}x{N}x{K}")
    A = randn((M, K), 76, torch.bfloat16)
    W = randn((N, K), 77, torch.bfloat16, 0.05)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    bd.g4_linear(A.data_ptr(), W.data_ptr(), C.data_ptr(), M, N, K, bd.G4_BF16, bd.G4_BF16, None, 0, stream())
    torch.cuda.synchronize()
    rows = _sample_rows(M)
    ref = O.f64(A[rows]) @ O.f64(W).T
    # every column block within the bf16 bound
    for c0 in range(0, N, 2048):
        assert_close(C[rows, c0:c0 + 2048], ref[:, c0:c0 + 2048], "bf16", f"columns {c0}..")


def test_ffn_geglu_e4b_rows():
    """E4B FFN (H 2560, F 10240) at T = 2048: the gate/up GEMM with its GEGLU epilogue, then down; sampled rows."""
    M, H, F = 2048, 2560, 10240
    log("ffn geglu E4B T=2048")
    x = randn((M, H), 84, torch.bfloat16)
    wg, wu = randn((F, H), 85, torch.bfloat16, 0.02), randn((F, H), 86, torch.bfloat16, 0.02)
    wd = randn((H, F), 87, torch.bfloat16, 0.02)
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    wsb = bd.g4_ffn_geglu_ws(M, H, F, bd.G4_BF16)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    bd.g4_ffn_geglu(x.data_ptr(), wg.data_ptr(), wu.data_ptr(), wd.data_ptr(), out.data_ptr(), M, H, F, ws.data_ptr(),
                    wsb, bd.G4_BF16, stream())
    torch.cuda.synchronize()
    rows = _sample_rows(M)
    xv = O.f64(x[rows])
    ref = (O.gelu_tanh(xv @ O.f64(wg).T) * (xv @ O.f64(wu).T)) @ O.f64(wd).T
    assert_close(out[rows], ref, "bf16", "ffn rows")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_ffn_geglu_vs_oracle(dt):
    gdt, tdt = DT[dt]
    M, H, F = 33, 256, 1024
    x = randn((M, H), 80, tdt)
    wg, wu = randn((F, H), 81, tdt, 0.05), randn((F, H), 82, tdt, 0.05)
    wd = randn((H, F), 83, tdt, 0.05)
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    wsb = bd.g4_ffn_geglu_ws(M, H, F, gdt)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    bd.g4_ffn_geglu(x.data_ptr(), wg.data_ptr(), wu.data_ptr(), wd.data_ptr(), out.data_ptr(), M, H, F, ws.data_ptr(),
                    wsb, gdt, stream())
    torch.cuda.synchronize()
    xv = O.f64(x)
    ref = (O.gelu_tanh(xv @ O.f64(wg).T) * (xv @ O.f64(wu).T)) @ O.f64(wd).T
    assert_close(out, ref, dt, "ffn")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("scalar", [1.0, 0.5])
def test_ple_inject_vs_oracle(dt, scalar):
    gdt, tdt = DT[dt]
    M, H, d, L = 21, 256, 32, 3
    h = randn((M, H), 90)
    h0 = h.clone()
    ple = randn((M, L * d), 91)
    wg, wp = randn((d, H), 92, tdt, 0.05), randn((H, d), 93, tdt, 0.05)
    wpost = randn((H,), 94, tdt, 0.1, 1.0)
    wsb = bd.g4_ple_inject_ws(M, H, d, gdt)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    bd.g4_ple_inject(h.data_ptr(), wg.data_ptr(), ple[:, d:].data_ptr(), L * d, wp.data_ptr(), wpost.data_ptr(),
                     scalar, M, H, d, 1e-6, ws.data_ptr(), wsb, gdt, stream())
    torch.cuda.synchronize()
    hv = O.f64(h0)
    gmix = O.gelu_tanh(hv @ O.f64(wg).T) * O.f64(ple)[:, d:2 * d]
    ref = (hv + O.rms_norm(gmix @ O.f64(wp).T, wpost, 1e-6)) * scalar
    assert_close(h, ref, "f32" if dt == "f32" else "bf16", "h")


@pytest.mark.parametrize("M,scalar", [(1000, 1.0), (70, 0.5), (4096, 1.0), (65, 1.0), (129, 0.5)])
def test_ple_inject_e4b_widths_vs_oracle(M, scalar):
    """The PLE block at E4B widths (H 2560, d 256), bf16, at prefill row counts (the gate GEMM on 64 x 64
    tiles over the whole K with gelu(g) x input in the store, the projection GEMM and the row tail;
    M = 1000, 70, 65 and 129 leave ragged tiles, 65 a last tile of one row). The branch itself,
    h_out / scalar - h, is compared at the bf16 bound, and h within it."""
    H, d, L = 2560, 256, 4
    h = randn((M, H), 95)
    h0 = h.clone()
    ple = randn((M, L * d), 96)
    wg, wp = randn((d, H), 97, torch.bfloat16, 0.02), randn((H, d), 98, torch.bfloat16, 0.02)
    wpost = randn((H,), 99, torch.bfloat16, 0.1, 1.0)
    wsb = bd.g4_ple_inject_ws(M, H, d, bd.G4_BF16)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    bd.g4_ple_inject(h.data_ptr(), wg.data_ptr(), ple[:, 2 * d:].data_ptr(), L * d, wp.data_ptr(), wpost.data_ptr(),
                     scalar, M, H, d, 1e-6, ws.data_ptr(), wsb, bd.G4_BF16, stream())
    torch.cuda.synchronize()
    hv = O.f64(h0)
    gmix = O.gelu_tanh(hv @ O.f64(wg).T) * O.f64(ple)[:, 2 * d:3 * d]
    branch = O.rms_norm(gmix @ O.f64(wp).T, wpost, 1e-6)
    e = assert_close(O.f64(h) / scalar - hv, branch, "bf16", "PLE branch")
    assert_close(h, (hv + branch) * scalar, "bf16", "h")
    log(f"PLE block M={M}: branch rel L2 {e:.2e}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_embed_ple_vs_oracle(dt):
    from synth import configs, gen
    cfg = configs.get(1, dtype=dt)
    glob = gen.model_globals(cfg, "cuda")
    m_ids = [0, 5, 511, 300, 512, 7000, -3, 42]
    ids = torch.tensor(m_ids, dtype=torch.int32, device="cuda")
    from gemma_decoder_forward_amd.model import G4Model
    layers = [gen.layer_weights(cfg, l, "cuda") for l in range(cfg["n_layers"])]
    model = G4Model(cfg, layers, glob)
    h, ple = model.embed(ids.view(1, -1))
    torch.cuda.synchronize()
    e_ref, p_ref = O.entry(cfg, {k: v.cpu() for k, v in glob.items()}, np.array([m_ids]))
    assert_close(h, e_ref, "f32", "h0")
    assert_close(ple, p_ref, "f32" if dt == "f32" else "bf16", "ple_in")
    assert torch.all(h[0, 4:7] == 0)


def test_embed_ple_e4b_widths_vs_oracle():
    """The entry at the 42-layer model's widths: H = 2560, 42 layers of 256 per-layer inputs, vocabulary
    262144 (5.6 GB PLE table), 300 token ids including out-of-range ones, bf16."""
    from gemma_decoder_forward_amd.model import G4Model
    from synth import configs, gen
    cfg = configs.get(3)
    glob = gen.model_globals(cfg, "cuda")
    g = torch.Generator(device="cuda").manual_seed(77)
    ids = torch.randint(0, cfg["vocab"], (300,), generator=g, device="cuda", dtype=torch.int64).to(torch.int32)
    ids[[3, 100, 299]] = torch.tensor([cfg["vocab"], -1, 2 ** 30], dtype=torch.int32, device="cuda")
    ids[7] = cfg["vocab"] - 1
    lw = gen.layer_weights(cfg, 0, "cuda")
    model = G4Model(cfg, [lw] * cfg["n_layers"], glob)  # the entry reads only the tables
    h, ple = model.embed(ids.view(1, -1))
    torch.cuda.synchronize()
    m_ids = ids.cpu().numpy()
    valid = (m_ids >= 0) & (m_ids < cfg["vocab"])
    uniq, inv = np.unique(np.where(valid, m_ids, 0), return_inverse=True)
    idx = torch.from_numpy(uniq).cuda()
    sub = dict(cfg, vocab=len(uniq), ple_vocab=len(uniq))
    gh = dict(embed=glob["embed"][idx].cpu(), ple_embed=glob["ple_embed"][idx].cpu(),
              ple_model_proj=glob["ple_model_proj"].cpu(), ple_norm=glob["ple_norm"].cpu())
    local = np.where(valid, inv, len(uniq)).reshape(1, -1)  # out-of-range ids stay out of range
    e_ref, p_ref = O.entry(sub, gh, local)
    assert_close(h, e_ref, "f32", "h0")
    e = assert_close(ple, p_ref, "bf16", "ple_in")
    log(f"entry at E4B widths: ple_in rel L2 {e:.2e}")
    # an out-of-range id: zero embedding row, so a zero projection, and no table term
    assert torch.all(h[0, [3, 100, 299]] == 0) and torch.all(ple[0, [3, 100, 299]] == 0)


# ------------------------------------------------------------------------------- output head
@pytest.mark.parametrize("dt,M,H,V,cap", [("f32", 5, 256, 512, 30.0), ("f32", 70, 64, 200, 0.0),
                                          ("bf16", 1, 2560, 262144, 30.0), ("bf16", 7, 2560, 262144, 30.0),
                                          ("bf16", 64, 2560, 262144, 30.0),
                                          ("bf16", 300, 256, 4096, 30.0), ("bf16", 33, 256, 960, 0.0),
                                          ("bf16", 33, 256, 960, 30.0), ("bf16", 20, 256, 1000, 30.0),
                                          ("f32", 5, 256, 510, 30.0), ("bf16", 5, 256, 960, 30.0),
                                          ("bf16", 3, 64, 512, 30.0), ("bf16", 2, 256, 1000, 30.0)])
def test_logits_vs_oracle(dt, M, H, V, cap):
    """Final norm + output projection + softcap; the E4B vocabulary at decode batch sizes. 17 to 64 rows
    apply the softcap in the 64-row tiles' store (64, 128 or 256 columns wide: vocabularies of 960 and
    262144), up to 16 in the few-row product's finishing pass (1, 5 and 7 rows); other rows, and shapes
    those kernels do not take (K = 64, a vocabulary of 1000), a separate pass, four floats per thread or
    (a length not a multiple of 4) one."""
    log(f"logits {dt} M={M} H={H} V={V} cap={cap}")
    gdt, tdt = DT[dt]
    h = randn((M, H), 90 + M, torch.float32, 2.0)
    wn = randn((H,), 91, tdt, 0.1, 1.0)
    W = randn((V, H), 92, tdt, 0.5)  # large enough that many logits reach the softcap's curved part
    out = torch.empty((M, V), dtype=torch.float32, device="cuda")
    wsb = bd.g4_logits_ws(M, H, V, gdt)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    bd.g4_logits(h.data_ptr(), M, H, wn.data_ptr(), W.data_ptr(), V, 1e-6, cap, out.data_ptr(), ws.data_ptr(), wsb,
                 gdt, stream())
    torch.cuda.synchronize()
    ref = O.logits(O.f64(h), O.f64(wn), O.f64(W), cap)
    assert_close(out, ref, dt, "logits")
    if cap > 0:
        assert float(out.abs().max()) < cap

