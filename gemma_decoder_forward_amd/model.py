"""Model-level driver over libg4.so: descriptors, KV caches, workspace, prefill and decode calls.

PyTorch supplies device memory and the stream; every step of the forward runs in the library.
"""
import ctypes as C
import os

import torch

from . import binding as bd

DTYPES = {"f32": (bd.G4_F32, torch.float32), "bf16": (bd.G4_BF16, torch.bfloat16)}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


class G4Model:
    """A Gemma-4 E-series text stack resident on one GPU.

    cfg: a workload dict (hidden, n_heads, ..., layer_types "S"/"F" per layer, n_shared, dtype; optional
    n_kv_heads_full, k_eq_v and per-layer ffn_dims).
    layers: list of per-layer dicts of device tensors (names as in g4_layer_desc; each layer's FFN width
    is read from its w_gate).
    glob: optional dict with embed, ple_embed, ple_model_proj, ple_norm (device tensors).
    """

    def __init__(self, cfg, layers, glob=None):
        self.cfg = cfg
        self.g4_dtype, self.torch_dtype = DTYPES[cfg["dtype"]]
        L = len(cfg["layer_types"])
        self.L = L
        self.desc = bd.ModelDesc(
            hidden=cfg["hidden"], n_heads=cfg["n_heads"], n_kv_heads=cfg["n_kv_heads"],
            head_dim_swa=cfg["head_dim_swa"], head_dim_full=cfg["head_dim_full"],
            ffn=max([cfg["ffn"]] + [int(f) for f in cfg.get("ffn_dims") or []]),
            ple_dim=cfg["ple_dim"], n_layers=L, window=cfg["window"], vocab=cfg.get("vocab", 1),
            ple_vocab=cfg.get("ple_vocab", 1), eps=cfg["eps"], theta_swa=cfg["theta_swa"],
            theta_full=cfg["theta_full"], partial_rotary=cfg["partial_rotary"], dtype=self.g4_dtype,
            k_eq_v=1 if cfg.get("k_eq_v") else 0, n_kv_heads_full=int(cfg.get("n_kv_heads_full") or 0))
        self.sliding = [1 if t == "S" else 0 for t in cfg["layer_types"]]
        self.kv_src = bd.g4_kv_sources(self.sliding, cfg["n_shared"])
        self.layers = layers
        self.glob = glob
        self.descs = (bd.LayerDesc * L)()
        for l, lw in enumerate(layers):
            d = self.descs[l]
            d.sliding = self.sliding[l]
            d.kv_src = self.kv_src[l]
            d.layer_scalar = float(lw.get("layer_scalar", 1.0))
            d.ffn = int(lw["w_gate"].shape[0])
            own = self.kv_src[l] == l
            for name in bd.LAYER_PTRS:
                t = lw.get(name)
                if name in ("wk", "wv", "k_norm") and not own:
                    t = None
                setattr(d, name, _ptr(t))
        self._ws = None

    def head_dim(self, l):
        return self.cfg["head_dim_swa"] if self.sliding[l] else self.cfg["head_dim_full"]

    def kv_heads(self, l):
        if self.sliding[l] or not self.cfg.get("n_kv_heads_full"):
            return self.cfg["n_kv_heads"]
        return self.cfg["n_kv_heads_full"]

    def new_caches(self, B, cap, fill=None, ring=0):
        """Device K/V caches [B, nkv, rows, hd] for every owning layer, plus the C table.

        rows = cap, position p in row p; with ring > 0 the sliding layers' caches are rings of `ring` rows
        (position p in row p mod ring, ring >= window), which bounds their memory by the window instead of
        the context; a call then takes at most ring - window + 1 tokens per sequence."""
        caches = {}
        table = (bd.KvEntry * self.L)()
        for l in range(self.L):
            if self.kv_src[l] != l:
                continue
            hd = self.head_dim(l)
            is_ring = 1 if (ring and self.sliding[l]) else 0
            rows = ring if is_ring else cap
            if fill is not None:
                k, v = fill(l)
            else:
                k = torch.zeros((B, self.kv_heads(l), rows, hd), dtype=self.torch_dtype, device="cuda")
                v = torch.zeros_like(k)
            caches[l] = (k, v)
            table[l] = bd.KvEntry(k=k.data_ptr(), v=v.data_ptr(), cap=rows, hd=hd, sliding=self.sliding[l],
                                  ring=is_ring)
        return caches, table

    def workspace(self, B, T, cap, mode):
        need = bd.g4_workspace_size(self.desc, B, T, cap, mode)
        if need == 0:
            raise RuntimeError("invalid model descriptor")
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        return self._ws

    def embed(self, ids, h=None, ple=None):
        """ids int32 [B, T] (device) -> (h0 float32 [B, T, H], ple_in float32 [B, T, L, d]), written into
        h and ple when given (contiguous float32 tensors of those shapes), else into new tensors."""
        B, T = ids.shape
        M = B * T
        H, L, d = self.cfg["hidden"], self.L, self.cfg["ple_dim"]
        if h is None:
            h = torch.empty((B, T, H), dtype=torch.float32, device="cuda")
        if ple is None:
            ple = torch.empty((B, T, L, d), dtype=torch.float32, device="cuda")
        for t, shape in ((h, (B, T, H)), (ple, (B, T, L, d))):
            if tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous():
                raise ValueError(f"embed output must be a contiguous float32 tensor of shape {shape}")
        ws = self.workspace(B, T, 1, bd.G4_PREFILL)
        g = self.glob
        bd.g4_embed_ple(ids.data_ptr(), M, g["embed"].data_ptr(), g["ple_embed"].data_ptr(),
                        g["ple_model_proj"].data_ptr(), g["ple_norm"].data_ptr(), self.desc, h.data_ptr(),
                        ple.data_ptr(), ws.data_ptr(), ws.numel(), _stream())
        return h, ple

    def forward(self, h, ple_in, pos, table, cap, mode=bd.G4_PREFILL, layer=None, dump=None, caches=None):
        """Run all layers (or one, if `layer` is given) in place on h [B, T, H] float32.

        dump: a directory (default: the G4_DUMP environment variable, if set) for a per-layer dump to diff
        against an oracle, as cortiq-engine `g4e_forward` writes one (`CMF_LAYER_DUMP`: the hidden state
        after every block). The layers then run one library call each, and the
        hidden state goes to `l_in.f32` before the first layer and `lNN.f32` after layer NN, float32
        little-endian [B, T, H]. With `caches` (from new_caches) every owning layer's K and V rows at the
        call's positions go to `lNN_k.f32` / `lNN_v.f32`, [B, nkv, T, hd] upcast to float32."""
        B, T = h.shape[0], h.shape[1]
        if dump is None:
            dump = os.environ.get("G4_DUMP") or None
        if dump is not None and layer is None:
            return self._forward_dump(h, ple_in, pos, table, cap, mode, dump, caches)
        ws = self.workspace(B, T, cap, mode)
        if layer is None:
            bd.g4_stack_forward(self.desc, self.descs, h.data_ptr(), ple_in.data_ptr(), table, self.L, pos.data_ptr(),
                                B, T, mode, ws.data_ptr(), ws.numel(), _stream())
        else:
            bd.g4_layer_forward(self.desc, self.descs[layer], layer, h.data_ptr(), ple_in.data_ptr(), table, self.L,
                                pos.data_ptr(), B, T, mode, ws.data_ptr(), ws.numel(), _stream())
        return h

    def _forward_dump(self, h, ple_in, pos, table, cap, mode, path, caches):
        os.makedirs(path, exist_ok=True)
        B, T = h.shape[0], h.shape[1]

        def write(name, t):
            torch.cuda.synchronize()
            t.detach().to(torch.float32).contiguous().cpu().numpy().astype("<f4").tofile(os.path.join(path, name))

        write("l_in.f32", h)
        # cache row of token t of sequence b: position pos[b] + t, wrapped on a ring
        steps = torch.arange(T, device=h.device, dtype=torch.int64)
        for l in range(self.L):
            self.forward(h, ple_in, pos, table, cap, mode, layer=l)
            write(f"l{l:02d}.f32", h)
            if caches is not None and l in caches:
                k, v = caches[l]
                rows = pos.to(torch.int64)[:, None] + steps[None, :]
                if table[l].ring:
                    rows = rows % table[l].cap
                idx = rows[:, None, :, None].expand(B, k.shape[1], T, k.shape[3])
                write(f"l{l:02d}_k.f32", torch.gather(k, 2, idx))
                write(f"l{l:02d}_v.f32", torch.gather(v, 2, idx))
        return h


def capture(step, warmup=1):
    """Record `step` (a function issuing library calls on the current stream) as one HIP graph.

    The step runs `warmup` times first on a side stream, so that every buffer it needs (workspace,
    outputs) is allocated before capture; a replay then re-issues all of its kernels with one launch.
    Inputs and outputs are the same device buffers on every replay. Returns the torch CUDAGraph.
    """
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g

