"""Pure-Python brute force for tiny inputs: an independent check of the oracle.

Written with explicit loops and a different formulation wherever one exists (RoPE as a complex
rotation, softmax as explicit sums with math.exp, matvecs as loops over a row-major weight), so a
dropped term, wrong sign, transposed operand or wrong head index in the numpy oracle shows up as a
mismatch. Sizes must stay tiny (hidden <= 64, T <= 8).
"""
import cmath
import math


def matvec(W, x):
    """W is a list of rows (out x in); returns W x."""
    return [sum(W[r][c] * x[c] for c in range(len(x))) for r in range(len(W))]


def rms(x, w, eps):
    n = len(x)
    ms = 0.0
    for v in x:
        ms += v * v
    ms /= n
    inv = 1.0 / math.sqrt(ms + eps)
    return [x[i] * inv * (1.0 if w is None else w[i]) for i in range(n)]


def gelu(x):
    return 0.5 * x * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def rope_complex(x, pos, theta, n_rot):
    """Rotate pairs (x_j, x_{j+h}) as the complex number x_j + i x_{j+h} times exp(i pos w_j)."""
    hd = len(x)
    h = hd // 2
    out = list(x)
    for j in range(h):
        w = theta ** (-2.0 * j / hd) if j < n_rot else 0.0
        z = complex(x[j], x[j + h]) * cmath.exp(1j * pos * w)
        out[j], out[j + h] = z.real, z.imag
    return out


def attend(qh, keys, vals):
    """softmax(q . k_j) weighted sum of v_j over the given (already selected) keys."""
    s = [sum(qh[d] * k[d] for d in range(len(qh))) for k in keys]
    m = max(s)
    e = [math.exp(v - m) for v in s]
    z = sum(e)
    return [sum(e[j] * vals[j][d] for j in range(len(keys))) / z for d in range(len(vals[0]))]


def layer(cfg, lw, layer_idx, own_kv, h_rows, ple_rows, positions, cache, bidirectional=False):
    """One layer for one sequence. h_rows: list of T lists (H); cache: dict with 'k','v' lists
    indexed [g][pos] -> list(hd) (mutated when own_kv). Returns the new list of rows.
    bidirectional: the encoder's mask, every key of the call within W positions on either side (sliding)
    or every key of the call (full)."""
    eps, nh = cfg["eps"], cfg["n_heads"]
    sliding = cfg["layer_types"][layer_idx] == "S"
    # variants: a full layer may have its own KV head count, and with K=V its V comes from the K weight
    nkv = cfg["n_kv_heads"] if sliding or not cfg.get("n_kv_heads_full") else cfg["n_kv_heads_full"]
    wv = lw["wk"] if (cfg.get("k_eq_v") and not sliding) else lw["wv"]
    hd = cfg["head_dim_swa"] if sliding else cfg["head_dim_full"]
    theta = cfg["theta_swa"] if sliding else cfg["theta_full"]
    n_rot = hd // 2 if sliding else int(hd * cfg["partial_rotary"] / 2)
    grp = nh // nkv
    W = cfg["window"]
    T = len(h_rows)
    # projections for every token first (keys of later tokens must exist before attention of none:
    # causal masking only ever looks back, so a token-by-token order gives the same result)
    qs, out = [], []
    for t in range(T):
        xn = rms(h_rows[t], lw["input_norm"], eps)
        q = matvec(lw["wq"], xn)
        heads = []
        for hh in range(nh):
            qh = rms(q[hh * hd:(hh + 1) * hd], lw["q_norm"], eps)
            heads.append(rope_complex(qh, positions[t], theta, n_rot))
        qs.append(heads)
        if own_kv:
            k = matvec(lw["wk"], xn)
            v = matvec(wv, xn)
            for g in range(nkv):
                kg = rms(k[g * hd:(g + 1) * hd], lw["k_norm"], eps)
                cache["k"][g][positions[t]] = rope_complex(kg, positions[t], theta, n_rot)
                cache["v"][g][positions[t]] = rms(v[g * hd:(g + 1) * hd], None, eps)
    for t in range(T):
        i = positions[t]
        if bidirectional:
            sel = [j for j in positions if not sliding or abs(i - j) <= W]
        else:
            sel = list(range(max(0, i - W + 1) if sliding else 0, i + 1))
        o = []
        for hh in range(nh):
            g = hh // grp
            keys = [cache["k"][g][j] for j in sel]
            vals = [cache["v"][g][j] for j in sel]
            o.extend(attend(qs[t][hh], keys, vals))
        a = matvec(lw["wo"], o)
        an = rms(a, lw["post_attn_norm"], eps)
        h = [h_rows[t][c] + an[c] for c in range(len(an))]
        xn2 = rms(h, lw["pre_ffn_norm"], eps)
        gt = matvec(lw["w_gate"], xn2)
        up = matvec(lw["w_up"], xn2)
        act = [gelu(gt[c]) * up[c] for c in range(len(gt))]
        f = rms(matvec(lw["w_down"], act), lw["post_ffn_norm"], eps)
        h = [h[c] + f[c] for c in range(len(h))]
        pg = matvec(lw["ple_gate"], h)
        mixed = [gelu(pg[c]) * ple_rows[t][c] for c in range(len(pg))]
        pn = rms(matvec(lw["ple_proj"], mixed), lw["post_ple_norm"], eps)
        s = lw.get("layer_scalar", 1.0)
        out.append([(h[c] + pn[c]) * s for c in range(len(h))])
    return out


def ple_row(cfg, tok, E, Tab, Wpm, ple_norm):
    """(h0 row, per-layer inputs [L][d]) for one token id."""
    H, L, d, eps = cfg["hidden"], cfg["n_layers"], cfg["ple_dim"], cfg["eps"]
    e = [E[tok][c] * math.sqrt(H) for c in range(H)] if 0 <= tok < cfg["vocab"] else [0.0] * H
    P = [v / math.sqrt(H) for v in matvec(Wpm, e)]
    rows = []
    for l in range(L):
        pn = rms(P[l * d:(l + 1) * d], ple_norm, eps)
        tab = [Tab[tok][l * d + j] * math.sqrt(d) if 0 <= tok < cfg["ple_vocab"] else 0.0 for j in range(d)]
        rows.append([(pn[j] + tab[j]) / math.sqrt(2.0) for j in range(d)])
    return e, rows
