"""Planted mistakes in the oracle must make the pins fail (opt-in: G4_MUTATIONS=1, about two minutes).

Each case copies the oracle and the pins to a scratch directory, changes one line of the oracle's
arithmetic into a plausible mistake, and runs the pins there. A mistake that no pin catches means a
step of the oracle is not tied to anything outside itself. Runs on the CPU only.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name: (original text in the oracle, the planted mistake)
MUTATIONS = {
    "rope_sin_sign": ("a * c - b * s, b * c + a * s", "a * c + b * s, b * c - a * s"),
    "gqa_head_mod": ("g = h // grp", "g = h % nkv"),
    "ple_missing_inv_sqrt2": ("* (1.0 / math.sqrt(2.0))", ""),
    "window_off_by_one": ("vis &= j[None, :] > p[:, None] - window", "vis &= j[None, :] >= p[:, None] - window"),
    "ple_gate_on_xn2": ('g = gelu_tanh(h @ f64(lw["ple_gate"]).T)', 'g = gelu_tanh(xn2 @ f64(lw["ple_gate"]).T)'),
    "drop_attn_residual": ('h = h + rms_norm(a, lw["post_attn_norm"], eps)', 'h = rms_norm(a, lw["post_attn_norm"], eps)'),
    "v_norm_weighted": ('v = rms_norm((xn @ f64(value_weight(cfg, lw, layer)).T).reshape(B, T, nkv, hd), None, eps)',
                        'v = rms_norm((xn @ f64(value_weight(cfg, lw, layer)).T).reshape(B, T, nkv, hd), lw["k_norm"], eps)'),
    "k_eq_v_on_sliding_layers": ('if cfg.get("k_eq_v") and cfg["layer_types"][layer] != "S":', 'if cfg.get("k_eq_v"):'),
    "k_eq_v_value_is_rotated_k": ('v = rms_norm((xn @ f64(value_weight(cfg, lw, layer)).T).reshape(B, T, nkv, hd), None, eps)',
                                  'v = rms_norm(k, None, eps) if cfg.get("k_eq_v") and not sliding else '
                                  'rms_norm((xn @ f64(value_weight(cfg, lw, layer)).T).reshape(B, T, nkv, hd), None, eps)'),
    "full_kv_heads_ignored": ('return cfg.get("n_kv_heads_full") or cfg["n_kv_heads"]', 'return cfg["n_kv_heads"]'),
    "bidir_band_one_sided": ("vis &= np.abs(j[None, :] - p[:, None]) <= window",
                             "vis &= (j[None, :] - p[:, None] <= 0) & (p[:, None] - j[None, :] <= window)"),
    "bidir_band_strict": ("vis &= np.abs(j[None, :] - p[:, None]) <= window",
                          "vis &= np.abs(j[None, :] - p[:, None]) < window"),
    "bidir_flag_dropped": ("h = layer_forward(cfg, lw, l, srcs[l], h, ple_in[:, :, l, :], pos, caches, bidirectional=bidirectional)",
                           "h = layer_forward(cfg, lw, l, srcs[l], h, ple_in[:, :, l, :], pos, caches)"),
    "eps_outside_mean": ("y = x * (ms + eps) ** -0.5", "y = x * (ms ** -0.5 + eps)"),
    "partial_rotary_denominator": ("inv = float(theta) ** (-2.0 * j / hd)",
                                   "inv = float(theta) ** (-2.0 * j / (2 * max(n_rot, 1)))"),
    "ple_proj_unscaled": ("P = (e @ f64(W_pm).T) * (H ** -0.5)", "P = (e @ f64(W_pm).T)"),
    "gelu_on_up": ('act = gelu_tanh(xn2 @ f64(lw["w_gate"]).T) * (xn2 @ f64(lw["w_up"]).T)',
                   'act = (xn2 @ f64(lw["w_gate"]).T) * gelu_tanh(xn2 @ f64(lw["w_up"]).T)'),
    "layer_scalar_ignored": ('h = h * float(lw.get("layer_scalar", 1.0))', "h = h"),
    "q_norm_dropped": ('q = rope(rms_norm(q, lw["q_norm"], eps), pos[:, :, None], inv)',
                       "q = rope(rms_norm(q, None, eps), pos[:, :, None], inv)"),
    "embedding_unscaled": ('* math.sqrt(cfg["hidden"])', ""),
    "ple_table_unscaled": ("* math.sqrt(d)\n", "\n"),
    "route_first_same_type": ("src.append(cands[-1] if cands else l)", "src.append(cands[0] if cands else l)"),
    "softcap_unscaled": ("return cap * np.tanh(x / cap)", "return np.tanh(x / cap)"),
    "logits_without_final_norm": ("return softcap(rms_norm(h, out_norm, eps) @ f64(w_out).T, cap)",
                                  "return softcap(f64(h) @ f64(w_out).T, cap)"),
}

pytestmark = pytest.mark.skipif(os.environ.get("G4_MUTATIONS") != "1", reason="opt-in: set G4_MUTATIONS=1")


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_oracle_mistake_is_caught(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "g4_oracle.py")).read()
    a, b = MUTATIONS[name]
    assert src.count(a) >= 1, f"{name}: the original text is no longer in the oracle"
    for d in ("oracle", "tests", "synth"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d, ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "oracle" / "g4_oracle.py").write_text(src.replace(a, b))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"{name}: no pin failed\n{r.stdout[-2000:]}"


def test_unchanged_copy_passes(tmp_path):
    """The harness itself: the pins pass on an unchanged copy."""
    for d in ("oracle", "tests", "synth"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d, ignore=shutil.ignore_patterns("__pycache__"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
