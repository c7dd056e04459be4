"""The oracle's pins must catch plausible slips: each case plants one mistake
in a temporary copy of the oracle (on the CPU) and expects the pin suite to fail."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    "gate_up_swapped": ('gate, up = gu[:, :p.ffn], gu[:, p.ffn:]', 'up, gate = gu[:, :p.ffn], gu[:, p.ffn:]'),
    "gqa_interleaved": ('j = h // group', 'j = h % n_kv'),
    "v_normed": ('v = (xn @ f64(w["wv"]).T).reshape(R, nkv, d)',
                 'v = rms_norm((xn @ f64(w["wv"]).T).reshape(R, nkv, d), w["k_norm"], eps)'),
    "eps_outside_root": ('return x / np.sqrt(ms + eps) * f64(gain)', 'return x / (np.sqrt(ms) + eps) * f64(gain)'),
    "rope_sign": ('np.concatenate([a * c - b * s, a * s + b * c]', 'np.concatenate([a * c + b * s, -a * s + b * c]'),
    "rope_frequency": ('-2.0 * i / d', '-1.0 * i / d'),
    "no_score_scale": ('/ np.sqrt(d)', '/ 1.0'),
    "residual_from_normed": ('h = x + o @ f64(w["wo"]).T', 'h = xn + o @ f64(w["wo"]).T'),
    "ffn_norm_of_x": ('hn = rms_norm(hs, w["ffn_norm"], eps)', 'hn = rms_norm(x[rows], w["ffn_norm"], eps)'),
    "causal_extent_short": ('positions[r] + 1).reshape(-1)', 'positions[r]).reshape(-1)'),
    "q_norm_uses_k_gain": ('q = rope_neox(rms_norm(q, w["q_norm"], eps)', 'q = rope_neox(rms_norm(q, w["k_norm"], eps)'),
    "argmax_highest_index": ('return int(np.argmax(l32))', 'return int(len(l32) - 1 - np.argmax(l32[::-1]))'),
    "silu_sign": ('return z / (1.0 + np.exp(-z))', 'return z / (1.0 + np.exp(z))'),
    "down_rows_permuted": ('(silu(gate) * up) @ f64(w["w_down"]).T', '(silu(gate) * up) @ f64(w["w_down"]).T[::-1]'),
    "inject_keep_on_audio": ('return rows * f64(keep)[:, None] + f64(audio_dense)',
                             'return rows + f64(audio_dense) * f64(keep)[:, None]'),
    "loop_context_off_by_one": ('cur + 1 <= n_ctx', 'cur + 1 < n_ctx'),
    "loop_budget_excludes_first": ('len(tokens) < max_new', 'len(tokens) <= max_new'),
    "margin_to_smallest": ('second = np.max(l)', 'second = np.min(np.where(np.isinf(l), np.inf, l))'),
    "margin_keeps_nan": ('l[np.isnan(l)] = -np.inf\n    i = int(np.argmax(l))',
                         'i = int(np.argmax(l))'),
}


def run_pins_on_copy(tmp_path, old=None, new=None, name=""):
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in ["conftest.py", "test_oracle_pins.py"]:
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    src = tmp_path / "oracle" / "decoder.py"
    text = src.read_text()
    if old is not None:
        assert text.count(old) >= 1, name
        src.write_text(text.replace(old, new))
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_oracle_pins.py"],
                          cwd=tmp_path, capture_output=True, text=True, timeout=300)


def test_unmutated_copy_passes(tmp_path):
    """Control: the copied pin suite passes on the unchanged oracle, so a failure
    below comes from the planted mistake and not from the copy itself."""
    r = run_pins_on_copy(tmp_path)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    r = run_pins_on_copy(tmp_path, old, new, name)
    assert r.returncode == 1, f"planted mistake {name} was not caught:\n{r.stdout[-2000:]}"
