"""The pins must catch plausible mistakes: each case plants one in a temporary
copy of the oracle (on the CPU, never in the repository) and expects the pin
suite to fail on the mutated copy."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (file, original text, planted mistake)
MUTATIONS = {
    "rope_sign": ("csa_oracle.py", "z = z * np.exp(1j * ang)", "z = z * np.exp(-1j * ang)"),
    "rope_half_split": ("csa_oracle.py",
                        "z = x[..., D - rope_dim::2] + 1j * x[..., D - rope_dim + 1::2]",
                        "z = x[..., D - rope_dim:D - rope_dim // 2] + 1j * x[..., D - rope_dim // 2:]"),
    "rope_freq": ("csa_oracle.py", "return base ** (-2.0 * j / rope_dim)",
                  "return base ** (-1.0 * j / rope_dim)"),
    "yarn_ramp_direction": ("csa_oracle.py",
                            "return theta * (1.0 - r) + (theta / base.factor) * r",
                            "return theta * r + (theta / base.factor) * (1.0 - r)"),
    "yarn_correction_half": ("csa_oracle.py",
                             "return rope_dim * math.log(context / (2.0 * math.pi * n_turns)) / (2.0 * math.log(base))",
                             "return rope_dim * math.log(context / (2.0 * math.pi * n_turns)) / math.log(base)"),
    "yarn_lo_rounding": ("csa_oracle.py", "lo = math.floor(yarn_correction_index(",
                         "lo = math.ceil(yarn_correction_index("),
    "yarn_betas_swapped": ("csa_oracle.py",
                           "lo = math.floor(yarn_correction_index(base.beta_fast,",
                           "lo = math.floor(yarn_correction_index(base.beta_slow,"),
    "pool_axis": ("csa_oracle.py", "alpha = e / e.sum(axis=0, keepdims=True)",
                  "alpha = e / e.sum(axis=1, keepdims=True)"),
    "pool_window_edge": ("csa_oracle.py", "return max((w - overlap) * ratio, p0), (w + 1) * ratio",
                         "return max((w - overlap) * ratio + 1, p0), (w + 1) * ratio"),
    "pool_rope_pos": ("csa_oracle.py", "w * ratio,\n                                 rope_dim",
                      "(w + 1) * ratio - 1,\n                                 rope_dim"),
    "visibility": ("csa_oracle.py", "return range(p0 // ratio, (t + 1) // ratio)",
                   "return range(p0 // ratio, t // ratio)"),
    "window_edge": ("csa_oracle.py", "return range(max(p0, t - window + 1), t + 1)",
                    "return range(max(p0, t - window), t + 1)"),
    "relu_place": ("csa_oracle.py",
                   "return (np.asarray(wi_t, np.float64)[:, None] * np.maximum(dots, 0.0)).sum(axis=0)",
                   "return np.maximum(np.asarray(wi_t, np.float64)[:, None] * dots, 0.0).sum(axis=0)"),
    "tie_break": ("csa_oracle.py", "order = np.lexsort((np.arange(n), -s))",
                  "order = np.lexsort((-np.arange(n), -s))"),
    "sink_dropped": ("csa_oracle.py", "Z = Z + np.exp(sinks - M)", "Z = Z + 0.0 * np.exp(sinks - M)"),
    "no_unrotate": ("csa_oracle.py", "o = rope(o, t, rope_dim, base, -1)",
                    "o = rope(o, t, rope_dim, base, +1)"),
    "query_unrotated": ("csa_oracle.py", "q = round_to(rope(q_t, t, rope_dim, base, +1), dtype)",
                        "q = round_to(np.asarray(q_t, np.float64), dtype)"),
    "oproj_group_order": ("csa_oracle.py", "xg = x.reshape(T, G, ig)",
                          "xg = x.reshape(T, ig, G).transpose(0, 2, 1)"),
    "oproj_weight_transposed": ("csa_oracle.py",
                                "wa = np.asarray(w_a, dtype=np.float64).reshape(G, R, ig)",
                                "wa = np.asarray(w_a, dtype=np.float64).reshape(G, ig, R).transpose(0, 2, 1)"),
    "oproj_no_intermediate_rounding": ("csa_oracle.py", "    y = round_to(y, dtype)\n",
                                       "    y = y\n"),
    "proj_norm_axis": ("csa_oracle.py",
                       "out = y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)",
                       "out = y / np.sqrt(np.mean(y * y, axis=0, keepdims=True) + eps)"),
    "proj_segment_order": ("csa_oracle.py",
                           "cuts = np.cumsum([0, sz.q_lora, sz.head_dim, sz.comp,",
                           "cuts = np.cumsum([0, sz.head_dim, sz.q_lora, sz.comp,"),
    "proj_latent_unrounded": ("csa_oracle.py",
                              "yq = round_to(latent @ np.asarray(w_q, dtype=np.float64).T, dtype)",
                              "yq = round_to(_rms_rows(seg[0], g_qa, eps) @ np.asarray(w_q, dtype=np.float64).T, dtype)"),
    "round_bits": ("csa_oracle.py", "q = np.ldexp(np.round(np.ldexp(x, 8 - e)), e - 8)",
                   "q = np.ldexp(np.round(np.ldexp(x, 9 - e)), e - 9)"),
    "round_double": ("csa_oracle.py", "_, e = np.frexp(x)",
                     "x = x.astype(np.float32).astype(np.float64)\n    _, e = np.frexp(x)"),
}


def _run_mutant(name, tmp_root):
    fname, old, new = MUTATIONS[name]
    d = os.path.join(tmp_root, name)
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"))
    shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(d, "synth"))
    os.makedirs(os.path.join(d, "tests"))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(d, "tests", "golden"))
    shutil.copy(os.path.join(ROOT, "tests", "test_oracle_pins.py"), os.path.join(d, "tests"))
    shutil.copy(os.path.join(ROOT, "tests", "conftest.py"), os.path.join(d, "tests"))
    path = os.path.join(d, "oracle", fname)
    src = open(path).read()
    assert src.count(old) == 1, f"mutation {name} does not match the oracle source"
    open(path, "w").write(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(d, "tests", "test_oracle_pins.py")],
                       cwd=d, capture_output=True, text=True, timeout=300)
    return r.returncode


def test_every_planted_mistake_fails_a_pin(tmp_path):
    names = sorted(MUTATIONS)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        codes = dict(zip(names, ex.map(lambda n: _run_mutant(n, str(tmp_path)), names)))
    # exit code 1 means tests ran and at least one failed (not a collection error)
    survivors = [n for n, c in codes.items() if c != 1]
    assert not survivors, f"mutations not caught by a failing pin: {survivors} {codes}"
