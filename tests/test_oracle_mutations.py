"""Planted mistakes in a copy of the oracle must be caught by its pins (CPU only).

Each mutation is a plausible slip (a sign, an index, a dropped term, a swapped
operand). The oracle pin tests are re-run in a subprocess with the mutated
copy first on sys.path; the run must fail.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("forward.py", "a * c - b * s, b * c + a * s", "a * c + b * s, b * c - a * s"),        # RoPE direction
    ("forward.py", "qg = q[i].reshape(m.Hkv, G, m.dh)",
     "qg = q[i].reshape(G, m.Hkv, m.dh).transpose(1, 0, 2)"),                                # GQA head map
    ("forward.py", "[: p + 1]", "[: p]"),                                                       # causal limit
    ("forward.py", "x = x + o.reshape", "x = o.reshape"),                                       # dropped residual
    ("forward.py", "/ np.sqrt(m.dh)", "/ m.dh"),                                                # attention scale
    ("forward.py", "(silu(gate) * up)", "(silu(up) * gate)"),                                   # gate/up swap
    ("forward.py", "keepdims=True) + eps)", "keepdims=True))"),                                 # RMSNorm eps
    ("forward.py", "kc[local(slots)] = k", "pass"),                                             # no KV write
    ("expand.py", "ids[o] = tid[j + 1]", "ids[o] = tid[j]"),                                   # input shift
    ("expand.py", "pos[o] = p_ntp + mm", "pos[o] = p_ntp + mm - 1"),                           # MASK positions
    ("expand.py", "slot[o] = -1 if is_rej[o] else _slot(bt[r], int(pos[o]), block_size)",
     "slot[o] = _slot(bt[r], int(pos[o]), block_size)"),                                       # -1 for rejected
    ("expand.py", "new_idx[r * K] = out_start + v - 1", "new_idx[r * K] = out_start + v"),     # NTP index
    ("forward.py", 'kvf["k"][l][sl] = kk', "pass"),                                           # AR: no KV carry-over
    ("expand.py", "pos_prev[new_idx[i]] + 1 for i in last", "pos_prev[new_idx[i]] + 2 for i in last"),  # AR position
    ("forward.py", 'nxt["hidden_d"] = res["hidden_out"] if', 'nxt["hidden_d"] = 0 * res["hidden_out"] if'),  # AR feedback
    ("partition.py", "seg[d][p] = dep", "seg[d][p] = _segment_of_index(b, p)"),             # deeper depths by index
    ("partition.py", "dep = seg[d - 1][p - 1] if", "dep = seg[d - 1][p] if"),                  # wrong dependency
    ("partition.py", "for p in range(b[s]) if keep[0][p]", "for p in range(b[s] - 1) if keep[0][p]"),  # context short
    ("partition.py", "seg[1][p] = _segment_of_index(b, p)", "seg[1][p] = _segment_of_index(b, p - 1)"),  # depth 1 index
    ("partition.py", "            else:\n                bad = True\n    owned", "            else:\n                pass\n    owned"),  # broken chain unreported
    ("rounds.py", "p_ntp = int(pos[nti[r * K]])", "p_ntp = int(pos[nti[r * K]]) + 1"),          # window one position late
    ("rounds.py", "ids.append(int(nxt[r]))", "ids.append(int(d[r, 0]))"),                     # sampled token dropped
    ("rounds.py", '"num_rejected": (K - a).astype(np.int32)', '"num_rejected": a.astype(np.int32)'),  # rejected count
    ("rounds.py", 'kvf["k"][l][sl] = kk', "pass"),                                            # no KV carry-over
    ("fp8.py", "(frac == 0.5) & (lo % 2 == 1)", "(frac == 0.5) & (lo % 2 == 0)"),             # ties to odd
    ("fp8.py", "E4M3_MAX = 448.0", "E4M3_MAX = 480.0"),                                        # wrong saturation bound
    ("fp8.py", "(1.0 + m / 8.0) * np.exp2(e - 7.0)", "(1.0 + m / 8.0) * np.exp2(e - 8.0)"),    # exponent bias
    ("forward.py", 'k = fp8_roundtrip(k, float(kv_fp8["k_scale"][l]))', "k = fp8_roundtrip(k, 1.0)"),  # K scale ignored
]

PIN_FILES = {
    "partition.py": ["tests/test_oracle_partition.py"],
    "rounds.py": ["tests/test_oracle_rounds.py"],
    "fp8.py": ["tests/test_oracle_fp8.py"],
}
DEFAULT_PINS = ["tests/test_oracle_expand.py", "tests/test_oracle_forward.py", "tests/test_oracle_ar.py",
                "tests/test_oracle_fp8.py"]


@pytest.mark.parametrize("fname,old,new", MUTATIONS, ids=[m[2][:24] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, fname, old, new):
    dst = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("__pycache__", "*.so", "*.o"))
    src = (dst / fname).read_text()
    assert src.count(old) == 1, f"mutation anchor not unique in {fname}: {old}"
    (dst / fname).write_text(src.replace(old, new))
    env = dict(os.environ, PD_ORACLE_MUTANT_DIR=str(tmp_path), PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_FILES.get(fname, DEFAULT_PINS)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "the oracle pins did not catch: " + new + "\n" + r.stdout[-2000:]
