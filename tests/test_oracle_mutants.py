"""Planted mistakes in the oracle are caught by its pins.

Each case copies the oracle package to a temporary directory, plants one plausible
mistake in ``attention.py`` (a textual edit), and runs the pin suite
``tests/test_oracle.py`` against the copy in a fresh process; the suite must fail.  An
unmodified copy must pass, so a broken harness cannot make every mistake look caught.
CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in oracle/attention.py, replacement)
MUTANTS = [
    ("strict_causal_mask", "visible = np.arange(L)[None, :] <= np.asarray(positions)[:, None]",
     "visible = np.arange(L)[None, :] < np.asarray(positions)[:, None]"),
    ("dropped_scale", "s = (q @ K.T) * float(scale)", "s = (q @ K.T)"),
    ("gqa_heads_interleaved", "            g = h // G\n", "            g = h % Hkv\n"),
    ("gather_rows_reversed", "return pool[blocks, :, j % BLOCK_SIZE, :]",
     "return pool[blocks, :, BLOCK_SIZE - 1 - j % BLOCK_SIZE, :]"),
    ("missing_prefix_offset", "pos = P[b] + np.arange(C)", "pos = np.arange(C)"),
    ("normalised_by_max", "den = w.sum(axis=1, keepdims=True)", "den = w.max(axis=1, keepdims=True)"),
    ("decode_position_off_by_one", "V[:, h // G], [n - 1], scale)", "V[:, h // G], [n - 2], scale)"),
    ("chunk_k_read_from_v", "Ks = decode_bits(k_self, dtype)", "Ks = decode_bits(v_self, dtype)"),
    ("bf16_payload_shift", "(bits.astype(np.uint32) << 16)", "(bits.astype(np.uint32) << 15)"),
    ("slot_row_off_by_one", "int(slot) // BLOCK_SIZE, int(slot) % BLOCK_SIZE",
     "int(slot) // BLOCK_SIZE, (int(slot) + 1) % BLOCK_SIZE"),
    ("out_of_pool_slot_written", "if slot < 0 or slot >= n_slots:", "if slot < 0:"),
    ("lse_merge_log_dropped", "lse = np.where(den > 0, Mf + np.log(safe), -np.inf)",
     "lse = np.where(den > 0, Mf + safe, -np.inf)"),
]


def _run_pins(tmp_path, old=None, new=None):
    dst = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("__pycache__"))
    if old is not None:
        path = dst / "attention.py"
        src = path.read_text()
        assert src.count(old) >= 1, f"mutation text not found: {old!r}"
        path.write_text(src.replace(old, new))
    # the copy shadows the repository's oracle: it sits in the working directory (first
    # on sys.path) and the repository root is on PYTHONPATH for everything else
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT]),
               PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=300)
    return r


def test_unmodified_copy_passes(tmp_path):
    r = _run_pins(tmp_path)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    # and the copy is what the pins imported
    r = subprocess.run([sys.executable, "-c", "import oracle; print(oracle.__file__)"],
                       cwd=str(tmp_path), env=dict(os.environ, PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT])),
                       capture_output=True, text=True, timeout=60)
    assert r.stdout.strip().startswith(str(tmp_path)), r.stdout


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    r = _run_pins(tmp_path, old, new)
    assert r.returncode != 0, f"the pins did not catch {name}"
