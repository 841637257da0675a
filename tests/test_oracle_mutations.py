"""Planted mistakes in a copy of the oracle must each make its pins fail.

Each case copies the oracle with one plausible error (an off-by-one window,
a dropped term, a wrong sign or index, a wrong bound) and runs the pins of
tests/test_oracle.py against it in a child process; the run must fail.
This shows that the pins are sensitive to the errors an implementation of
the pages' mask, attention, gradients, RoPE and cache is likely to make.
The mistakes live only in the temporary copy, on the CPU.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "sepllm_oracle.py")

# (what goes wrong, text in the oracle, replacement)
MISTAKES = [
    ("window one token wider", "(i - j < n)", "(i - j <= n)"),
    ("separators dropped from the mask", "(j < a) | (i - j < n) | sep", "(j < a) | (i - j < n)"),
    ("dK without the softmax scale", "dk[b, kh, cols] += scale * (ds.T @ q[b, h, r0:r1])",
     "dk[b, kh, cols] += (ds.T @ q[b, h, r0:r1])"),
    ("wrong sign in dS", "ds = p * (dp - D)", "ds = p * (dp + D)"),
    ("RoPE rotates the other way", "np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s]",
     "np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s]"),
    ("RoPE frequencies halved in the exponent", "w = theta ** (-2.0 * np.arange(half) / d)",
     "w = theta ** (-1.0 * np.arange(half) / d)"),
    ("separator FIFO keeps one entry too many", "            if len(self.sep) > self.s:",
     "            if len(self.sep) > self.s + 1:"),
    ("window keeps one entry too many", "        if len(self.win) > self.n + self.P:",
     "        if len(self.win) > self.n + self.P + 1:"),
    ("query takes a rank past the cache", "            return np.arange(len(ordr)), len(ordr) - 1",
     "            return np.arange(len(ordr)), len(ordr)"),
    ("sinks listed as separators", "            if j >= a and f[b, j]:", "            if f[b, j]:"),
    ("LSE without the running maximum", "lse[b, h, r0:r1] = (mx + np.log(l))[:, 0]",
     "lse[b, h, r0:r1] = (np.log(l))[:, 0]"),
    ("tile band starts one key early", "            lo = max(0, q0 - n + 1)\n            m = mask_rows",
     "            lo = max(0, q0 - n)\n            m = mask_rows"),
    ("tile anchors counted from the sinks' end", "out[b, t] = (int(seen[:a].sum()), int(seen[a:].sum()), lo, q1)",
     "out[b, t] = (int(seen[:a].sum()), int(seen[a + 1:].sum()), lo, q1)"),
]


def _run_pins(tmp_path, oracle_src):
    """Runs the oracle's pins on a copy of the tree whose oracle is oracle_src."""
    for d in ("oracle", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__", "*.pyc"))
    pkg = tmp_path / "separator_kv_cache_amd"
    pkg.mkdir()
    for f in ("__init__.py", "synth.py"):
        shutil.copy(os.path.join(ROOT, "separator_kv_cache_amd", f), pkg / f)
    (tmp_path / "oracle" / "sepllm_oracle.py").write_text(oracle_src)
    return subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle.py", "-x", "-q", "-m", "not gpu",
                           "-p", "no:cacheprovider"], cwd=tmp_path, capture_output=True, text=True, timeout=900)


def test_unchanged_copy_passes(tmp_path):
    """The harness itself: the copied tree with the oracle as it stands passes."""
    r = _run_pins(tmp_path, open(ORACLE).read())
    assert r.returncode == 0, f"{r.stdout[-2000:]}\n{r.stderr[-2000:]}"


@pytest.mark.parametrize("what,old,new", MISTAKES, ids=[m[0].replace(" ", "-") for m in MISTAKES])
def test_planted_mistake_fails_a_pin(what, old, new, tmp_path):
    src = open(ORACLE).read()
    assert src.count(old) == 1, f"the text to change is not in the oracle once: {old!r}"
    r = _run_pins(tmp_path, src.replace(old, new))
    # 1: tests ran and one failed (a broken import would be 2, a collection error)
    assert r.returncode == 1, f"the pins did not catch: {what}\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}"
