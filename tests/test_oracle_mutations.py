"""Strength of the oracle's pins: each case plants one plausible mistake in a scratch copy of
the oracle (a wrong log base, a count off by one block, a mean with the wrong denominator, the
tie band measured against the wrong distance, ...), runs the pins of test_oracle_pins.py
against that copy in a child process, and requires at least one of them to fail. The product
oracle is never modified; every mutation touches only the copy."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (what the mistake is, exact source text, replacement)
MUTATIONS = [
    ("top-two gap over the smaller distance",
     "gap = np.where(d2 > 0, (d2 - d1) / d2, 0.0)", "gap = np.where(d1 > 0, (d2 - d1) / d1, 0.0)"),
    ("tie band ten times wider", "TIE_BAND = 1e-4", "TIE_BAND = 1e-3"),
    ("band membership against the smallest distance",
     "return (d - d1) <= TIE_BAND * d\n", "return (d - d1) <= TIE_BAND * d1\n"),
    ("key variance around the cached centroid",
     '"kvar": key_variance(K, a, mu1),', '"kvar": key_variance(K, a, mu0),'),
    ("log2 of the count as the cluster bias",
     "np.log(counts[b, cs].astype(np.float64))", "np.log2(counts[b, cs].astype(np.float64))"),
    ("the raw count as the cluster bias",
     "np.log(counts[b, cs].astype(np.float64))", "(counts[b, cs].astype(np.float64))"),
    ("inside and outside of the exact blocks swapped in the counts",
     "        outside = mask[b][blk] == 0\n", "        outside = mask[b][blk] != 0\n"),
    ("key block index off by one",
     "    blk = np.arange(n_tok) // (block if kblock is None else kblock)",
     "    blk = (np.arange(n_tok) + 1) // (block if kblock is None else kblock)"),
    ("mean with a wrong denominator",
     "    mu1[has] = ksum[has] / sizes[has, None]", "    mu1[has] = ksum[has] / (sizes[has, None] + 1)"),
    ("exact logits without the scale",
     "        logits = np.concatenate([scale * (q @ K[ex].T), comp], axis=1)",
     "        logits = np.concatenate([(q @ K[ex].T), comp], axis=1)"),
    ("compensation values dropped",
     "        vals = np.concatenate([V[ex], vbar[cs]], axis=0)",
     "        vals = np.concatenate([V[ex], 0 * vbar[cs]], axis=0)"),
    ("empty cluster loses its cached centroid", "    mu1 = mu0.copy()", "    mu1 = np.zeros_like(mu0)"),
    ("ties to the highest index",
     "        order = np.lexsort((cols, dx, rows))", "        order = np.lexsort((-cols, dx, rows))"),
]


def _pins_on_a_copy(tmp_path, old=None, new=None):
    """Run the pins against a scratch copy of the oracle, with `old` replaced by `new`."""
    for d in ("oracle", "datagen", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path / "pytest.ini")
    if old is not None:
        path = tmp_path / "oracle" / "decoupattn_oracle.py"
        src = path.read_text()
        assert src.count(old) >= 1, f"the mutation site is gone: {old!r}"
        path.write_text(src.replace(old, new, 1))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q",
                           "-p", "no:cacheprovider", "-x"],
                          cwd=tmp_path, capture_output=True, text=True, env=env, timeout=600)


def test_pins_pass_on_an_unmodified_copy(tmp_path):
    r = _pins_on_a_copy(tmp_path)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("what,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_a_planted_mistake(tmp_path, what, old, new):
    r = _pins_on_a_copy(tmp_path, old, new)
    # exit 1: some pin failed (an import or collection error would be 2 and does not count)
    assert r.returncode == 1, (f"planted mistake not caught ({what}): pytest exit {r.returncode}\n"
                               + r.stdout[-2000:])
