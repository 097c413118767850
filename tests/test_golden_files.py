"""Consistency of the stored oracle samples used by the full-size GPU tests (CPU only)."""
import glob
import hashlib
import json
import os
import re

import numpy as np
import pytest

from wan_inputs import get_config

HERE = os.path.dirname(os.path.abspath(__file__))
FILES = sorted(glob.glob(os.path.join(HERE, "golden", "forward_cfg*_L*.npz")))
HASHES = json.load(open(os.path.join(HERE, "golden", "oracle_hashes.json")))


def oracle_source_hash() -> str:
    with open(os.path.join(os.path.dirname(HERE), "oracle", "wan_oracle.py"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def test_hash_list_names_the_current_oracle():
    """Editing the oracle forces a decision on the stored goldens (keep them as equivalent, or regenerate)."""
    assert HASHES["current"] == oracle_source_hash()


@pytest.mark.parametrize("path", FILES, ids=[os.path.basename(f) for f in FILES])
def test_golden_file_is_consistent(path):
    m = re.match(r"forward_cfg(\d+)_L(\d+)\.npz", os.path.basename(path))
    cfg = get_config(int(m.group(1))).with_layers(int(m.group(2)))
    g = np.load(path)
    shape = tuple(int(s) for s in g["shape"])
    assert shape == cfg.out_shape
    n = int(np.prod(shape))
    idx, val = g["index"], g["value"]
    assert idx.dtype == np.int64 and idx.ndim == 1 and idx.size == val.size
    assert np.all(np.diff(idx) > 0) and idx[0] == 0 and idx[-1] == n - 1
    assert np.array_equal(idx[:64], np.arange(64)) and np.array_equal(idx[-64:], np.arange(n - 64, n))
    assert np.isfinite(val).all()
    sumsq = float(g["sumsq"][0])
    assert sumsq >= float((val * val).sum())
    # the sampled positions are a uniform random subset: their mean square estimates the whole output's
    ms_all, ms_sample = sumsq / n, float((val * val).mean())
    assert 0.8 < ms_sample / ms_all < 1.25
    tag = str(g["oracle"][0])
    assert tag == HASHES["current"] or tag in HASHES["equivalent"], (os.path.basename(path), tag)
