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
    m = re.match(r"forward_cfg(\d+)(i?)_L(\d+)\.npz", os.path.basename(path))
    cfg = get_config(int(m.group(1))).with_layers(int(m.group(3)))
    g = np.load(path)
    if m.group(2):
        assert int(g["image_len"][0]) > 0
        cfg = cfg.replace(image_len=int(g["image_len"][0]))
    shape = tuple(int(s) for s in g["shape"])
    assert shape == cfg.out_shape
    tag = str(g["oracle"][0])
    assert tag == HASHES["current"] or tag in HASHES["equivalent"], (os.path.basename(path), tag)
    if "rows_only" in g.files:
        # sampled token rows of a one-block stack: every proj_out value of each row, first and last 32 tokens in
        tok, z = g["tokens"], g["z"]
        assert cfg.num_layers == 1
        assert tok.ndim == 1 and np.all(np.diff(tok) > 0) and tok[0] == 0 and tok[-1] == cfg.tokens - 1
        assert np.array_equal(tok[:32], np.arange(32)) and np.array_equal(tok[-32:], np.arange(cfg.tokens - 32, cfg.tokens))
        assert z.shape == (cfg.batch, tok.size, cfg.out_k) and np.isfinite(z).all()
        assert 0.1 < float(np.sqrt((z.astype(np.float64) ** 2).mean())) < 10.0
        return
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


def test_row_positions_follow_the_oracle_unpatchify():
    """The map from a row-only golden's z to output positions, against the oracle's own unpatchify."""
    from golden_index import rows_positions
    from oracle import wan_oracle as O

    cfg = get_config(1).replace(batch=2, frames=3, height=4, width=6, out_channels=3)
    rng = np.random.default_rng(0)
    z = rng.standard_normal((2, cfg.tokens, cfg.out_k))
    out = O.unpatchify(z, cfg.frames, cfg.height, cfg.width, cfg.out_channels)
    tokens = np.array([0, 2, 5, cfg.tokens - 1])
    pos = rows_positions(cfg, tokens)
    assert np.array_equal(out.reshape(-1)[pos], z[:, tokens])
