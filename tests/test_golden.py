"""The CPU oracle against the hand-derived fixtures in tests/golden/.

Each fixture works one small case out by hand from the method's definitions
(the files give the derivation and the section of the SVG-EAR paper followed).
"""
import ast
import os

import numpy as np
import pytest

from oracle import svgear_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split("=", 1)
            out[k.strip()] = ast.literal_eval(v.strip())
    return out


@pytest.mark.parametrize("fill", ["skip", "stop"])
def test_route_worked_case(fill):
    g = load("route_skip_continue.txt")
    off = np.concatenate([[0], np.cumsum(g["sizes"])]).astype(np.int64)
    mask, lst, count, keys = O.route(np.asarray([g["ratios"]]), off, g["budget"], fill=fill)
    want = g[f"selected_{fill}"]
    assert sorted(np.nonzero(mask[0])[0].tolist()) == want
    assert lst[0, :count[0]].tolist() == want
    assert int(keys[0]) == g[f"used_{fill}"]


@pytest.mark.parametrize("fill", ["skip", "stop"])
def test_route_global_worked_case(fill):
    g = load("route_global.txt")
    qo = np.concatenate([[0], np.cumsum(g["q_sizes"])]).astype(np.int64)
    ko = np.concatenate([[0], np.cumsum(g["k_sizes"])]).astype(np.int64)
    mask, lst, count, keys, used = O.route_global(np.asarray(g["ratios"]), qo, ko, g["budget"],
                                                  fill=fill)
    want = g[f"selected_{fill}"]
    for c in range(2):
        assert np.nonzero(mask[c])[0].tolist() == want[c]
        assert lst[c, :count[c]].tolist() == want[c]
    assert keys.tolist() == g[f"keys_{fill}"]
    assert used == g[f"used_{fill}"]


def test_probe_worked_case():
    g = load("probe_two_keys.txt")
    keys = np.asarray(g["keys"])
    ratio, log_norm = O.probe(np.asarray([g["q_centroid"]]), keys, keys.mean(0, keepdims=True),
                              np.asarray([0, 2]), 1.0)
    assert ratio[0, 0] == pytest.approx(g["ratio"], rel=1e-13)
    assert log_norm[0] == pytest.approx(g["log_norm"], rel=1e-13)


def test_probe_values_worked_case():
    g = load("probe_values_two_keys.txt")
    keys, values = np.asarray(g["keys"]), np.asarray(g["values"])
    ratio, log_norm = O.probe_values(np.asarray([g["q_centroid"]]), keys,
                                     keys.mean(0, keepdims=True), values,
                                     values.mean(0, keepdims=True), np.asarray([0, 2]), 1.0)
    assert ratio[0, 0] == pytest.approx(g["ratio"], rel=1e-13)
    assert log_norm[0] == pytest.approx(g["log_norm"], rel=1e-13)


def test_attend_worked_case():
    g = load("attend_density_zero.txt")
    k, v = np.asarray(g["keys"]), np.asarray(g["values"])
    off = np.asarray(g["k_offsets"])
    kc = np.stack([k[off[i]:off[i + 1]].mean(0) for i in range(2)])
    vc = np.stack([v[off[i]:off[i + 1]].mean(0) for i in range(2)])
    out = O.attend(np.asarray([g["query"]]), k, v, np.asarray([0, 1]), off, kc, vc,
                   np.zeros((1, 2), np.uint8), 1.0)
    np.testing.assert_allclose(out[0], g["output"], rtol=1e-13)


def test_block_scores_worked_case():
    g = load("block_scores_two_centroids.txt")
    sc = O.block_scores(np.asarray(g["q_centroids"]), np.asarray(g["k_centroids"]),
                        np.asarray(g["k_offsets"]), 1.0)
    np.testing.assert_allclose(sc, np.asarray(g["scores"]), rtol=1e-13, atol=0)
