"""CPU tests of the seeded input generator (no method arithmetic here)."""
import json
import os

import numpy as np
import pytest

import synth
from synth.workloads import CONFIGS

GOLD = os.path.join(os.path.dirname(__file__), "golden")
GAMMA = 0x9E3779B97F4A7C15
M64 = (1 << 64) - 1


def test_splitmix64_reference_vector():
    ref = json.load(open(os.path.join(GOLD, "splitmix64_seed1234567.json")))
    s = ref["state"]
    got = []
    for _ in ref["outputs"]:
        s = (s + GAMMA) & M64
        got.append(str(synth.lib().synth_mix64(s)))
    assert got == ref["outputs"]


def test_normal_is_counter_based_and_deterministic():
    a = synth.normal(7, 3, 0, 1001)
    b = synth.normal(7, 3, 0, 1001)
    assert np.array_equal(a, b)
    # any sub-range, odd or even start, gives the same elements
    for start, n in ((1, 10), (5, 1), (500, 501), (999, 2)):
        assert np.array_equal(synth.normal(7, 3, start, n), a[start:start + n])
    one = [synth.lib().synth_normal_one(7, 3, i) for i in (0, 1, 2, 999, 1000)]
    assert np.array_equal(np.array(one), a[[0, 1, 2, 999, 1000]])
    # different streams / seeds differ
    assert not np.array_equal(a, synth.normal(7, 4, 0, 1001))
    assert not np.array_equal(a, synth.normal(8, 3, 0, 1001))


def test_normal_moments():
    x = synth.normal(11, 2, 0, 2_000_000)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    # Box-Muller pair members are uncorrelated
    assert abs(np.corrcoef(x[0::2], x[1::2])[0, 1]) < 5e-3


def _bf16_neighbours(x):
    """The two bf16 values bracketing float64 x, by brute force over bit patterns."""
    f = np.float32(x)
    bits = int(np.array(f).view(np.uint32)) >> 16
    cands = [(bits + o) & 0xFFFF for o in (-1, 0, 1)]
    vals = [float(np.array(c << 16, np.uint32).view(np.float32)) for c in cands]
    return list(zip(cands, vals))


def test_bf16_rounding_is_nearest_even_from_double():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=2000), rng.normal(size=200) * 1e-20,
                        rng.normal(size=200) * 1e20])
    # exact halfway cases between bf16 neighbours (ties -> even) and near-ties
    base = np.array([1.0, 1.5, 3.0, -2.25], np.float64)
    ulp = 2.0 ** -7 * np.array([1, 1, 2, 2], np.float64)
    x = np.concatenate([x, base + ulp / 2, base + 3 * ulp / 2, base + ulp / 2 + 1e-12,
                        base + ulp / 2 - 1e-12])
    r = synth.round_to(x, "bf16")
    for xi, ri in zip(x, r):
        nb = _bf16_neighbours(xi)
        best = min(abs(v - xi) for _, v in nb)
        ties = [c for c, v in nb if abs(v - xi) == best]
        want = ties[0] if len(ties) == 1 else [c for c in ties if c % 2 == 0][0]
        assert int(ri) == want, (xi, ri, ties)
    assert int(synth.round_to(np.array([0.0]), "bf16")[0]) == 0
    assert int(synth.round_to(np.array([-0.0]), "bf16")[0]) == 0x8000


def test_widen_roundtrip():
    b = synth.normal(3, 2, 0, 4096, "bf16")
    w = synth.widen(b, "bf16")
    assert np.array_equal(synth.round_to(w, "bf16"), b)
    f = synth.normal(3, 2, 0, 4096, "f32")
    assert np.array_equal(synth.round_to(synth.widen(f, "f32"), "f32"), f)


def test_workload_shapes():
    c = CONFIGS
    assert (c[1].nb, c[1].max_selected, c[1].G) == (64, 8 + 4 + 1, 1)
    assert (c[2].nb, c[2].max_selected) == (512, 64 + 8 + 1)
    assert (c[3].nb, c[3].max_selected, c[3].G, c[3].units) == (4096, 128 + 16 + 1, 4, 32)
    assert (c[4].nb, c[4].nc, c[4].max_selected) == (4096, 256, 128 + 8 + 1)
    assert (c[5].top_k, c[5].max_selected, c[5].layers, c[5].steps) == (102, 102 + 8 + 1, 8, 16)


def test_page_table_is_a_permutation():
    w = CONFIGS[5].scaled(batch=3, T=4096)
    pt = w.page_table()
    assert pt.shape == (3, 64)
    assert np.array_equal(np.sort(pt.ravel()), np.arange(3 * 64))
    assert not np.array_equal(pt.ravel(), np.arange(3 * 64))
    assert np.array_equal(pt, w.page_table())
    ident = CONFIGS[3].scaled(batch=2, T=4096).page_table()
    assert np.array_equal(ident.ravel(), np.arange(ident.size))


def test_needles_planted_before_window():
    w = CONFIGS[3].scaled(batch=1, hkv=2, hq=8, T=8192)
    for g in range(2):
        blocks = w.needle_blocks(0, g)
        assert len(blocks) == 16 and len(set(blocks.tolist())) == 16
        assert np.all((blocks + 1) * w.S <= w.T - w.window)
        k = synth.widen(w.k_unit(0, 0, g), "bf16")
        qd = w.q_dir(0, g)
        proj = k @ qd
        inside = np.zeros(w.T, bool)
        for beta in blocks:
            inside[beta * w.S:(beta + 1) * w.S] = True
        # needle keys carry 3 * q_dir: their projection is ~3, the rest ~0
        assert proj[inside].mean() > 2.5 and abs(proj[~inside].mean()) < 0.1


def test_drift_recursion():
    w = CONFIGS[5].scaled(batch=2, T=1024)
    q0, q1, q2 = (w.q_master(1, t) for t in range(3))
    n = w.batch * w.hq * w.d
    z1 = synth.normal(w.seed, 7 + 16, 0, n).reshape(q0.shape)
    z2 = synth.normal(w.seed, 7 + 16, n, n).reshape(q0.shape)
    assert np.allclose(q1, 0.9 * q0 + 0.44 * z1, rtol=0, atol=0)
    assert np.allclose(q2, 0.9 * q1 + 0.44 * z2, rtol=0, atol=0)
