"""The synthetic workloads carry the statistics the STEPQuant pages print
(fixture tests/golden/pages_figures.json, each value cited there)."""
import json
import math
import os

import numpy as np
import torch

from quantized_recurrent_state_gated_amd import inputs as I

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def test_serving_shape_matches_pages():
    w = I.WORKLOADS["serving"]
    assert w.n_heads == GOLDEN["recurrent_heads_qwen"]["value"]
    assert w.n_req == GOLDEN["concurrency_crossover"]["value"]
    bits = I.head_bits(w)
    assert abs((bits == 16).mean() - GOLDEN["pivot_head_fraction"]["value"]) < 5e-4
    assert I.pool_stats(w)["mean_bits_nonpivot"] == 6.0
    assert abs(I.pool_stats(I.WORKLOADS["highconc"])["mean_bits_nonpivot"] - 4.225) < 1e-3
    assert I.WORKLOADS["drift"].steps == GOLDEN["outlier_persistence_steps"]["value"]


def test_outlier_ratios_match_pages():
    w = I.scaled(I.WORKLOADS["serving"], n_req=2, n_heads=64)
    S = torch.cat([I.initial_state(w, p) for p in range(w.n_req)])
    rr, cr = I._ratios(S.double())
    assert abs(float(rr.median()) / GOLDEN["row_max_over_median"]["value"] - 1) < 0.1
    assert abs(float(cr.median()) / GOLDEN["col_max_over_median"]["value"] - 1) < 0.1
    frac3 = float(((rr > 3) & (cr > 3)).double().mean())
    assert frac3 >= GOLDEN["fraction_of_states_ratio_above_3x"]["value"]


def test_bits_follow_half_life_rank():
    w = I.WORKLOADS["layer"]
    hl, bits = I.half_lives(w), I.head_bits(w)
    order = {16: 0, 8: 1, 6: 2, 4: 3}
    ranks = np.array([order[int(b)] for b in bits])
    # a longer half-life never gets a narrower width than a shorter one
    idx = np.argsort(-hl)
    assert np.all(np.diff(ranks[idx]) >= 0)


def test_scales_never_clip_the_initial_state():
    w = I.scaled(I.WORKLOADS["layer"], n_req=3, n_heads=8)
    r, c = I.scales(w)
    bits = I.head_bits(w)
    S = torch.stack([I.initial_state(w, p) for p in range(w.n_req)])
    for h in range(w.n_heads):
        if bits[h] > 8:
            continue
        Q = 2 ** (int(bits[h]) - 1) - 1
        s = (r[h][:, None] * c[h][None, :]).double()
        assert float((S[:, h].double().abs() / s).max()) <= Q * (1 + 1e-6)


def test_step_inputs_distributions():
    w = I.WORKLOADS["layer"]
    si = I.step_inputs(w, 3)
    assert si.q.dtype == torch.bfloat16 and si.q.shape == (8, 48, 128)
    kn = si.k.float().norm(dim=-1)
    assert float((kn - 1).abs().max()) < 2 ** -7  # unit norm before the bf16 cast
    assert float(si.alpha.max()) <= 1.0 and float(si.alpha.min()) > 0.0
    assert 0.05 <= float(si.beta.min()) and float(si.beta.max()) <= 0.95
    # mean log-retention is -ln2 / half-life (averaged over many draws)
    hl = I.half_lives(w)
    la = torch.stack([torch.log(I.step_inputs(w, t).alpha) for t in range(200)]).double()
    est = -la.mean(dim=(0, 1)).numpy() * hl / math.log(2)
    assert abs(float(np.median(est)) - 1) < 0.05
    # reproducible
    assert torch.equal(I.step_inputs(w, 3).q, si.q)


def test_tiny_recipe():
    w = I.WORKLOADS["tiny"]
    r, c = I.scales(w)
    assert torch.all(r == 1)
    ranges = c * 127
    assert float(ranges.min()) >= 0.5 and float(ranges.max()) <= 2.0
    S = I.initial_state(w, 0)
    assert abs(float(S.std()) - 0.1) < 0.01
    si = I.step_inputs(w, 0)
    assert si.q.dtype == torch.float32
    assert float((si.k.norm(dim=-1) - 1).abs().max()) < 1e-6


def test_spearman_helper_matches_scipy():
    from scipy.stats import spearmanr
    from quantized_recurrent_state_gated_amd.drift import spearman
    rng = np.random.default_rng(3)
    a = rng.standard_normal(200)
    b = a + rng.standard_normal(200)
    b[:20] = b[0]  # ties
    assert abs(spearman(a, b) - spearmanr(a, b).correlation) < 1e-12


def test_channel_gates_distribution():
    w = I.WORKLOADS["layer"]
    a = I.channel_gates(w, 3)
    assert a.shape == (w.n_req, w.n_heads, w.dk) and a.dtype == torch.float32
    assert float(a.max()) <= 1.0 and float(a.min()) > 0.0
    # channels of one head differ; their mean log-retention is the head's -ln2/h
    assert float(a.std(dim=-1).min()) > 0
    hl = I.half_lives(w)
    la = torch.stack([torch.log(I.channel_gates(w, t)) for t in range(50)]).double()
    est = -la.mean(dim=(0, 1, 3)).numpy() * hl / math.log(2)
    assert abs(float(np.median(est)) - 1) < 0.05
    assert torch.equal(I.channel_gates(w, 3), a)
    assert not torch.equal(I.channel_gates(w, 4), a)
    t = I.channel_gates(I.WORKLOADS["tiny"], 0)
    assert t.shape == (1, 4, 16) and float(t.max()) < 1.0
