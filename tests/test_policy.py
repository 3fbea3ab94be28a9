"""Adaptive K: the policy reproduces the pages' best depths from their own costs.

The blog's L4 table ("Results") gives, per mode, the autoregressive step cost
(1000 / tok/s at k = 0: 23.4 ms eager, 6.3 ms with CUDA graphs), the k = 3
step cost (32.9 / 15.9 ms, i.e. about 3.2 ms per draft pass in both modes) and
the acceptance at each k.  From those alone the policy must pick k = 3 in eager
mode and k = 1 with graphs, the depths the pages report as best.
"""
import json
import os

from speculative_moe_decoding_amd import policy

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "l4_fastmtp_table.json")


def _rows():
    t = json.load(open(GOLDEN))
    cols = t["columns"]
    return [dict(zip(cols, r)) for r in t["rows"]]


def test_policy_reproduces_pages_best_depths():
    rows = _rows()
    for mode, best in (("eager", 3), ("graph", 1)):
        r = {int(x["k"]): x for x in rows if x["mode"] == mode}
        t0 = 1000.0 / r[0]["tok_per_s"]
        t3 = 1000.0 * r[3]["tau"] / r[3]["tok_per_s"]
        costs = policy.linear_step_costs(t0, (t3 - t0) / 3.0, 3)
        alpha = {k: r[k]["acceptance"] for k in (1, 2, 3)}
        assert policy.choose_k(costs, alpha) == best, mode


def test_expected_tokens_identity():
    for x in _rows():
        if int(x["k"]) > 0:
            assert abs(policy.expected_tokens(int(x["k"]), x["acceptance"]) - x["tau"]) < 0.011


def test_policy_on_measured_mi355x_costs():
    """The MI355X sweep (graph-replayed steps: 0.668 / 0.901 / 1.120 / 1.321 ms
    for K = 0..3 at the table's graph-mode acceptance) favours K = 2."""
    costs = {0: 0.668, 1: 0.901, 2: 1.120, 3: 1.321}
    assert policy.choose_k(costs, {1: 0.829, 2: 0.693, 3: 0.579}) == 2


def test_online_depth_learns_acceptance_and_picks_the_best_depth():
    """Fed steps whose drafts are accepted with a fixed per-draft probability
    (the controlled benchmark's model) and the MI355X step costs, the run-time
    controller's tau estimate converges to the geometric acceptance and it
    settles on the depth with the best tokens per unit time."""
    import numpy as np
    rng = np.random.default_rng(0)
    costs = {1: 0.705, 2: 0.867, 3: 1.005}         # measured ms per step, base page, graphs
    q = 0.78                                         # per-draft acceptance
    ctl = policy.OnlineDepth(3, explore_every=0)
    picks = []
    for _ in range(200):
        k = ctl.choose()
        picks.append(k)
        n = []
        for _ in range(8):
            a = 0
            while a < k and rng.random() < q:
                a += 1
            n.append(a)
        ctl.observe(k, n, costs[k])
    for k in (1, 2, 3):
        exact = sum(q ** i for i in range(k + 1))
        assert abs(ctl.tau(k) - exact) < 0.08, (k, ctl.tau(k), exact)
    best = max((sum(q ** i for i in range(k + 1)) / costs[k], k) for k in costs)[1]
    assert picks[-50:].count(best) == 50
    # a controller told the k = 3 step costs as much as k = 1 moves to k = 3
    ctl2 = policy.OnlineDepth(3, explore_every=0)
    for k in (1, 2, 3) * 5:
        ctl2.observe(k, [min(k, 2)] * 8, 1.0)
    assert ctl2.choose() == 3
