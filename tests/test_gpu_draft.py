"""GPU parity of the FastMTP draft block's catch-up and of the decode-step
graphs against the oracle, under controlled acceptance.

The random-init draft block never proposes what the random-init verifier
accepts, so with its own proposals every catch-up pass would carry one row.
Here acceptance is driven by the controlled drafts (the verifier's own
sequence with each slot replaced at probability p), which makes the accepted
count -- and so the rows of the next catch-up pass -- range over 0..K; the
block's real proposals are captured before the override and compared with
the oracle's draft_propose under the same history.  Decode-step graphs are
checked the same way through the step taps (real proposals, accepted lengths)
and the by-position routing tap.  Tolerances: fp32 model 1e-3, bf16 model
5e-2, excuses only at near ties of the oracle's margins."""
import dataclasses

import pytest

from speculative_moe_decoding_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import forced_spec_parity, log, make_pair  # noqa: E402
from speculative_moe_decoding_amd import ocrdec  # noqa: E402

SMALL32 = dataclasses.replace(synth.FULL, n_layers=2, vocab=5003, dtype="f32")
SMALL16 = dataclasses.replace(synth.FULL, n_layers=2, vocab=5003, dtype="bf16")


@pytest.mark.parametrize("K,p", [(3, 0.2), (7, 0.12)])
@pytest.mark.parametrize("arith", ["vector_f32", "matrix_bf16"])
@pytest.mark.parametrize("graphs", [False, True], ids=["eager", "graphs"])
def test_draft_catch_up_vs_oracle(arith, K, p, graphs):
    cfg, path, tol = ((SMALL32, ocrdec.OCRDEC_PATH_VECTOR, 1e-3) if arith == "vector_f32"
                      else (SMALL16, ocrdec.OCRDEC_PATH_MATRIX, 5e-2))
    log(f"case {arith} K={K} p={p} graphs={graphs}")
    w, dec, orc = make_pair(cfg, 71, max_k=K, max_positions=256, path=path)
    page = synth.make_pages(cfg, 72, [20], [5], [64])[0]
    N = 64
    r = forced_spec_parity(dec, orc, page, N, K, tol, p, graphs=graphs)
    log(f"{arith} K={K} graphs={graphs}: {r.steps} steps, n_prev seen {sorted(r.n_values)}, "
        f"real drafts {r.drafts_compared - r.drafts_excused}/{r.drafts_compared} exact "
        f"({r.drafts_excused} near ties), greedy rows {r.greedy_compared} ({r.greedy_excused} near ties), "
        f"max |dlogit| {r.worst_logit:.2e}; {r.picker.summary()}")
    # the catch-up pass carried 1 .. K + 1 rows over the run: n_prev took 0, K and values between
    assert 0 in r.n_values and K in r.n_values and len(r.n_values) >= 3
    assert r.drafts_compared >= 2 * K * 4
    assert r.drafts_excused <= max(2, r.steps // 4)


@pytest.mark.parametrize("arith", ["vector_f32", "matrix_bf16"])
@pytest.mark.parametrize("graphs", [False, True], ids=["eager", "graphs"])
def test_depth_changes_between_steps(arith, graphs):
    """Run-time adaptive K: one page decoded with the depth going 3 -> 1 -> 2
    (a few steps each, repeated), controlled acceptance: lossless, accepted
    lengths as predicted, and the draft block's proposals -- including the
    catch-up of up to 4 rows into a depth-1 step -- equal to the oracle's."""
    cfg, path, tol = ((SMALL32, ocrdec.OCRDEC_PATH_VECTOR, 1e-3) if arith == "vector_f32"
                      else (SMALL16, ocrdec.OCRDEC_PATH_MATRIX, 5e-2))
    log(f"case {arith} graphs={graphs}")
    w, dec, orc = make_pair(cfg, 73, max_k=3, max_positions=256, path=path)
    page = synth.make_pages(cfg, 74, [18], [6], [64])[0]
    sched = ([3] * 4 + [1] * 4 + [2] * 4) * 8
    r = forced_spec_parity(dec, orc, page, 64, 3, tol, 0.15, graphs=graphs, k_sched=lambda s: sched[s])
    log(f"{arith} 3->1->2 graphs={graphs}: {r.steps} steps, real drafts {r.drafts_compared - r.drafts_excused}/"
        f"{r.drafts_compared} exact, max |dlogit| {r.worst_logit:.2e}; {r.picker.summary()}")
    assert r.steps >= 12 and 3 in r.n_values


def test_generate_adaptive_is_lossless():
    """Decoder.generate_adaptive chooses K per window from measured step times
    and the acceptance it sees (policy.OnlineDepth); with controlled drafts the
    page equals the AR sequence and more than one depth is used."""
    from speculative_moe_decoding_amd import policy
    cfg = SMALL16
    w, dec, orc = make_pair(cfg, 75, max_k=3, max_positions=512)
    page = synth.make_pages(cfg, 76, [20], [4], [160])[0]
    N = 160
    ar, _, _ = dec.generate([page], N + 8, 0, check_every=16)
    trace = torch.from_numpy(ar.astype("int32")).cuda()
    thr = int(0.2 * float(1 << 53))
    ctl = policy.OnlineDepth(3, explore_every=3)
    toks, hist = dec.generate_adaptive([page], N, ctl, window=4, trace=trace, seed=3000, threshold=thr)
    assert toks[0].tolist() == ar[0][:N].tolist()
    used = sorted({k for k, _, _ in hist})
    log(f"adaptive K: depths used {used}, windows {len(hist)}, tau(1..3) "
        f"{[round(ctl.tau(k), 2) for k in (1, 2, 3)]}, ms/step {ctl.ms}")
    assert len(used) >= 2
