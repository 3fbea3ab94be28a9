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
