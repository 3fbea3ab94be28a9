"""GPU checks of the prefill pass: the prefix in entries of 32 rows through the
prefill attention (matrix cores for the bf16 cache), against the oracle at a
long prefix, and a row's result independent of the pass it falls in.

The model is the 2-layer bf16 one with a ragged vocabulary (5003); the pages
are the method's page shapes stretched to long prefixes: 300 + 12, 1850 + 20
and 40 + 5 rows, 71 entries in all, so that a call of the three pages takes
two passes (64 entries per pass) and the long page is split between them."""
import dataclasses

import numpy as np
import pytest

from speculative_moe_decoding_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import log, make_pair  # noqa: E402
from oracle import decoder as od  # noqa: E402
from speculative_moe_decoding_amd import ocrdec  # noqa: E402

SMALL16 = dataclasses.replace(synth.FULL, n_layers=2, vocab=5003, dtype="bf16")
TOL = 5e-2


def _pages(cfg):
    return synth.make_pages(cfg, 81, [300, 1850, 40], [12, 20, 5], [4, 4, 4])


def _ar_step_logits(dec, B):
    """One K = 0 verify over slots 0..B-1: (greedy [B], logits [B][V])."""
    draft = dec.i32(B, 1)
    greedy = dec.i32(B, 1)
    logits = torch.empty(B, 1, dec.cfg.vocab, dtype=torch.float32, device="cuda")
    dec.verify(B, 0, draft, greedy=greedy, logits=logits)
    torch.cuda.synchronize()
    return greedy.cpu().numpy()[:, 0], logits.cpu().numpy()[:, 0]


def test_prefill_split_across_passes_is_invariant():
    """Three pages prefilled in one call (two passes; the 1870-row page spans
    both) give bitwise the first token and the next step's logits of each page
    prefilled alone (one pass)."""
    cfg = SMALL16
    w = synth.Weights(cfg, 82)
    pages = _pages(cfg)
    log(f"prefix lengths {[p.prefix_len for p in pages]}, entries "
        f"{sum((p.prefix_len + 31) // 32 for p in pages)}")
    dec3 = ocrdec.Decoder(cfg, w.device_arrays(), max_batch=3, max_k=0, max_positions=2048)
    pend3 = dec3.prefill(pages).cpu().numpy()
    g3, l3 = _ar_step_logits(dec3, 3)
    for b, page in enumerate(pages):
        dec1 = ocrdec.Decoder(cfg, w.device_arrays(), max_batch=1, max_k=0, max_positions=2048)
        pend1 = dec1.prefill([page]).cpu().numpy()
        g1, l1 = _ar_step_logits(dec1, 1)
        assert pend1[0] == pend3[b], f"page {b}: first token {pend1[0]} alone, {pend3[b]} in the batch"
        assert g1[0] == g3[b]
        assert np.array_equal(l1[0], l3[b]), f"page {b}: logits differ by {np.abs(l1[0] - l3[b]).max():.3e}"
        del dec1
    log("first tokens and next-step logits bitwise equal alone and in a two-pass call")


def test_long_prefill_vs_oracle():
    """The 1870-row page: first token and the logits of the next step against
    the oracle (fp64) within the bf16 tolerance (token excused only at a near
    tie of the oracle's margins)."""
    cfg = SMALL16
    w, dec, orc = make_pair(cfg, 82, max_batch=1, max_k=0, max_positions=2048)
    page = _pages(cfg)[1]
    pend = int(dec.prefill([page]).item())
    g, lg = _ar_step_logits(dec, 1)
    st = orc.new_state(page.prefix_len + 4)
    y0 = orc.prefill(st, page.vision, page.prompt, with_draft=False)
    m0 = od.top2_margin(st.first_logits[None])[0]
    if pend != y0:
        assert m0 < TOL, f"first token {pend} vs oracle {y0} with margin {m0:.3e}"
        log(f"first token differs at a near tie (margin {m0:.2e}); the oracle follows the GPU's")
    P = page.prefix_len
    h = orc.verifier_forward(st, orc.embed([pend]), [P])
    ref = orc.lm_logits(h)[0]
    diff = float(np.abs(lg[0] - ref).max())
    log(f"prefix {P}: first token {pend} (oracle {y0}), next-step logits within {diff:.2e}")
    assert diff < TOL
    if int(g[0]) != int(od.greedy(ref[None])[0]):
        assert od.top2_margin(ref[None])[0] < TOL
