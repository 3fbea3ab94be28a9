"""GPU parity at the workloads' full sizes.

* 2-layer fp32 model, vocab 129,280, prefix 256 vision + 16 prompt rows, 64
  output tokens: AR and FastMTP K=3 with the real draft block, step by step
  against the oracle (tokens, drafts, accepted lengths exact; logits 1e-3).
* 12-layer bf16 model (the benchmarked decoder), prefix 256 + 32:
  speculative output equal to AR output for the real draft and for the
  controlled-acceptance drafts at K = 1, 2, 3, with accepted lengths equal to
  the oracle's prediction (batch 1, one stream, eager).
* Gundam page (1,156 + 32 prefix, 3,568 tokens, cache past 4,096 positions):
  lossless with graphs, accepted lengths.
The bf16 decoder's tokens, routing and logits are checked against the oracle
in test_gpu_teacher.py (teacher-forced, whole pages).
"""
import dataclasses
import time

import numpy as np
import pytest

from oracle import decoder as od
from speculative_moe_decoding_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import compare_steps, log, make_pair, run_gpu_steps  # noqa: E402


def test_two_layer_fp32_full_vocab():
    wl = synth.WORKLOADS["tiny_fp32_2layer"]
    cfg = wl["cfg"]
    w, dec, orc = make_pair(cfg, wl["weight_seed"], max_positions=1024)
    page = synth.make_pages(cfg, wl["input_seed"], [wl["n_vision"]], [wl["n_prompt"]], [wl["n_out"]])[0]
    N = wl["n_out"]
    t = time.time()
    g_ar, g_steps = run_gpu_steps(dec, page, N, 0)
    log(f"GPU AR {N} tokens: {time.time() - t:.1f}s")
    t = time.time()
    r_ar, r_logits = orc.generate_ar(page.vision, page.prompt, N, keep_logits=True)
    log(f"oracle AR: {time.time() - t:.1f}s")
    ref = [od.StepRecord(0, [], [r_ar[i + 1]], 0, r_logits[i + 1][None]) for i in range(N - 1)]
    n, worst, note = compare_steps(g_steps, ref, 1e-3)
    log(f"AR: {n}/{N - 1} steps agree, max |dlogit| {worst:.2e}, {note}")
    assert worst < 1e-3 and n >= 16
    g_sp, g_ss = run_gpu_steps(dec, page, N, 3)
    assert g_sp == g_ar
    t = time.time()
    r_sp, r_ss = orc.generate_spec(page.vision, page.prompt, N, 3, keep_logits=True)
    log(f"oracle spec: {time.time() - t:.1f}s")
    assert r_sp == r_ar
    n, worst, note = compare_steps(g_ss, r_ss, 1e-3)
    log(f"spec K=3: {n}/{len(r_ss)} steps agree, max |dlogit| {worst:.2e}, {note}; "
        f"accepted {[s['n'] for s in g_ss][:24]}")
    assert worst < 1e-3 and n >= 8


@pytest.fixture(scope="module")
def full():
    wl = synth.WORKLOADS["base_page_bf16"]
    cfg = wl["cfg"]
    w, dec, orc = make_pair(cfg, wl["weight_seed"], max_positions=2048)
    page = synth.make_pages(cfg, wl["input_seed"], [wl["n_vision"]], [wl["n_prompt"]], [wl["n_out"]])[0]
    return w, dec, orc, page


def test_full_model_lossless(full):
    w, dec, orc, page = full
    N = 400
    t = time.time()
    ar, _, _ = dec.generate([page], N + 8, 0, check_every=32)
    log(f"GPU AR {N + 8} tokens: {time.time() - t:.2f}s")
    trace = torch.from_numpy(ar.astype(np.int32)).cuda()
    for K, alpha in ((1, 0.826), (2, 0.691), (3, 0.576)):
        p = synth.replacement_probability(alpha, K)
        t = time.time()
        toks, acc, steps = dec.generate([page], N, K, trace=trace, seed=3000, threshold=od.replace_threshold(p),
                                        record=True, check_every=8)
        assert toks[0].tolist() == ar[0][:N].tolist(), K
        assert acc[0] == od.controlled_accepts(N, K, 3000, p), K
        log(f"K={K} controlled: lossless, tau {np.mean(np.array(acc[0]) + 1):.3f}, {time.time() - t:.2f}s")
    # the real draft block
    toks, acc, _ = dec.generate([page], 96, 3, record=True, check_every=4)
    assert toks[0].tolist() == ar[0][:96].tolist()
    log(f"real draft K=3: lossless; accepted {acc[0][:20]}")


def test_gundam_page_lossless(full):
    """Gundam-mode page: 1,156 vision + 32 prompt rows, 3,568 output tokens, K = 3
    at 57.6 % controlled acceptance, so the cache grows from 1,188 to 4,756
    positions (a handle past 4,096 positions uses 256-key attention chunks).
    The whole page is lossless against the K = 0 run (decode-step graphs);
    accepted lengths equal the SplitMix64 prediction over the first 600 tokens."""
    w, _, _, _ = full
    wl = synth.WORKLOADS["gundam_page_bf16"]
    cfg = wl["cfg"]
    from speculative_moe_decoding_amd import ocrdec
    page = synth.make_pages(cfg, wl["input_seed"], [wl["n_vision"]], [wl["n_prompt"]], [wl["n_out"]])[0]
    N = wl["n_out"]
    P = page.prefix_len
    dec = ocrdec.Decoder(cfg, w.device_arrays(), max_batch=1, max_k=3, max_positions=P + N + 160)
    t = time.time()
    ar, _, _ = dec.generate([page], N + 8, 0, check_every=64)
    log(f"Gundam page: GPU AR {N + 8} tokens in {time.time() - t:.1f}s")
    trace = torch.from_numpy(ar.astype(np.int32)).cuda()
    p = synth.replacement_probability(0.576, 3)
    thr = od.replace_threshold(p)
    t = time.time()
    toks, _, steps = dec.generate([page], N, 3, trace=trace, seed=3000, threshold=thr, check_every=16, graphs=True)
    assert toks[0].tolist() == ar[0][:N].tolist()
    log(f"Gundam page K=3 graphs: lossless over {N} tokens, {steps} steps, {time.time() - t:.1f}s")
    n_rec = 600
    toks, acc, _ = dec.generate([page], n_rec, 3, trace=trace, seed=3000, threshold=thr, record=True, check_every=8)
    assert toks[0].tolist() == ar[0][:n_rec].tolist()
    assert acc[0] == od.controlled_accepts(n_rec, 3, 3000, p)
