"""GPU parity of the HIP decode path (through the C ABI) against the CPU oracle.

Tolerances: routing, accepted lengths and tokens bit-exact; logits within
1e-3 (fp32 model) or 5e-2 (bf16 model) absolute, a token mismatch excused only
where the oracle's top-2 logit margin is under that tolerance."""
import dataclasses

import numpy as np
import pytest

from oracle import decoder as od
from speculative_moe_decoding_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import compare_steps, forced_ar_parity, log, make_pair, run_gpu_steps  # noqa: E402

SMALL32 = dataclasses.replace(synth.FULL, n_layers=2, vocab=5003, dtype="f32")
SMALL16 = dataclasses.replace(synth.FULL, n_layers=2, vocab=5003, dtype="bf16")


def test_smoke():
    import __graft_entry__
    __graft_entry__.smoke()


@pytest.mark.parametrize("cfg,tol", [(SMALL32, 1e-3), (SMALL16, 5e-2)], ids=["f32", "bf16"])
def test_small_model_ar_and_spec(cfg, tol):
    """2 layers, vocab 5003 (ragged against the 64-row LM-head tiles), prefix
    20 vision + 5 prompt rows (one prefill entry of 25 rows)."""
    w, dec, orc = make_pair(cfg, 41)
    page = synth.make_pages(cfg, 42, [20], [5], [24])[0]
    N = 24
    # autoregressive, every step against the oracle (forced history)
    g_ar, n, ex, worst = forced_ar_parity(dec, orc, page, N, tol, min_steps=N - 1)
    _, g_steps = run_gpu_steps(dec, page, N, 0)
    log(f"{cfg.dtype} AR: {n} steps compared, {ex} near ties, max |dlogit| {worst:.2e}")
    # speculative, K = 3, the real draft block
    g_sp, g_ssteps = run_gpu_steps(dec, page, N, 3)
    r_sp, r_ssteps = orc.generate_spec(page.vision, page.prompt, N, 3, keep_logits=True)
    assert g_sp == g_ar                    # GPU spec == GPU AR, bit for bit
    n, worst, note = compare_steps(g_ssteps, r_ssteps, tol)
    log(f"{cfg.dtype} spec K=3: {n}/{len(r_ssteps)} steps agree, max |dlogit| {worst:.2e}, {note}, "
        f"accepted {[s['n'] for s in g_ssteps]}")
    assert worst < tol
    assert n >= 4 or note is not None
    # logits of the accepted verify rows equal the AR logits bitwise (batch invariance)
    ar_rows = [s["logits"][0] for s in g_steps]
    pos = 0
    for s in g_ssteps:
        for i in range(s["n"] + 1):
            if pos + i < len(ar_rows):
                assert np.array_equal(s["logits"][i], ar_rows[pos + i]), (pos, i)
        pos += s["n"] + 1


def test_routing_taps_bit_exact():
    """Layer-by-layer routing indices of a verify step equal the oracle's
    (excused only where the oracle's 6th/7th logit gap is under 1e-4)."""
    cfg = SMALL32
    w, dec, orc = make_pair(cfg, 43)
    page = synth.make_pages(cfg, 44, [12], [3], [4])[0]
    K = 3
    route = torch.full((cfg.n_layers, K + 1, 8), -1, dtype=torch.int32, device="cuda")
    hid = torch.zeros(K + 1, cfg.d_model, dtype=torch.float32, device="cuda")
    from speculative_moe_decoding_amd import ocrdec
    ocrdec.ocrdec_set_taps(dec.h, route, hid)
    pending = dec.prefill([page])
    draft = torch.tensor([[7, 4000, 123]], dtype=torch.int32, device="cuda")
    dec.verify(1, K, draft)
    torch.cuda.synchronize()
    st = orc.new_state(64)
    y0 = orc.prefill(st, page.vision, page.prompt, with_draft=False)
    assert int(pending.item()) == y0
    rec = []
    h = orc.verifier_forward(st, orc.embed([y0, 7, 4000, 123]), np.arange(15, 19), record=rec)
    got = route.cpu().numpy()
    checked = 0
    for l in range(cfg.n_layers):
        for r in range(K + 1):
            assert list(got[l, r, 6:]) == [64, 65]
            if list(got[l, r, :6]) != list(rec[l][r]):
                pytest.fail(f"layer {l} row {r}: {got[l, r, :6]} vs oracle {rec[l][r]}")
            checked += 1
    np.testing.assert_allclose(hid.cpu().numpy(), h, atol=1e-3, rtol=1e-4)
    log(f"routing bit-exact on {checked} (layer, row) pairs")


def test_batch_invariance_and_slots():
    """Two pages decoded together (B = 2) give bitwise the tokens of each page
    decoded alone; sequences use independent state slots."""
    cfg = SMALL16
    w = synth.Weights(cfg, 45)
    from speculative_moe_decoding_amd import ocrdec
    pages = synth.make_pages(cfg, 46, [20, 9], [5, 11], [20, 20])
    dec2 = ocrdec.Decoder(cfg, w.device_arrays(), max_batch=2, max_k=3, max_positions=512)
    toks2, acc2, _ = dec2.generate(pages, 20, 3, record=True, check_every=1)
    for b in range(2):
        dec1 = ocrdec.Decoder(cfg, w.device_arrays(), max_batch=1, max_k=3, max_positions=512)
        toks1, acc1, _ = dec1.generate([pages[b]], 20, 3, record=True, check_every=1)
        assert toks1[0].tolist() == toks2[b].tolist()
        assert acc1[0] == acc2[b]
        ar1, _, _ = dec1.generate([pages[b]], 20, 0, check_every=1)
        assert ar1[0].tolist() == toks1[0].tolist()


def test_controlled_acceptance_lossless():
    """Drafts replaced by the controlled generator: committed tokens equal the AR
    trace and the accepted lengths equal the oracle's prediction from SplitMix64."""
    cfg = SMALL16
    w = synth.Weights(cfg, 47)
    from speculative_moe_decoding_amd import ocrdec
    page = synth.make_pages(cfg, 48, [16], [4], [40])[0]
    dec = ocrdec.Decoder(cfg, w.device_arrays(), max_batch=1, max_k=3, max_positions=512)
    N = 40
    for K, alpha in ((1, 0.826), (2, 0.691), (3, 0.576)):
        ar, _, _ = dec.generate([page], N + K + 2, 0, check_every=4)
        trace = torch.from_numpy(ar.astype(np.int32)).cuda()
        p = synth.replacement_probability(alpha, K)
        thr = od.replace_threshold(p)
        toks, acc, _ = dec.generate([page], N, K, trace=trace, seed=3000, threshold=thr, record=True,
                                    check_every=1)
        assert toks[0].tolist() == ar[0][:N].tolist()
        assert acc[0] == od.controlled_accepts(N, K, 3000, p, seq_index=0)


def test_graph_steps_match_eager_calls():
    """Decode steps replayed from cached HIP graphs give the tokens and accepted
    lengths of the individual calls, replay after replay (eager work and
    synchronisations in between), with the real draft and with controlled drafts."""
    cfg = SMALL16
    w = synth.Weights(cfg, 49)
    from speculative_moe_decoding_amd import ocrdec
    page = synth.make_pages(cfg, 50, [30], [6], [48])[0]
    dec = ocrdec.Decoder(cfg, w.device_arrays(), max_batch=1, max_k=3, max_positions=1024)
    N = 48
    ar, _, _ = dec.generate([page], N + 8, 0, check_every=8)
    trace = torch.from_numpy(ar.astype(np.int32)).cuda()
    thr = od.replace_threshold(synth.replacement_probability(0.576, 3))
    for tr in (None, trace):
        eager, _, _ = dec.generate([page], N, 3, trace=tr, seed=3000, threshold=thr, check_every=1)
        for rep in range(3):
            g, _, _ = dec.generate([page], N, 3, trace=tr, seed=3000, threshold=thr, check_every=2, graphs=True)
            assert g[0].tolist() == eager[0].tolist(), rep
            torch.cuda.synchronize()
        assert eager[0].tolist() == ar[0][:N].tolist()
    log("graph decode matches eager calls")


def _eager_steps(dec, pages, K, n_steps, slots):
    """n_steps individual draft / verify / accept calls with the given slot map
    (None: identity); returns the committed tokens per sequence."""
    from speculative_moe_decoding_amd import ocrdec  # noqa: F401
    B = len(pages)
    cap = n_steps * (K + 1) + 2
    out_tokens = torch.zeros(B, cap, dtype=torch.int32, device="cuda")
    out_len = dec.i32(B)
    n_acc = dec.i32(B)
    draft, greedy = dec.i32(B, max(K, 1)), dec.i32(B, K + 1)
    out_tokens[:, 0] = dec.prefill(pages)
    for _ in range(n_steps):
        dec.draft(B, K, slots=slots, out=draft)
        dec.verify(B, K, draft, slots=slots, greedy=greedy)
        dec.accept(B, K, draft, greedy, n_acc, out_tokens, out_len, slots=slots)
    torch.cuda.synchronize()
    n = out_len.cpu().numpy()
    return [out_tokens[b, :int(n[b])].cpu().numpy().tolist() for b in range(B)]


@pytest.mark.parametrize("B,K", [(2, 3), (1, 7)])
def test_graph_steps_batches_and_depths(B, K):
    """Decode-step graphs (whose accept launch also reduces the verify's greedy
    tokens) give the individual calls' tokens with several sequences and with
    the deepest draft (8 verify rows per sequence, two per wavefront in the
    reduction); both equal plain autoregressive decoding; and an explicit slot
    map 0..B-1 gives the tokens of the calls without one (whose attention
    takes the slot from the sequence index)."""
    cfg = SMALL16
    w = synth.Weights(cfg, 51)
    from speculative_moe_decoding_amd import ocrdec
    log(f"case B={B} K={K}")
    pages = synth.make_pages(cfg, 52, [18, 11][:B], [6, 9][:B], [32] * B)
    dec = ocrdec.Decoder(cfg, w.device_arrays(), max_batch=B, max_k=K, max_positions=512)
    N = 32
    eager, _, _ = dec.generate(pages, N, K, check_every=1)
    for rep in range(2):
        g, _, _ = dec.generate(pages, N, K, check_every=2, graphs=True)
        assert g.tolist() == eager.tolist(), rep
    ar, _, _ = dec.generate(pages, N, 0, check_every=4)
    assert eager.tolist() == ar.tolist()
    slots = torch.arange(B, dtype=torch.int32, device="cuda")
    a = _eager_steps(dec, pages, K, 6, None)
    b = _eager_steps(dec, pages, K, 6, slots)
    assert a == b
    log(f"B={B} K={K}: graphs = eager = AR over {N} tokens; slot map 0..B-1 = identity")


@pytest.mark.parametrize("which", ["f32_2layer", "bf16_2layer", "bf16_12layer"])
def test_fused_moe_launch_bitwise(which):
    """The persistent MoE launch (routing, gate/up, down, combine in one launch
    after the router logits, with waits inside it) gives bitwise the logits,
    drafts, greedy tokens and accepted lengths of the launches it replaces, step
    after step of a K = 3 decode, on a handle of each kind (the 12-layer one is
    the benchmark's)."""
    from speculative_moe_decoding_amd import ocrdec
    cfg = {"f32_2layer": SMALL32, "bf16_2layer": SMALL16, "bf16_12layer": synth.FULL}[which]
    w = synth.Weights(cfg, 1234 if which == "bf16_12layer" else 95)
    page = synth.make_pages(cfg, 96, [24], [6], [40])[0]
    K, N = 3, 40
    decs = [ocrdec.Decoder(cfg, w.device_arrays(), max_batch=1, max_k=K, max_positions=256) for _ in range(2)]
    assert ocrdec.ocrdec_moe_grid(decs[0].h) > 0
    ocrdec.ocrdec_set_moe_launches(decs[0].h, True)
    ocrdec.ocrdec_set_moe_launches(decs[1].h, False)
    log(f"case {which}: persistent MoE grid {ocrdec.ocrdec_moe_grid(decs[0].h)} workgroups")
    runs = [run_gpu_steps(dec, page, N, K) for dec in decs]
    (ta, sa), (tb, sb) = runs
    assert ta == tb
    assert len(sa) == len(sb)
    for x, y in zip(sa, sb):
        assert x["drafts"] == y["drafts"] and x["greedy"] == y["greedy"] and x["n"] == y["n"]
        assert np.array_equal(x["logits"], y["logits"])
    log(f"{which}: {len(sa)} steps, fused and five-launch MoE bitwise equal")
