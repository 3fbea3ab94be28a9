"""Long-context layer: one MoE layer + final norm + LM head (bf16, full
vocabulary) verifying 4 rows per sequence at positions 32,764..32,767 against a
loaded cache of 32,764 positions (keys / values ~ N(0, 1) in bf16), with the
skewed synthetic routing (router logits = log pi + Gumbel, pi ~ rank^-1.1).

Batch 1 runs the vector path, batches 4, 16 and 64 the matrix path (16, 64
and 256 rows per call).  The logits of the first and last sequence's rows
match the oracle (5e-2; greedy tokens exact unless the oracle's top-2 margin
is under that), and the routing taps equal the oracle's selection from the
same logits."""
import dataclasses

import numpy as np
import pytest

from oracle import decoder as od
from speculative_moe_decoding_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import log  # noqa: E402
from speculative_moe_decoding_amd import ocrdec  # noqa: E402

TOL = 5e-2


@pytest.fixture(scope="module")
def setup():
    wl = synth.WORKLOADS["longctx_layer_bf16"]
    cfg = wl["cfg"]
    w = synth.Weights(cfg, wl["weight_seed"])
    n_pos = wl["n_cached"]
    kv_bits = synth.longctx_kv(cfg, wl["kv_seed"], n_pos)
    kv_dev = torch.from_numpy(kv_bits.view(np.int16)).cuda()
    orc = od.Oracle(cfg, w.f32)
    return wl, cfg, w, n_pos, kv_bits, kv_dev, orc


@pytest.mark.parametrize("B", [1, 4, 16, 64])
def test_longctx_layer_vs_oracle(setup, B):
    wl, cfg, w, n_pos, kv_bits, kv_dev, orc = setup
    K = 3
    log(f"case B={B}")
    dec = ocrdec.Decoder(cfg, w.device_arrays(), max_batch=B, max_k=K, max_positions=n_pos + K + 1)
    rng = np.random.default_rng([wl["input_seed"], B])
    pend = rng.integers(0, cfg.vocab, size=B)
    drafts = rng.integers(0, cfg.vocab, size=(B, K)).astype(np.int32)
    for b in range(B):
        ocrdec.ocrdec_load_sequence(dec.h, dec.stream, b, n_pos, int(pend[b]), kv_dev)
    rl = synth.zipf_router_logits(wl["input_seed"] + B, B * (K + 1))
    rl_dev = torch.from_numpy(rl).cuda()
    ocrdec.ocrdec_set_router_logits(dec.h, rl_dev)
    route = torch.full((1, B * (K + 1), 8), -1, dtype=torch.int32, device="cuda")
    ocrdec.ocrdec_set_taps(dec.h, route, None)
    draft = torch.from_numpy(drafts).cuda()
    logits = torch.empty(B, K + 1, cfg.vocab, dtype=torch.float32, device="cuda")
    greedy = dec.verify(B, K, draft, logits=logits)
    torch.cuda.synchronize()
    g_logits = logits.cpu().numpy()
    g_tok = greedy.cpu().numpy()
    g_route = route.cpu().numpy()[0]
    # oracle: the loaded cache (bf16 values), rows [pending, d1, d2, d3]
    st = orc.new_state(n_pos + K + 1)
    kv = synth.bf16_bits_to_f32(kv_bits)            # [1][K|V][head][pos][dim]
    st.kv[0, :, :n_pos] = np.transpose(kv[0], (0, 2, 1, 3))
    checked = 0
    for b in sorted({0, B - 1}):
        ids = [int(pend[b])] + drafts[b].tolist()
        rows = slice(b * (K + 1), (b + 1) * (K + 1))
        rec = []
        h = orc.verifier_forward(st, orc.embed(ids), np.arange(n_pos, n_pos + K + 1), record=rec,
                                 router_logits=rl[:, rows])
        ref = orc.lm_logits(h)
        assert [list(r) for r in g_route[rows, :6]] == [list(r) for r in rec[0]]
        assert (g_route[rows, 6:] == [64, 65]).all()
        diff = float(np.abs(g_logits[b] - ref).max())
        log(f"B={B} seq {b}: max |dlogit| {diff:.3e}")
        assert diff < TOL
        margins = od.top2_margin(ref)
        for i in range(K + 1):
            if g_tok[b, i] != od.greedy(ref[i:i + 1])[0]:
                assert margins[i] < TOL, (b, i, margins[i])
        checked += 1
    assert checked >= 1
