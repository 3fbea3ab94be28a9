"""Helpers shared by the GPU parity tests: build a decoder and an oracle over
the same seeded weights, run step-by-step loops through the C ABI, and compare
with the tolerance rules (tokens exact unless the oracle's top-2 margin is under
the tolerance; logits within an absolute tolerance)."""
import dataclasses
import sys
import time

import numpy as np

from oracle import decoder as od
from speculative_moe_decoding_amd import synth


def log(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def make_pair(cfg, wseed, max_batch=1, max_k=3, max_positions=512, cache_dense=True, path=0):
    import torch
    from speculative_moe_decoding_amd import ocrdec
    t = time.time()
    w = synth.Weights(cfg, wseed)
    dec = ocrdec.Decoder(cfg, w.device_arrays(), max_batch=max_batch, max_k=max_k, max_positions=max_positions,
                         path=path)
    orc = od.Oracle(cfg, w.f32, cache_dense=cache_dense)
    torch.cuda.synchronize()
    log(f"weights + upload for {cfg.n_layers} layers / V={cfg.vocab} / {cfg.dtype}: {time.time() - t:.1f}s")
    return w, dec, orc


def run_gpu_steps(dec, page, n_out, K, with_logits=True, proposer=None):
    """Step-by-step decode of one page through the C ABI; returns
    (tokens, [dict(drafts, greedy, n, logits)])."""
    import torch
    V = dec.cfg.vocab
    pending = dec.prefill([page])
    toks = [int(pending.item())]
    steps = []
    draft = dec.i32(1, max(K, 1))
    greedy = dec.i32(1, K + 1)
    n_acc = dec.i32(1)
    out_tokens = torch.zeros(1, n_out + K + 2, dtype=torch.int32, device="cuda")
    out_len = dec.i32(1)
    logits = torch.empty(1, K + 1, V, dtype=torch.float32, device="cuda") if with_logits else None
    while len(toks) < n_out:
        if K > 0:
            if proposer is None:
                dec.draft(1, K, out=draft)
            else:
                draft.copy_(torch.tensor([proposer(len(steps), list(toks), K)], dtype=torch.int32))
        dec.verify(1, K, draft, greedy=greedy, logits=logits)
        dec.accept(1, K, draft, greedy, n_acc, out_tokens, out_len)
        torch.cuda.synchronize()
        n = int(n_acc.item())
        d = draft.cpu().numpy()[0][:K].tolist() if K > 0 else []
        g = greedy.cpu().numpy()[0].tolist()
        steps.append(dict(drafts=d, greedy=g, n=n, logits=logits.cpu().numpy()[0] if with_logits else None))
        toks += d[:n] + [g[n]]
    return toks[:n_out], steps


def compare_steps(gpu_steps, ref_steps, tol, check_drafts=True):
    """Step records must agree exactly (drafts, greedy tokens, accepted lengths);
    a mismatch is excused only where the oracle's top-2 logit margin is under
    tol, and comparison stops there (the two runs then follow different
    sequences).  Logits must agree within tol on every compared row.  Returns
    (steps compared, max |logit diff|, note on an excused flip or None)."""
    worst = 0.0
    for s, (g, r) in enumerate(zip(gpu_steps, ref_steps)):
        n_rows = r.accepted + 1
        margins = od.top2_margin(r.logits[:n_rows])
        if g["logits"] is not None:
            worst = max(worst, float(np.abs(g["logits"][:n_rows] - r.logits[:n_rows]).max()))
        near = bool((margins < tol).any())
        if check_drafts and g["drafts"] != r.drafts:
            j = next(i for i in range(len(r.drafts)) if g["drafts"][i] != r.drafts[i])
            if r.draft_margins is not None and r.draft_margins[j] < tol:
                return s, worst, f"step {s}: draft {j} differs at a near tie (margin {r.draft_margins[j]:.2e})"
            raise AssertionError(f"step {s}: drafts {g['drafts']} != oracle {r.drafts} "
                                 f"(margins {r.draft_margins})")
        if g["greedy"][:n_rows] != r.greedy[:n_rows] or g["n"] != r.accepted:
            if near:
                return s, worst, f"step {s}: greedy differs at a near tie (margin {margins.min():.2e})"
            raise AssertionError(f"step {s}: greedy {g['greedy']} n={g['n']} != oracle {r.greedy} n={r.accepted}; "
                                 f"margins {margins}")
    return min(len(gpu_steps), len(ref_steps)), worst, None
