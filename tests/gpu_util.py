"""Helpers shared by the GPU parity tests: build a decoder and an oracle over
the same seeded weights, run decode loops through the C ABI, and compare with
the tolerance rules.

Rules (a reading of the tolerances the parity target states):
  * tokens exact, a mismatch excused only where the oracle's top-2 logit
    margin at that row is under the tolerance (1e-3 fp32, 5e-2 bf16);
  * logits within the same absolute tolerance;
  * routing exact, a different choice excused only where every expert the GPU
    put at rank k has an oracle logit within ``route_tol`` of the oracle's k-th
    largest logit (a near tie), and then the oracle follows the GPU's choice;
  * wherever a choice is excused, the oracle continues with the GPU's choice
    (forced history), so one mismatch never ends the comparison."""
import dataclasses
import sys
import time

import numpy as np

from oracle import decoder as od
from speculative_moe_decoding_amd import synth

ROUTE_TOL = {"f32": 1e-4, "bf16": 1e-3}


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
    """Free-running comparison of step records (drafts, greedy tokens,
    accepted lengths exact; logits within tol on the rows both runs commit).
    The first differing draft or greedy row is excused only if the oracle's
    top-2 margin at that very row is under tol; comparison then stops (the two
    runs follow different sequences from there).  Returns (steps compared,
    max |logit diff|, note on an excused flip or None)."""
    worst = 0.0
    for s, (g, r) in enumerate(zip(gpu_steps, ref_steps)):
        if check_drafts and g["drafts"] != r.drafts:
            j = next(i for i in range(len(r.drafts)) if g["drafts"][i] != r.drafts[i])
            if r.draft_margins is not None and r.draft_margins[j] < tol:
                return s, worst, f"step {s}: draft {j} differs at a near tie (margin {r.draft_margins[j]:.2e})"
            raise AssertionError(f"step {s}: drafts {g['drafts']} != oracle {r.drafts} "
                                 f"(margins {r.draft_margins})")
        n_rows = r.accepted + 1
        if g["logits"] is not None:
            worst = max(worst, float(np.abs(g["logits"][:n_rows] - r.logits[:n_rows]).max()))
        diff = [i for i in range(n_rows) if g["greedy"][i] != r.greedy[i]]
        if diff:
            i = diff[0]
            m = float(od.top2_margin(r.logits[i]))
            if m < tol:
                return s, worst, f"step {s}: greedy row {i} differs at a near tie (margin {m:.2e})"
            raise AssertionError(f"step {s}: greedy {g['greedy']} n={g['n']} != oracle {r.greedy} n={r.accepted}; "
                                 f"row {i} margin {m:.3e}")
        assert g["n"] == r.accepted, (s, g["n"], r.accepted)
    return min(len(gpu_steps), len(ref_steps)), worst, None


class RoutePicker:
    """The oracle's routing hook for a parity run: where the GPU's routing of a
    row is known (route(layer, position) -> 6 experts, or None), the oracle
    compares it with its own; a different choice is accepted only as a near
    tie (see the module rules) and then followed.  Counts every decision."""

    def __init__(self, route, tol):
        self.route, self.tol = route, tol
        self.decisions = self.exact = self.near = 0
        self.max_dev = 0.0
        self.hard = []

    def __call__(self, layer, positions, logits, idx):
        out = idx.copy()
        lf = np.asarray(logits, np.float64).astype(np.float32).astype(np.float64)
        for r, p in enumerate(positions):
            g = self.route(layer, int(p))
            if g is None:
                continue
            g = [int(e) for e in g]
            self.decisions += 1
            if g == [int(e) for e in idx[r]]:
                self.exact += 1
                continue
            top = np.sort(lf[r])[::-1]
            ok = len(set(g)) == len(g) and all(0 <= e < lf.shape[1] for e in g)
            dev = max(abs(lf[r][e] - top[k]) for k, e in enumerate(g)) if ok else np.inf
            if dev < self.tol:
                self.near += 1
                self.max_dev = max(self.max_dev, dev)
                out[r] = g
            else:
                self.hard.append((layer, int(p), [int(e) for e in idx[r]], g, float(dev)))
        return out

    def summary(self):
        return (f"routing: {self.decisions} decisions, {self.exact} exact, {self.near} near ties followed "
                f"(largest logit gap {self.max_dev:.1e}), {len(self.hard)} mismatches")


def position_route_tap(dec, slot, cap):
    """Device buffer for the by-position routing tap of one slot."""
    import torch
    from speculative_moe_decoding_amd import ocrdec
    buf = torch.full((dec.cfg.n_layers, cap, 8), -1, dtype=torch.int32, device="cuda")
    return buf


@dataclasses.dataclass
class ForcedRun:
    steps: int
    drafts_compared: int
    drafts_excused: int
    greedy_compared: int
    greedy_excused: int
    worst_logit: float
    n_values: set
    picker: RoutePicker


def forced_spec_parity(dec, orc, page, N, K, tol, p_replace, seed=3000, graphs=False, route_tol=None,
                       min_steps=4, k_sched=None):
    """FastMTP at depth K on one page with acceptance driven by the controlled
    drafts (the GPU's own K = 0 sequence, each slot replaced with probability
    p_replace), so that the catch-up pass of the real draft block carries 1 ..
    K + 1 rows; the block's own proposals are captured before the override
    (drafts tap) and compared with the oracle's draft_propose under the same
    history.  Eager: verify logits (all K + 1 rows) and greedy tokens compared
    at every step, routing from the per-call tap.  graphs: decode-step graph
    replays; accepted lengths from the accepted tap, greedy tokens of the
    committed rows from the output, routing from the by-position tap.  The
    oracle follows the GPU at excused near ties (forced history).  Accepted
    lengths must equal the SplitMix64 prediction (the run is lossless).
    k_sched(step) -> depth (optional, at most K) changes the depth per step
    (graphs: one decode-step call per step)."""
    import torch
    from speculative_moe_decoding_amd import ocrdec
    cfg = dec.cfg
    V = cfg.vocab
    P = page.prefix_len
    route_tol = ROUTE_TOL[cfg.dtype] if route_tol is None else route_tol
    ar, _, _ = dec.generate([page], N + K + 2, 0, check_every=8)
    trace_np = ar[0].astype(np.int32)
    trace = torch.from_numpy(trace_np[None].copy()).cuda()
    thr = od.replace_threshold(p_replace)
    cap = N + 2
    acc_tap = torch.full((dec.max_batch, cap), -9, dtype=torch.int32, device="cuda")
    dr_tap = torch.full((dec.max_batch, cap, 8), -9, dtype=torch.int32, device="cuda")
    pos_cap = P + N + K + 4
    route_pos = torch.full((cfg.n_layers, pos_cap, 8), -1, dtype=torch.int32, device="cuda")
    rows = K + 1
    route_call = torch.full((cfg.n_layers, rows, 8), -1, dtype=torch.int32, device="cuda")
    ocrdec.ocrdec_set_taps(dec.h, route_idx=None if graphs else route_call, route_pos=route_pos,
                           route_pos_slot=0, accepted=acc_tap, drafts=dr_tap)
    gsteps = []
    ks = (lambda s_: K) if k_sched is None else k_sched
    try:
        if graphs:
            if k_sched is None:
                toks, _, nst = dec.generate([page], N, K, trace=trace, seed=seed, threshold=thr, check_every=2,
                                            graphs=True)
                toks = toks[0].tolist()
            else:
                draft, greedy = dec.i32(1, K), dec.i32(1, K + 1)
                n_acc, out_len = dec.i32(1), dec.i32(1)
                out_tokens = torch.zeros(1, N + K + 2, dtype=torch.int32, device="cuda")
                out_tokens[:, 0] = dec.prefill([page])
                s = 0
                while True:
                    dec.decode_steps(1, ks(s), 1, draft, greedy, n_acc, out_tokens, out_len, trace, seed, thr)
                    s += 1
                    ocrdec.ocrdec_sync_positions(dec.h, dec.stream)
                    if int(out_len.item()) >= N:
                        break
                toks = out_tokens.cpu().numpy()[0][:N].tolist()
            torch.cuda.synchronize()
            acc = acc_tap.cpu().numpy()[0]
            drs = dr_tap.cpu().numpy()[0]
            c = 1
            s = 0
            while c < N:
                n = int(acc[s])
                Ks = ks(s)
                assert 0 <= n <= Ks, (s, n)
                g_rows = toks[c:c + n + 1] if c + n + 1 <= N else None
                gsteps.append(dict(real=drs[s, :Ks].tolist(), n=n, greedy=g_rows, logits=None, route=None))
                c += n + 1
                s += 1
            y0 = toks[0]
        else:
            pend = dec.prefill([page])
            y0 = int(pend.item())
            draft, greedy = dec.i32(1, K), dec.i32(1, K + 1)
            n_acc, out_len = dec.i32(1), dec.i32(1)
            out_tokens = torch.zeros(1, N + K + 2, dtype=torch.int32, device="cuda")
            out_tokens[:, 0] = pend
            lg = torch.empty(1, K + 1, V, dtype=torch.float32, device="cuda")
            c = 1
            while c < N:
                Ks = ks(len(gsteps))
                dk, gk, lk = draft[:, :Ks], greedy[:, :Ks + 1], lg[:, :Ks + 1]
                dec.draft(1, Ks, out=dk)
                real = dk.clone()
                dec.controlled(1, Ks, trace, seed, thr, dk)
                dec.verify(1, Ks, dk, greedy=gk, logits=lk)
                dec.accept(1, Ks, dk, gk, n_acc, out_tokens, out_len)
                torch.cuda.synchronize()
                n = int(n_acc.item())
                gsteps.append(dict(real=real.cpu().numpy()[0].tolist(), n=n, greedy=gk.cpu().numpy()[0].tolist(),
                                   logits=lk.cpu().numpy()[0],
                                   route=route_call.flatten()[:cfg.n_layers * (Ks + 1) * 8].cpu().numpy().reshape(
                                       cfg.n_layers, Ks + 1, 8)))
                c += n + 1
                if len(gsteps) % 8 == 0:
                    ocrdec.ocrdec_sync_positions(dec.h, dec.stream)
            toks = out_tokens.cpu().numpy()[0][:N].tolist()
        rpos = route_pos.cpu().numpy()
    finally:
        ocrdec.ocrdec_set_taps(dec.h)
    assert toks == trace_np[:N].tolist(), "speculative output differs from the GPU's K = 0 output"
    pred = od.controlled_accepts(N, K, seed, p_replace, k_schedule=k_sched)
    assert [s["n"] for s in gsteps] == pred[:len(gsteps)], "accepted lengths differ from the SplitMix64 prediction"

    # the oracle on the same history
    ctx = {"step": -1, "q": P}

    def gpu_route(layer, pos):
        if pos < P:
            r = rpos[layer, pos, :6]
            return None if r[0] < 0 else r
        s = ctx["step"]
        if s < 0 or s >= len(gsteps):
            return None
        i = pos - ctx["q"]
        st_ = gsteps[s]
        if st_["route"] is not None:
            return st_["route"][layer, i, :6] if 0 <= i < st_["route"].shape[1] else None
        if 0 <= i <= st_["n"]:                      # committed rows: the by-position tap
            r = rpos[layer, pos, :6]
            return None if r[0] < 0 else r
        return None

    picker = RoutePicker(gpu_route, route_tol)
    base_prop = od.controlled_proposer(trace_np.tolist(), seed, p_replace, V)

    def proposer(step, out, K_):
        ctx["step"] = step
        ctx["q"] = P + len(out) - 1
        return base_prop(step, out, K_)

    stats = dict(gc=0, ge=0, worst=0.0)

    def hook(step, g, lg):
        st_ = gsteps[step]
        if st_["logits"] is not None:
            stats["worst"] = max(stats["worst"], float(np.abs(st_["logits"] - lg).max()))
        ref = st_["greedy"]
        if ref is None:                             # last step past N: nothing committed to compare
            return g
        out = list(g)
        for i in range(len(ref)):
            stats["gc"] += 1
            if int(ref[i]) != g[i]:
                m = float(od.top2_margin(lg[i]))
                assert m < tol, f"step {step} row {i}: GPU {ref[i]} oracle {g[i]}, margin {m:.3e}"
                stats["ge"] += 1
                out[i] = int(ref[i])
        return out

    states = []
    otoks, osteps = orc.generate_spec(page.vision, page.prompt, N, K, proposer=proposer, draft_for_cost=True,
                                      greedy_hook=hook, pick=picker, first_token=y0, state_out=states,
                                      k_schedule=k_sched)
    fl = states[0].first_logits
    if int(od.greedy(fl[None])[0]) != y0:
        assert float(od.top2_margin(fl)) < tol, "first token differs without a near tie"
    assert otoks == toks
    assert [s.accepted for s in osteps] == [s["n"] for s in gsteps]
    dc = de = 0
    for s, (g, r) in enumerate(zip(gsteps, osteps)):
        for j in range(len(r.real_drafts)):
            dc += 1
            if g["real"][j] != r.real_drafts[j]:
                assert r.draft_margins[j] < tol, \
                    f"step {s}: real draft {j}: GPU {g['real']} oracle {r.real_drafts} margins {r.draft_margins}"
                de += 1
                break                                # later passes take the differing token as input
    assert not picker.hard, picker.hard[:5]
    assert stats["worst"] < tol, stats["worst"]
    assert len(gsteps) >= min_steps
    prev = [0] + [s["n"] for s in gsteps[:-1]]
    return ForcedRun(len(gsteps), dc, de, stats["gc"], stats["ge"], stats["worst"], set(prev), picker)


def forced_ar_parity(dec, orc, page, N, tol, min_steps=8):
    """Greedy AR decode of one page (K = 0) against the oracle under forced
    history: every token equal to the oracle's greedy token or excused at a
    near tie (then the oracle takes the GPU's token), logits within tol at
    every step.  Returns (GPU tokens, steps compared, near ties, max |dlogit|)."""
    g_toks, g_steps = run_gpu_steps(dec, page, N, 0)
    stats = dict(ex=0, worst=0.0)

    def hook(step, g, lg):
        ref = g_steps[step]
        stats["worst"] = max(stats["worst"], float(np.abs(ref["logits"] - lg).max()))
        if ref["greedy"][0] != g[0]:
            m = float(od.top2_margin(lg[0]))
            assert m < tol, f"step {step}: GPU {ref['greedy'][0]} oracle {g[0]}, margin {m:.3e}"
            stats["ex"] += 1
        return [ref["greedy"][0]]

    states = []
    o_toks, o_steps = orc.generate_spec(page.vision, page.prompt, N, 0, proposer=lambda s, out, K: [],
                                        greedy_hook=hook, first_token=g_toks[0], state_out=states)
    fl = states[0].first_logits
    if int(od.greedy(fl[None])[0]) != g_toks[0]:
        assert float(od.top2_margin(fl)) < tol, "first token differs without a near tie"
        stats["ex"] += 1
    assert o_toks == g_toks
    assert len(o_steps) >= min_steps
    assert stats["worst"] < tol, stats["worst"]
    return g_toks, len(o_steps), stats["ex"], stats["worst"]
