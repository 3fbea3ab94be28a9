"""Plain CPU oracle of the jina-ocr-v1 decoder with FastMTP speculative decoding.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The product
path (the ``ocrdec`` HIP library and its Python binding) never calls it, and
this module imports nothing from the product: it shares only the seeded input
generator (``speculative_moe_decoding_amd.synth``), which holds no decoder
arithmetic.

Everything here is computed in float64 with NumPy, one obvious step at a time,
on the exact values the model stores (bf16 matrices widened to float).  Where a
floating-point value decides an integer (router top-k, greedy argmax) the
decision is taken on the float32 rounding of the float64 value, the precision
the GPU path decides in.

Sources (jina-ocr-v1 pages):
  * announcement / blog spec table ("Model and training" section, spec table):
    12-layer DeepSeek-3B-MoE decoder, d = 1280, 64 routed + 2 shared experts,
    top-6, vocabulary 129,280, RoPE theta = 10^6 with a 32,768 position limit,
    one shared dense MTP block applied recursively for K = 3 steps;
  * blog, "Model and training": the verifier checks each proposal greedily and
    keeps the longest prefix on which draft and verifier agree, so the committed
    sequence is the verifier's greedy sequence;
  * blog, "Speculative decoding on L4" table caption: tau counts the bonus token
    the verifier adds after the accepted prefix;
  * blog, "Getting started": the draft head is trained with recursive
    hidden-state feedback (registered as an EAGLE-style proposer).

Readings of what the pages leave open:
  pre-norm residual blocks with RMSNorm (eps 1e-6, per-channel gain); MHA with
  10 heads of 128, no biases, scale 1/sqrt(128), causal; rotate-half RoPE over
  all 128 dims with inv_freq_i = theta^(-2i/128); every decoder layer is MoE;
  router = softmax over the 64 routed experts, top-6 taken on the logits
  (softmax is strictly increasing, so it is the same set), ties to the lower
  index, gate = the softmax probability (no renormalisation); the two shared
  experts have gate 1; experts are SwiGLU, F(b) = W_d (silu(W_g b) * W_u b);
  untied embedding and LM head; greedy argmax takes the lowest id on ties.
  Precision: a bf16 model stores its matrices and its KV cache in bf16; the
  oracle computes on the stored values and rounds keys (after RoPE) and values
  to bf16 where they enter the cache; everything else stays float64.
  Draft: the row at position p takes (h_{p-1}, e_p) -- the verifier's pre-norm
  final hidden of the previous position and the input embedding of p -- fuses
  u = W_f [RMSNorm(h); RMSNorm(e)], runs one dense pre-norm block (attention
  over the draft's own KV cache, SwiGLU of width 3,584) and predicts the token
  at p+1 through RMSNorm and the shared LM head; its output u is fed back as the
  hidden of the next draft row.  Accepted rows are recomputed by the next draft
  call from verifier hiddens ("catch-up").
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# single operations
# ----------------------------------------------------------------------------

def linear(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """y = W x for every row x of ``x``; W has shape [out, in]."""
    return np.asarray(x, F64) @ np.asarray(W, F64).T


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, F64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, F64)


def rope(x: np.ndarray, pos: Sequence[int], theta: float) -> np.ndarray:
    """Rotary position embedding, rotate-half form.

    x: [T, H, hd] at positions pos[T].  Dimension i (< hd/2) is paired with
    i + hd/2 and the pair is rotated by the angle pos * theta^(-2i/hd)
    (RoPE with theta = 10^6 per the spec table)."""
    x = np.asarray(x, F64)
    hd = x.shape[-1]
    half = hd // 2
    inv_freq = float(theta) ** (-(2.0 * np.arange(half, dtype=F64)) / hd)
    ang = np.asarray(pos, F64)[:, None] * inv_freq[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def causal_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, q_pos: Sequence[int]) -> np.ndarray:
    """Softmax attention, one head group at a time.

    q: [T, H, hd] queries at positions q_pos; K, V: [L, H, hd] cached keys and
    values of positions 0..L-1.  Query t sees keys 0..q_pos[t] (causal);
    scores are scaled by 1/sqrt(hd)."""
    q = np.asarray(q, F64)
    hd = q.shape[-1]
    s = np.einsum("thd,lhd->htl", q, np.asarray(K, F64)) / np.sqrt(hd)
    L = K.shape[0]
    future = np.arange(L)[None, :] > np.asarray(q_pos)[:, None]
    s = np.where(future[None, :, :], -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("htl,lhd->thd", p, np.asarray(V, F64))


def softmax(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, F64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def route_logits(logits: np.ndarray, top_k: int):
    """Softmax top-k selection from router logits [T, E].

    Returns (idx [T, k] int, gate [T, k] float64).  idx lists the chosen experts
    by decreasing score; the choice is made on the float32 rounding of the
    logits with ties going to the lower expert index.  gate is the softmax
    probability over all routed experts (not renormalised)."""
    logits = np.asarray(logits, F64)
    lf = logits.astype(np.float32).astype(F64)
    E = logits.shape[-1]
    idx = np.empty((logits.shape[0], top_k), dtype=np.int64)
    for t in range(logits.shape[0]):
        order = np.lexsort((np.arange(E), -lf[t]))
        idx[t] = order[:top_k]
    probs = softmax(logits)
    gate = np.take_along_axis(probs, idx, axis=-1)
    return idx, gate


def route(b: np.ndarray, W_r: np.ndarray, top_k: int):
    """Softmax top-k router: route_logits of the logits W_r b.
    Returns (idx, gate, logits)."""
    logits = linear(b, W_r)
    idx, gate = route_logits(logits, top_k)
    return idx, gate, logits


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, F64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(b: np.ndarray, W_g: np.ndarray, W_u: np.ndarray, W_d: np.ndarray) -> np.ndarray:
    """F(b) = W_d (silu(W_g b) * W_u b)."""
    return linear(silu(linear(b, W_g)) * linear(b, W_u), W_d)


def moe(b: np.ndarray, W_r, W_g, W_u, W_d, n_experts: int, n_shared: int, top_k: int, router_logits=None,
        pick=None):
    """y = sum_shared F_s(b) + sum_{j<k} gate_j F_{idx_j}(b).

    Expert tensors hold the routed experts first, then the shared ones.  With
    router_logits [T, E] given, the routing is taken from them instead of W_r b
    (the long-context benchmark's synthetic skewed routing).  pick (optional)
    is called as pick(logits [T, E], idx [T, k]) and returns the selection to
    use (a parity harness that follows another implementation's choice at a
    near tie); the gates stay the softmax probabilities of the experts used."""
    b = np.asarray(b, F64)
    if router_logits is None:
        logits = linear(b, W_r)
    else:
        logits = np.asarray(router_logits, F64)
    idx, gate = route_logits(logits, top_k)
    if pick is not None:
        idx = np.asarray(pick(logits, idx), dtype=np.int64)
        gate = np.take_along_axis(softmax(logits), idx, axis=-1)
    y = np.zeros_like(b)
    for s in range(n_shared):
        e = n_experts + s
        y += swiglu(b, W_g[e], W_u[e], W_d[e])
    for e in np.unique(idx):
        rows, slot = np.nonzero(idx == e)
        y[rows] += gate[rows, slot][:, None] * swiglu(b[rows], W_g[e], W_u[e], W_d[e])
    return y, idx


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value (8 significant bits, ties to even),
    directly from float64.  A bf16 model stores its KV cache in bf16."""
    x = np.asarray(x, F64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def greedy(logits: np.ndarray) -> np.ndarray:
    """Greedy token: argmax of the float32-rounded logits, lowest id on ties."""
    return np.argmax(np.asarray(logits, F64).astype(np.float32), axis=-1)


def top2_margin(logits: np.ndarray) -> np.ndarray:
    """Largest minus second-largest logit along the last axis (0 at a tie of
    the two largest): the gap a rounding difference must close to change the
    greedy token, so token mismatches are excused only where it is small."""
    lf = np.sort(np.asarray(logits, F64), axis=-1)
    return lf[..., -1] - lf[..., -2]


# ----------------------------------------------------------------------------
# counter-based generator for the controlled-acceptance drafts
# ----------------------------------------------------------------------------

_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """SplitMix64 output function applied to state x (Steele, Lea & Flood 2014;
    the form Vigna publishes as splitmix64.c): add the golden gamma, then two
    xor-shift-multiply rounds and a final xor-shift."""
    z = (x + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def draft_hash(seed: int, seq: int, step: int, slot: int) -> int:
    """H(seed, b, s, j): chained SplitMix64 over the counter (b, s, j)."""
    h = splitmix64(seed & _M64)
    for v in (seq, step, slot):
        h = splitmix64(h ^ (v & _M64))
    return h


def replace_threshold(p: float) -> int:
    """Integer threshold on the top 53 bits of H: replace iff (H >> 11) < floor(p * 2^53)."""
    return int(p * float(1 << 53))


def controlled_token(true_tok: int, h: int, thr: int, vocab: int) -> int:
    """Keep the verifier's own next token unless the top 53 bits of h fall under
    thr; a replaced token is always different from the true one."""
    if (h >> 11) < thr:
        return (true_tok + 1 + (h & 0xFFFFFFFF) % (vocab - 1)) % vocab
    return true_tok


# ----------------------------------------------------------------------------
# model
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class StepRecord:
    position: int               # position of the pending token (first verify row)
    drafts: List[int]           # d_1..d_K proposed
    greedy: List[int]           # g_0..g_K of the verifier
    accepted: int               # n
    logits: Optional[np.ndarray] = None   # [K+1, V] verifier logits (kept on request)
    draft_margins: Optional[List[float]] = None   # top-2 margin of each draft pass's logits
    real_drafts: Optional[List[int]] = None       # the draft block's proposals (also when a proposer replaced them)


class Oracle:
    """The decoder, its draft block, and the AR / speculative greedy loops.

    ``weights``: mapping name -> float array (see synth.weight_specs for names
    and shapes); values are used exactly as given.  One ``Oracle`` serves any
    number of independent sequences (``SeqState``)."""

    def __init__(self, cfg, weights: Dict[str, np.ndarray], cache_dense: bool = True):
        self.cfg = cfg
        self.w = weights
        self._cache: Dict[str, np.ndarray] = {}
        self.cache_dense = cache_dense

    # matrices used on every row are widened to float64 once
    def W(self, name: str) -> np.ndarray:
        if not self.cache_dense:
            return self.w[name]
        a = self._cache.get(name)
        if a is None:
            a = np.asarray(self.w[name], F64)
            self._cache[name] = a
        return a

    def embed(self, ids) -> np.ndarray:
        return np.asarray(self.w["embed"][np.asarray(ids, dtype=np.int64)], F64)

    # -- verifier ------------------------------------------------------------
    def new_state(self, max_pos: int) -> "SeqState":
        c = self.cfg
        return SeqState(
            kv=np.zeros((c.n_layers, 2, max_pos, c.n_heads, c.head_dim), F64),
            dkv=np.zeros((2, max_pos, c.n_heads, c.head_dim), F64))

    def attention_block(self, x, pos, norm, wqkv, wo, K_cache, V_cache):
        """x += W_o Attn(RoPE(q), RoPE(k), v) of RMSNorm(x); writes k, v at pos."""
        c = self.cfg
        T = x.shape[0]
        a = rmsnorm(x, self.w[norm], c.norm_eps)
        qkv = linear(a, self.W(wqkv))
        Hd = c.qkv_dim
        q = qkv[:, :Hd].reshape(T, c.n_heads, c.head_dim)
        k = qkv[:, Hd:2 * Hd].reshape(T, c.n_heads, c.head_dim)
        v = qkv[:, 2 * Hd:].reshape(T, c.n_heads, c.head_dim)
        q = rope(q, pos, c.rope_theta)
        k = rope(k, pos, c.rope_theta)
        if getattr(c, "dtype", "f32") == "bf16":
            k, v = round_bf16(k), round_bf16(v)
        K_cache[pos] = k
        V_cache[pos] = v
        L = int(pos[-1]) + 1
        o = causal_attention(q, K_cache[:L], V_cache[:L], pos)
        return x + linear(o.reshape(T, Hd), self.W(wo))

    def verifier_forward(self, st: "SeqState", x_in: np.ndarray, pos: Sequence[int], record=None,
                         router_logits=None, pick=None):
        """Rows x_in [T, d] at consecutive positions ``pos`` through all layers.
        Returns the pre-norm final hidden [T, d].  router_logits (optional
        [n_layers][T][E]) replaces each layer's router logits; pick (optional)
        is called as pick(layer, positions, logits, idx) and may replace the
        selection (see moe)."""
        c = self.cfg
        x = np.asarray(x_in, F64).copy()
        pos = np.asarray(pos, dtype=np.int64)
        for l in range(c.n_layers):
            x = self.attention_block(x, pos, f"l{l}.attn_norm", f"l{l}.wqkv", f"l{l}.wo",
                                     st.kv[l, 0], st.kv[l, 1])
            b = rmsnorm(x, self.w[f"l{l}.ffn_norm"], c.norm_eps)
            lp = None if pick is None else (lambda lg, ix, _l=l: pick(_l, pos, lg, ix))
            y, idx = moe(b, self.W(f"l{l}.router"), self.w[f"l{l}.w_gate"], self.w[f"l{l}.w_up"],
                         self.w[f"l{l}.w_down"], c.n_experts, c.n_shared, c.top_k,
                         None if router_logits is None else router_logits[l], lp)
            if record is not None:
                record.append(idx)
            x = x + y
        return x

    def lm_logits(self, h: np.ndarray, norm: str = "final_norm") -> np.ndarray:
        return linear(rmsnorm(h, self.w[norm], self.cfg.norm_eps), self.W("lm_head"))

    # -- draft ---------------------------------------------------------------
    def draft_forward(self, st: "SeqState", h: np.ndarray, e: np.ndarray, pos: Sequence[int]) -> np.ndarray:
        """Draft rows: (h_{p-1}, e_p) at positions pos -> block output u (fed back as h)."""
        c = self.cfg
        pos = np.asarray(pos, dtype=np.int64)
        hn = rmsnorm(h, self.w["draft.norm_h"], c.norm_eps)
        en = rmsnorm(e, self.w["draft.norm_e"], c.norm_eps)
        u = linear(np.concatenate([hn, en], axis=-1), self.W("draft.fuse"))
        u = self.attention_block(u, pos, "draft.attn_norm", "draft.wqkv", "draft.wo", st.dkv[0], st.dkv[1])
        b = rmsnorm(u, self.w["draft.ffn_norm"], c.norm_eps)
        return u + swiglu(b, self.W("draft.w_gate"), self.W("draft.w_up"), self.W("draft.w_down"))

    def draft_logits(self, u: np.ndarray) -> np.ndarray:
        return self.lm_logits(u, "draft.out_norm")

    # -- loops ---------------------------------------------------------------
    def prefix_rows(self, vision: np.ndarray, prompt: Sequence[int]) -> np.ndarray:
        """Prefix layout: the vision rows, then the embeddings of the prompt ids."""
        return np.concatenate([np.asarray(vision, F64), self.embed(prompt)], axis=0)

    def prefill(self, st: "SeqState", vision, prompt, with_draft: bool, chunk: int = 512, pick=None,
                first_token: Optional[int] = None):
        """Prefix rows through the verifier (and the draft block when with_draft);
        output token 0 is the greedy token of the last prefix row, or
        first_token when given (a parity harness following another
        implementation's choice at a near tie)."""
        e = self.prefix_rows(vision, prompt)
        P = e.shape[0]
        h = np.empty_like(e)
        for lo in range(0, P, chunk):
            hi = min(P, lo + chunk)
            h[lo:hi] = self.verifier_forward(st, e[lo:hi], np.arange(lo, hi), pick=pick)
        logits = self.lm_logits(h[-1:])
        y0 = int(greedy(logits)[0]) if first_token is None else int(first_token)
        if with_draft:
            hprev = np.concatenate([np.zeros((1, e.shape[1]), F64), h[:-1]], axis=0)
            for lo in range(0, P, chunk):
                hi = min(P, lo + chunk)
                self.draft_forward(st, hprev[lo:hi], e[lo:hi], np.arange(lo, hi))
        st.prefix_len = P
        st.kv_len = P
        st.draft_len = P
        st.out = [y0]
        st.hbuf = h[-1:].copy()
        st.cu = [y0]
        st.first_logits = logits[0]
        return y0

    def generate_ar(self, vision, prompt, n_out: int, keep_logits: bool = False):
        """Plain greedy autoregressive decoding: n_out output tokens (the first one
        comes from the prefix's last row)."""
        P = vision.shape[0] + len(prompt)
        st = self.new_state(P + n_out + 1)
        self.prefill(st, vision, prompt, with_draft=False)
        logits_rows = [st.first_logits] if keep_logits else None
        while len(st.out) < n_out:
            h = self.verifier_forward(st, self.embed([st.out[-1]]), [st.kv_len])
            lg = self.lm_logits(h)
            st.out.append(int(greedy(lg)[0]))
            st.kv_len += 1
            if keep_logits:
                logits_rows.append(lg[0])
        return st.out[:n_out], logits_rows

    def teacher_forced(self, vision, prompt, tokens: Sequence[int], chunk: int = 512, pick=None,
                       keep_at: Sequence[int] = ()):
        """The verifier along a given output sequence (teacher forcing): the
        prefix rows, then tokens[0..N-2] as inputs at positions P..P+N-2, in
        batched forwards of ``chunk`` rows.  Output token t (0..N-1) is
        predicted by the row at position P-1+t.  Returns (greedy [N] -- argmax
        of the float32-rounded logits, lowest id on ties --, top-2 margin [N],
        {t: logits [V]} for t in keep_at, the state, whose cache holds all
        P+N-1 positions)."""
        e = np.concatenate([self.prefix_rows(vision, prompt), self.embed(list(tokens)[:-1])], axis=0)
        P = vision.shape[0] + len(prompt)
        N = len(tokens)
        st = self.new_state(P + N + 8)
        keep = set(int(t) for t in keep_at)
        g = np.empty(N, dtype=np.int64)
        mg = np.empty(N, dtype=F64)
        kept = {}
        for lo in range(0, e.shape[0], chunk):
            hi = min(e.shape[0], lo + chunk)
            h = self.verifier_forward(st, e[lo:hi], np.arange(lo, hi), pick=pick)
            r0 = max(lo, P - 1)                # rows that predict output tokens
            if r0 >= hi:
                continue
            lg = self.lm_logits(h[r0 - lo:])
            t0 = r0 - (P - 1)
            g[t0:t0 + lg.shape[0]] = greedy(lg)
            mg[t0:t0 + lg.shape[0]] = top2_margin(lg)
            for i in range(lg.shape[0]):
                if t0 + i in keep:
                    kept[t0 + i] = lg[i].copy()
        st.kv_len = e.shape[0]
        return g, mg, kept, st

    def draft_propose(self, st: "SeqState", K: int) -> List[int]:
        """K recursive passes of the shared draft block.  Pass 1 re-runs the
        catch-up rows draft_len..kv_len from verifier hiddens; passes 2..K feed
        the block's own output back."""
        pos = np.arange(st.draft_len, st.kv_len + 1)
        assert len(pos) == len(st.cu) == st.hbuf.shape[0]
        u = self.draft_forward(st, st.hbuf, self.embed(st.cu), pos)
        lg = self.draft_logits(u[-1:])
        d = [int(greedy(lg)[0])]
        st.draft_margins = [float(top2_margin(lg)[0])]
        prev = u[-1:]
        for j in range(2, K + 1):
            u = self.draft_forward(st, prev, self.embed([d[-1]]), [st.kv_len + j - 1])
            lg = self.draft_logits(u)
            d.append(int(greedy(lg)[0]))
            st.draft_margins.append(float(top2_margin(lg)[0]))
            prev = u
        return d

    def generate_spec(self, vision, prompt, n_out: int, K: int,
                      proposer: Optional[Callable] = None, keep_logits: bool = False,
                      seq_index: int = 0, draft_for_cost: bool = False, max_steps: Optional[int] = None,
                      greedy_hook: Optional[Callable] = None, pick: Optional[Callable] = None,
                      first_token: Optional[int] = None, state_out: Optional[list] = None,
                      k_schedule: Optional[Callable] = None):
        """FastMTP speculative decoding with greedy longest-prefix acceptance.

        proposer(step, committed_tokens, K) -> K tokens replaces the draft block
        (losslessness tests, controlled acceptance); None runs the draft block.
        draft_for_cost runs the draft block even when a proposer replaces its
        tokens (as the controlled-acceptance benchmark does); its proposals are
        recorded as real_drafts.  max_steps bounds the number of speculative
        steps.  greedy_hook(step, g, logits) -> tokens (optional) may replace
        the verifier's greedy tokens of a step before acceptance, and pick the
        routing (see verifier_forward): a parity harness uses them to follow
        another implementation's choice at a near tie, so both keep one history;
        first_token likewise replaces output token 0, and state_out (a list)
        receives the sequence state.  k_schedule(step) -> depth (optional, at
        most K) changes the draft depth from step to step; the catch-up pass
        recomputes whatever the previous step accepted, whatever its depth.
        Returns (tokens[:n_out], [StepRecord])."""
        P = vision.shape[0] + len(prompt)
        st = self.new_state(P + n_out + K + 2)
        self.prefill(st, vision, prompt, with_draft=proposer is None or draft_for_cost, pick=pick,
                     first_token=first_token)
        if state_out is not None:
            state_out.append(st)
        steps: List[StepRecord] = []
        K_max = K
        while len(st.out) < n_out and (max_steps is None or len(steps) < max_steps):
            K = K_max if k_schedule is None else int(k_schedule(len(steps)))
            assert 0 <= K <= K_max
            real = None
            if proposer is None:
                d = self.draft_propose(st, K)
                real = list(d)
            else:
                if draft_for_cost and K > 0:
                    real = self.draft_propose(st, K)
                d = [int(t) for t in proposer(len(steps), list(st.out), K)]
            q = st.kv_len
            rows = [st.out[-1]] + d
            h = self.verifier_forward(st, self.embed(rows), np.arange(q, q + K + 1), pick=pick)
            lg = self.lm_logits(h)
            g = [int(t) for t in greedy(lg)]
            if greedy_hook is not None:
                g = [int(t) for t in greedy_hook(len(steps), g, lg)]
            n = 0
            while n < K and d[n] == g[n]:
                n += 1
            st.out += d[:n] + [g[n]]
            steps.append(StepRecord(q, d, g, n, lg if keep_logits else None,
                                    st.draft_margins if real is not None else None, real))
            # rollback: verifier KV keeps positions < q + n + 1; the draft KV keeps
            # position q (computed from a true verifier hidden); the next catch-up
            # recomputes draft rows q+1 .. q+n+1 from the verifier hiddens h[0..n].
            st.draft_len = q + 1
            st.hbuf = h[:n + 1].copy()
            st.cu = d[:n] + [g[n]]
            st.kv_len = q + n + 1
        return st.out[:n_out], steps


@dataclasses.dataclass
class SeqState:
    kv: np.ndarray
    dkv: np.ndarray
    prefix_len: int = 0
    kv_len: int = 0
    draft_len: int = 0
    out: list = dataclasses.field(default_factory=list)
    hbuf: Optional[np.ndarray] = None
    cu: list = dataclasses.field(default_factory=list)
    first_logits: Optional[np.ndarray] = None
    draft_margins: Optional[list] = None


# ----------------------------------------------------------------------------
# proposers used by tests and the controlled-acceptance workloads
# ----------------------------------------------------------------------------

def trace_proposer(trace: Sequence[int]):
    """Always-right drafts: the verifier's own greedy continuation."""
    def propose(step, out, K):
        c = len(out)
        return [trace[c - 1 + j] if c - 1 + j < len(trace) else 0 for j in range(1, K + 1)]
    return propose


def wrong_proposer(trace: Sequence[int], vocab: int):
    """Always-wrong first draft."""
    def propose(step, out, K):
        c = len(out)
        return [((trace[c] if c < len(trace) else 0) + 1) % vocab for _ in range(K)]
    return propose


def random_proposer(seed: int, vocab: int):
    rng = np.random.default_rng(seed)

    def propose(step, out, K):
        return [int(t) for t in rng.integers(0, vocab, size=K)]
    return propose


def controlled_proposer(trace: Sequence[int], seed: int, p: float, vocab: int, seq_index: int = 0):
    """Draft slot j of verify step s proposes the verifier's true next token,
    replaced with probability p by a different token drawn from H(seed, b, s, j)."""
    thr = replace_threshold(p)

    def propose(step, out, K):
        c = len(out)
        res = []
        for j in range(1, K + 1):
            t = c - 1 + j
            true_tok = int(trace[t]) if t < len(trace) else 0
            res.append(controlled_token(true_tok, draft_hash(seed, seq_index, step, j), thr, vocab))
        return res
    return propose


def controlled_accepts(n_out: int, K: int, seed: int, p: float, seq_index: int = 0,
                       k_schedule: Optional[Callable] = None) -> List[int]:
    """Accepted lengths of a lossless speculative run whose drafts come from
    controlled_proposer: n = number of leading slots that were not replaced
    (depth K, or k_schedule(step) at each step)."""
    thr = replace_threshold(p)
    K_max = K
    out_len, step, res = 1, 0, []
    while out_len < n_out:
        K = K_max if k_schedule is None else int(k_schedule(step))
        n = 0
        while n < K and (draft_hash(seed, seq_index, step, n + 1) >> 11) >= thr:
            n += 1
        res.append(n)
        out_len += n + 1
        step += 1
    return res


def active_params(cfg) -> Dict[str, int]:
    """Parameter counts of the decoder (without the draft): total and active per token."""
    d, Hd = cfg.d_model, cfg.qkv_dim
    attn = 3 * Hd * d + d * Hd
    expert = 3 * d * cfg.d_expert
    router = cfg.n_experts * d
    per_layer_total = attn + router + (cfg.n_experts + cfg.n_shared) * expert
    per_layer_active = attn + router + (cfg.top_k + cfg.n_shared) * expert
    head = cfg.vocab * d
    return dict(total=cfg.n_layers * per_layer_total + 2 * head,
                active=cfg.n_layers * per_layer_active + head)
