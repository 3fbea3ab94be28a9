"""Python binding of the ``ocrdec`` C ABI (include/ocrdec.h, and the harness
calls of include/ocrdec_harness.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libocrdec.so.  PyTorch supplies device memory and the stream.
The library must have been built (``python -m speculative_moe_decoding_amd.build``);
loading fails loudly otherwise -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libocrdec.so")

OCRDEC_OK, OCRDEC_EINVAL, OCRDEC_ECAPACITY, OCRDEC_EHIP = 0, -1, -2, -3
OCRDEC_F32, OCRDEC_BF16 = 0, 1
OCRDEC_PATH_AUTO, OCRDEC_PATH_VECTOR, OCRDEC_PATH_MATRIX = 0, 1, 2

SYMBOLS = (
    "ocrdec_state_bytes", "ocrdec_workspace_bytes", "ocrdec_num_weights", "ocrdec_create", "ocrdec_destroy",
    "ocrdec_prefill", "ocrdec_draft", "ocrdec_verify", "ocrdec_accept_rollback", "ocrdec_controlled_drafts",
    "ocrdec_set_taps", "ocrdec_expert_timing", "ocrdec_expert_stats", "ocrdec_replay_expert_gate_up",
    "ocrdec_decode_steps", "ocrdec_sync_positions", "ocrdec_load_sequence", "ocrdec_set_router_logits",
    "ocrdec_read_probe", "ocrdec_last_error", "ocrdec_decode_steps_noalloc", "ocrdec_set_moe_launches",
    "ocrdec_moe_grid", "ocrdec_release_slot", "ocrdec_kv_pages",
)


class ocrdec_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("n_layers", "d_model", "n_heads", "head_dim", "n_experts", "n_shared",
                                            "top_k", "d_expert", "d_draft_ffn", "vocab")] + [
        ("rope_theta", ctypes.c_float), ("norm_eps", ctypes.c_float), ("dtype", ctypes.c_int),
        ("max_batch", ctypes.c_int), ("max_k", ctypes.c_int), ("max_positions", ctypes.c_int),
        ("path", ctypes.c_int), ("kv_pages", ctypes.c_int)]


class ocrdec_controlled_cfg(ctypes.Structure):
    _fields_ = [("trace", ctypes.c_void_p), ("trace_stride", ctypes.c_int), ("trace_len", ctypes.c_int),
                ("seed", ctypes.c_uint64), ("threshold", ctypes.c_uint64)]


class ocrdec_taps(ctypes.Structure):
    _fields_ = [("route_idx", ctypes.c_void_p), ("hidden", ctypes.c_void_p), ("route_pos", ctypes.c_void_p),
                ("route_pos_slot", ctypes.c_int), ("route_pos_cap", ctypes.c_int), ("accepted", ctypes.c_void_p),
                ("drafts", ctypes.c_void_p), ("step_cap", ctypes.c_int)]


class OcrdecError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libocrdec.so not found at {path}: build it with "
                           f"`python -m speculative_moe_decoding_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, U64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64
    cfgp = ctypes.POINTER(ocrdec_config)
    sig = {
        "ocrdec_state_bytes": (ctypes.c_size_t, [cfgp]),
        "ocrdec_workspace_bytes": (ctypes.c_size_t, [cfgp]),
        "ocrdec_num_weights": (I, [cfgp]),
        "ocrdec_create": (I, [cfgp, ctypes.POINTER(P), I, P, P, P, ctypes.POINTER(P)]),
        "ocrdec_destroy": (I, [P]),
        "ocrdec_prefill": (I, [P, P, I, P, P, I, P, P, I, P, P]),
        "ocrdec_draft": (I, [P, P, I, P, I, P]),
        "ocrdec_verify": (I, [P, P, I, P, I, P, P, P]),
        "ocrdec_accept_rollback": (I, [P, P, I, P, I, P, P, P, P, P, I]),
        "ocrdec_controlled_drafts": (I, [P, P, I, P, I, P, I, I, U64, U64, P]),
        "ocrdec_set_taps": (I, [P, ctypes.POINTER(ocrdec_taps)]),
        "ocrdec_expert_timing": (I, [P, I]),
        "ocrdec_expert_stats": (I, [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong),
                                    ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong),
                                    ctypes.POINTER(ctypes.c_longlong)]),
        "ocrdec_replay_expert_gate_up": (I, [P, P, I, ctypes.POINTER(I)]),
        "ocrdec_decode_steps": (I, [P, P, I, P, I, I, ctypes.POINTER(ocrdec_controlled_cfg), P, P, P, P, P, I]),
        "ocrdec_decode_steps_noalloc": (I, [P, P, I, P, I, I, P, P, P, P, P, I]),
        "ocrdec_sync_positions": (I, [P, P]),
        "ocrdec_load_sequence": (I, [P, P, I, I, I, P]),
        "ocrdec_set_router_logits": (I, [P, P]),
        "ocrdec_set_moe_launches": (I, [P, I]),
        "ocrdec_moe_grid": (I, [P]),
        "ocrdec_release_slot": (I, [P, P, I]),
        "ocrdec_kv_pages": (I, [P, ctypes.POINTER(I), ctypes.POINTER(I)]),
        "ocrdec_read_probe": (I, [P, P, ctypes.c_size_t, I, I, P]),
        "ocrdec_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, rc: int) -> None:
    if rc != OCRDEC_OK:
        raise OcrdecError(fn, rc, load_library().ocrdec_last_error().decode())


def make_config(cfg, max_batch: int, max_k: int, max_positions: int, path: int = 0,
                kv_pages: int = 0) -> ocrdec_config:
    return ocrdec_config(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.head_dim, cfg.n_experts, cfg.n_shared,
                         cfg.top_k, cfg.d_expert, cfg.d_draft_ffn, cfg.vocab, float(cfg.rope_theta),
                         float(cfg.norm_eps), OCRDEC_BF16 if cfg.dtype == "bf16" else OCRDEC_F32,
                         max_batch, max_k, max_positions, path, kv_pages)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# C-ABI wrappers with the same names (tensors in, data pointers out)
def ocrdec_state_bytes(c: ocrdec_config) -> int:
    return int(load_library().ocrdec_state_bytes(ctypes.byref(c)))


def ocrdec_workspace_bytes(c: ocrdec_config) -> int:
    return int(load_library().ocrdec_workspace_bytes(ctypes.byref(c)))


def ocrdec_num_weights(c: ocrdec_config) -> int:
    n = load_library().ocrdec_num_weights(ctypes.byref(c))
    _check("ocrdec_num_weights", n if n < 0 else 0)
    return int(n)


def ocrdec_create(c: ocrdec_config, weights: Sequence, state, workspace, stream: int) -> int:
    arr = (ctypes.c_void_p * len(weights))(*[w.data_ptr() for w in weights])
    h = ctypes.c_void_p()
    _check("ocrdec_create", load_library().ocrdec_create(ctypes.byref(c), arr, len(weights), state.data_ptr(),
                                                         workspace.data_ptr(), stream, ctypes.byref(h)))
    return h.value


def ocrdec_destroy(h: int) -> None:
    _check("ocrdec_destroy", load_library().ocrdec_destroy(h))


def ocrdec_prefill(h, stream, B, slots_host, vision, nv_stride, n_vision_host, prompt, np_stride, n_prompt_host,
                   pending_out) -> None:
    _check("ocrdec_prefill", load_library().ocrdec_prefill(
        h, stream, B, None if slots_host is None else slots_host.ctypes.data, _ptr(vision), nv_stride,
        n_vision_host.ctypes.data, _ptr(prompt), np_stride, n_prompt_host.ctypes.data, _ptr(pending_out)))


def ocrdec_draft(h, stream, B, slots, K, draft_out) -> None:
    _check("ocrdec_draft", load_library().ocrdec_draft(h, stream, B, _ptr(slots), K, _ptr(draft_out)))


def ocrdec_verify(h, stream, B, slots, K, draft, greedy_out, logits_out=None) -> None:
    _check("ocrdec_verify", load_library().ocrdec_verify(h, stream, B, _ptr(slots), K, _ptr(draft), _ptr(greedy_out),
                                                         _ptr(logits_out)))


def ocrdec_accept_rollback(h, stream, B, slots, K, draft, greedy, n_accepted_out, out_tokens, out_len, out_cap):
    _check("ocrdec_accept_rollback", load_library().ocrdec_accept_rollback(
        h, stream, B, _ptr(slots), K, _ptr(draft), _ptr(greedy), _ptr(n_accepted_out), _ptr(out_tokens),
        _ptr(out_len), out_cap))


def ocrdec_controlled_drafts(h, stream, B, slots, K, trace, trace_stride, trace_len, seed, threshold, draft_inout):
    _check("ocrdec_controlled_drafts", load_library().ocrdec_controlled_drafts(
        h, stream, B, _ptr(slots), K, _ptr(trace), trace_stride, trace_len, seed, threshold, _ptr(draft_inout)))


def ocrdec_sync_positions(h, stream: int):
    _check("ocrdec_sync_positions", load_library().ocrdec_sync_positions(h, stream))


def ocrdec_load_sequence(h, stream: int, slot: int, n_pos: int, pending_token: int, kv) -> None:
    _check("ocrdec_load_sequence", load_library().ocrdec_load_sequence(h, stream, slot, n_pos, pending_token,
                                                                          kv.data_ptr()))


def ocrdec_release_slot(h, stream: int, slot: int) -> None:
    _check("ocrdec_release_slot", load_library().ocrdec_release_slot(h, stream, slot))


def ocrdec_kv_pages(h):
    """(pages in the pool, free pages)."""
    total, free = ctypes.c_int(0), ctypes.c_int(0)
    _check("ocrdec_kv_pages", load_library().ocrdec_kv_pages(h, ctypes.byref(total), ctypes.byref(free)))
    return total.value, free.value


def ocrdec_set_router_logits(h, logits=None) -> None:
    _check("ocrdec_set_router_logits", load_library().ocrdec_set_router_logits(h, _ptr(logits)))


def ocrdec_set_moe_launches(h, fused: bool):
    _check("ocrdec_set_moe_launches", load_library().ocrdec_set_moe_launches(h, 1 if fused else 0))


def ocrdec_moe_grid(h) -> int:
    n = load_library().ocrdec_moe_grid(h)
    _check("ocrdec_moe_grid", n if n < 0 else 0)
    return int(n)


def ocrdec_set_taps(h, route_idx=None, hidden=None, route_pos=None, route_pos_slot=0, accepted=None, drafts=None):
    """Parity taps (see ocrdec_harness.h).  route_pos: int32 [n_layers][cap][8] for slot
    route_pos_slot; accepted: int32 [max_batch][cap]; drafts: int32 [max_batch][cap][8]."""
    if all(t is None for t in (route_idx, hidden, route_pos, accepted, drafts)):
        _check("ocrdec_set_taps", load_library().ocrdec_set_taps(h, None))
        return
    cap = 0
    for t in (accepted, drafts):
        if t is not None:
            cap = int(t.shape[1])
    taps = ocrdec_taps(_ptr(route_idx), _ptr(hidden), _ptr(route_pos), int(route_pos_slot),
                       0 if route_pos is None else int(route_pos.shape[1]), _ptr(accepted), _ptr(drafts), cap)
    _check("ocrdec_set_taps", load_library().ocrdec_set_taps(h, ctypes.byref(taps)))


def ocrdec_expert_timing(h, enable: bool):
    _check("ocrdec_expert_timing", load_library().ocrdec_expert_timing(h, 1 if enable else 0))


def ocrdec_expert_stats(h):
    a, b = ctypes.c_double(), ctypes.c_double()
    na, nb, sets = ctypes.c_longlong(), ctypes.c_longlong(), ctypes.c_longlong()
    _check("ocrdec_expert_stats", load_library().ocrdec_expert_stats(h, ctypes.byref(a), ctypes.byref(na),
                                                                     ctypes.byref(b), ctypes.byref(nb),
                                                                     ctypes.byref(sets)))
    return dict(ms_gate_up=a.value, n_gate_up=na.value, ms_down=b.value, n_down=nb.value, expert_sets=sets.value)


def ocrdec_decode_steps(h, stream, B, slots, K, n_steps, ctrl, draft, greedy, n_accepted_out, out_tokens, out_len,
                        out_cap):
    _check("ocrdec_decode_steps", load_library().ocrdec_decode_steps(
        h, stream, B, _ptr(slots), K, n_steps, None if ctrl is None else ctypes.byref(ctrl), _ptr(draft),
        _ptr(greedy), _ptr(n_accepted_out), _ptr(out_tokens), _ptr(out_len), out_cap))


def ocrdec_decode_steps_noalloc(h, stream, B, slots, K, n_steps, draft, greedy, n_accepted_out, out_tokens, out_len,
                                out_cap):
    _check("ocrdec_decode_steps_noalloc", load_library().ocrdec_decode_steps_noalloc(
        h, stream, B, _ptr(slots), K, n_steps, _ptr(draft), _ptr(greedy), _ptr(n_accepted_out), _ptr(out_tokens),
        _ptr(out_len), out_cap))


def ocrdec_replay_expert_gate_up(h, stream, n_rounds: int, want_count: bool = False):
    na = ctypes.c_int()
    _check("ocrdec_replay_expert_gate_up", load_library().ocrdec_replay_expert_gate_up(
        h, stream, n_rounds, ctypes.byref(na) if want_count else None))
    return na.value if want_count else None


def ocrdec_read_probe(stream, buf, nbytes: int, n_regions: int, n_launches: int, sink):
    _check("ocrdec_read_probe", load_library().ocrdec_read_probe(stream, _ptr(buf), nbytes, n_regions, n_launches,
                                                                  _ptr(sink)))


class Decoder:
    """One model on one GPU: uploads the weights, owns state + workspace
    (torch allocations) and drives the four decode calls on one stream."""

    def __init__(self, cfg, weight_arrays: List[np.ndarray], max_batch: int, max_k: int, max_positions: int,
                 device: str = "cuda", path: int = 0, kv_pages: int = 0):
        import torch
        self.torch = torch
        load_library()
        self.cfg = cfg
        self.device = torch.device(device)
        self.c = make_config(cfg, max_batch, max_k, max_positions, path, kv_pages)
        n = ocrdec_num_weights(self.c)
        if n != len(weight_arrays):
            raise ValueError(f"expected {n} weight tensors, got {len(weight_arrays)}")
        self.weights = []
        for a in weight_arrays:
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            self.weights.append(torch.from_numpy(a).to(self.device))
        self.state = torch.empty(ocrdec_state_bytes(self.c), dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(ocrdec_workspace_bytes(self.c), dtype=torch.uint8, device=self.device)
        self.stream = torch.cuda.current_stream(self.device).cuda_stream
        self.h = ocrdec_create(self.c, self.weights, self.state, self.workspace, self.stream)
        self.max_batch, self.max_k, self.max_positions = max_batch, max_k, max_positions

    def close(self):
        if getattr(self, "h", None):
            ocrdec_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def release(self, slot: int):
        """Return the KV pages of ``slot`` to the pool (prefill it before its next decode)."""
        ocrdec_release_slot(self.h, self.stream, slot)

    def kv_pages(self):
        """(pages in the KV pool, free pages); a page holds 64 positions of one sequence."""
        return ocrdec_kv_pages(self.h)

    # -- helpers -------------------------------------------------------------
    def i32(self, *shape):
        return self.torch.empty(*shape, dtype=self.torch.int32, device=self.device)

    def stage_pages(self, pages):
        """Upload the prefixes of ``pages`` (list of synth.Page) to the device: the
        vision rows [B, nvs, d] fp32 and prompt ids [B, nps] int32, zero-padded,
        with the host-side lengths.  The result feeds ``prefill_staged``."""
        torch = self.torch
        B = len(pages)
        nv = np.array([p.vision.shape[0] for p in pages], dtype=np.int32)
        npr = np.array([p.prompt.shape[0] for p in pages], dtype=np.int32)
        nvs, nps = max(1, int(nv.max())), max(1, int(npr.max()))
        vis = np.zeros((B, nvs, self.cfg.d_model), dtype=np.float32)
        pr = np.zeros((B, nps), dtype=np.int32)
        for b, p in enumerate(pages):
            vis[b, :p.vision.shape[0]] = p.vision
            pr[b, :p.prompt.shape[0]] = p.prompt
        return (torch.from_numpy(vis).to(self.device), nvs, nv, torch.from_numpy(pr).to(self.device), nps, npr)

    def prefill_staged(self, staged, slots: Optional[Sequence[int]] = None, pending=None):
        """Prefill from device-resident prefixes (``stage_pages``).  Returns the
        device int32 [B] first output tokens (into ``pending`` when given)."""
        vis_t, nvs, nv, pr_t, nps, npr = staged
        B = len(nv)
        if pending is None:
            pending = self.i32(B)
        sl = None if slots is None else np.asarray(slots, dtype=np.int32)
        ocrdec_prefill(self.h, self.stream, B, sl, vis_t, nvs, nv, pr_t, nps, npr, pending)
        return pending

    def prefill(self, pages, slots: Optional[Sequence[int]] = None):
        """pages: list of synth.Page.  Returns the device int32 [B] first output tokens."""
        return self.prefill_staged(self.stage_pages(pages), slots)

    def draft(self, B, K, slots=None, out=None):
        out = self.i32(B, K) if out is None else out
        ocrdec_draft(self.h, self.stream, B, slots, K, out)
        return out

    def verify(self, B, K, draft, slots=None, greedy=None, logits=None):
        greedy = self.i32(B, K + 1) if greedy is None else greedy
        ocrdec_verify(self.h, self.stream, B, slots, K, draft, greedy, logits)
        return greedy

    def accept(self, B, K, draft, greedy, n_acc, out_tokens, out_len, slots=None):
        ocrdec_accept_rollback(self.h, self.stream, B, slots, K, draft, greedy, n_acc, out_tokens, out_len,
                               out_tokens.shape[1])

    def controlled(self, B, K, trace, seed, threshold, draft, slots=None):
        ocrdec_controlled_drafts(self.h, self.stream, B, slots, K, trace, trace.shape[1], trace.shape[1], seed,
                                 threshold, draft)

    def decode_steps(self, B, K, n_steps, draft, greedy, n_acc, out_tokens, out_len, trace=None, seed=0,
                     threshold=0, slots=None):
        """n_steps graph-replayed speculative steps (see ocrdec_decode_steps)."""
        ctrl = None
        if trace is not None:
            ctrl = ocrdec_controlled_cfg(trace.data_ptr(), trace.shape[1], trace.shape[1], seed, threshold)
        ocrdec_decode_steps(self.h, self.stream, B, slots, K, n_steps, ctrl, draft, greedy, n_acc, out_tokens,
                            out_len, out_tokens.shape[1])

    def generate(self, pages, n_out: int, K: int, trace=None, seed: int = 0, threshold: int = 0,
                 record: bool = False, check_every: int = 16, graphs: bool = False):
        """Decode B pages to n_out tokens each with K draft tokens per step (K = 0: plain
        autoregressive).  With ``trace`` (device int32 [B, T]) the drafts are replaced by the
        controlled-acceptance tokens.  Returns (tokens [B, n_out] numpy, per-sequence lists of
        accepted lengths up to the step that reached n_out (if record), steps run)."""
        torch = self.torch
        B = len(pages)
        cap = n_out + self.max_k + 2
        out_tokens = torch.zeros(B, cap, dtype=torch.int32, device=self.device)
        out_len = self.i32(B)
        n_acc = self.i32(B)
        pending = self.prefill(pages)
        out_tokens[:, 0] = pending
        draft = self.i32(B, max(K, 1))
        greedy = self.i32(B, K + 1)
        accs, lens = [], []
        steps = 0
        while True:
            if graphs and not record:
                self.decode_steps(B, K, check_every, draft, greedy, n_acc, out_tokens, out_len, trace, seed,
                                  threshold)
                steps += check_every
                ocrdec_sync_positions(self.h, self.stream)
                if int(out_len.min().item()) >= n_out:
                    break
                continue
            for _ in range(check_every):
                if K > 0:
                    self.draft(B, K, out=draft)
                    if trace is not None:
                        self.controlled(B, K, trace, seed, threshold, draft)
                self.verify(B, K, draft, greedy=greedy)
                self.accept(B, K, draft, greedy, n_acc, out_tokens, out_len)
                steps += 1
                if record:
                    accs.append(n_acc.clone())
                    lens.append(out_len.clone())
            ocrdec_sync_positions(self.h, self.stream)
            if int(out_len.min().item()) >= n_out:
                break
        toks = out_tokens[:, :n_out].cpu().numpy()
        acc = None
        if record:
            # keep, per sequence, the steps taken before it reached n_out tokens
            a = torch.stack(accs).cpu().numpy()
            ln = torch.stack(lens).cpu().numpy()
            acc = [a[:int(np.argmax(ln[:, b] >= n_out)) + 1, b].tolist() for b in range(B)]
        return toks, acc, steps

    def generate_adaptive(self, pages, n_out: int, controller, window: int = 8, trace=None, seed: int = 0,
                          threshold: int = 0):
        """Decode B pages to n_out tokens each with the draft depth chosen at run
        time: every window of `window` steps runs at the depth controller.choose()
        returns (decode-step graphs), timed with events on the stream; the
        window's accepted lengths (read from the accepted-length tap) and its
        time per step go back to controller.observe(K, accepted, ms_per_step).
        ``trace`` switches on the controlled drafts.  Returns (tokens [B, n_out]
        numpy, [(K, steps, ms_per_step)] per window)."""
        torch = self.torch
        B = len(pages)
        Kmax = self.max_k
        cap = n_out + Kmax + 2
        out_tokens = torch.zeros(B, cap, dtype=torch.int32, device=self.device)
        out_len, n_acc = self.i32(B), self.i32(B)
        draft, greedy = self.i32(B, max(Kmax, 1)), self.i32(B, Kmax + 1)
        steps_cap = n_out + window + 2
        acc_tap = torch.full((self.max_batch, steps_cap), -1, dtype=torch.int32, device=self.device)
        ocrdec_set_taps(self.h, accepted=acc_tap)
        hist = []
        try:
            out_tokens[:, 0] = self.prefill(pages)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0 = 0
            while True:
                K = int(controller.choose())
                if not 1 <= K <= Kmax:
                    raise ValueError(f"controller chose K = {K}, outside 1..{Kmax}")
                e0.record()
                self.decode_steps(B, K, window, draft, greedy, n_acc, out_tokens, out_len, trace, seed, threshold)
                e1.record()
                ocrdec_sync_positions(self.h, self.stream)
                ms = e0.elapsed_time(e1) / window
                acc = acc_tap[:B, s0:s0 + window].cpu().numpy()
                controller.observe(K, acc.reshape(-1).tolist(), ms)
                hist.append((K, window, ms))
                s0 += window
                if int(out_len.min().item()) >= n_out or s0 + window > steps_cap:
                    break
        finally:
            ocrdec_set_taps(self.h)
        return out_tokens[:, :n_out].cpu().numpy(), hist

    def _ragged_buffers(self, B: int, K: int, cap: int, T: int):
        """Per-shape scratch of generate_ragged, kept so that repeated runs pass the same
        pointers (the decode-step graphs are cached by call shape and pointers)."""
        key = (B, K, cap, T)
        if not hasattr(self, "_rag"):
            self._rag = {}
        if key not in self._rag:
            torch = self.torch
            self._rag[key] = dict(
                slots=self.i32(B), out=torch.zeros(B, cap, dtype=torch.int32, device=self.device),
                trace=torch.zeros(B, max(T, 1), dtype=torch.int32, device=self.device),
                out_len=self.i32(B), n_acc=self.i32(B), draft=self.i32(B, max(K, 1)), greedy=self.i32(B, K + 1))
        return self._rag[key]

    def generate_ragged(self, pages, n_out, K: int, trace=None, seed: int = 0, threshold: int = 0,
                        check_every: int = 8, record: bool = False, graphs: bool = False, timer=None):
        """Static batch with per-sequence output lengths: sequence b (slot b) leaves the
        batch once it has n_out[b] tokens; the others go on (no refill).  ``trace``
        (device int32 [B, T]) switches on the controlled drafts.  ``timer`` (optional
        callable) is called after the prefill, synchronised.  Returns (list of token
        arrays, per-sequence accepted lengths of the steps up to n_out[b] if record, total
        sequence-steps run)."""
        torch = self.torch
        B = len(pages)
        n_out = np.asarray(n_out, dtype=np.int64)
        cap = int(n_out.max()) + self.max_k + 2
        T = 0 if trace is None else int(trace.shape[1])
        buf = self._ragged_buffers(B, K, cap, T)
        full = torch.zeros(B, cap, dtype=torch.int32, device=self.device)
        full[:, 0] = self.prefill(pages)
        if timer is not None:
            torch.cuda.synchronize()
            timer()
        active = np.arange(B)
        accs = [[] for _ in range(B)]
        done_len = np.ones(B, dtype=np.int64)
        seq_steps = 0
        while len(active):
            Bb = len(active)
            idx = torch.from_numpy(active).to(self.device)
            slots = buf["slots"][:Bb]
            slots.copy_(idx.to(torch.int32))
            out_t = buf["out"][:Bb]
            out_t.copy_(full[idx])
            tr = None
            if trace is not None:
                tr = buf["trace"][:Bb]
                tr.copy_(trace[idx])
            out_len, n_acc = buf["out_len"][:Bb], buf["n_acc"][:Bb]
            draft, greedy = buf["draft"][:Bb], buf["greedy"][:Bb]
            while True:
                rec = []
                if graphs and not record:
                    self.decode_steps(Bb, K, check_every, draft, greedy, n_acc, out_t, out_len, tr, seed,
                                      threshold, slots=slots)
                else:
                    for _ in range(check_every):
                        if K > 0:
                            self.draft(Bb, K, slots=slots, out=draft)
                            if tr is not None:
                                self.controlled(Bb, K, tr, seed, threshold, draft, slots=slots)
                        self.verify(Bb, K, draft, slots=slots, greedy=greedy)
                        self.accept(Bb, K, draft, greedy, n_acc, out_t, out_len, slots=slots)
                        if record:
                            rec.append((n_acc.clone(), out_len.clone()))
                seq_steps += Bb * check_every
                if record:
                    for a, ln in rec:
                        a, ln = a.cpu().numpy(), ln.cpu().numpy()
                        for i, b in enumerate(active):
                            if done_len[b] < n_out[b]:
                                accs[b].append(int(a[i]))
                                done_len[b] = ln[i]
                ocrdec_sync_positions(self.h, self.stream)
                lens = out_len.cpu().numpy()
                if (lens >= n_out[active]).any():
                    break
            full[idx] = out_t
            active = active[lens < n_out[active]]
        host = full.cpu().numpy()
        return [host[b, :n_out[b]] for b in range(B)], (accs if record else None), seq_steps

    def generate_stream(self, pages, n_out, K: int, concurrency: int, trace=None, seed: int = 0,
                        threshold: int = 0, check_every: int = 8, graphs: bool = False, refill_min: int = 1):
        """Continuous batching over a queue of pages: at most ``concurrency`` pages in
        flight, one state slot each; when a page has its n_out[i] tokens, its slot is
        prefilled with the next queued page (all refills of a check in one prefill call;
        with refill_min > 1, free slots wait until that many are free or nothing else
        runs, so prefills run several pages per pass) while the other slots keep decoding.
        A page is admitted only while the KV page pool can hold every page in flight
        at its full length (prefix + n_out[i] + the positions a check can run past
        it), in queue order; a finished page's slot returns its pages at once.
        ``trace`` (device int32 [n_pages, T]) switches on the controlled drafts (each
        page reads its own row).  Returns (list of token arrays per page, total
        sequence-steps run)."""
        torch = self.torch
        n = len(pages)
        n_out = np.asarray(n_out, dtype=np.int64)
        C = min(concurrency, self.max_batch, n)
        cap = int(n_out.max()) + self.max_k + 2
        T = 0 if trace is None else int(trace.shape[1])
        buf = self._ragged_buffers(C, K, cap, T)
        out_full = torch.zeros(C, cap, dtype=torch.int32, device=self.device)
        tr_full = None if trace is None else torch.zeros(C, T, dtype=torch.int32, device=self.device)
        slot_page = [-1] * C
        results = [None] * n
        queue = 0
        seq_steps = 0
        pool, _ = self.kv_pages()
        run_past = (check_every + 2) * (K + 1) + 1
        need = [-(-(pg.prefix_len + int(n_out[i]) + run_past) // 64) for i, pg in enumerate(pages)]
        if max(need) > pool:
            raise ValueError(f"a page needs {max(need)} KV pages, the pool has {pool}")
        reserved = 0

        def refill(free):
            """Admit queued pages into the free slots; returns the slots left free."""
            nonlocal queue, reserved
            take = []
            for s in free:
                if queue < n and reserved + need[queue] <= pool:
                    slot_page[s] = queue
                    reserved += need[queue]
                    queue += 1
                    take.append(s)
                else:
                    slot_page[s] = -1
            if take:
                pend = self.prefill([pages[slot_page[s]] for s in take], slots=take)
                for j, s in enumerate(take):
                    out_full[s].zero_()
                    out_full[s, 0] = pend[j]
                    if tr_full is not None:
                        tr_full[s].copy_(trace[slot_page[s]])
            return [s for s in free if s not in take]

        free = refill(list(range(C)))
        while any(p >= 0 for p in slot_page):
            active = np.array([s for s in range(C) if slot_page[s] >= 0], dtype=np.int64)
            Bb = len(active)
            idx = torch.from_numpy(active).to(self.device)
            slots = buf["slots"][:Bb]
            slots.copy_(idx.to(torch.int32))
            out_t = buf["out"][:Bb]
            out_t.copy_(out_full[idx])
            tr = None
            if tr_full is not None:
                tr = buf["trace"][:Bb]
                tr.copy_(tr_full[idx])
            out_len, n_acc = buf["out_len"][:Bb], buf["n_acc"][:Bb]
            draft, greedy = buf["draft"][:Bb], buf["greedy"][:Bb]
            target = np.array([n_out[slot_page[s]] for s in active])
            while True:
                if graphs:
                    self.decode_steps(Bb, K, check_every, draft, greedy, n_acc, out_t, out_len, tr, seed,
                                      threshold, slots=slots)
                else:
                    for _ in range(check_every):
                        if K > 0:
                            self.draft(Bb, K, slots=slots, out=draft)
                            if tr is not None:
                                self.controlled(Bb, K, tr, seed, threshold, draft, slots=slots)
                        self.verify(Bb, K, draft, slots=slots, greedy=greedy)
                        self.accept(Bb, K, draft, greedy, n_acc, out_t, out_len, slots=slots)
                seq_steps += Bb * check_every
                ocrdec_sync_positions(self.h, self.stream)
                lens = out_len.cpu().numpy()
                if (lens >= target).any():
                    break
            out_full[idx] = out_t
            done = [int(s) for i, s in enumerate(active) if lens[i] >= target[i]]
            host = out_full.cpu().numpy()
            for s in done:
                results[slot_page[s]] = host[s, :n_out[slot_page[s]]].copy()
                reserved -= need[slot_page[s]]
                slot_page[s] = -1
                self.release(s)  # its KV pages go back to the pool at once
            free += done
            if queue < n and (len(free) >= refill_min or all(p < 0 for p in slot_page)):
                free = refill(free)
        return results, seq_steps
