"""ocrdec_decode_steps_noalloc -- the entry point for callers that cannot
allocate -- against ocrdec_decode_steps (the same steps recorded as HIP
graphs, scratch in the handle's workspace): two calls in a row on one handle,
the second with fewer sequences, each equal bit for bit (tokens, accepted
lengths, committed counts) to the graph entry point on a twin handle; and a
call whose scratch would pass the static array's size is refused before any
launch."""
import dataclasses

import numpy as np
import pytest

from speculative_moe_decoding_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_util import log  # noqa: E402
from speculative_moe_decoding_amd import ocrdec  # noqa: E402


def _run(dec, pages, K, n_steps, noalloc):
    B = len(pages)
    slots = torch.arange(B, dtype=torch.int32, device="cuda")
    draft, greedy = dec.i32(B, K), dec.i32(B, K + 1)
    n_acc, out_len = dec.i32(B), dec.i32(B)
    cap = n_steps * (K + 1) + 2
    out = torch.zeros(B, cap, dtype=torch.int32, device="cuda")
    acc_tap = torch.full((dec.max_batch, n_steps + 2), -9, dtype=torch.int32, device="cuda")
    ocrdec.ocrdec_set_taps(dec.h, accepted=acc_tap)
    try:
        out[:, 0] = dec.prefill(pages)
        fn = ocrdec.ocrdec_decode_steps_noalloc if noalloc else None
        for _ in range(n_steps):
            if noalloc:
                ocrdec.ocrdec_decode_steps_noalloc(dec.h, dec.stream, B, slots, K, 1, draft, greedy, n_acc, out,
                                                   out_len, cap)
            else:
                ocrdec.ocrdec_decode_steps(dec.h, dec.stream, B, slots, K, 1, None, draft, greedy, n_acc, out,
                                           out_len, cap)
        torch.cuda.synchronize()
        return out.cpu().numpy(), out_len.cpu().numpy(), acc_tap.cpu().numpy()[:B, :n_steps]
    finally:
        ocrdec.ocrdec_set_taps(dec.h)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_steps_match_graph_steps(dtype):
    cfg = dataclasses.replace(synth.FULL, n_layers=2, vocab=5003, dtype=dtype)
    w = synth.Weights(cfg, 91)
    K = 3
    pages = synth.make_pages(cfg, 92, [20, 7, 13], [4, 9, 2], [40, 40, 40])
    a = ocrdec.Decoder(cfg, w.device_arrays(), max_batch=3, max_k=K, max_positions=256)
    b = ocrdec.Decoder(cfg, w.device_arrays(), max_batch=3, max_k=K, max_positions=256)
    for B, n_steps in ((3, 12), (2, 9)):          # the second call is smaller
        t_ref, l_ref, acc_ref = _run(a, pages[:B], K, n_steps, noalloc=False)
        t_got, l_got, acc_got = _run(b, pages[:B], K, n_steps, noalloc=True)
        assert np.array_equal(l_got, l_ref), (B, l_got, l_ref)
        for i in range(B):
            assert np.array_equal(t_got[i, :l_ref[i]], t_ref[i, :l_ref[i]]), (B, i)
        assert np.array_equal(acc_got, acc_ref)
        assert (acc_ref >= 0).all()
        log(f"no-allocation steps ({dtype}), B={B}, {n_steps} steps: equal to the graph steps "
            f"({int(l_ref.sum())} tokens)")
    # AR steps (K = 0) on the same handles
    t_ref, l_ref, _ = _run(a, pages[:1], 0, 6, noalloc=False)
    t_got, l_got, _ = _run(b, pages[:1], 0, 6, noalloc=True)
    assert np.array_equal(t_got[:, :7], t_ref[:, :7]) and np.array_equal(l_got, l_ref)


def test_noalloc_refuses_oversized_calls():
    cfg = dataclasses.replace(synth.FULL, n_layers=1, vocab=301, dtype="bf16")
    w = synth.Weights(cfg, 93)
    B, K = 256, 3                                  # 1,024 rows: far past the static scratch
    dec = ocrdec.Decoder(cfg, w.device_arrays(), max_batch=B, max_k=K, max_positions=32)
    draft, greedy = dec.i32(B, K), dec.i32(B, K + 1)
    n_acc, out_len = dec.i32(B), dec.i32(B)
    out = torch.zeros(B, 8, dtype=torch.int32, device="cuda")
    with pytest.raises(ocrdec.OcrdecError) as e:
        ocrdec.ocrdec_decode_steps_noalloc(dec.h, dec.stream, B, None, K, 1, draft, greedy, n_acc, out, out_len, 8)
    assert e.value.code == ocrdec.OCRDEC_ECAPACITY and "no-allocation limit" in str(e.value)
    torch.cuda.synchronize()
