"""GPU checks of the paged KV cache: a pool of pages of 64 positions shared by
the slots (the concurrency-32 serving of the French model card, where pages
of different lengths are in flight together).

Where a sequence's cache rows live must not change any result: the same
pages decoded on a handle whose pool is small, fragmented and handed out in
reverse order give bitwise the tokens and logits of a handle with one page per
64 positions of every slot.  A call the pool cannot serve is refused with
OCRDEC_ECAPACITY and changes nothing; releasing a slot lets it through.

The model is the 2-layer one with a ragged vocabulary (5003), bf16 on the
matrix cores and fp32 on the vector path."""
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

SMALL = dataclasses.replace(synth.FULL, n_layers=2, vocab=5003)
PATHS = {"bf16": ocrdec.OCRDEC_PATH_MATRIX, "f32": ocrdec.OCRDEC_PATH_VECTOR}


def _dec(cfg, w, max_batch, max_k, max_positions, kv_pages=0):
    return ocrdec.Decoder(cfg, w.device_arrays(), max_batch=max_batch, max_k=max_k, max_positions=max_positions,
                          path=PATHS[cfg.dtype], kv_pages=kv_pages)


def _verify_logits(dec, B, K, draft):
    greedy = dec.i32(B, K + 1)
    logits = torch.empty(B, K + 1, dec.cfg.vocab, dtype=torch.float32, device="cuda")
    dec.verify(B, K, draft, greedy=greedy, logits=logits)
    torch.cuda.synchronize()
    return greedy.cpu().numpy(), logits.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fragmented_pool_bitwise_equal_to_full_pool(dtype):
    """Three pages (prefixes of 155, 73 and 204 rows) decoded to 40 tokens with
    K = 3, eagerly and with graphs, on a 14-page pool whose free pages were
    left fragmented by earlier sequences, equal bitwise the same decode on the
    full pool (3 slots x 8 pages)."""
    cfg = dataclasses.replace(SMALL, dtype=dtype)
    w = synth.Weights(cfg, 91)
    pages = synth.make_pages(cfg, 92, [150, 70, 200], [5, 3, 4], [40, 40, 40])
    fill = synth.make_pages(cfg, 93, [128, 250, 66], [2, 10, 4], [1, 1, 1])  # 3 + 5 + 2 pages
    full = _dec(cfg, w, 3, 3, 512)
    ref, _, _ = full.generate(pages, 40, 3, check_every=4)
    paged = _dec(cfg, w, 3, 3, 512, kv_pages=14)
    assert paged.kv_pages() == (14, 14)
    # earlier sequences take pages 0-2, 3-7 and 8-9; freeing slots 1 then 0
    # leaves the free stack out of order, so the next prefill's slots get
    # pages like 9, 8, 2, ... rather than consecutive ones
    paged.prefill(fill)
    assert paged.kv_pages() == (14, 4)
    paged.release(1)
    paged.release(0)
    assert paged.kv_pages() == (14, 12)
    got, _, _ = paged.generate(pages, 40, 3, check_every=4)
    assert np.array_equal(ref, got), "tokens differ between the full and the fragmented pool"
    # one more verify of every slot at the positions the decode reached: the
    # logits themselves, bitwise
    draft = torch.from_numpy(ref[:, 1:4].astype(np.int32)).cuda()
    g0, l0 = _verify_logits(full, 3, 3, draft)
    g1, l1 = _verify_logits(paged, 3, 3, draft)
    assert np.array_equal(g0, g1) and np.array_equal(l0, l1), float(np.abs(l0 - l1).max())
    got_g, _, _ = paged.generate(pages, 40, 3, check_every=4, graphs=True)
    assert np.array_equal(ref, got_g), "graph decode on the fragmented pool differs"
    total, free = paged.kv_pages()
    log(f"{dtype}: 3 pages x 40 tokens bitwise equal on a fragmented 14-page pool ({free} pages left free)")


def test_pool_exhaustion_is_refused_and_release_frees_pages():
    """A 4-page pool holding two 2-page prefixes: a verify whose rows would
    cross into a third page of slot 0 is refused (ECAPACITY) with the pool
    unchanged; a prefill that needs more pages than the pool has is refused the
    same way and leaves the slots' pages alone; after slot 1 is released the
    verify runs and equals bitwise the same verify on the full pool."""
    cfg = dataclasses.replace(SMALL, dtype="bf16")
    w = synth.Weights(cfg, 94)
    pages = synth.make_pages(cfg, 95, [120, 90], [5, 6], [8, 8])  # 125 and 96 rows: 2 pages each
    big = synth.make_pages(cfg, 96, [300], [4], [8])
    full = _dec(cfg, w, 2, 3, 512)
    paged = _dec(cfg, w, 2, 3, 512, kv_pages=4)
    p_full = full.prefill(pages).cpu().numpy()
    p_paged = paged.prefill(pages).cpu().numpy()
    assert np.array_equal(p_full, p_paged)
    assert paged.kv_pages() == (4, 0)
    draft = torch.from_numpy(np.stack([p_full, p_full, p_full], 1).astype(np.int32)).cuda()
    with pytest.raises(ocrdec.OcrdecError) as e:
        _verify_logits(paged, 2, 3, draft)  # slot 0 would write positions 125..128
    assert e.value.code == ocrdec.OCRDEC_ECAPACITY and "pool" in str(e.value)
    assert paged.kv_pages() == (4, 0)
    with pytest.raises(ocrdec.OcrdecError) as e:
        paged.prefill(big, slots=[1])  # 304 rows: 5 pages of a 4-page pool
    assert e.value.code == ocrdec.OCRDEC_ECAPACITY
    assert paged.kv_pages() == (4, 0)
    paged.release(1)
    assert paged.kv_pages() == (4, 2)
    g1, l1 = _verify_logits(paged, 1, 3, draft[:1])
    g0, l0 = _verify_logits(full, 1, 3, draft[:1])
    assert np.array_equal(g0, g1) and np.array_equal(l0, l1), float(np.abs(l0 - l1).max())
    assert paged.kv_pages() == (4, 1)
    log("exhausted pool refused with nothing changed; after a release the verify equals the full pool's")


def test_continuous_batching_on_a_small_pool():
    """Nine pages streamed through 3 slots on a 6-page pool (the full pool
    would be 12): finished slots give their pages back, refills take them, and
    every page's tokens equal bitwise the stream on the full pool; at the end
    every page is free again."""
    cfg = dataclasses.replace(SMALL, dtype="bf16")
    w = synth.Weights(cfg, 97)
    n = 9
    rng = np.random.default_rng(98)
    nv = rng.integers(3, 60, size=n).tolist()
    npr = rng.integers(1, 6, size=n).tolist()
    n_out = rng.integers(5, 40, size=n)
    pages = synth.make_pages(cfg, 99, nv, npr, n_out.tolist())
    full = _dec(cfg, w, 3, 3, 256)
    ref, _ = full.generate_stream(pages, n_out, 3, 3, check_every=2, refill_min=2)
    paged = _dec(cfg, w, 3, 3, 256, kv_pages=6)
    got, _ = paged.generate_stream(pages, n_out, 3, 3, check_every=2, refill_min=2)
    for i in range(n):
        assert ref[i].tolist() == got[i].tolist(), i
    assert paged.kv_pages() == (6, 6)
    log(f"continuous batching: {n} pages through 3 slots on a 6-page pool, bitwise equal to the full pool")


def test_load_sequence_on_a_small_pool():
    """A caller's cache loaded into the pages of a slot (ocrdec_load_sequence):
    on a 6-page pool a second 200-position sequence (4 pages) is refused with
    the pool unchanged, and once the first slot is released it loads into the
    pages that slot gave back; a verify over it then equals bitwise the same
    verify on the full pool."""
    cfg = dataclasses.replace(SMALL, dtype="bf16")
    w = synth.Weights(cfg, 101)
    n_pos = 200
    kv_dev = torch.from_numpy(synth.longctx_kv(cfg, 102, n_pos).view(np.int16)).cuda()
    other = torch.from_numpy(synth.longctx_kv(cfg, 103, n_pos).view(np.int16)).cuda()
    full = _dec(cfg, w, 2, 3, 512)
    paged = _dec(cfg, w, 2, 3, 512, kv_pages=6)
    ocrdec.ocrdec_load_sequence(full.h, full.stream, 0, n_pos, 17, kv_dev)
    ocrdec.ocrdec_load_sequence(paged.h, paged.stream, 1, n_pos, 5, other)
    assert paged.kv_pages() == (6, 2)
    with pytest.raises(ocrdec.OcrdecError) as e:
        ocrdec.ocrdec_load_sequence(paged.h, paged.stream, 0, n_pos, 17, kv_dev)
    assert e.value.code == ocrdec.OCRDEC_ECAPACITY
    assert paged.kv_pages() == (6, 2)
    paged.release(1)
    ocrdec.ocrdec_load_sequence(paged.h, paged.stream, 0, n_pos, 17, kv_dev)
    assert paged.kv_pages() == (6, 2)
    draft = torch.tensor([[3, 4, 5]], dtype=torch.int32, device="cuda")
    g0, l0 = _verify_logits(full, 1, 3, draft)
    g1, l1 = _verify_logits(paged, 1, 3, draft)
    assert np.array_equal(g0, g1) and np.array_equal(l0, l1), float(np.abs(l0 - l1).max())
    log("loaded cache on a small pool: refused when full, equal to the full pool after a release")


def test_stream_on_a_small_pool_matches_the_oracle():
    """Continuous batching on a small KV pool checked against the oracle
    itself (fp32 model on the vector path): six pages through two slots on a
    4-page pool, K = 3 with the real draft block; for the first and the last
    page the oracle's teacher-forced pass over the GPU's tokens gives the same
    greedy token at every position (a mismatch excused only where the
    oracle's top-2 margin is under 1e-3)."""
    from oracle import decoder as od
    cfg = dataclasses.replace(SMALL, dtype="f32")
    w = synth.Weights(cfg, 104)
    rng = np.random.default_rng(105)
    n = 6
    nv = rng.integers(3, 40, size=n).tolist()
    npr = rng.integers(1, 6, size=n).tolist()
    n_out = rng.integers(8, 24, size=n)
    pages = synth.make_pages(cfg, 106, nv, npr, n_out.tolist())
    paged = _dec(cfg, w, 2, 3, 128, kv_pages=4)
    toks, _ = paged.generate_stream(pages, n_out, 3, 2, check_every=2, refill_min=1)
    assert paged.kv_pages() == (4, 4)
    orc = od.Oracle(cfg, w.f32)
    for i in (0, n - 1):
        g, mg, _, _ = orc.teacher_forced(pages[i].vision, pages[i].prompt, toks[i].tolist())
        bad = [t for t in range(len(toks[i])) if int(g[t]) != int(toks[i][t])]
        hard = [(t, int(toks[i][t]), int(g[t]), float(mg[t])) for t in bad if mg[t] >= 1e-3]
        assert not hard, hard[:5]
        log(f"stream page {i}: {len(toks[i])} tokens, {len(toks[i]) - len(bad)} equal to the oracle's greedy token, "
            f"{len(bad)} near ties")
