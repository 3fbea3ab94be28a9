"""The C-ABI library loads, exports every function include/ocrdec.h and
include/ocrdec_harness.h declare,
and its host-only entry points (sizes, argument checks) behave as documented.
No GPU compute is launched here."""
import ctypes
import os
import re
import subprocess

import pytest

from speculative_moe_decoding_amd import ocrdec, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(ocrdec_\w+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ocrdec.LIB_PATH):
        pytest.fail("libocrdec.so is not built (run __graft_entry__.build())")
    return ocrdec.load_library()


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", ocrdec.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (ocrdec_\w+)", out))
    declared = declared_functions()
    assert len(declared) >= 14
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    assert set(ocrdec.SYMBOLS) == set(declared)
    for f in declared:
        getattr(lib, f)


def test_sizes_scale_with_capacity(lib):
    c1 = ocrdec.make_config(synth.FULL, 1, 3, 2048)
    c2 = ocrdec.make_config(synth.FULL, 2, 3, 2048)
    s1, s2 = ocrdec.ocrdec_state_bytes(c1), ocrdec.ocrdec_state_bytes(c2)
    # verifier KV: 12 layers x 2 x 1280 x 2048 positions x 2 bytes per slot, plus the draft's layer
    kv_per_slot = 13 * 2 * 1280 * 2048 * 2
    assert s1 >= kv_per_slot and s2 >= 2 * kv_per_slot
    assert ocrdec.ocrdec_workspace_bytes(c1) > 0
    assert ocrdec.ocrdec_num_weights(c1) == len(synth.weight_specs(synth.FULL)) == 3 + 8 * 12 + 11


def test_rejects_bad_configs(lib):
    import dataclasses
    bad = ocrdec.make_config(dataclasses.replace(synth.FULL, d_model=1024), 1, 3, 2048)
    assert ocrdec.ocrdec_state_bytes(bad) == 0
    assert "unsupported shape" in lib.ocrdec_last_error().decode()
    with pytest.raises(ocrdec.OcrdecError) as e:
        ocrdec.ocrdec_num_weights(bad)
    assert e.value.code == ocrdec.OCRDEC_EINVAL
    for mb, mk, mp in ((0, 3, 2048), (1, 8, 2048), (1, 3, 40000), (1025, 0, 2048), (257, 3, 2048)):
        c = ocrdec.make_config(synth.FULL, mb, mk, mp)
        assert ocrdec.ocrdec_state_bytes(c) == 0
    # rows of one verify call: max_batch * (max_k + 1) up to 1024
    assert ocrdec.ocrdec_state_bytes(ocrdec.make_config(synth.FULL, 256, 3, 64)) > 0
    assert ocrdec.ocrdec_state_bytes(ocrdec.make_config(synth.FULL, 1024, 0, 64)) > 0
    # create checks the weight list before touching the device
    c = ocrdec.make_config(synth.FULL, 1, 3, 2048)
    h = ctypes.c_void_p()
    arr = (ctypes.c_void_p * 3)()
    rc = lib.ocrdec_create(ctypes.byref(c), arr, 3, None, None, None, ctypes.byref(h))
    assert rc == ocrdec.OCRDEC_EINVAL and h.value is None
    # calls on a null handle
    assert lib.ocrdec_verify(None, None, 1, None, 0, None, None, None) == ocrdec.OCRDEC_EINVAL
    assert lib.ocrdec_draft(None, None, 1, None, 3, None) == ocrdec.OCRDEC_EINVAL


def test_rejects_bad_paths_and_null_handles(lib):
    import dataclasses
    # the matrix-core path needs bf16 weights and a vocabulary of at least 64
    f32 = dataclasses.replace(synth.FULL, dtype="f32")
    c = ocrdec.make_config(f32, 4, 3, 2048, ocrdec.OCRDEC_PATH_MATRIX)
    assert ocrdec.ocrdec_state_bytes(c) == 0
    assert "matrix" in lib.ocrdec_last_error().decode()
    small = dataclasses.replace(synth.FULL, vocab=32)
    assert ocrdec.ocrdec_state_bytes(ocrdec.make_config(small, 4, 3, 2048, ocrdec.OCRDEC_PATH_MATRIX)) == 0
    assert ocrdec.ocrdec_state_bytes(ocrdec.make_config(synth.FULL, 4, 3, 2048, 7)) == 0
    for p in (ocrdec.OCRDEC_PATH_AUTO, ocrdec.OCRDEC_PATH_VECTOR, ocrdec.OCRDEC_PATH_MATRIX):
        assert ocrdec.ocrdec_state_bytes(ocrdec.make_config(synth.FULL, 4, 3, 2048, p)) > 0
    # every handle-taking entry point rejects a null handle without touching the device
    E = ocrdec.OCRDEC_EINVAL
    assert lib.ocrdec_destroy(None) == E
    assert lib.ocrdec_accept_rollback(None, None, 1, None, 0, None, None, None, None, None, 1) == E
    assert lib.ocrdec_controlled_drafts(None, None, 1, None, 1, None, 1, 1, 0, 0, None) == E
    assert lib.ocrdec_decode_steps(None, None, 1, None, 1, 1, None, None, None, None, None, None, 1) == E
    assert lib.ocrdec_sync_positions(None, None) == E
    assert lib.ocrdec_load_sequence(None, None, 0, 16, 0, None) == E
    assert lib.ocrdec_set_router_logits(None, None) == E
    assert lib.ocrdec_set_taps(None, None) == E
    assert lib.ocrdec_expert_timing(None, 1) == E
    assert lib.ocrdec_replay_expert_gate_up(None, None, 1, None) == E
    assert lib.ocrdec_read_probe(None, None, 256, 1, 1, None) == E
    assert lib.ocrdec_set_moe_launches(None, 1) == E
    assert lib.ocrdec_moe_grid(None) == E
    assert lib.ocrdec_release_slot(None, None, 0) == E
    assert lib.ocrdec_kv_pages(None, None, None) == E


def test_kv_page_pool_sizes_the_state(lib):
    """The KV cache is a pool of pages of 64 positions: its size follows
    kv_pages (0 = every slot at max_positions), clipped to that full size;
    a negative pool is refused."""
    full = ocrdec.ocrdec_state_bytes(ocrdec.make_config(synth.FULL, 8, 3, 2048))
    assert ocrdec.ocrdec_state_bytes(ocrdec.make_config(synth.FULL, 8, 3, 2048, kv_pages=8 * 32)) == full
    assert ocrdec.ocrdec_state_bytes(ocrdec.make_config(synth.FULL, 8, 3, 2048, kv_pages=10 ** 6)) == full
    small = ocrdec.ocrdec_state_bytes(ocrdec.make_config(synth.FULL, 8, 3, 2048, kv_pages=64))
    esz = 2 if synth.FULL.dtype == "bf16" else 4
    page = 2 * synth.FULL.n_heads * 64 * synth.FULL.head_dim * esz  # keys and values of one page, one layer
    # every verifier layer and the draft block hold the pages (256-byte alignment per region)
    saved = (8 * 32 - 64) * page * (synth.FULL.n_layers + 1)
    assert abs((full - small) - saved) < 4096
    assert ocrdec.ocrdec_state_bytes(ocrdec.make_config(synth.FULL, 8, 3, 2048, kv_pages=-1)) == 0
    assert "kv_pages" in lib.ocrdec_last_error().decode()


def test_prefill_argument_checks_need_no_device(lib):
    # a null handle, then a too-long prefix: both refused before any launch
    nv = (ctypes.c_int32 * 1)(10)
    npr = (ctypes.c_int32 * 1)(0)
    assert lib.ocrdec_prefill(None, None, 1, None, None, 10, nv, None, 1, npr, None) == ocrdec.OCRDEC_EINVAL
