"""The C ABI library loads and exports every symbol include/csa.h declares; host-only calls
(shape helpers, workspace sizes, argument errors) behave as documented.  CPU only: no call here
launches device work."""
import ctypes
import os
import re

import pytest

import long_context_sparse_15_amd as csa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "csa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+((?:csa|hca)_\w+)\s*\(", src,
                                 flags=re.M)))


def _cfg(mode=csa.MODE_CSA, **kw):
    d = dict(mode=mode, m=4 if mode == csa.MODE_CSA else 128, top_k=512, n_win=128, n_heads=64,
             head_dim=512, rope_dim=64, idx_heads=64, idx_dim=128, hidden=4096,
             softmax_scale=512 ** -0.5, rms_eps=1e-6, rope_inv_freq=0x1000)
    d.update(kw)
    return csa.Config(**d)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(csa.LIB_PATH):
        pytest.fail("libcsa.so is not built; run __graft_entry__.build()")
    return csa.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) == 26, names
    for n in names:
        assert hasattr(L, n), n
        assert n in csa._SIGS, n


def test_version_and_helpers(L):
    assert csa.version() == 10300
    c = _cfg()
    assert csa.weight_cols(c) == 5 * 512 + 4 * 128
    assert csa.tail_shape(c) == (8, 4 * 512 + 4 * 128)
    h = _cfg(csa.MODE_HCA)
    assert csa.weight_cols(h) == 3 * 512
    assert csa.tail_shape(h) == (128, 1024)


def test_workspace_sizes_are_monotone(L):
    c = _cfg()
    a = csa.workspace_size(c, csa.OP_INDEX_TOPK, 32, 1, 32768)
    b = csa.workspace_size(c, csa.OP_INDEX_TOPK, 32, 1, 65536)
    assert 0 < a < b
    d = csa.workspace_size(c, csa.OP_DECODE, 32, 1, 32768)
    assert d >= a
    p = csa.workspace_size(c, csa.OP_PREFILL, 1, 2048, 512)
    assert p > 0
    h = _cfg(csa.MODE_HCA)
    assert csa.workspace_size(h, csa.OP_HCA_MQA, 16, 1, 8192) >= 0


@pytest.mark.parametrize("field,value", [("head_dim", 96), ("rope_dim", 3), ("rope_dim", 0),
                                         ("n_heads", 0), ("n_heads", 129), ("idx_dim", 48),
                                         ("top_k", 0), ("top_k", 5000), ("mode", 7), ("m", 0),
                                         ("softmax_scale", 0.0), ("rope_inv_freq", None)])
def test_invalid_config_is_rejected_without_launch(L, field, value):
    c = _cfg(**{field: value})
    b = ctypes.c_size_t()
    rc = L.csa_workspace_size(ctypes.byref(c), csa.OP_DECODE, 1, 1, 16, ctypes.byref(b))
    assert rc == -1
    assert len(csa.last_error()) > 0


def test_null_arguments_are_rejected(L):
    c = _cfg()
    assert L.csa_workspace_size(None, 0, 1, 1, 1, None) == -1
    assert "NULL" in csa.last_error()
    # every compute entry point rejects a NULL config before touching the device
    assert L.csa_compress(None, 1, 1, None, None, None, None, None, 0, None) == -1
    assert L.csa_index_topk(None, 1, 1, None, None, None, None, None, None, None, None, 0,
                            None) == -1
    assert L.csa_sparse_mqa(None, 1, 1, None, None, None, None, None, None, None, None, 0,
                            None) == -1
    assert L.hca_dense_mqa(None, 1, 1, None, None, None, None, None, None, None, 0, None) == -1
    assert L.csa_decode(None, 1, None, None, None, None, None, None, None, None, None, None,
                        None, None, 0, None) == -1
    assert L.csa_prefill(None, 1, 1, None, None, None, None, None, None, None, None, None, None,
                         None, None, 0, None) == -1
    # a valid config with a NULL cache
    assert L.csa_index_topk(ctypes.byref(c), 1, 1, None, None, None, None, None, None, None,
                            None, 0, None) == -1
    assert "cache" in csa.last_error()
    assert L.hca_dense_mqa(ctypes.byref(_cfg(csa.MODE_HCA)), 1, 1, None, None, None, None,
                           None, None, None, 0, None) == -1


def test_projection_configs_are_checked(L):
    c = _cfg(hidden=4096, q_rank=1024, out_groups=8, out_rank=1024)
    q = csa.workspace_size(c, csa.OP_QUERY_PROJ, 1, 4096, 1)
    o = csa.workspace_size(c, csa.OP_OUTPUT_PROJ, 1, 4096, 1)
    assert q >= 4096 * 1024 * 2 and o >= 4096 * 8 * 1024 * 2
    for bad in (dict(q_rank=1000), dict(hidden=4000)):
        with pytest.raises(csa.CsaError):
            csa.workspace_size(_cfg(**dict(dict(hidden=4096, q_rank=1024), **bad)),
                               csa.OP_QUERY_PROJ, 1, 16, 1)
    for bad in (dict(out_groups=3), dict(out_rank=10)):
        with pytest.raises(csa.CsaError):
            csa.workspace_size(_cfg(**dict(dict(hidden=4096, out_groups=8, out_rank=1024), **bad)),
                               csa.OP_OUTPUT_PROJ, 1, 16, 1)


@pytest.mark.parametrize("mode,be,bps,nb,n_max,msg", [
    (csa.MODE_CSA, 24, 4, 8, 96, "power of two"),
    (csa.MODE_CSA, 8, 4, 8, 32, ">= 16"),
    (csa.MODE_CSA, 32, 4, 8, 100, "n_max"),
    (csa.MODE_CSA, 32, 4, 0, 128, "n_blocks"),
    (csa.MODE_HCA, 1, 0, 8, 1, "blocks_per_seq"),
    (csa.MODE_HCA, 1 << 20, 1, 1 << 12, 1 << 20, "2^31"),
    (csa.MODE_HCA, 1, 64, 8, 64, None),  # valid: the next check (NULL q) fails instead
])
def test_paged_cache_layout_is_checked(L, mode, be, bps, nb, n_max, msg):
    c = _cfg(mode)
    k = csa.Cache(n_max, 128, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, be, bps, nb,
                  0x7000)
    rc = L.hca_dense_mqa(ctypes.byref(c), 1, 1, None, ctypes.byref(k), None, None, None, None,
                         None, 0, None)
    assert rc == -1
    err = csa.last_error()
    assert ("NULL" if msg is None else msg) in err, err


def test_entry_format_is_checked(L):
    b = ctypes.c_size_t()
    ok = _cfg(entry_format=csa.ENT_MIXED)
    assert L.csa_workspace_size(ctypes.byref(ok), csa.OP_DECODE, 1, 1, 16, ctypes.byref(b)) == 0
    bad_dim = _cfg(entry_format=csa.ENT_MIXED, head_dim=256)
    assert L.csa_workspace_size(ctypes.byref(bad_dim), csa.OP_DECODE, 1, 1, 16,
                                ctypes.byref(b)) == -2  # CSA_ERR_UNSUPPORTED
    assert "mixed" in csa.last_error()
    bad_rope = _cfg(entry_format=csa.ENT_MIXED, rope_dim=40)
    assert L.csa_workspace_size(ctypes.byref(bad_rope), csa.OP_DECODE, 1, 1, 16,
                                ctypes.byref(b)) == -2
    bad = _cfg(entry_format=5)
    assert L.csa_workspace_size(ctypes.byref(bad), csa.OP_DECODE, 1, 1, 16, ctypes.byref(b)) == -1


def test_long_rows_in_big_batches_are_refused(L):
    """Selection over caches of more than 32768 entries takes at most 4096 query rows a call."""
    c = _cfg()
    b = ctypes.c_size_t()
    assert L.csa_workspace_size(ctypes.byref(c), csa.OP_INDEX_TOPK, 1, 4096, 65536,
                                ctypes.byref(b)) == 0
    assert L.csa_workspace_size(ctypes.byref(c), csa.OP_INDEX_TOPK, 1, 4097, 65536,
                                ctypes.byref(b)) == -2
    assert "4096" in csa.last_error()
    assert L.csa_workspace_size(ctypes.byref(c), csa.OP_PREFILL, 2, 4096, 65536,
                                ctypes.byref(b)) == -2
    assert L.csa_workspace_size(ctypes.byref(c), csa.OP_INDEX_TOPK, 1, 65536, 32768,
                                ctypes.byref(b)) == 0   # rows of at most 32768 entries: any count


def test_misaligned_workspace_is_rejected(L):
    """Every compute entry point checks the workspace's documented 256-byte alignment before
    anything is launched (the other pointers here are aligned stand-ins that are never used)."""
    c = _cfg()
    h = _cfg(csa.MODE_HCA)
    k = csa.Cache(8192, 128, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0, 0, 0, 0)
    ws, n = 0x10010, 1 << 40
    P = 0x20000
    calls = [
        lambda: L.csa_index_topk(ctypes.byref(c), 1, 1, P, P, P, ctypes.byref(k), P, P, None, ws,
                                 n, None),
        lambda: L.csa_sparse_mqa(ctypes.byref(c), 1, 1, P, ctypes.byref(k), P, P, P, P, None, ws,
                                 n, None),
        lambda: L.hca_dense_mqa(ctypes.byref(h), 1, 1, P, ctypes.byref(k), P, P, P, None, ws, n,
                                None),
        lambda: L.csa_decode(ctypes.byref(c), 1, None, None, ctypes.byref(k), P, P, P, P, P, P, P,
                             None, ws, n, None),
    ]
    for f in calls:
        assert f() == -1
        assert "256-byte aligned" in csa.last_error(), csa.last_error()


def test_attention_plan_does_not_depend_on_the_batch(L):
    """The attention workspace (span partials) grows exactly linearly with the batch: the number
    of spans a query's list is cut into is the same for every batch size."""
    for cfg, op, n_max in ((_cfg(), csa.OP_SPARSE_MQA, 32768),
                           (_cfg(n_heads=128, top_k=2048), csa.OP_SPARSE_MQA, 262144),
                           (_cfg(csa.MODE_HCA, n_heads=128), csa.OP_HCA_MQA, 8192)):
        one = csa.workspace_size(cfg, op, 1, 1, n_max)
        assert one > 0
        for B in (2, 5, 16, 32, 128):
            assert csa.workspace_size(cfg, op, B, 1, n_max) == B * one


def test_chunked_prefill_window_ring_is_checked(L):
    """A chunk that continues a sequence (pos0 given) needs a window ring that still holds the
    last n_win - 1 rows of the earlier chunks: win_slots >= T + n_win - 1.  Refused before any
    launch (the pointers are stand-ins that are never used)."""
    c = _cfg()
    P = 0x20000
    wts = csa.Weights(P, P, P, P, P, P, P)
    T = 1000
    for slots, ok in ((T, False), (T + c.n_win - 2, False), (T + c.n_win - 1, True)):
        k = csa.Cache(8192, slots, P, P, P, P, P, P, 0, 0, 0, 0)
        # a too small workspace makes the valid case stop at the workspace check instead
        rc = L.csa_prefill(ctypes.byref(c), 1, T, P, P, ctypes.byref(wts), ctypes.byref(k), P, P,
                           P, P, P, P, None, 0x100000, 16, None)
        err = csa.last_error()
        assert rc == (-3 if ok else -1), err
        assert ("T + n_win - 1" in err) != ok, err
