"""Host-side block manager of the block cache layout (csa_blocks_*): reference counts, free and
idle blocks, the prefix registry and the prefix key chain.  CPU only: nothing here touches the
device."""
import os

import pytest

import long_context_sparse_15_amd as csa


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(csa.LIB_PATH):
        pytest.fail("libcsa.so is not built; run __graft_entry__.build()")


def test_alloc_share_release_counts():
    m = csa.BlockManager(8)
    assert m.counts() == (8, 0)
    a = m.alloc(3)
    assert sorted(a) == [0, 1, 2] and len(set(a)) == 3
    assert m.counts() == (5, 0)
    m.share([a[0]])
    assert m.refcount(a[0]) == 2
    m.release([a[0]])
    assert m.refcount(a[0]) == 1 and m.counts() == (5, 0)
    m.release(a)
    assert m.counts() == (8, 0)
    assert all(m.refcount(b) == 0 for b in range(8))


def test_errors_change_nothing():
    m = csa.BlockManager(4)
    a = m.alloc(2)
    with pytest.raises(csa.CsaError, match="free"):
        m.alloc(3)                        # only 2 free: nothing allocated
    assert m.counts() == (2, 0)
    with pytest.raises(csa.CsaError, match="released more often"):
        m.release([a[0], a[0]])           # one reference, listed twice
    assert m.refcount(a[0]) == 1
    with pytest.raises(csa.CsaError, match="not in use"):
        m.share([3])                      # never allocated
    with pytest.raises(csa.CsaError, match="out of range"):
        m.release([7])
    with pytest.raises(csa.CsaError, match="not in use"):
        m.publish(123, 3)
    with pytest.raises(csa.CsaError):
        csa.BlockManager(0)


def test_prefix_registry_and_idle_recycling():
    m = csa.BlockManager(4)
    x, y = m.alloc(2)
    m.publish(111, x)
    m.publish(222, y)
    m.publish(111, y)                     # the key keeps its first block
    assert m.lookup([111]) == [x]
    m.release([x])                        # back to one reference (the owner's)
    m.release([x, y])                     # both registered: idle, still found
    assert m.counts() == (4, 2)
    assert m.lookup([111, 222, 333]) == [x, y]   # longest leading run; idle blocks revive
    assert m.refcount(x) == 1 and m.counts() == (2, 0)
    m.release([y])                        # y idle
    m.release([x])                        # then x idle: y is the least recently released
    fresh = m.alloc(2)                    # never-registered blocks go first
    assert set(fresh).isdisjoint({x, y}) and m.counts() == (2, 2)
    z = m.alloc(1)[0]                     # no free block left: recycle y, unregister 222
    assert z == y
    assert m.lookup([222]) == []
    assert m.lookup([111]) == [x]


def test_chain_keys():
    toks = list(range(1000, 1000 + 3 * 128 + 50))
    k = csa.chain_keys(toks, 128)
    assert len(k) == 3 and len(set(k)) == 3
    assert csa.chain_keys(toks[:2 * 128 + 7], 128) == k[:2]      # only whole blocks, prefix-wise
    t2 = list(toks)
    t2[128 + 5] += 1                                            # change a token of block 1
    k2 = csa.chain_keys(t2, 128)
    assert k2[0] == k[0] and k2[1] != k[1] and k2[2] != k[2]
    assert csa.chain_keys(toks, 128, seed=1) != k               # seed separates namespaces
    # blocks with the same tokens at different depths get different keys
    rep = [7] * (2 * 128)
    kr = csa.chain_keys(rep, 128)
    assert kr[0] != kr[1]


def test_two_requests_share_a_prefix():
    """Block tables of two requests whose first 300 tokens agree: the second maps the first's
    two whole blocks (256 tokens) and allocates the rest; releasing the first leaves the shared
    blocks in use."""
    m = csa.BlockManager(16)
    a_tok = list(range(700))
    b_tok = a_tok[:300] + list(range(5000, 5200))
    ka = csa.chain_keys(a_tok)
    ta = m.alloc((len(a_tok) + 127) // 128)
    for key, blk in zip(ka, ta):
        m.publish(key, blk)
    kb = csa.chain_keys(b_tok)
    hit = m.lookup(kb)
    assert hit == ta[:2]
    tb = hit + m.alloc((len(b_tok) + 127) // 128 - len(hit))
    assert len(tb) == 4 and set(tb[2:]).isdisjoint(ta)
    m.release(ta)
    assert all(m.refcount(b) == 1 for b in tb)
    assert m.counts()[0] == 16 - 4
