"""The Python binding checks every tensor's dtype and size against the config, the batch and
the query count before a call (the C layer sees raw device pointers only, so an undersized
tensor would be read or written out of bounds).  CPU only: a check that passes reaches the
pointer conversion, which refuses host tensors; nothing is launched."""
import pytest
import torch

import long_context_sparse_15_amd as csa


def _cfg(**kw):
    d = dict(mode=csa.MODE_CSA, m=4, top_k=64, n_win=128, n_heads=8, head_dim=128, rope_dim=64,
             idx_heads=4, idx_dim=64, hidden=512, softmax_scale=128 ** -0.5, rms_eps=1e-6,
             rope_inv_freq=0x1000)
    d.update(kw)
    return csa.Config(**d)


def _cache(B=2, N=100, slots=128, c=128, dI=64, key_bytes=None, tail=None):
    k = csa.Cache(N, slots, 0x1000, 0x2000, 0x3000, 0x4000, 0, 0x5000, 0, 0, 0, 0)
    k._keep = (torch.zeros(B, N, c, dtype=torch.int16), torch.zeros(B, slots, c, dtype=torch.int16),
               torch.zeros(B, dtype=torch.int32),
               torch.zeros(B, N, key_bytes or dI, dtype=torch.uint8),
               torch.zeros(B, N, dtype=torch.float32), tail, None)
    return k


def _decode_args(B=2, n_h=8, c=128, H_I=4, dI=64, k=64):
    return dict(pos=torch.zeros(B, dtype=torch.int32),
                q=torch.zeros(B, n_h, c, dtype=torch.bfloat16),
                sink=torch.zeros(n_h), out=torch.zeros(B, n_h, c, dtype=torch.bfloat16),
                qi=torch.zeros(B, 1, H_I, dI, dtype=torch.uint8),
                qi_scale=torch.zeros(B, 1, H_I), wi=torch.zeros(B, 1, H_I),
                idx_out=torch.zeros(B, k, dtype=torch.int32))


def _decode(cfg, cache, a):
    csa.decode(cfg, cache, a["pos"], a["q"], a["sink"], a["out"], None, qi=a["qi"],
               qi_scale=a["qi_scale"], wi=a["wi"], idx_out=a["idx_out"])


def test_valid_decode_arguments_reach_the_pointer_conversion():
    with pytest.raises(csa.CsaError, match="on the GPU"):
        _decode(_cfg(), _cache(), _decode_args())


@pytest.mark.parametrize("name,bad,msg", [
    ("pos", torch.zeros(3, dtype=torch.int32), "pos holds 3"),
    ("pos", torch.zeros(2, dtype=torch.int64), "pos has dtype int64"),
    ("out", torch.zeros(2, 8, 64, dtype=torch.bfloat16), "out holds"),
    ("out", torch.zeros(2, 8, 128, dtype=torch.float32), "out has dtype float32"),
    ("sink", torch.zeros(7), "sink holds 7"),
    ("qi", torch.zeros(2, 1, 4, 32, dtype=torch.uint8), "qi holds"),
    ("qi_scale", torch.zeros(2, 1, 3), "qi_scale holds"),
    ("wi", torch.zeros(2, 1, 5), "wi holds"),
    ("idx_out", torch.zeros(2, 63, dtype=torch.int32), "idx_out holds 126"),
])
def test_decode_arguments_are_checked(name, bad, msg):
    a = _decode_args()
    a[name] = bad
    with pytest.raises(csa.CsaError, match=msg):
        _decode(_cfg(), _cache(), a)


def test_cache_tensors_are_checked():
    k = _cache(N=100)
    k._keep = (torch.zeros(2, 99, 128, dtype=torch.int16),) + k._keep[1:]
    with pytest.raises(csa.CsaError, match="cache entries"):
        _decode(_cfg(), k, _decode_args())
    k = _cache()
    k._keep = k._keep[:3] + (torch.zeros(2, 100, 32, dtype=torch.uint8),) + k._keep[4:]
    with pytest.raises(csa.CsaError, match="cache idx_keys"):
        _decode(_cfg(), k, _decode_args())
    k = _cache()
    k._keep = k._keep[:1] + (torch.zeros(2, 64, 128, dtype=torch.int16),) + k._keep[2:]
    with pytest.raises(csa.CsaError, match="cache window"):
        _decode(_cfg(), k, _decode_args())


def test_mxfp4_query_sizes():
    """An MXFP4 indexer query holds d_I/2 bytes per head and 4 scale bytes per head."""
    cfg = _cfg(idx_key_format=csa.IDX_MXFP4, idx_query_format=csa.IDX_MXFP4)
    a = _decode_args()
    a["qi"] = torch.zeros(2, 1, 4, 32, dtype=torch.uint8)
    a["qi_scale"] = torch.zeros(2, 1, 4, 4, dtype=torch.uint8)
    with pytest.raises(csa.CsaError, match="on the GPU"):
        _decode(cfg, _cache(key_bytes=32), a)
    a["qi"] = torch.zeros(2, 1, 4, 64, dtype=torch.uint8)
    with pytest.raises(csa.CsaError, match="qi holds"):
        _decode(cfg, _cache(key_bytes=32), a)


def test_sparse_mqa_and_index_topk_are_checked():
    cfg = _cfg()
    B, nq = 1, 16
    q = torch.zeros(B, nq, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(csa.CsaError, match="idx holds"):
        csa.sparse_mqa(cfg, q, _cache(B=1), torch.zeros(B, nq, 10, dtype=torch.int32),
                       torch.zeros(B, nq, dtype=torch.int32), torch.zeros(8), torch.zeros_like(q),
                       None)
    with pytest.raises(csa.CsaError, match="lse_out holds"):
        csa.sparse_mqa(cfg, q, _cache(B=1), torch.zeros(B, nq, 64, dtype=torch.int32),
                       torch.zeros(B, nq, dtype=torch.int32), torch.zeros(8), torch.zeros_like(q),
                       None, lse_out=torch.zeros(B, nq, 7))
    with pytest.raises(csa.CsaError, match="score_out holds"):
        csa.index_topk(cfg, torch.zeros(B, nq, 4, 64, dtype=torch.uint8), torch.zeros(B, nq, 4),
                       torch.zeros(B, nq, 4), _cache(B=1), torch.zeros(B, nq, dtype=torch.int32),
                       torch.zeros(B, nq, 64, dtype=torch.int32), None,
                       score_out=torch.zeros(B, nq, 63))
