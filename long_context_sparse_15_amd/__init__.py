"""Python binding of libcsa.so, the MI355X CSA/HCA library.

Argument marshalling only: every step of the path runs in the HIP kernels behind the C ABI
declared in include/csa.h.  Tensors are torch tensors on the GPU (torch provides device memory
and streams); bf16 arguments may be torch.bfloat16 or int16/uint16 bit patterns, E4M3
arguments torch.uint8 or torch.float8_e4m3fn.  Every call enqueues on the current torch stream
(or the stream passed) and raises CsaError with the library's message on a non-zero status.
There is no fallback: if libcsa.so is missing or fails to load, every call raises.
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")

MODE_CSA, MODE_HCA = 0, 1
IDX_E4M3, IDX_MXFP4 = 0, 1
SCORE_FP32, SCORE_BF16 = 0, 1
ENT_BF16, ENT_MIXED = 0, 1
(OP_COMPRESS, OP_INDEX_TOPK, OP_SPARSE_MQA, OP_HCA_MQA, OP_DECODE, OP_PREFILL, OP_QUERY_PROJ,
 OP_OUTPUT_PROJ) = range(8)
NOALLOC_SCRATCH_BYTES = 64 << 20  # CSA_NOALLOC_SCRATCH_BYTES


class CsaError(RuntimeError):
    pass


class Config(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("m", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_win", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
                ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("rope_inv_freq", ctypes.c_void_p),
                ("idx_key_format", ctypes.c_int32), ("q_rank", ctypes.c_int32),
                ("out_groups", ctypes.c_int32), ("out_rank", ctypes.c_int32),
                ("entry_format", ctypes.c_int32), ("idx_query_format", ctypes.c_int32),
                ("score_format", ctypes.c_int32)]


class Cache(ctypes.Structure):
    _fields_ = [("n_max", ctypes.c_int32), ("win_slots", ctypes.c_int32),
                ("entries", ctypes.c_void_p), ("idx_keys", ctypes.c_void_p),
                ("idx_scale", ctypes.c_void_p), ("window", ctypes.c_void_p),
                ("tail", ctypes.c_void_p), ("n_entries", ctypes.c_void_p),
                ("block_entries", ctypes.c_int32), ("blocks_per_seq", ctypes.c_int32),
                ("n_blocks", ctypes.c_int32), ("block_table", ctypes.c_void_p)]


class QProjWeights(ctypes.Structure):
    _fields_ = [("w_dq", ctypes.c_void_p), ("w_w", ctypes.c_void_p), ("w_uq", ctypes.c_void_p),
                ("w_iuq", ctypes.c_void_p), ("gamma_q", ctypes.c_void_p)]


class OProjWeights(ctypes.Structure):
    _fields_ = [("w_down", ctypes.c_void_p), ("w_proj", ctypes.c_void_p)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 40), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double)]


class Weights(ctypes.Structure):
    _fields_ = [("w_cat", ctypes.c_void_p), ("bias_a", ctypes.c_void_p),
                ("bias_b", ctypes.c_void_p), ("bias_ia", ctypes.c_void_p),
                ("bias_ib", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("gamma_win", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_SIGS = {
    "csa_version": ([], ctypes.c_int),
    "csa_last_error": ([], ctypes.c_char_p),
    "csa_profile_start": ([], ctypes.c_int),
    "csa_profile_stop": ([_P, _I, _P], ctypes.c_int),
    "csa_weight_cols": ([_P, _P], ctypes.c_int),
    "csa_tail_shape": ([_P, _P, _P], ctypes.c_int),
    "csa_workspace_size": ([_P, _I, _I, _I, _I, _P], ctypes.c_int),
    "csa_compress": ([_P, _I, _I, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "csa_index_topk": ([_P, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "csa_sparse_mqa": ([_P, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "hca_dense_mqa": ([_P, _I, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "csa_decode": ([_P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
                   ctypes.c_int),
    "csa_prefill": ([_P, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
                    ctypes.c_int),
    "csa_decode_noalloc": ([_P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
                           ctypes.c_int),
    "csa_query_proj": ([_P, _I, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "csa_output_proj": ([_P, _I, _I, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "csa_blocks_create": ([_I, _P], ctypes.c_int),
    "csa_blocks_destroy": ([_P], ctypes.c_int),
    "csa_blocks_counts": ([_P, _P, _P], ctypes.c_int),
    "csa_blocks_refcount": ([_P, _I, _P], ctypes.c_int),
    "csa_blocks_alloc": ([_P, _I, _P], ctypes.c_int),
    "csa_blocks_share": ([_P, _I, _P], ctypes.c_int),
    "csa_blocks_release": ([_P, _I, _P], ctypes.c_int),
    "csa_blocks_publish": ([_P, ctypes.c_uint64, _I], ctypes.c_int),
    "csa_blocks_lookup": ([_P, _I, _P, _P, _P], ctypes.c_int),
    "csa_blocks_chain_keys": ([_P, _I, _I, ctypes.c_uint64, _P], ctypes.c_int),
}

_lib = None


def lib():
    """Load libcsa.so (raises CsaError if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CsaError("libcsa.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def version():
    return lib().csa_version()


def last_error():
    return lib().csa_last_error().decode()


def profile_start():
    """Start bracketing every kernel launch of the library with hipEvents."""
    _check(lib().csa_profile_start(), "csa_profile_start")


def profile_stop():
    """Stop; returns {kernel name: (launches, summed event milliseconds)}."""
    buf = (KernelTime * 64)()
    n = ctypes.c_int32()
    _check(lib().csa_profile_stop(buf, 64, ctypes.byref(n)), "csa_profile_stop")
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(n.value)}


def _check(rc, what):
    if rc != 0:
        raise CsaError("%s failed (%d): %s" % (what, rc, last_error()))


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise CsaError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise CsaError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ---- argument checks: the library sees raw device pointers only, so every tensor's dtype and
# size is checked here against the config, the batch and the query count before the call (an
# undersized tensor would otherwise be read or written out of bounds on the device).

def _bytes(t):
    return t.numel() * t.element_size()


def _want(t, name, dtypes, numel=None, min_numel=None, min_bytes=None):
    """Raise CsaError unless t is a tensor of one of `dtypes` (names, e.g. "bfloat16") holding
    exactly `numel` elements / at least `min_numel` elements / at least `min_bytes` bytes."""
    if t is None:
        raise CsaError("%s is required" % name)
    dt = str(t.dtype).replace("torch.", "")
    if dtypes and dt not in dtypes:
        raise CsaError("%s has dtype %s, expected one of %s" % (name, dt, ", ".join(dtypes)))
    if numel is not None and t.numel() != numel:
        raise CsaError("%s holds %d elements, expected %d" % (name, t.numel(), numel))
    if min_numel is not None and t.numel() < min_numel:
        raise CsaError("%s holds %d elements, needs at least %d" % (name, t.numel(), min_numel))
    if min_bytes is not None and _bytes(t) < min_bytes:
        raise CsaError("%s holds %d bytes, needs at least %d" % (name, _bytes(t), min_bytes))


_BF16 = ("bfloat16", "int16", "uint16")
_U8 = ("uint8", "float8_e4m3fn", "int8")
_F32 = ("float32",)
_I32 = ("int32",)
_ANY4 = ("float32", "int32", "uint8", "uint32")  # 4-byte scale words (fp32, or 4 E8M0 bytes)


def _qi_width(cfg):
    """Bytes per indexer-query head: E4M3 codes, or packed MXFP4 codes."""
    return cfg.idx_dim // 2 if cfg.idx_query_format == IDX_MXFP4 else cfg.idx_dim


def _check_indexer_query(cfg, rows, qi, qi_scale, wi):
    _want(qi, "qi", _U8, numel=rows * cfg.idx_heads * _qi_width(cfg))
    _want(qi_scale, "qi_scale", _ANY4, min_bytes=rows * cfg.idx_heads * 4)
    if _bytes(qi_scale) != rows * cfg.idx_heads * 4:
        raise CsaError("qi_scale holds %d bytes, expected %d (4 per head)" %
                       (_bytes(qi_scale), rows * cfg.idx_heads * 4))
    _want(wi, "wi", _F32, numel=rows * cfg.idx_heads)


def _check_cache(cfg, cache, B, keys=False, tail=False):
    """The cache's tensors hold what B sequences of n_max entries (or the block pools) and their
    window rings need."""
    entries, window, n_entries, idx_keys, idx_scale, tail_t, table = cache._keep
    rows = (cache.n_blocks * cache.block_entries if cache.block_entries
            else B * cache.n_max)
    row_bytes = (cfg.head_dim + cfg.rope_dim if cfg.entry_format == ENT_MIXED
                 else 2 * cfg.head_dim)
    _want(entries, "cache entries", None, min_bytes=rows * row_bytes)
    _want(window, "cache window", _BF16, min_numel=B * cache.win_slots * cfg.head_dim)
    _want(n_entries, "cache n_entries", _I32, min_numel=B)
    if cache.block_entries:
        _want(table, "cache block_table", _I32, min_numel=B * cache.blocks_per_seq)
    if keys:
        kb = cfg.idx_dim // 2 if cfg.idx_key_format == IDX_MXFP4 else cfg.idx_dim
        _want(idx_keys, "cache idx_keys", _U8, min_bytes=rows * kb)
        _want(idx_scale, "cache idx_scale", None, min_bytes=rows * 4)
    if tail and tail_t is not None:
        r, c = tail_shape(cfg)
        _want(tail_t, "cache tail", _F32, min_numel=B * r * c)


def _check_attention(cfg, B, nq, q, pos, sink, out, lse_out=None):
    n = B * nq * cfg.n_heads * cfg.head_dim
    _want(q, "q", _BF16, numel=n)
    _want(out, "out", _BF16, numel=n)
    if pos is not None:
        _want(pos, "pos", _I32, numel=B * nq)
    _want(sink, "sink", _F32, numel=cfg.n_heads)
    if lse_out is not None:
        _want(lse_out, "lse_out", _F32, min_numel=B * nq * cfg.n_heads)


def make_config(mode, m, n_heads, head_dim, rope_dim, inv_freq, top_k=0, n_win=128,
                idx_heads=0, idx_dim=0, hidden=0, softmax_scale=None, rms_eps=1e-6,
                idx_key_format=0, q_rank=0, out_groups=0, out_rank=0, entry_format=0,
                idx_query_format=0, score_format=0):
    """A Config; keeps a reference to the device inv_freq tensor for the config's lifetime."""
    cfg = Config(mode, m, top_k, n_win, n_heads, head_dim, rope_dim, idx_heads, idx_dim, hidden,
                 float(softmax_scale if softmax_scale is not None else head_dim ** -0.5),
                 float(rms_eps), _ptr(inv_freq).value, int(idx_key_format), int(q_rank),
                 int(out_groups), int(out_rank), int(entry_format), int(idx_query_format),
                 int(score_format))
    cfg._keep = inv_freq
    return cfg


def make_cache(n_max, win_slots, entries, window, n_entries, idx_keys=None, idx_scale=None,
               tail=None, block_table=None, block_entries=0, n_blocks=0):
    """Contiguous cache, or (block_table [B, blocks_per_seq] int32 given) the block layout:
    entries / idx_keys / idx_scale are then pools of n_blocks blocks of block_entries rows and
    n_max must be blocks_per_seq * block_entries."""
    bps = int(block_table.shape[-1]) if block_table is not None else 0
    c = Cache(n_max, win_slots, _ptr(entries).value, _ptr(idx_keys) and _ptr(idx_keys).value,
              _ptr(idx_scale) and _ptr(idx_scale).value, _ptr(window).value,
              _ptr(tail) and _ptr(tail).value, _ptr(n_entries).value,
              block_entries if block_table is not None else 0, bps,
              n_blocks if block_table is not None else 0,
              _ptr(block_table) and _ptr(block_table).value)
    c._keep = (entries, window, n_entries, idx_keys, idx_scale, tail, block_table)
    return c


def make_weights(w_cat, bias_a, gamma, gamma_win, bias_b=None, bias_ia=None, bias_ib=None):
    v = lambda t: _ptr(t) and _ptr(t).value
    w = Weights(v(w_cat), v(bias_a), v(bias_b), v(bias_ia), v(bias_ib), v(gamma), v(gamma_win))
    w._keep = (w_cat, bias_a, bias_b, bias_ia, bias_ib, gamma, gamma_win)
    return w


def make_qproj_weights(w_dq, w_uq, gamma_q, w_w=None, w_iuq=None):
    v = lambda t: _ptr(t) and _ptr(t).value
    w = QProjWeights(v(w_dq), v(w_w), v(w_uq), v(w_iuq), v(gamma_q))
    w._keep = (w_dq, w_w, w_uq, w_iuq, gamma_q)
    return w


def make_oproj_weights(w_down, w_proj):
    w = OProjWeights(_ptr(w_down).value, _ptr(w_proj).value)
    w._keep = (w_down, w_proj)
    return w


def query_proj(cfg, H, weights, q_out, ws, qi_out=None, qi_scale_out=None, wi_out=None,
               stream=None):
    """csa_query_proj: H [B, T, hidden] -> q_out [B, T, n_heads, head_dim] (and the indexer
    query, its scales and head weights in CSA mode)."""
    B, T = H.shape[0], H.shape[1]
    _want(H, "H", _BF16, numel=B * T * cfg.hidden)
    _want(q_out, "q_out", _BF16, numel=B * T * cfg.n_heads * cfg.head_dim)
    if cfg.mode == MODE_CSA:
        _check_indexer_query(cfg, B * T, qi_out, qi_scale_out, wi_out)
    wp, wn = _ws(ws)
    _check(lib().csa_query_proj(ctypes.byref(cfg), B, T, _ptr(H), ctypes.byref(weights),
                                _ptr(q_out), _ptr(qi_out), _ptr(qi_scale_out), _ptr(wi_out), wp,
                                wn, _stream(stream)), "csa_query_proj")


def output_proj(cfg, O, weights, y_out, ws, stream=None):
    """csa_output_proj: O [B, T, n_heads, head_dim] -> y_out [B, T, hidden]."""
    B, T = O.shape[0], O.shape[1]
    _want(O, "O", _BF16, numel=B * T * cfg.n_heads * cfg.head_dim)
    _want(y_out, "y_out", _BF16, numel=B * T * cfg.hidden)
    wp, wn = _ws(ws)
    _check(lib().csa_output_proj(ctypes.byref(cfg), B, T, _ptr(O), ctypes.byref(weights),
                                 _ptr(y_out), wp, wn, _stream(stream)), "csa_output_proj")


def weight_cols(cfg):
    n = ctypes.c_int32()
    _check(lib().csa_weight_cols(ctypes.byref(cfg), ctypes.byref(n)), "csa_weight_cols")
    return n.value


def tail_shape(cfg):
    r, c = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().csa_tail_shape(ctypes.byref(cfg), ctypes.byref(r), ctypes.byref(c)),
           "csa_tail_shape")
    return r.value, c.value


def workspace_size(cfg, op, B, nq, n_max):
    b = ctypes.c_size_t()
    _check(lib().csa_workspace_size(ctypes.byref(cfg), op, B, nq, n_max, ctypes.byref(b)),
           "csa_workspace_size")
    return b.value


def _ws(ws):
    return (_ptr(ws), ws.numel() * ws.element_size()) if ws is not None else (None, 0)


def compress(cfg, H, pos0, weights, cache, ws, stream=None):
    B, T = H.shape[0], H.shape[1]
    _want(H, "H", _BF16, numel=B * T * cfg.hidden)
    _want(pos0, "pos0", _I32, numel=B)
    _check_cache(cfg, cache, B, keys=cfg.mode == MODE_CSA, tail=True)
    wp, wn = _ws(ws)
    _check(lib().csa_compress(ctypes.byref(cfg), B, T, _ptr(H), _ptr(pos0),
                              ctypes.byref(weights), ctypes.byref(cache), wp, wn,
                              _stream(stream)), "csa_compress")


def index_topk(cfg, qi, qi_scale, wi, cache, pos, idx_out, ws, score_out=None, stream=None):
    B, nq = qi.shape[0], qi.shape[1]
    _check_indexer_query(cfg, B * nq, qi, qi_scale, wi)
    _want(pos, "pos", _I32, numel=B * nq)
    _want(idx_out, "idx_out", _I32, min_numel=B * nq * cfg.top_k)
    if score_out is not None:
        _want(score_out, "score_out", _F32, min_numel=B * nq * cfg.top_k)
    _check_cache(cfg, cache, B, keys=True)
    wp, wn = _ws(ws)
    _check(lib().csa_index_topk(ctypes.byref(cfg), B, nq, _ptr(qi), _ptr(qi_scale), _ptr(wi),
                                ctypes.byref(cache), _ptr(pos), _ptr(idx_out), _ptr(score_out),
                                wp, wn, _stream(stream)), "csa_index_topk")


def sparse_mqa(cfg, q, cache, idx, pos, sink, out, ws, lse_out=None, stream=None):
    B, nq = q.shape[0], q.shape[1]
    _check_attention(cfg, B, nq, q, pos, sink, out, lse_out)
    _want(pos, "pos", _I32, numel=B * nq)
    _want(idx, "idx", _I32, min_numel=B * nq * cfg.top_k)
    _check_cache(cfg, cache, B)
    wp, wn = _ws(ws)
    _check(lib().csa_sparse_mqa(ctypes.byref(cfg), B, nq, _ptr(q), ctypes.byref(cache),
                                _ptr(idx), _ptr(pos), _ptr(sink), _ptr(out), _ptr(lse_out),
                                wp, wn, _stream(stream)), "csa_sparse_mqa")


def hca_dense_mqa(cfg, q, cache, pos, sink, out, ws, lse_out=None, stream=None):
    B, nq = q.shape[0], q.shape[1]
    _check_attention(cfg, B, nq, q, pos, sink, out, lse_out)
    _want(pos, "pos", _I32, numel=B * nq)
    _check_cache(cfg, cache, B)
    wp, wn = _ws(ws)
    _check(lib().hca_dense_mqa(ctypes.byref(cfg), B, nq, _ptr(q), ctypes.byref(cache),
                               _ptr(pos), _ptr(sink), _ptr(out), _ptr(lse_out), wp, wn,
                               _stream(stream)), "hca_dense_mqa")


def _check_decode(cfg, B, cache, pos, q, sink, out, h_new, qi, qi_scale, wi, idx_out):
    _check_attention(cfg, B, 1, q, pos, sink, out)
    _want(pos, "pos", _I32, numel=B)
    if h_new is not None:
        _want(h_new, "h_new", _BF16, numel=B * cfg.hidden)
    csa_mode = cfg.mode == MODE_CSA
    if csa_mode:
        _check_indexer_query(cfg, B, qi, qi_scale, wi)
        if idx_out is not None:
            _want(idx_out, "idx_out", _I32, min_numel=B * cfg.top_k)
    _check_cache(cfg, cache, B, keys=csa_mode, tail=h_new is not None)


def decode(cfg, cache, pos, q, sink, out, ws, h_new=None, weights=None, qi=None, qi_scale=None,
           wi=None, idx_out=None, stream=None):
    B = q.shape[0]
    _check_decode(cfg, B, cache, pos, q, sink, out, h_new, qi, qi_scale, wi, idx_out)
    wp, wn = _ws(ws)
    _check(lib().csa_decode(ctypes.byref(cfg), B, _ptr(h_new),
                            ctypes.byref(weights) if weights is not None else None,
                            ctypes.byref(cache), _ptr(pos), _ptr(q), _ptr(qi), _ptr(qi_scale),
                            _ptr(wi), _ptr(sink), _ptr(out), _ptr(idx_out), wp, wn,
                            _stream(stream)), "csa_decode")


def decode_noalloc(cfg, cache, pos, q, sink, out, h_new=None, weights=None, qi=None,
                   qi_scale=None, wi=None, idx_out=None, stream=None):
    """csa_decode_noalloc: csa_decode with the library's static device scratch instead of a
    workspace (for callers that cannot allocate; calls overlapping on one GPU race)."""
    B = q.shape[0]
    _check_decode(cfg, B, cache, pos, q, sink, out, h_new, qi, qi_scale, wi, idx_out)
    _check(lib().csa_decode_noalloc(ctypes.byref(cfg), B, _ptr(h_new),
                                    ctypes.byref(weights) if weights is not None else None,
                                    ctypes.byref(cache), _ptr(pos), _ptr(q), _ptr(qi),
                                    _ptr(qi_scale), _ptr(wi), _ptr(sink), _ptr(out),
                                    _ptr(idx_out), _stream(stream)), "csa_decode_noalloc")


def prefill(cfg, H, weights, cache, q, sink, out, ws, qi=None, qi_scale=None, wi=None,
            idx_out=None, pos0=None, stream=None):
    """pos0=None: tokens 0..T-1 of every sequence; an int32 [B] device tensor: a chunk that
    continues sequence b at position pos0[b] (chunked prefill)."""
    B, T = H.shape[0], H.shape[1]
    _want(H, "H", _BF16, numel=B * T * cfg.hidden)
    if pos0 is not None:
        _want(pos0, "pos0", _I32, numel=B)
    _check_attention(cfg, B, T, q, None, sink, out)
    csa_mode = cfg.mode == MODE_CSA
    if csa_mode:
        _check_indexer_query(cfg, B * T, qi, qi_scale, wi)
        if idx_out is not None:
            _want(idx_out, "idx_out", _I32, min_numel=B * T * cfg.top_k)
    _check_cache(cfg, cache, B, keys=csa_mode, tail=True)
    wp, wn = _ws(ws)
    _check(lib().csa_prefill(ctypes.byref(cfg), B, T, _ptr(H), _ptr(pos0), ctypes.byref(weights),
                             ctypes.byref(cache), _ptr(q), _ptr(qi), _ptr(qi_scale), _ptr(wi),
                             _ptr(sink), _ptr(out), _ptr(idx_out), wp, wn, _stream(stream)),
           "csa_prefill")


class BlockManager:
    """Host-side block manager of the block cache layout (csa_blocks_*): reference counts, free
    blocks, and a registry of full blocks by token-prefix key for prefix reuse."""

    def __init__(self, n_blocks):
        self._m = ctypes.c_void_p()
        _check(lib().csa_blocks_create(int(n_blocks), ctypes.byref(self._m)), "csa_blocks_create")

    def close(self):
        if self._m:
            lib().csa_blocks_destroy(self._m)
            self._m = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _ids(blocks):
        a = (ctypes.c_int32 * len(blocks))(*[int(b) for b in blocks])
        return a, len(blocks)

    def counts(self):
        f, i = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().csa_blocks_counts(self._m, ctypes.byref(f), ctypes.byref(i)),
               "csa_blocks_counts")
        return f.value, i.value

    def refcount(self, block):
        c = ctypes.c_int32()
        _check(lib().csa_blocks_refcount(self._m, int(block), ctypes.byref(c)),
               "csa_blocks_refcount")
        return c.value

    def alloc(self, n):
        a = (ctypes.c_int32 * max(n, 1))()
        _check(lib().csa_blocks_alloc(self._m, int(n), a), "csa_blocks_alloc")
        return list(a[:n])

    def share(self, blocks):
        a, n = self._ids(blocks)
        _check(lib().csa_blocks_share(self._m, n, a), "csa_blocks_share")

    def release(self, blocks):
        a, n = self._ids(blocks)
        _check(lib().csa_blocks_release(self._m, n, a), "csa_blocks_release")

    def publish(self, key, block):
        _check(lib().csa_blocks_publish(self._m, ctypes.c_uint64(key), int(block)),
               "csa_blocks_publish")

    def lookup(self, keys):
        k = (ctypes.c_uint64 * max(len(keys), 1))(*[int(x) for x in keys])
        b = (ctypes.c_int32 * max(len(keys), 1))()
        h = ctypes.c_int32()
        _check(lib().csa_blocks_lookup(self._m, len(keys), k, b, ctypes.byref(h)),
               "csa_blocks_lookup")
        return list(b[:h.value])


def chain_keys(tokens, block_tokens=128, seed=0):
    """Prefix keys of the whole blocks of a token-id sequence (csa_blocks_chain_keys)."""
    t = (ctypes.c_int32 * max(len(tokens), 1))(*[int(x) for x in tokens])
    nb = len(tokens) // block_tokens
    k = (ctypes.c_uint64 * max(nb, 1))()
    _check(lib().csa_blocks_chain_keys(t, len(tokens), int(block_tokens), ctypes.c_uint64(seed),
                                       k), "csa_blocks_chain_keys")
    return list(k[:nb])
