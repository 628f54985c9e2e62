"""Python binding of libhca.so, the MI355X (gfx950) CSA + HCA hybrid-attention library.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in include/hca.h. Tensors are torch CUDA tensors (device memory) and
work is enqueued on the current torch stream unless `stream` is given. There is
no fallback: if libhca.so is missing or fails to load, importing this module
raises.

Function names, argument order and meaning follow include/hca.h.
"""

import ctypes
import os

import torch

__all__ = [
    "F32", "BF16", "FP8_E4M3", "MXFP4", "LAYOUT_F32", "LAYOUT_BF16", "LAYOUT_SPLIT", "LAYOUT_MXFP4",
    "HcaError", "Store", "DecodeLayer", "abi_version", "csa_compress", "hca_compress", "decode_append",
    "lightning_index_topk_workspace", "lightning_index_topk", "mqa_attn_workspace",
    "csa_sparse_mqa_attn", "hca_dense_mqa_attn", "hca_dense_mqa_attn_noalloc", "AttnPartials",
    "csa_sparse_mqa_attn_partials", "hca_dense_mqa_attn_partials", "mqa_attn_merge", "PendingSelect",
    "lightning_index_select_pending", "hca_dense_mqa_attn_partials_select", "grouped_out_proj",
    "library_path",
]

F32, BF16, FP8_E4M3, MXFP4 = 0, 1, 2, 3
LAYOUT_F32, LAYOUT_BF16, LAYOUT_SPLIT, LAYOUT_MXFP4 = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libhca.so")

if not os.path.exists(library_path):
    raise ImportError(f"{library_path} is not built; run `python long_context_attention_hca_amd/build.py` "
                      "(or __graft_entry__.build())")
_lib = ctypes.CDLL(library_path)


class _StoreC(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("n_rows", ctypes.c_int64), ("data", ctypes.c_void_p),
                ("row_stride", ctypes.c_int64), ("scale", ctypes.c_void_p), ("rope", ctypes.c_void_p),
                ("rope_stride", ctypes.c_int64)]


class _DecodeLayerC(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("w", ctypes.c_int32), ("m_prime", ctypes.c_int32), ("W", ctypes.c_int32),
                ("R", ctypes.c_int32), ("d_idx", ctypes.c_int32),
                ("bias_csa", ctypes.c_void_p), ("bias_hca", ctypes.c_void_p), ("bias_idx", ctypes.c_void_p),
                ("ring_x", ctypes.c_void_p), ("ring_z_csa", ctypes.c_void_p), ("ring_z_hca", ctypes.c_void_p),
                ("ring_k_idx", ctypes.c_void_p), ("ring_z_idx", ctypes.c_void_p), ("hca_state", ctypes.c_void_p),
                ("window", _StoreC), ("win_row_begin", ctypes.c_void_p), ("win_pos0", ctypes.c_void_p),
                ("csa", _StoreC), ("csa_row_begin", ctypes.c_void_p),
                ("hca", _StoreC), ("hca_row_begin", ctypes.c_void_p),
                ("idx", _StoreC), ("idx_row_begin", ctypes.c_void_p)]


_P, _I32, _I64, _SZ, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_SP = ctypes.POINTER(_StoreC)


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_abi = _sig("hca_abi_version", ctypes.c_int, [])
_status_string = _sig("hca_status_string", ctypes.c_char_p, [ctypes.c_int])
_last_error = _sig("hca_last_error", ctypes.c_char_p, [])
_compress_args = [_P, _I32, _I64, _I64, _I64, _P, _I64, _I64, _P]
_csa_compress = _sig("csa_compress", ctypes.c_int, _compress_args + [_I32, _I32, _I64, _I64, _SP, _I64, _P])
_hca_compress = _sig("hca_compress", ctypes.c_int, _compress_args + [_I32, _I64, _I64, _SP, _I64, _P])
_proj = _sig("grouped_out_proj", ctypes.c_int, [_P, _I64, _I64, _I32, _I32, _P, _I32, _P, _I32, _I64, _P])
_decode_append = _sig("decode_append", ctypes.c_int,
                      [ctypes.POINTER(_DecodeLayerC), _I32, _P, _P, _P, _P, _P, _P, _P])
_index_ws = _sig("lightning_index_topk_workspace", _SZ, [_I32, _I64, _I32])
_index_argtypes = [_P, _P, _P, _I32, _I32, _I32, _P, _P, _I64, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32, _P, _P,
                   _SZ, _P]
_index = _sig("lightning_index_topk", ctypes.c_int, _index_argtypes)
_index_phase = {"both": _index, "scores": _sig("lightning_index_scores", ctypes.c_int, _index_argtypes),
                "select": _sig("lightning_index_select", ctypes.c_int, _index_argtypes)}
_attn_ws = _sig("mqa_attn_workspace", _SZ, [_I32, _I32, _I32, _I32, _I64])
_attn_tail = [_SP, _P, _P, _I32, _P, _P, _P, _F, _P, _I32, _P, _P, _SZ, _P]
_csa_attn = _sig("csa_sparse_mqa_attn", ctypes.c_int, [_P, _I32, _I32, _I32, _SP, _P, _P, _I32] + _attn_tail)
_hca_attn = _sig("hca_dense_mqa_attn", ctypes.c_int, [_P, _I32, _I32, _I32, _SP, _P, _I32, _I64] + _attn_tail)
_hca_attn_noalloc = _sig("hca_dense_mqa_attn_noalloc", ctypes.c_int,
                         [_P, _I32, _I32, _I32, _SP, _P, _I32, _I64] + _attn_tail[:-3] + [_P])


class AttnPartials(ctypes.Structure):
    """hca_attn_partials: where a deferred attention call left its split-K partials."""
    _fields_ = [("part_o", ctypes.c_void_p), ("part_lse", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("nq", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("d", ctypes.c_int32),
                ("n_split", ctypes.c_int32), ("o_dtype", ctypes.c_int32)]


_AP = ctypes.POINTER(AttnPartials)
_csa_attn_partials = _sig("csa_sparse_mqa_attn_partials", ctypes.c_int,
                          [_P, _I32, _I32, _I32, _SP, _P, _P, _I32] + _attn_tail + [_AP])
_hca_attn_partials = _sig("hca_dense_mqa_attn_partials", ctypes.c_int,
                          [_P, _I32, _I32, _I32, _SP, _P, _I32, _I64] + _attn_tail + [_AP])
_attn_merge = _sig("mqa_attn_merge", ctypes.c_int, [_AP, _AP, _P])


class PendingSelect(ctypes.Structure):
    """hca_pending_select: a top-k selection recorded by lightning_index_select_pending."""
    _fields_ = [("opaque", ctypes.c_uint64 * 48)]


_PS = ctypes.POINTER(PendingSelect)
_index_pending = _sig("lightning_index_select_pending", ctypes.c_int, _index_argtypes + [_PS])
_hca_attn_partials_select = _sig("hca_dense_mqa_attn_partials_select", ctypes.c_int,
                                 [_P, _I32, _I32, _I32, _SP, _P, _I32, _I64] + _attn_tail + [_PS, _AP])


class HcaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"[{status}] {message}")
        self.status = status


def _check(status):
    if status != 0:
        raise HcaError(status, _last_error().decode())


def abi_version():
    return _abi()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    if t.dtype == torch.uint8:
        return MXFP4
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


class Store:
    """A view of KV rows (compressed entries or raw window tokens) for the C ABI.

    dense: `data` [n_rows, >=D] float32 or bf16 (torch.bfloat16 / int16 bits).
    split: `data` uint8 E4M3 codes [n_rows, >=d_nope], `scale` float32 [n_rows],
           `rope` bf16 bits [n_rows, >=d_rope].
    mxfp4: `data` uint8 E2M1 codes [n_rows, >=D/2], the E8M0 scales uint8
           [n_rows, >=D/32] in the `rope` slot (d_nope = D, d_rope = 0).
    Tensors are kept referenced by the Store.
    """

    def __init__(self, layout, d_nope, d_rope, data, scale=None, rope=None):
        self.layout, self.d_nope, self.d_rope = layout, int(d_nope), int(d_rope)
        self.data, self.scale, self.rope = data, scale, rope
        self._c = _StoreC(layout, self.d_nope, self.d_rope, 0, data.shape[0], data.data_ptr(), data.stride(0),
                          scale.data_ptr() if scale is not None else None,
                          rope.data_ptr() if rope is not None else None,
                          rope.stride(0) if rope is not None else 0)

    @classmethod
    def dense(cls, data, d_nope, d_rope):
        layout = LAYOUT_F32 if data.dtype == torch.float32 else LAYOUT_BF16
        return cls(layout, d_nope, d_rope, data)

    @classmethod
    def split(cls, nope, scale, rope):
        return cls(LAYOUT_SPLIT, nope.shape[1], rope.shape[1], nope, scale, rope)

    @classmethod
    def mxfp4(cls, codes, scales):
        return cls(LAYOUT_MXFP4, codes.shape[1] * 2, 0, codes, None, scales)

    @property
    def n_rows(self):
        return self.data.shape[0]

    def c(self):
        return ctypes.byref(self._c)


def csa_compress(raw, first_pos, logits, pos_bias, m, w, first_entry, n_entries, out, out_row0=0,
                 scalar_logits=False, stream=None):
    _check(_csa_compress(_ptr(raw), _dtype_code(raw), raw.stride(0), raw.shape[0], first_pos, _ptr(logits),
                         logits.stride(0), 0 if scalar_logits else 1, _ptr(pos_bias), m, w, first_entry,
                         n_entries, out.c(), out_row0, _stream(stream)))


def hca_compress(raw, first_pos, logits, pos_bias, m_prime, first_entry, n_entries, out, out_row0=0,
                 scalar_logits=False, stream=None):
    _check(_hca_compress(_ptr(raw), _dtype_code(raw), raw.stride(0), raw.shape[0], first_pos, _ptr(logits),
                         logits.stride(0), 0 if scalar_logits else 1, _ptr(pos_bias), m_prime, first_entry,
                         n_entries, out.c(), out_row0, _stream(stream)))


class DecodeLayer:
    """One layer's decode-time state for decode_append (the hca_decode_layer of include/hca.h).

    rings: dict of bf16 tensors "x", "z_csa", "z_hca" [B * R, D] and, with indexer keys,
    "k_idx", "z_idx" [B * R, d_idx]; hca_state: float32 [B, 3, D]; window / csa / hca / idx:
    Stores; *_row_begin: int64 [B] device tensors; win_pos0: int64 [B] (written by
    decode_append). Tensors are kept referenced.
    """

    def __init__(self, m, w, m_prime, W, R, bias_csa, bias_hca, rings, hca_state, window, win_row_begin, win_pos0,
                 csa, csa_row_begin, hca, hca_row_begin, idx=None, idx_row_begin=None, bias_idx=None):
        self.keep = (bias_csa, bias_hca, bias_idx, rings, hca_state, window, win_row_begin, win_pos0, csa,
                     csa_row_begin, hca, hca_row_begin, idx, idx_row_begin)
        d_idx = 0 if idx is None else idx.d_nope + idx.d_rope
        p = lambda t: None if t is None else t.data_ptr()
        self._c = _DecodeLayerC(m, w, m_prime, W, R, d_idx, p(bias_csa), p(bias_hca), p(bias_idx),
                                p(rings["x"]), p(rings["z_csa"]), p(rings["z_hca"]),
                                p(rings.get("k_idx")), p(rings.get("z_idx")), p(hca_state),
                                window._c, p(win_row_begin), p(win_pos0), csa._c, p(csa_row_begin), hca._c,
                                p(hca_row_begin), idx._c if idx is not None else _StoreC(),
                                p(idx_row_begin))

    def c(self):
        return ctypes.byref(self._c)


def decode_append(layer, pos, x, z_csa, z_hca, k_idx=None, z_idx=None, stream=None):
    """One decode step: pos int64 [B] (negative = idle slot), x / z_csa / z_hca bf16 [B, D],
    k_idx / z_idx bf16 [B, d_idx] (with indexer keys)."""
    _check(_decode_append(layer.c(), pos.shape[0], _ptr(pos), _ptr(x), _ptr(z_csa), _ptr(z_hca), _ptr(k_idx),
                          _ptr(z_idx), _stream(stream)))


def grouped_out_proj(x, w, y, stream=None):
    """x: bf16 [n, G * K] (e.g. the attention output [n, h, D] viewed as [n, h * D]); w: bf16
    [G, N, K]; y: bf16 or float32 [n, G * N] (row strides from the tensors)."""
    G, N, K = w.shape
    _check(_proj(_ptr(x), x.shape[0], x.stride(0), G, K, _ptr(w), N, _ptr(y), _dtype_code(y), y.stride(0),
                 _stream(stream)))


def lightning_index_topk_workspace(nq, max_visible, k):
    return _index_ws(nq, max_visible, k)


def lightning_index_topk(q_idx, w_idx, k_idx, k_row_begin, q_seq, q_pos, max_visible, m, k, out_idx, ws,
                         q_idx_scale=None, k_idx_scale=None, idx_dtype=None, q_lo=None, w=None, phase="both",
                         stream=None):
    """q_idx [nq, H, d] (f32/bf16) or [nq, H, d/2] uint8 (MXFP4, with scales). q_lo: int64 [nq]
    document starts (None: no document mask); w: the CSA window (default 2m). phase "scores" /
    "select" calls lightning_index_scores / lightning_index_select (the two halves)."""
    _check(_index_phase[phase](*_index_call_args(q_idx, w_idx, k_idx, k_row_begin, q_seq, q_pos, max_visible, m, k,
                                                 out_idx, ws, q_idx_scale, k_idx_scale, idx_dtype, q_lo, w, stream)))


def _index_call_args(q_idx, w_idx, k_idx, k_row_begin, q_seq, q_pos, max_visible, m, k, out_idx, ws, q_idx_scale,
                     k_idx_scale, idx_dtype, q_lo, w, stream):
    dt = _dtype_code(q_idx) if idx_dtype is None else idx_dtype
    nq, H = q_idx.shape[0], q_idx.shape[1]
    d = q_idx.shape[2] * (2 if dt == MXFP4 else 1)
    return (_ptr(q_idx), _ptr(q_idx_scale), _ptr(w_idx), H, d, dt, _ptr(k_idx), _ptr(k_idx_scale), k_idx.shape[0],
            _ptr(k_row_begin), _ptr(q_seq), _ptr(q_pos), _ptr(q_lo), nq, max_visible, m, 2 * m if w is None else w, k,
            _ptr(out_idx), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))


def lightning_index_select_pending(q_idx, w_idx, k_idx, k_row_begin, q_seq, q_pos, max_visible, m, k, out_idx, ws,
                                   q_idx_scale=None, k_idx_scale=None, idx_dtype=None, q_lo=None, w=None):
    """lightning_index_topk's selection phase recorded, not enqueued: returns the PendingSelect that
    hca_dense_mqa_attn_partials_select runs. The tensors must stay alive until then."""
    out = PendingSelect()
    _check(_index_pending(*_index_call_args(q_idx, w_idx, k_idx, k_row_begin, q_seq, q_pos, max_visible, m, k,
                                            out_idx, ws, q_idx_scale, k_idx_scale, idx_dtype, q_lo, w, None),
                          ctypes.byref(out)))
    return out


def mqa_attn_workspace(q_dtype, nq, n_heads, d, max_entries):
    return _attn_ws(q_dtype, nq, n_heads, d, max_entries)


def _ws_args(ws):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def csa_sparse_mqa_attn(q, cache, cache_row_begin, idx, window, win_row_begin, win_pos0, W, q_seq, q_pos, scale,
                        o, lse, ws=None, q_lo=None, stream=None):
    if not idx.is_contiguous():
        raise ValueError("idx must be contiguous [nq, k] (rows of k slots)")
    wp, wb = _ws_args(ws)
    _check(_csa_attn(_ptr(q), _dtype_code(q), q.shape[0], q.shape[1], cache.c(), _ptr(cache_row_begin),
                     _ptr(idx), idx.shape[1], window.c(), _ptr(win_row_begin), _ptr(win_pos0), W, _ptr(q_seq),
                     _ptr(q_pos), _ptr(q_lo), scale, _ptr(o), _dtype_code(o), _ptr(lse), wp, wb, _stream(stream)))


def hca_dense_mqa_attn(q, cache, cache_row_begin, m_prime, max_visible, window, win_row_begin, win_pos0, W, q_seq,
                       q_pos, scale, o, lse, ws=None, q_lo=None, stream=None):
    wp, wb = _ws_args(ws)
    _check(_hca_attn(_ptr(q), _dtype_code(q), q.shape[0], q.shape[1], cache.c(), _ptr(cache_row_begin), m_prime,
                     max_visible, window.c(), _ptr(win_row_begin), _ptr(win_pos0), W, _ptr(q_seq), _ptr(q_pos),
                     _ptr(q_lo), scale, _ptr(o), _dtype_code(o), _ptr(lse), wp, wb, _stream(stream)))


def csa_sparse_mqa_attn_partials(q, cache, cache_row_begin, idx, window, win_row_begin, win_pos0, W, q_seq, q_pos,
                                 scale, o, lse, ws=None, q_lo=None, stream=None):
    """csa_sparse_mqa_attn without its split-K merge: returns the AttnPartials that mqa_attn_merge takes."""
    if not idx.is_contiguous():
        raise ValueError("idx must be contiguous [nq, k] (rows of k slots)")
    wp, wb = _ws_args(ws)
    out = AttnPartials()
    _check(_csa_attn_partials(_ptr(q), _dtype_code(q), q.shape[0], q.shape[1], cache.c(), _ptr(cache_row_begin),
                              _ptr(idx), idx.shape[1], window.c(), _ptr(win_row_begin), _ptr(win_pos0), W,
                              _ptr(q_seq), _ptr(q_pos), _ptr(q_lo), scale, _ptr(o), _dtype_code(o), _ptr(lse), wp, wb,
                              _stream(stream), ctypes.byref(out)))
    return out


def hca_dense_mqa_attn_partials(q, cache, cache_row_begin, m_prime, max_visible, window, win_row_begin, win_pos0, W,
                                q_seq, q_pos, scale, o, lse, ws=None, q_lo=None, stream=None):
    """hca_dense_mqa_attn without its split-K merge: returns the AttnPartials that mqa_attn_merge takes."""
    wp, wb = _ws_args(ws)
    out = AttnPartials()
    _check(_hca_attn_partials(_ptr(q), _dtype_code(q), q.shape[0], q.shape[1], cache.c(), _ptr(cache_row_begin),
                              m_prime, max_visible, window.c(), _ptr(win_row_begin), _ptr(win_pos0), W, _ptr(q_seq),
                              _ptr(q_pos), _ptr(q_lo), scale, _ptr(o), _dtype_code(o), _ptr(lse), wp, wb,
                              _stream(stream), ctypes.byref(out)))
    return out


def hca_dense_mqa_attn_partials_select(q, cache, cache_row_begin, m_prime, max_visible, window, win_row_begin,
                                       win_pos0, W, q_seq, q_pos, scale, o, lse, sel, ws=None, q_lo=None,
                                       stream=None):
    """hca_dense_mqa_attn_partials with the recorded selection `sel` (a PendingSelect) enqueued as one
    unit: returns the AttnPartials that mqa_attn_merge takes."""
    wp, wb = _ws_args(ws)
    out = AttnPartials()
    _check(_hca_attn_partials_select(_ptr(q), _dtype_code(q), q.shape[0], q.shape[1], cache.c(),
                                     _ptr(cache_row_begin), m_prime, max_visible, window.c(), _ptr(win_row_begin),
                                     _ptr(win_pos0), W, _ptr(q_seq), _ptr(q_pos), _ptr(q_lo), scale, _ptr(o),
                                     _dtype_code(o), _ptr(lse), wp, wb, _stream(stream), ctypes.byref(sel),
                                     ctypes.byref(out)))
    return out


def mqa_attn_merge(a, b=None, stream=None):
    """Merges the partials of one deferred attention call, or of two in one launch."""
    _check(_attn_merge(ctypes.byref(a), None if b is None else ctypes.byref(b), _stream(stream)))


def hca_dense_mqa_attn_noalloc(q, cache, cache_row_begin, m_prime, max_visible, window, win_row_begin, win_pos0, W,
                               q_seq, q_pos, scale, o, lse, q_lo=None, stream=None):
    """hca_dense_mqa_attn without a workspace (the library's static 16 MiB scratch; allocates nothing)."""
    _check(_hca_attn_noalloc(_ptr(q), _dtype_code(q), q.shape[0], q.shape[1], cache.c(), _ptr(cache_row_begin),
                             m_prime, max_visible, window.c(), _ptr(win_row_begin), _ptr(win_pos0), W, _ptr(q_seq),
                             _ptr(q_pos), _ptr(q_lo), scale, _ptr(o), _dtype_code(o), _ptr(lse), _stream(stream)))
