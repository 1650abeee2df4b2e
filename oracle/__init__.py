"""CPU oracle for the BF16 DiT row epilogues -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it.

Everything here is a thin ctypes marshalling layer over ``dit_oracle.c``;
bf16 tensors are numpy ``uint16`` arrays holding bit patterns.  Row tensors
are 2-D ``[rows, dim]`` (any row stride, unit element stride).
"""
import contextlib
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


class QkvStream(ctypes.Structure):
    _fields_ = [
        ("q", _u16p), ("k", _u16p), ("v", _u16p),
        ("tok_stride", _i64), ("batch_stride", _i64),
        ("q_weight", _u16p), ("k_weight", _u16p),
        ("tokens", _i64),
    ]


def load(path=None):
    """Loads liboracle.so, building it first only if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            _build.build()
    lib = ctypes.CDLL(path)
    lib.orc_bf16_round.restype = ctypes.c_uint16
    lib.orc_bf16_round.argtypes = [ctypes.c_float]
    lib.orc_bf16_value.restype = ctypes.c_float
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_round_f64.restype = ctypes.c_uint16
    lib.orc_bf16_round_f64.argtypes = [ctypes.c_double]
    lib.orc_sum_wave.restype = ctypes.c_float
    lib.orc_sum_wave.argtypes = [_f32p, _i64]
    lib.orc_sum_head.restype = ctypes.c_float
    lib.orc_sum_head.argtypes = [_f32p, _i64]
    for name in ("orc_one_plus", "orc_tanh", "orc_rms_rstd"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_uint16
        fn.argtypes = [ctypes.c_uint16]
    lib.orc_ln_row.argtypes = [_u16p, _i64, ctypes.c_float, _u16p, _f32p]
    lib.orc_rms_row.argtypes = [_u16p, _u16p, _i64, ctypes.c_float, _u16p, _f32p]
    lib.orc_qk_head.argtypes = [_u16p, _u16p, _f32p, _f32p, _i64, ctypes.c_float, _u16p]
    lib.orc_ln_modulate.restype = ctypes.c_int
    lib.orc_ln_modulate.argtypes = [_u16p, _i64, _u16p, _i64, _u16p, _u16p, _i64, _i64, _i64,
                                    _i64, ctypes.c_float]
    lib.orc_rmsnorm_scale.restype = ctypes.c_int
    lib.orc_rmsnorm_scale.argtypes = [_u16p, _i64, _u16p, _i64, _u16p, _u16p, _i64, _i64, _i64,
                                      _i64, ctypes.c_float]
    lib.orc_rmsnorm_tanh_residual.restype = ctypes.c_int
    lib.orc_rmsnorm_tanh_residual.argtypes = [_u16p, _i64, _u16p, _i64, _u16p, _i64, _u16p,
                                              _u16p, _i64, _i64, _i64, _i64, ctypes.c_float]
    lib.orc_residual_gate_add.restype = ctypes.c_int
    lib.orc_residual_gate_add.argtypes = [_u16p, _i64, _u16p, _i64, _u16p, _i64, _u16p, _i64,
                                          _i64, _i64, _i64]
    lib.orc_gate_add_ln_modulate.restype = ctypes.c_int
    lib.orc_gate_add_ln_modulate.argtypes = [_u16p, _i64, _u16p, _i64, _u16p, _i64, _u16p, _i64,
                                             _u16p, _u16p, _u16p, _i64, _i64, _i64, _i64,
                                             ctypes.c_float]
    lib.orc_wan_mod_table.restype = ctypes.c_int
    lib.orc_wan_mod_table.argtypes = [_f32p, _f32p, _u16p, _i64, _i64, _i64, _i64]
    lib.orc_modulate_scale_shift.restype = ctypes.c_int
    lib.orc_modulate_scale_shift.argtypes = [_u16p, _i64, _u16p, _i64, _u16p, _u16p, _i64, _i64,
                                             _i64, _i64]
    lib.orc_qk_norm_rope.restype = ctypes.c_int
    lib.orc_qk_norm_rope.argtypes = [_u16p, _u16p, _u16p, _i64, _i64,
                                     ctypes.POINTER(QkvStream), ctypes.POINTER(QkvStream),
                                     _f32p, _f32p, _i64, _i64, _i64, ctypes.c_float]
    lib.orc_qk_norm_rope_dest.restype = ctypes.c_int
    lib.orc_qk_norm_rope_dest.argtypes = [_u16p, _u16p, _u16p, _i64, _i64, _i64, _i64,
                                          ctypes.POINTER(QkvStream), ctypes.POINTER(QkvStream),
                                          _f32p, _f32p, _i64, _i64, _i64, ctypes.c_float]
    lib.orc_bf16_round_array.argtypes = [_f32p, _u16p, _i64]
    lib.orc_bf16_round_bits_range.argtypes = [ctypes.c_uint32, _i64, _u16p]
    lib.orc_e4m3.restype = ctypes.c_uint8
    lib.orc_e4m3.argtypes = [ctypes.c_float]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_array.argtypes = [_f32p, _u8p, _i64]
    lib.orc_e4m3_bits_range.argtypes = [ctypes.c_uint32, _i64, _u8p]
    lib.orc_ln_modulate_fp8.restype = ctypes.c_int
    lib.orc_ln_modulate_fp8.argtypes = [_u16p, _i64, _u8p, _i64, _u16p, _i64, _u16p, _u16p, _i64,
                                        _i64, _i64, _i64, ctypes.c_float, ctypes.c_float]
    lib.orc_gate_add_ln_modulate_fp8.restype = ctypes.c_int
    lib.orc_gate_add_ln_modulate_fp8.argtypes = [_u16p, _i64, _u16p, _i64, _u8p, _i64, _u16p,
                                                 _i64, _u16p, _i64, _u16p, _u16p, _u16p, _i64,
                                                 _i64, _i64, _i64, ctypes.c_float,
                                                 ctypes.c_float]
    for name in ("orc_tanh_array", "orc_one_plus_array", "orc_rms_rstd_array"):
        getattr(lib, name).argtypes = [_u16p, _u16p, _i64]
    lib.orc_tanh_check_ld.argtypes = [_u16p, _u16p, _f64p, _i64]
    _lib = lib
    return lib


@contextlib.contextmanager
def using_library(path):
    """Temporarily routes every function here to another build of the oracle
    source (used by the tests that plant mistakes in a copy of it)."""
    global _lib
    saved = _lib
    _lib = None
    try:
        load(path)
        yield
    finally:
        _lib = saved


def _p16(a):
    assert a.dtype == np.uint16
    return a.ctypes.data_as(_u16p)


def _p32(a):
    assert a.dtype == np.float32
    return a.ctypes.data_as(_f32p)


def _rows(a):
    """(row_stride, array) of a 2-D uint16 array with unit element stride."""
    assert a.ndim == 2 and a.dtype == np.uint16 and a.strides[1] == 2
    return a.strides[0] // 2, a


# --- scalar and array primitives -------------------------------------------------------

def bf16_round(v):
    """binary32 -> bf16 bits (array or scalar)."""
    lib = load()
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    out = np.empty(a.shape, dtype=np.uint16)
    lib.orc_bf16_round_array(_p32(a), _p16(out), a.size)
    return out


def _p8(a):
    assert a.dtype == np.uint8
    return a.ctypes.data_as(_u8p)


def e4m3(v):
    """binary32 -> OCP E4M3 codes (uint8; round to nearest even, saturating
    at 448, NaN kept)."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    out = np.empty(a.shape, dtype=np.uint8)
    load().orc_e4m3_array(_p32(a), _p8(out), a.size)
    return out


def e4m3_value(codes):
    """E4M3 codes -> their values (float64)."""
    lib = load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.orc_e4m3_value(int(v)) for v in c.ravel()]).reshape(c.shape)


def e4m3_bits_range(first, n):
    out = np.empty(n, dtype=np.uint8)
    load().orc_e4m3_bits_range(ctypes.c_uint32(first), n, _p8(out))
    return out


def bf16_round_bits_range(first, n):
    lib = load()
    out = np.empty(n, dtype=np.uint16)
    lib.orc_bf16_round_bits_range(ctypes.c_uint32(first), n, _p16(out))
    return out


def bf16_value(h):
    """bf16 bits -> exact binary32 values."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def bf16_round_f64(v):
    return load().orc_bf16_round_f64(float(v))


def sum_wave(t):
    t = np.ascontiguousarray(t, dtype=np.float32)
    return np.float32(load().orc_sum_wave(_p32(t), t.size))


def sum_head(t):
    t = np.ascontiguousarray(t, dtype=np.float32)
    return np.float32(load().orc_sum_head(_p32(t), t.size))


def _unary(name, h):
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16))
    out = np.empty(h.shape, dtype=np.uint16)
    getattr(load(), name)(_p16(h), _p16(out), h.size)
    return out


def one_plus(scale_bits):
    return _unary("orc_one_plus_array", scale_bits)


def tanh_bf16(gate_bits):
    return _unary("orc_tanh_array", gate_bits)


def rms_rstd(v_bits):
    return _unary("orc_rms_rstd_array", v_bits)


def tanh_check_ld(gate_bits):
    h = np.ascontiguousarray(np.asarray(gate_bits, dtype=np.uint16))
    out = np.empty(h.shape, dtype=np.uint16)
    margin = np.empty(h.shape, dtype=np.float64)
    load().orc_tanh_check_ld(_p16(h), _p16(out), margin.ctypes.data_as(_f64p), h.size)
    return out, margin


# --- row pieces ------------------------------------------------------------------------

def ln_row(x, eps):
    """LayerNorm of one row: (n bits, (mean, var, rho))."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    n = np.empty_like(x)
    st = np.empty(3, dtype=np.float32)
    load().orc_ln_row(_p16(x), x.size, ctypes.c_float(eps), _p16(n), _p32(st))
    return n, tuple(st)


def rms_row(x, w, eps):
    """Native-bf16 RMSNorm of one row: (y2 bits, (ms, ms+eps, rstd))."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    y2 = np.empty_like(x)
    st = np.empty(3, dtype=np.float32)
    load().orc_rms_row(_p16(x), _p16(w), x.size, ctypes.c_float(eps), _p16(y2), _p32(st))
    return y2, tuple(st)


def qk_head(x, w, c, z, eps):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    c = np.ascontiguousarray(c, dtype=np.float32)
    z = np.ascontiguousarray(z, dtype=np.float32)
    o = np.empty_like(x)
    load().orc_qk_head(_p16(x), _p16(w), _p32(c), _p32(z), x.size, ctypes.c_float(eps), _p16(o))
    return o


# --- whole ops ---------------------------------------------------------------------------

def _check(rc):
    if rc != 0:
        raise ValueError("oracle rejected the problem shape")


def _mod(t, dim):
    t = t.reshape(-1, dim) if t.ndim != 2 else t
    return _rows(t)


def ln_modulate(x, scale, shift, eps=1e-6):
    """x [rows, D]; scale, shift [mod_rows, D] (same row stride) -> out [rows, D]."""
    x_rs, x = _rows(x)
    rows, dim = x.shape
    m_rs, scale = _mod(scale, dim)
    m_rs2, shift = _mod(shift, dim)
    assert m_rs == m_rs2 and scale.shape == shift.shape
    out = np.empty((rows, dim), dtype=np.uint16)
    _check(load().orc_ln_modulate(_p16(out), dim, _p16(x), x_rs, _p16(scale), _p16(shift),
                                  m_rs, scale.shape[0], rows, dim, ctypes.c_float(eps)))
    return out


def modulate_scale_shift(x, scale, shift):
    """x [rows, D]; scale, shift [mod_rows, D] -> bf(bf(x * bf(1 + scale)) + shift)."""
    x_rs, x = _rows(x)
    rows, dim = x.shape
    m_rs, scale = _mod(scale, dim)
    m_rs2, shift = _mod(shift, dim)
    assert m_rs == m_rs2 and scale.shape == shift.shape
    out = np.empty((rows, dim), dtype=np.uint16)
    _check(load().orc_modulate_scale_shift(_p16(out), dim, _p16(x), x_rs, _p16(scale),
                                           _p16(shift), m_rs, scale.shape[0], rows, dim))
    return out


def rmsnorm_scale(x, w, scale, eps=1e-6):
    x_rs, x = _rows(x)
    rows, dim = x.shape
    m_rs, scale = _mod(scale, dim)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    out = np.empty((rows, dim), dtype=np.uint16)
    _check(load().orc_rmsnorm_scale(_p16(out), dim, _p16(x), x_rs, _p16(w), _p16(scale), m_rs,
                                    scale.shape[0], rows, dim, ctypes.c_float(eps)))
    return out


def rmsnorm_tanh_residual(x, residual, w, gate, eps=1e-6):
    x_rs, x = _rows(x)
    r_rs, residual = _rows(residual)
    rows, dim = x.shape
    m_rs, gate = _mod(gate, dim)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    out = np.empty((rows, dim), dtype=np.uint16)
    _check(load().orc_rmsnorm_tanh_residual(_p16(out), dim, _p16(x), x_rs, _p16(residual), r_rs,
                                            _p16(w), _p16(gate), m_rs, gate.shape[0], rows, dim,
                                            ctypes.c_float(eps)))
    return out


def residual_gate_add(residual, y, gate):
    r_rs, residual = _rows(residual)
    y_rs, y = _rows(y)
    rows, dim = residual.shape
    m_rs, gate = _mod(gate, dim)
    out = np.empty((rows, dim), dtype=np.uint16)
    _check(load().orc_residual_gate_add(_p16(out), dim, _p16(residual), r_rs, _p16(y), y_rs,
                                        _p16(gate), m_rs, gate.shape[0], rows, dim))
    return out


def gate_add_ln_modulate(residual, y, gate, scale, shift, eps=1e-6):
    """residual, y [rows, D]; gate, scale, shift [mod_rows, D] (one row stride).
    Returns (r', out): r' = bf(residual + bf(gate * y)) and out = LN + AdaLN
    modulate of r'."""
    r_rs, residual = _rows(residual)
    y_rs, y = _rows(y)
    rows, dim = residual.shape
    m_rs, gate = _mod(gate, dim)
    m_rs2, scale = _mod(scale, dim)
    m_rs3, shift = _mod(shift, dim)
    assert m_rs == m_rs2 == m_rs3 and gate.shape == scale.shape == shift.shape
    out_res = np.empty((rows, dim), dtype=np.uint16)
    out = np.empty((rows, dim), dtype=np.uint16)
    _check(load().orc_gate_add_ln_modulate(_p16(out_res), dim, _p16(out), dim, _p16(residual),
                                           r_rs, _p16(y), y_rs, _p16(gate), _p16(scale),
                                           _p16(shift), m_rs, gate.shape[0], rows, dim,
                                           ctypes.c_float(eps)))
    return out_res, out


def ln_modulate_fp8(x, scale, shift, eps=1e-6, fp8_scale=1.0):
    """(out, out8): LN + AdaLN modulate and E4M3(out / fp8_scale)."""
    x_rs, x = _rows(x)
    rows, dim = x.shape
    m_rs, scale = _mod(scale, dim)
    m_rs2, shift = _mod(shift, dim)
    assert m_rs == m_rs2 and scale.shape == shift.shape
    out = np.empty((rows, dim), dtype=np.uint16)
    out8 = np.empty((rows, dim), dtype=np.uint8)
    _check(load().orc_ln_modulate_fp8(_p16(out), dim, _p8(out8), dim, _p16(x), x_rs, _p16(scale),
                                      _p16(shift), m_rs, scale.shape[0], rows, dim,
                                      ctypes.c_float(eps), ctypes.c_float(fp8_scale)))
    return out, out8


def gate_add_ln_modulate_fp8(residual, y, gate, scale, shift, eps=1e-6, fp8_scale=1.0):
    """(r', out, out8): the gated residual + LN + AdaLN producer and
    E4M3(out / fp8_scale)."""
    r_rs, residual = _rows(residual)
    y_rs, y = _rows(y)
    rows, dim = residual.shape
    m_rs, gate = _mod(gate, dim)
    _, scale = _mod(scale, dim)
    _, shift = _mod(shift, dim)
    out_res = np.empty((rows, dim), dtype=np.uint16)
    out = np.empty((rows, dim), dtype=np.uint16)
    out8 = np.empty((rows, dim), dtype=np.uint8)
    _check(load().orc_gate_add_ln_modulate_fp8(
        _p16(out_res), dim, _p16(out), dim, _p8(out8), dim, _p16(residual), r_rs, _p16(y), y_rs,
        _p16(gate), _p16(scale), _p16(shift), m_rs, gate.shape[0], rows, dim,
        ctypes.c_float(eps), ctypes.c_float(fp8_scale)))
    return out_res, out, out8


def wan_mod_table(table, temb):
    """table: float32 [n_mod, D]; temb: bf16 bits [B, S, n_mod, D].  Returns
    float32 [n_mod, B, S, D] = table[k] + temb[:, :, k] (binary32)."""
    table = np.ascontiguousarray(table, dtype=np.float32)
    temb = np.ascontiguousarray(temb, dtype=np.uint16)
    B, S, K, D = temb.shape
    assert table.shape == (K, D)
    out = np.empty((K, B, S, D), dtype=np.float32)
    _check(load().orc_wan_mod_table(_p32(out), _p32(table), _p16(temb), B, S, K, D))
    return out


def _stream(q, k, v, qw, kw):
    """q, k, v: uint16 views [B, S, H, Dh] sharing strides, head stride Dh."""
    assert q.strides == k.strides == v.strides and q.strides[3] == 2
    B, S, H, Dh = q.shape
    assert q.strides[2] == 2 * Dh
    keep = (q, k, v, qw, kw)
    st = QkvStream(
        q=q.ctypes.data_as(_u16p), k=k.ctypes.data_as(_u16p), v=v.ctypes.data_as(_u16p),
        tok_stride=q.strides[1] // 2, batch_stride=q.strides[0] // 2,
        q_weight=_p16(qw), k_weight=_p16(kw), tokens=S)
    return st, keep


def qk_norm_rope(txt, img, cos_t, sin_t, eps=1e-6):
    """txt, img: dicts with q, k, v ([B, S, H, Dh] uint16 views) and q_weight,
    k_weight ([Dh]).  cos_t, sin_t: float32 [S_txt + S_img, Dh/2].
    Returns contiguous joint (q, k, v), each [B, S_txt + S_img, H, Dh]."""
    B, S_txt, H, Dh = txt["q"].shape
    S_img = img["q"].shape[1]
    S = S_txt + S_img
    outs = [np.empty((B, S, H, Dh), dtype=np.uint16) for _ in range(3)]
    ts, tk = _stream(txt["q"], txt["k"], txt["v"], np.ascontiguousarray(txt["q_weight"]),
                     np.ascontiguousarray(txt["k_weight"]))
    ist, ik = _stream(img["q"], img["k"], img["v"], np.ascontiguousarray(img["q_weight"]),
                      np.ascontiguousarray(img["k_weight"]))
    cos_t = np.ascontiguousarray(cos_t, dtype=np.float32)
    sin_t = np.ascontiguousarray(sin_t, dtype=np.float32)
    assert cos_t.shape == (S, Dh // 2) and sin_t.shape == (S, Dh // 2)
    _check(load().orc_qk_norm_rope(_p16(outs[0]), _p16(outs[1]), _p16(outs[2]), H * Dh,
                                   S * H * Dh, ctypes.byref(ts), ctypes.byref(ist), _p32(cos_t),
                                   _p32(sin_t), B, H, Dh, ctypes.c_float(eps)))
    del tk, ik
    return tuple(outs)


def qk_norm_rope_packed(txt, img, cos_t, sin_t, dests, eps=1e-6):
    """The QKV epilogue written destination-major: returns the packed buffer
    [P, B, S_txt + S_img, 3, H / P, Dh] (P = dests) whose chunk p holds
    heads p H/P .. (p + 1) H/P - 1 of q, k, v."""
    B, S_txt, H, Dh = txt["q"].shape
    S_img = img["q"].shape[1]
    S = S_txt + S_img
    assert H % dests == 0
    hpd = H // dests
    buf = np.empty((dests, B, S, 3, hpd, Dh), dtype=np.uint16)
    ts, tk = _stream(txt["q"], txt["k"], txt["v"], np.ascontiguousarray(txt["q_weight"]),
                     np.ascontiguousarray(txt["k_weight"]))
    ist, ik = _stream(img["q"], img["k"], img["v"], np.ascontiguousarray(img["q_weight"]),
                      np.ascontiguousarray(img["k_weight"]))
    cos_t = np.ascontiguousarray(cos_t, dtype=np.float32)
    sin_t = np.ascontiguousarray(sin_t, dtype=np.float32)
    base = buf.reshape(-1)
    q = base[0:].ctypes.data_as(_u16p)
    k = base[hpd * Dh:].ctypes.data_as(_u16p)
    v = base[2 * hpd * Dh:].ctypes.data_as(_u16p)
    _check(load().orc_qk_norm_rope_dest(q, k, v, 3 * hpd * Dh, S * 3 * hpd * Dh, hpd,
                                        B * S * 3 * hpd * Dh, ctypes.byref(ts),
                                        ctypes.byref(ist), _p32(cos_t), _p32(sin_t), B, H, Dh,
                                        ctypes.c_float(eps)))
    del tk, ik
    return buf
