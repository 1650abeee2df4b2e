"""ctypes binding of libdit.so (argument marshalling only).

Each ``dit_*`` function takes torch tensors on a ROCm device, checks dtype,
device and layout, folds the leading dimensions into flat rows, and calls
the C entry point of the same name on the current torch stream.  Every step
of the computation runs in the HIP kernels; there is no CPU or PyTorch
fallback.  A problem outside the fast path raises ``DitUnsupported`` (the
caller decides what to run instead); bad arguments raise ``DitInvalid``.

The probes of the device primitives and the dispatch-timing hook live in
libdit_probe.so, which links the same kernel objects; ``instrumented()``
routes the epilogue calls made inside it through that library, so that
``dit_time_next_launch`` can time them.
"""
import contextlib
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdit.so")
PROBE_LIB_PATH = os.path.join(_PKG, "libdit_probe.so")

LOSSLESS = 0
FAST = 1
_MODES = {"lossless": LOSSLESS, "fast": FAST, LOSSLESS: LOSSLESS, FAST: FAST}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_int = ctypes.c_int


class DitError(RuntimeError):
    pass


class DitUnsupported(DitError):
    pass


class DitInvalid(DitError):
    pass


class DitHipError(DitError):
    pass


class QkvStream(ctypes.Structure):
    """dit_qkv_stream_t"""
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp), ("tok_stride", _i64),
                ("batch_stride", _i64), ("q_weight", _vp), ("k_weight", _vp), ("tokens", _i64)]


_lib = None
_probe_lib = None
_route_probe = False

# name -> argtypes of every entry point of libdit.so
SIGNATURES = {
    "dit_abi_version": [],
    "dit_status_string": [_int],
    "dit_status_reason": [],
    "dit_ln_modulate": [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _int, _vp],
    "dit_rmsnorm_scale": [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _int,
                          _vp],
    "dit_rmsnorm_tanh_residual": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _i64, _i64,
                                  _i64, _f32, _int, _vp],
    "dit_residual_gate_add": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _int,
                              _vp],
    "dit_gate_add_ln_modulate": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64,
                                 _i64, _i64, _i64, _f32, _int, _vp],
    "dit_ln_modulate_fp8": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64,
                            _f32, _vp, _int, _vp],
    "dit_gate_add_ln_modulate_fp8": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                                     _vp, _vp, _i64, _i64, _i64, _i64, _f32, _vp, _int, _vp],
    "dit_wan_modulation_table": [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp],
    "dit_qk_norm_rope": [_vp, _vp, _vp, _i64, _i64, ctypes.POINTER(QkvStream),
                         ctypes.POINTER(QkvStream), _vp, _vp, _i64, _i64, _i64, _f32, _int, _vp],
    "dit_modulate_scale_shift": [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _int,
                                 _vp],
    "dit_qk_norm_rope_dest": [_vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.POINTER(QkvStream),
                              ctypes.POINTER(QkvStream), _vp, _vp, _i64, _i64, _i64, _f32, _int,
                              _vp],
}

# the additional entry points of libdit_probe.so
PROBE_SIGNATURES = {
    "dit_probe_fp8": [_int, _vp, _vp, _i64, _vp, _vp],
    "dit_probe_bf16_round": [_vp, _vp, _i64, _vp],
    "dit_probe_unary": [_int, _vp, _vp, _i64, _int, _vp],
    "dit_probe_f32": [_int, _vp, _vp, _vp, _i64, _int, _vp],
    "dit_probe_row_sum": [_vp, _vp, _i64, _i64, _int, _vp],
    "dit_time_next_launch": [_vp, _vp],
    "dit_probe_copy": [_vp, _vp, _i64, _int, _vp],
}


def _load(path, signatures):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing; build it with "
                           "`python -m modulation_bf16_row_amd.build`")
    h = ctypes.CDLL(path)
    for name, args in signatures.items():
        fn = getattr(h, name)
        fn.argtypes = args
        fn.restype = _int
    h.dit_status_string.restype = ctypes.c_char_p
    h.dit_status_reason.restype = ctypes.c_char_p
    return h


def lib():
    """The loaded libdit.so.  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH, SIGNATURES)
    return _lib


def probe_lib():
    """The loaded libdit_probe.so (the product's kernels plus the probes and
    the timing hook)."""
    global _probe_lib
    if _probe_lib is None:
        _probe_lib = _load(PROBE_LIB_PATH, {**SIGNATURES, **PROBE_SIGNATURES})
    return _probe_lib


@contextlib.contextmanager
def instrumented():
    """Epilogue calls made (or prepared) inside go through libdit_probe.so:
    the same kernel objects, launched so that a pending dit_time_next_launch
    registration times them."""
    global _route_probe
    prev, _route_probe = _route_probe, True
    try:
        yield
    finally:
        _route_probe = prev


def _epilogue_lib():
    return probe_lib() if _route_probe else lib()


def _check(status, h=None):
    if status == 0:
        return
    reason = (h or lib()).dit_status_reason().decode()
    if status == 1:
        raise DitUnsupported(reason)
    if status == 2:
        raise DitInvalid(reason)
    raise DitHipError(reason)


def _mode(mode):
    try:
        return _MODES[mode]
    except KeyError:
        raise DitInvalid(f"unknown mode {mode!r}") from None


def _stream(t):
    return _vp(torch.cuda.current_stream(t.device).cuda_stream)


def _flat_rows(t, name, byte=False):
    """(rows, row_stride) of a [..., dim] tensor whose outer dimensions fold
    into one uniform row stride (the flat-row-stride rule).  byte: a uint8
    tensor (E4M3 codes) instead of bfloat16."""
    if t.dtype != (torch.uint8 if byte else torch.bfloat16):
        raise DitUnsupported(f"{name} must be {'uint8' if byte else 'bfloat16'}, got {t.dtype}")
    if t.device.type != "cuda":
        raise DitUnsupported(f"{name} must be on a ROCm device, got {t.device}")
    if t.dim() == 0:
        raise DitUnsupported(f"{name} must have a last dimension")
    dim = t.shape[-1]
    if t.dim() == 1:
        return 1, dim
    if t.stride(-1) != 1 and dim > 1:
        raise DitUnsupported(f"{name}: last dimension is not contiguous")
    rs = t.stride(-2)
    expected = rs * t.shape[-2]
    for d in range(t.dim() - 3, -1, -1):
        if t.shape[d] != 1 and t.stride(d) != expected:
            raise DitUnsupported(f"{name}: outer dimensions do not fold into flat rows")
        expected *= t.shape[d]
    rows = t.numel() // dim if dim else 0
    return rows, rs


def _same_device(*ts):
    dev = ts[0].device
    for t in ts[1:]:
        if t.device != dev:
            raise DitUnsupported("all tensors must be on the same device")


def _out_like(x, out):
    if out is None:
        return torch.empty(x.shape, dtype=x.dtype, device=x.device)
    if out.shape != x.shape:
        raise DitInvalid(f"out has shape {tuple(out.shape)}, expected {tuple(x.shape)}")
    return out


def _mod_rows(a, b, dim, names):
    ra, sa = _flat_rows(a, names[0])
    if a.shape[-1] != dim:
        raise DitInvalid(f"{names[0]} last dimension {a.shape[-1]} != {dim}")
    if b is not None:
        rb, sb = _flat_rows(b, names[1])
        if b.shape[-1] != dim or rb != ra:
            raise DitInvalid(f"{names[1]} shape does not match {names[0]}")
        if sb != sa and ra > 1:
            raise DitUnsupported(f"{names[0]} and {names[1]} must share one row stride")
    return ra, sa


class PreparedCall:
    """A fully marshalled epilogue call: checks and argument conversion were
    done once, on the stream that was current then; calling it only enqueues
    the kernel (one C call).  Returns the output tensor(s)."""
    __slots__ = ("_fn", "_args", "_result", "_lib")

    def __init__(self, fn, args, result, h):
        self._fn, self._args, self._result, self._lib = fn, args, result, h

    def __call__(self):
        status = self._fn(*self._args)
        if status:
            _check(status, self._lib)
        return self._result


def _call(name, result, prepare, *args):
    h = _epilogue_lib()
    fn = getattr(h, name)
    if prepare:
        conv = tuple(t(a) if not isinstance(a, (ctypes._SimpleCData, ctypes.Structure,
                                                 ctypes._Pointer)) and t is not None else a
                     for a, t in zip(args, SIGNATURES[name]))
        return PreparedCall(fn, conv, result, h)
    _check(fn(*args), h)
    return result


def dit_ln_modulate(x, scale, shift, eps=1e-6, mode="lossless", out=None, prepare=False):
    """LN(x) * (1 + scale) + shift with the lossless rounding contract.
    With prepare=True, returns a PreparedCall instead of launching."""
    _same_device(x, scale, shift)
    rows, x_rs = _flat_rows(x, "x")
    dim = x.shape[-1]
    mrows, mrs = _mod_rows(scale, shift, dim, ("scale", "shift"))
    out = _out_like(x, out)
    _same_device(x, out)
    _, o_rs = _flat_rows(out, "out")
    return _call("dit_ln_modulate", out, prepare, out.data_ptr(), o_rs, x.data_ptr(), x_rs,
                 scale.data_ptr(), shift.data_ptr(), mrs, mrows, rows, dim, eps, _mode(mode),
                 _stream(x))


def dit_rmsnorm_scale(x, weight, scale, eps=1e-6, mode="lossless", out=None, prepare=False):
    _same_device(x, weight, scale)
    rows, x_rs = _flat_rows(x, "x")
    dim = x.shape[-1]
    if weight.dtype != torch.bfloat16 or weight.numel() != dim or not weight.is_contiguous():
        raise DitUnsupported("weight must be a contiguous bfloat16 tensor of dim elements")
    mrows, mrs = _mod_rows(scale, None, dim, ("scale",))
    out = _out_like(x, out)
    _same_device(x, out)
    _, o_rs = _flat_rows(out, "out")
    return _call("dit_rmsnorm_scale", out, prepare, out.data_ptr(), o_rs, x.data_ptr(), x_rs,
                 weight.data_ptr(), scale.data_ptr(), mrs, mrows, rows, dim, eps, _mode(mode),
                 _stream(x))


def dit_rmsnorm_tanh_residual(x, residual, weight, gate, eps=1e-6, mode="lossless", out=None,
                              prepare=False):
    _same_device(x, residual, weight, gate)
    rows, x_rs = _flat_rows(x, "x")
    dim = x.shape[-1]
    rrows, r_rs = _flat_rows(residual, "residual")
    if residual.shape != x.shape:
        raise DitInvalid("residual must have the shape of x")
    if weight.dtype != torch.bfloat16 or weight.numel() != dim or not weight.is_contiguous():
        raise DitUnsupported("weight must be a contiguous bfloat16 tensor of dim elements")
    mrows, mrs = _mod_rows(gate, None, dim, ("gate",))
    out = _out_like(x, out)
    _same_device(x, out)
    _, o_rs = _flat_rows(out, "out")
    return _call("dit_rmsnorm_tanh_residual", out, prepare, out.data_ptr(), o_rs, x.data_ptr(),
                 x_rs, residual.data_ptr(), r_rs, weight.data_ptr(), gate.data_ptr(), mrs, mrows,
                 rows, dim, eps, _mode(mode), _stream(x))


def dit_residual_gate_add(residual, y, gate, mode="lossless", out=None, prepare=False):
    _same_device(residual, y, gate)
    rows, r_rs = _flat_rows(residual, "residual")
    dim = residual.shape[-1]
    if y.shape != residual.shape:
        raise DitInvalid("y must have the shape of residual")
    _, y_rs = _flat_rows(y, "y")
    mrows, mrs = _mod_rows(gate, None, dim, ("gate",))
    out = _out_like(residual, out)
    _same_device(residual, out)
    _, o_rs = _flat_rows(out, "out")
    return _call("dit_residual_gate_add", out, prepare, out.data_ptr(), o_rs, residual.data_ptr(),
                 r_rs, y.data_ptr(), y_rs, gate.data_ptr(), mrs, mrows, rows, dim, _mode(mode),
                 _stream(residual))


def dit_modulate_scale_shift(x, scale, shift, mode="lossless", out=None, prepare=False):
    """bf(bf(x * bf(1 + scale)) + shift) with modulation row r // (rows // mod_rows)."""
    _same_device(x, scale, shift)
    rows, x_rs = _flat_rows(x, "x")
    dim = x.shape[-1]
    mrows, mrs = _mod_rows(scale, shift, dim, ("scale", "shift"))
    out = _out_like(x, out)
    _same_device(x, out)
    _, o_rs = _flat_rows(out, "out")
    return _call("dit_modulate_scale_shift", out, prepare, out.data_ptr(), o_rs, x.data_ptr(),
                 x_rs, scale.data_ptr(), shift.data_ptr(), mrs, mrows, rows, dim, _mode(mode),
                 _stream(x))


def dit_gate_add_ln_modulate(residual, y, gate, scale, shift, eps=1e-6, mode="lossless",
                             out_residual=None, out=None, prepare=False):
    """r' = bf(residual + bf(gate * y)) and LN(r') * (1 + scale) + shift in one
    pass.  Returns (r', out); either output may be given (and may be residual
    or y itself)."""
    _same_device(residual, y, gate, scale, shift)
    rows, r_rs = _flat_rows(residual, "residual")
    dim = residual.shape[-1]
    if y.shape != residual.shape:
        raise DitInvalid("y must have the shape of residual")
    _, y_rs = _flat_rows(y, "y")
    mrows, mrs = _mod_rows(gate, scale, dim, ("gate", "scale"))
    _mod_rows(gate, shift, dim, ("gate", "shift"))
    out_residual = _out_like(residual, out_residual)
    out = _out_like(residual, out)
    _same_device(residual, out_residual, out)
    _, rr_rs = _flat_rows(out_residual, "out_residual")
    _, o_rs = _flat_rows(out, "out")
    return _call("dit_gate_add_ln_modulate", (out_residual, out), prepare,
                 out_residual.data_ptr(), rr_rs, out.data_ptr(), o_rs, residual.data_ptr(), r_rs,
                 y.data_ptr(), y_rs, gate.data_ptr(), scale.data_ptr(), shift.data_ptr(), mrs,
                 mrows, rows, dim, eps, _mode(mode), _stream(residual))


def _fp8_out(x, out_fp8):
    """The E4M3 output (float8_e4m3fn or uint8, shaped like x) and its row
    stride in bytes."""
    if out_fp8 is None:
        out_fp8 = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    if out_fp8.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise DitUnsupported("out_fp8 must be float8_e4m3fn or uint8")
    if out_fp8.shape != x.shape:
        raise DitInvalid(f"out_fp8 has shape {tuple(out_fp8.shape)}, expected {tuple(x.shape)}")
    if out_fp8.device != x.device:
        raise DitInvalid("out_fp8 is on another device")
    _, rs = _flat_rows(out_fp8.view(torch.uint8), "out_fp8", byte=True)
    return out_fp8, rs


def _fp8_scale(t, like):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.numel() != 1:
        raise DitUnsupported("fp8_scale must be a one-element float32 tensor")
    if t.device != like.device:
        raise DitInvalid("fp8_scale is on another device")
    return t


def dit_ln_modulate_fp8(x, scale, shift, fp8_scale, eps=1e-6, mode="lossless", out=None,
                        out_fp8=None, prepare=False):
    """LN(x) * (1 + scale) + shift in BF16 and its E4M3 copy E4M3(out / fp8_scale).
    fp8_scale: one-element float32 device tensor.  Returns (out, out_fp8)."""
    _same_device(x, scale, shift)
    rows, x_rs = _flat_rows(x, "x")
    dim = x.shape[-1]
    mrows, mrs = _mod_rows(scale, shift, dim, ("scale", "shift"))
    out = _out_like(x, out)
    _same_device(x, out)
    _, o_rs = _flat_rows(out, "out")
    out_fp8, q_rs = _fp8_out(x, out_fp8)
    fs = _fp8_scale(fp8_scale, x)
    return _call("dit_ln_modulate_fp8", (out, out_fp8), prepare, out.data_ptr(), o_rs,
                 out_fp8.data_ptr(), q_rs, x.data_ptr(), x_rs, scale.data_ptr(),
                 shift.data_ptr(), mrs, mrows, rows, dim, eps, fs.data_ptr(), _mode(mode),
                 _stream(x))


def dit_gate_add_ln_modulate_fp8(residual, y, gate, scale, shift, fp8_scale, eps=1e-6,
                                 mode="lossless", out_residual=None, out=None, out_fp8=None,
                                 prepare=False):
    """The gated residual + LN + AdaLN producer with an E4M3 copy of its LN
    output.  Returns (r', out, out_fp8)."""
    _same_device(residual, y, gate, scale, shift)
    rows, r_rs = _flat_rows(residual, "residual")
    dim = residual.shape[-1]
    if y.shape != residual.shape:
        raise DitInvalid("y must have the shape of residual")
    _, y_rs = _flat_rows(y, "y")
    mrows, mrs = _mod_rows(gate, scale, dim, ("gate", "scale"))
    _mod_rows(gate, shift, dim, ("gate", "shift"))
    out_residual = _out_like(residual, out_residual)
    out = _out_like(residual, out)
    _same_device(residual, out_residual, out)
    _, rr_rs = _flat_rows(out_residual, "out_residual")
    _, o_rs = _flat_rows(out, "out")
    out_fp8, q_rs = _fp8_out(residual, out_fp8)
    fs = _fp8_scale(fp8_scale, residual)
    return _call("dit_gate_add_ln_modulate_fp8", (out_residual, out, out_fp8), prepare,
                 out_residual.data_ptr(), rr_rs, out.data_ptr(), o_rs, out_fp8.data_ptr(), q_rs,
                 residual.data_ptr(), r_rs, y.data_ptr(), y_rs, gate.data_ptr(),
                 scale.data_ptr(), shift.data_ptr(), mrs, mrows, rows, dim, eps, fs.data_ptr(),
                 _mode(mode), _stream(residual))


def dit_wan_modulation_table(table, temb, out=None, prepare=False):
    """table: float32 [n_mod, D] (contiguous); temb: bfloat16 [B, S, n_mod, D]
    (contiguous).  Returns float32 [n_mod, B, S, D] = table[k] + temb[:, :, k]."""
    if table.dtype != torch.float32 or table.dim() != 2 or not table.is_contiguous():
        raise DitUnsupported("table must be a contiguous float32 [n_mod, D] tensor")
    if temb.dtype != torch.bfloat16 or temb.dim() != 4 or not temb.is_contiguous():
        raise DitUnsupported("temb must be a contiguous bfloat16 [B, S, n_mod, D] tensor")
    B, S, K, D = temb.shape
    if tuple(table.shape) != (K, D):
        raise DitInvalid(f"table shape {tuple(table.shape)} does not match temb {tuple(temb.shape)}")
    _same_device(table, temb)
    if out is None:
        out = torch.empty((K, B, S, D), dtype=torch.float32, device=temb.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (K, B, S, D) or not out.is_contiguous():
        raise DitInvalid("out must be a contiguous float32 [n_mod, B, S, D] tensor")
    _same_device(temb, out)
    return _call("dit_wan_modulation_table", out, prepare, out.data_ptr(), table.data_ptr(),
                 temb.data_ptr(), B, S, K, D, _stream(temb))


def _qkv_stream(st):
    """st: dict with q, k, v ([B, S, H, Dh] views sharing strides) and q_weight,
    k_weight ([Dh]); None means no tokens."""
    if st is None:
        return QkvStream(), (0, 0, 0, 0)
    q, k, v = st["q"], st["k"], st["v"]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise DitUnsupported(f"{n} must be a bfloat16 [B, S, H, Dh] view")
        if t.stride(3) != 1 or t.stride(2) != t.shape[3]:
            raise DitUnsupported(f"{n}: heads must be packed (head stride Dh, element stride 1)")
    if not (q.stride() == k.stride() == v.stride() and q.shape == k.shape == v.shape):
        raise DitUnsupported("q, k, v of one stream must share shape and strides")
    for w, n in ((st["q_weight"], "q_weight"), (st["k_weight"], "k_weight")):
        if w.dtype != torch.bfloat16 or not w.is_contiguous() or w.numel() != q.shape[3]:
            raise DitUnsupported(f"{n} must be a contiguous bfloat16 [Dh] tensor")
    s = QkvStream(q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), tok_stride=q.stride(1),
                  batch_stride=q.stride(0), q_weight=st["q_weight"].data_ptr(),
                  k_weight=st["k_weight"].data_ptr(), tokens=q.shape[1])
    return s, tuple(q.shape)


def dit_qk_norm_rope(txt, img, cos, sin, eps=1e-6, mode="lossless", out=None, prepare=False):
    """Q/K RMSNorm + interleaved RoPE + V copy into joint [B, S_txt + S_img, H, Dh]
    outputs (text tokens first).  ``out`` may be a (q, k, v) triple of views
    sharing token and batch strides.  With prepare=True, returns a
    PreparedCall instead of launching."""
    ts, tshape = _qkv_stream(txt)
    is_, ishape = _qkv_stream(img)
    ref = img["q"] if img is not None else txt["q"]
    B, _, H, Dh = ref.shape
    s_total = ts.tokens + is_.tokens
    if cos.dtype != torch.float32 or sin.dtype != torch.float32 or not cos.is_contiguous() \
            or not sin.is_contiguous():
        raise DitUnsupported("cos and sin must be contiguous float32 tensors")
    if cos.shape != (s_total, Dh // 2) or sin.shape != (s_total, Dh // 2):
        raise DitInvalid(f"cos/sin must be [{s_total}, {Dh // 2}]")
    for sh in (tshape, ishape):
        if sh[0] and (sh[0] != B or sh[2] != H or sh[3] != Dh):
            raise DitInvalid("text and image streams must agree on batch, heads and head_dim")
    if out is None:
        out = tuple(torch.empty((B, s_total, H, Dh), dtype=torch.bfloat16, device=ref.device)
                    for _ in range(3))
    qo, ko, vo = out
    for t in out:
        if t.shape != (B, s_total, H, Dh) or t.dtype != torch.bfloat16:
            raise DitInvalid("outputs must be bfloat16 [B, S_txt + S_img, H, Dh]")
        if t.stride(3) != 1 or t.stride(2) != Dh or t.stride() != qo.stride():
            raise DitUnsupported("outputs must share strides with packed heads")
    return _call("dit_qk_norm_rope", out, prepare, qo.data_ptr(), ko.data_ptr(), vo.data_ptr(),
                 qo.stride(1), qo.stride(0), ctypes.pointer(ts), ctypes.pointer(is_),
                 cos.data_ptr(), sin.data_ptr(), B, H, Dh, eps, _mode(mode), _stream(ref))


def dit_qk_norm_rope_packed(txt, img, cos, sin, dests, eps=1e-6, mode="lossless", out=None,
                            prepare=False):
    """The QKV epilogue written destination-major for Ulysses: returns the
    contiguous bfloat16 buffer [P, B, S_txt + S_img, 3, H / P, Dh] (P = dests)
    whose chunk p holds heads p H/P .. (p + 1) H/P - 1 of q, k and v, ready for
    one all-to-all.  ``out`` may be such a buffer."""
    ts, tshape = _qkv_stream(txt)
    is_, ishape = _qkv_stream(img)
    ref = img["q"] if img is not None else txt["q"]
    B, _, H, Dh = ref.shape
    s_total = ts.tokens + is_.tokens
    if dests <= 0 or H % dests:
        raise DitInvalid(f"dests={dests} must divide heads={H}")
    if cos.dtype != torch.float32 or sin.dtype != torch.float32 or not cos.is_contiguous() \
            or not sin.is_contiguous():
        raise DitUnsupported("cos and sin must be contiguous float32 tensors")
    if cos.shape != (s_total, Dh // 2) or sin.shape != (s_total, Dh // 2):
        raise DitInvalid(f"cos/sin must be [{s_total}, {Dh // 2}]")
    for sh in (tshape, ishape):
        if sh[0] and (sh[0] != B or sh[2] != H or sh[3] != Dh):
            raise DitInvalid("text and image streams must agree on batch, heads and head_dim")
    hpd = H // dests
    shape = (dests, B, s_total, 3, hpd, Dh)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=ref.device)
    if tuple(out.shape) != shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise DitInvalid(f"out must be a contiguous bfloat16 {list(shape)} buffer")
    base, esz = out.data_ptr(), out.element_size()
    ts_out = 3 * hpd * Dh
    return _call("dit_qk_norm_rope_dest", out, prepare, base, base + hpd * Dh * esz,
                 base + 2 * hpd * Dh * esz, ts_out, s_total * ts_out, hpd,
                 B * s_total * ts_out, ctypes.pointer(ts), ctypes.pointer(is_), cos.data_ptr(),
                 sin.data_ptr(), B, H, Dh, eps, _mode(mode), _stream(ref))


def dit_time_next_launch(start, stop):
    """Makes the next call on this thread into libdit_probe.so (an epilogue
    inside ``instrumented()``, or a probe) record `start` / `stop`
    (torch.cuda.Event objects that have been recorded once, so that they
    exist) around its kernel, from within the dispatch."""
    h = probe_lib()
    _check(h.dit_time_next_launch(_vp(start.cuda_event), _vp(stop.cuda_event)), h)


# --- probes of the device primitives (libdit_probe.so) ---------------------------------

def _pcheck(status):
    _check(status, probe_lib())


def dit_probe_bf16_round(x_f32, out=None):
    if out is None:
        out = torch.empty(x_f32.shape, dtype=torch.int16, device=x_f32.device)
    _pcheck(probe_lib().dit_probe_bf16_round(out.data_ptr(), x_f32.data_ptr(), x_f32.numel(),
                                             _stream(x_f32)))
    return out


def dit_probe_unary(op, h_i16, mode="lossless"):
    out = torch.empty_like(h_i16)
    _pcheck(probe_lib().dit_probe_unary(op, out.data_ptr(), h_i16.data_ptr(), h_i16.numel(),
                                        _mode(mode), _stream(h_i16)))
    return out


def dit_probe_f32(op, a, b=None, mode="lossless"):
    out = torch.empty_like(a)
    _pcheck(probe_lib().dit_probe_f32(op, out.data_ptr(), a.data_ptr(),
                                      b.data_ptr() if b is not None else None, a.numel(), _mode(mode),
                                      _stream(a)))
    return out


def dit_probe_copy(dst, src, flags=0):
    """Streaming device copy of src into dst (same number of bytes)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise DitInvalid("dst and src sizes differ")
    _pcheck(probe_lib().dit_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, flags, _stream(src)))
    return dst


def dit_probe_fp8(op, inp, scale=None):
    """op 0: E4M3 codes of a float32 tensor; op 1: E4M3 codes of a bfloat16
    tensor divided by scale (one-element float32 tensor).  Returns uint8."""
    out = torch.empty(inp.shape, dtype=torch.uint8, device=inp.device)
    _pcheck(probe_lib().dit_probe_fp8(op, out.data_ptr(), inp.data_ptr(), inp.numel(),
                                      scale.data_ptr() if scale is not None else None, _stream(inp)))
    return out


def dit_probe_row_sum(t, head=False):
    """t: float32 [rows, dim] contiguous -> float32 [rows] (head: [groups])."""
    rows, dim = t.shape
    out = torch.empty(rows, dtype=torch.float32, device=t.device)
    _pcheck(probe_lib().dit_probe_row_sum(out.data_ptr(), t.data_ptr(), rows, dim, int(head),
                                          _stream(t)))
    return out
