"""CPU tests of the C ABI: the built library exports every declared entry point,
and the host guards accept, reject and forward arguments as documented.

The guard tests link the real ABI layer (csrc/dit_abi.cpp) with stand-in
launchers (tests/host_stub.cpp) that record the launch instead of running it,
so no GPU is touched.  Pointers are fake, 16-byte aligned addresses.
"""
import ctypes
import os
import re
import subprocess

import pytest

import sanitizers

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "modulation_bf16_row_amd", "csrc")
LIB = os.path.join(ROOT, "modulation_bf16_row_amd", "libdit.so")

OK, UNSUPPORTED, INVALID, HIP = 0, 1, 2, 3
vp, i64, f32, cint = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int


PROBE_LIB = os.path.join(ROOT, "modulation_bf16_row_amd", "libdit_probe.so")
PRODUCT_HEADERS = ("dit.h", "dit_producers.h")
PROBE_HEADERS = ("dit_probe.h", "dit_timing.h")


def declared_functions(headers=None):
    names = set()
    for fn in os.listdir(INCLUDE):
        if fn.endswith(".h") and (headers is None or fn in headers):
            text = open(os.path.join(INCLUDE, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(dit_\w+)\s*\(", text))
    return sorted(names)


def exported(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    return sorted(l.split()[-1] for l in out.splitlines()
                  if l.strip() and not l.split()[-1].startswith("__hip_cuid_"))


def test_product_library_exports_exactly_the_product_headers():
    """libdit.so exports the entry points of dit.h and dit_producers.h and
    nothing else (no probes, no timing hook, no C++ internals)."""
    if not os.path.exists(LIB):
        pytest.skip("libdit.so not built")
    names = declared_functions(PRODUCT_HEADERS)
    assert len(names) >= 14
    assert exported(LIB) == names
    lib = ctypes.CDLL(LIB)
    lib.dit_abi_version.restype = cint
    assert lib.dit_abi_version() == 3


def test_probe_library_exports_every_declared_function():
    if not os.path.exists(PROBE_LIB):
        pytest.skip("libdit_probe.so not built")
    names = declared_functions()
    assert set(declared_functions(PROBE_HEADERS)) <= set(names)
    assert exported(PROBE_LIB) == names


@pytest.fixture(scope="module")
def stub(tmp_path_factory):
    san = sanitizers.sanitized_dir()
    d = tmp_path_factory.mktemp("stub")
    so = os.path.join(san, "libstub.so") if san else str(d / "libdit_hoststub.so")
    cmd = ["/opt/rocm/bin/hipcc", "-std=c++17", "-O1", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", CSRC,
           os.path.join(CSRC, "dit_abi.cpp"), os.path.join(CSRC, "dit_probe_abi.cpp"),
           os.path.join(ROOT, "tests", "host_stub.cpp"), "-o", so]
    if not san:
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
    lib = ctypes.CDLL(so)
    lib.dit_status_reason.restype = ctypes.c_char_p
    lib.dit_ln_modulate.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, f32, cint, vp]
    lib.dit_rmsnorm_scale.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, f32, cint,
                                      vp]
    lib.dit_rmsnorm_tanh_residual.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp, i64, i64, i64,
                                              i64, f32, cint, vp]
    lib.dit_residual_gate_add.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, cint,
                                          vp]
    lib.dit_gate_add_ln_modulate.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, vp, vp, vp, i64,
                                             i64, i64, i64, f32, cint, vp]
    lib.dit_ln_modulate_fp8.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp, i64, i64, i64, i64,
                                        f32, vp, cint, vp]
    lib.dit_gate_add_ln_modulate_fp8.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp,
                                                 vp, vp, i64, i64, i64, i64, f32, vp, cint, vp]
    lib.dit_probe_fp8.argtypes = [cint, vp, vp, i64, vp, vp]
    lib.dit_probe_unary.argtypes = [cint, vp, vp, i64, cint, vp]
    lib.dit_probe_copy.argtypes = [vp, vp, i64, cint, vp]
    lib.dit_wan_modulation_table.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp]
    return lib


class Rec:
    def __init__(self, lib):
        self.lib = lib

    @property
    def calls(self):
        return ctypes.c_int.in_dll(self.lib, "stub_calls").value

    @property
    def name(self):
        return ctypes.c_char_p(ctypes.addressof(ctypes.c_char.in_dll(self.lib, "stub_name"))
                               ).value.decode()

    @property
    def vals(self):
        return list((ctypes.c_int64 * 16).in_dll(self.lib, "stub_vals"))


A = 1 << 20          # fake device addresses, far apart and 16-byte aligned
X, OUT, SC, SH, W, RES, Y, G = (A * k for k in range(1, 9))


def ln(lib, out=OUT, out_rs=1024, x=X, x_rs=1024, sc=SC, sh=SH, mod_rs=1024, mod_rows=1,
       rows=8, dim=1024, mode=0):
    return lib.dit_ln_modulate(out, out_rs, x, x_rs, sc, sh, mod_rs, mod_rows, rows, dim,
                               1e-6, mode, None)


def test_ln_accepts_and_forwards(stub):
    r = Rec(stub)
    n0 = r.calls
    assert ln(stub, rows=12, mod_rows=3, x_rs=1536, out_rs=2048) == OK
    assert r.calls == n0 + 1 and r.name == "ln_modulate"
    assert r.vals[:6] == [12, 1024, 4, 2048, 1536, 1024]     # rows, dim, per_mod, strides
    assert ln(stub, out=X, out_rs=1024) == OK                   # exact in-place


@pytest.mark.parametrize("kw,status,why", [
    (dict(mode=2), INVALID, "mode"),
    (dict(rows=-1), INVALID, "negative"),
    (dict(dim=8200), UNSUPPORTED, "8192"),
    (dict(dim=1020), UNSUPPORTED, "% 8"),
    (dict(dim=0), UNSUPPORTED, "dim == 0"),
    (dict(rows=8, mod_rows=3), UNSUPPORTED, "mod_rows"),
    (dict(mod_rows=0), INVALID, "mod_rows == 0"),
    (dict(x=0), INVALID, "NULL"),
    (dict(sh=0), INVALID, "NULL"),
    (dict(x_rs=1000), UNSUPPORTED, "stride"),
    (dict(x_rs=1028), UNSUPPORTED, "stride"),
    (dict(x=X + 8), UNSUPPORTED, "aligned"),
    (dict(out=X + 2048, out_rs=1024), INVALID, "overlap"),       # out one row below x
    (dict(out=X, out_rs=2048, x_rs=2048 + 8), INVALID, "overlap"),
    (dict(out=SC), INVALID, "overlap"),                          # writes the modulation
])
def test_ln_rejections_touch_nothing(stub, kw, status, why):
    r = Rec(stub)
    n0 = r.calls
    assert ln(stub, **kw) == status
    assert r.calls == n0, "a rejected call must not launch"
    assert why.lower() in stub.dit_status_reason().decode().lower()


def test_empty_problem_is_ok_without_launch(stub):
    r = Rec(stub)
    n0 = r.calls
    assert ln(stub, rows=0, x=0, out=0) == OK
    assert r.calls == n0


def test_interleaved_views_in_one_buffer_are_not_overlap(stub):
    """x = columns [0, 1024) and out = columns [1024, 2048) of one [8, 2048]
    buffer share rows but no element."""
    assert ln(stub, x=X, x_rs=2048, out=X + 2048, out_rs=2048) == OK
    # ... but shifted by 512 columns they do overlap
    assert ln(stub, x=X, x_rs=2048, out=X + 1024, out_rs=2048) == INVALID


def test_other_row_ops(stub):
    r = Rec(stub)
    assert stub.dit_rmsnorm_scale(OUT, 3072, X, 3072, W, SC, 3072, 2, 10, 3072, 1e-6, 1,
                                  None) == OK
    assert r.name == "rmsnorm_scale" and r.vals[:3] == [10, 3072, 5]
    assert stub.dit_rmsnorm_scale(OUT, 3072, X, 3072, OUT, SC, 3072, 2, 10, 3072, 1e-6, 0,
                                  None) == INVALID                # out overwrites weight
    assert stub.dit_rmsnorm_tanh_residual(RES, 3072, X, 3072, RES, 3072, W, G, 3072, 10, 10,
                                          3072, 1e-6, 0, None) == OK   # in place on residual
    assert r.name == "rmsnorm_tanh_residual" and r.vals[2] == 1
    assert stub.dit_residual_gate_add(OUT, 512, RES, 512, Y, 512, G, 512, 1, 4, 512, 5,
                                      None) == INVALID            # bad mode
    assert stub.dit_residual_gate_add(OUT, 512, RES, 512, Y, 512, G, 512, 1, 4, 512, 0,
                                      None) == OK
    assert r.name == "residual_gate_add" and r.vals[:3] == [4, 512, 4]


def gate_ln(lib, out_res=OUT, out_res_rs=512, out=A * 10, out_rs=512, res=RES, res_rs=512, y=Y,
            y_rs=512, g=G, sc=SC, sh=SH, mod_rs=512, mod_rows=2, rows=8, dim=512, mode=0):
    return lib.dit_gate_add_ln_modulate(out_res, out_res_rs, out, out_rs, res, res_rs, y, y_rs, g,
                                        sc, sh, mod_rs, mod_rows, rows, dim, 1e-6, mode, None)


def test_gate_add_ln_accepts_and_forwards(stub):
    r = Rec(stub)
    n0 = r.calls
    assert gate_ln(stub, rows=12, mod_rows=3, res_rs=1024, out_rs=2048, mode=1) == OK
    assert r.calls == n0 + 1 and r.name == "gate_add_ln_modulate"
    assert r.vals[:8] == [12, 512, 4, 512, 2048, 1024, 512, 512]
    assert ctypes.c_int.in_dll(stub, "stub_mode").value == 1
    assert gate_ln(stub, out_res=RES) == OK                     # residual updated in place
    assert gate_ln(stub, out_res=RES, out=Y) == OK              # both outputs in place
    assert gate_ln(stub, rows=0, res=0, out=0) == OK


@pytest.mark.parametrize("kw,status,why", [
    (dict(out=OUT), INVALID, "outputs overlap"),                  # the two outputs coincide
    (dict(out=OUT + 1024, out_rs=512), INVALID, "outputs overlap"),
    (dict(out_res=RES + 16, out_res_rs=512), INVALID, "overlap"),  # partial overlap of residual
    (dict(out=SH), INVALID, "overlap"),                           # writes a modulation tensor
    (dict(out_res=G), INVALID, "overlap"),
    (dict(g=0), INVALID, "NULL"),
    (dict(out_res=0), INVALID, "NULL"),
    (dict(mod_rows=3), UNSUPPORTED, "mod_rows"),
    (dict(dim=8200), UNSUPPORTED, "8192"),
    (dict(y_rs=500), UNSUPPORTED, "stride"),
    (dict(mode=7), INVALID, "mode"),
])
def test_gate_add_ln_rejections_touch_nothing(stub, kw, status, why):
    r = Rec(stub)
    n0 = r.calls
    assert gate_ln(stub, **kw) == status
    assert r.calls == n0, "a rejected call must not launch"
    assert why.lower() in stub.dit_status_reason().decode().lower()


Q8, FS = A * 11, A * 12          # E4M3 output and the fp8 scale


def ln8(lib, q8=Q8, q8_rs=512, fs=FS, out=OUT, x=X, rows=8, dim=512, mode=0):
    return lib.dit_ln_modulate_fp8(out, 512, q8, q8_rs, x, 512, SC, SH, 512, 1, rows, dim, 1e-6,
                                   fs, mode, None)


def test_ln_modulate_fp8_guards(stub):
    r = Rec(stub)
    n0 = r.calls
    assert ln8(stub, q8_rs=1024) == OK
    assert r.calls == n0 + 1 and r.name == "ln_modulate_fp8"
    assert r.vals[6:8] == [1, 1024]
    for kw, status, why in [
            (dict(q8=0), INVALID, "out_fp8 is NULL"),
            (dict(fs=0), INVALID, "fp8_scale is NULL"),
            (dict(q8_rs=500), UNSUPPORTED, "out_fp8 row stride"),
            (dict(q8_rs=516), UNSUPPORTED, "out_fp8 row stride"),
            (dict(q8=Q8 + 4), UNSUPPORTED, "8-byte"),
            (dict(fs=FS + 2), UNSUPPORTED, "4-byte"),
            (dict(q8=X), INVALID, "overlaps"),                 # writes the input
            (dict(q8=OUT + 512), INVALID, "overlaps"),         # inside the bf16 output
            (dict(q8=FS - 1024, q8_rs=512), INVALID, "fp8_scale"),
            (dict(fs=OUT + 64), INVALID, "fp8_scale")]:
        n0 = r.calls
        assert ln8(stub, **kw) == status, kw
        assert r.calls == n0
        assert why.lower() in stub.dit_status_reason().decode().lower(), (kw, why)


def test_gate_add_ln_modulate_fp8_guards(stub):
    r = Rec(stub)
    f = stub.dit_gate_add_ln_modulate_fp8
    assert f(OUT, 512, A * 10, 512, Q8, 512, RES, 512, Y, 512, G, SC, SH, 512, 2, 8, 512, 1e-6, FS,
             1, None) == OK
    assert r.name == "gate_add_ln_modulate_fp8" and r.vals[8:10] == [1, 512]
    assert f(OUT, 512, A * 10, 512, RES, 512, RES, 512, Y, 512, G, SC, SH, 512, 2, 8, 512, 1e-6,
             FS, 0, None) == INVALID                                  # E4M3 over the residual
    assert f(OUT, 512, A * 10, 512, Q8, 512, RES, 512, Y, 512, G, SC, SH, 512, 2, 8, 512, 1e-6,
             OUT, 0, None) == INVALID                                 # scale inside an output


def test_probe_fp8_guards(stub):
    assert stub.dit_probe_fp8(2, Q8, X, 16, None, None) == INVALID
    assert stub.dit_probe_fp8(1, Q8, X, 16, None, None) == INVALID    # quant needs the scale
    assert stub.dit_probe_fp8(0, Q8, X, 16, None, None) == OK
    assert stub.dit_probe_fp8(0, Q8, X, 0, None, None) == OK


def test_probe_unary_guards(stub):
    f = stub.dit_probe_unary
    assert f(1, OUT, X, 16, 0, None) == INVALID     # reserved (no binary32 tanh evaluation)
    assert f(4, OUT, X, 16, 0, None) == INVALID
    assert f(0, OUT, X, 16, 2, None) == INVALID     # mode
    for op in (0, 2, 3):
        assert f(op, OUT, X, 16, 1, None) == OK


def test_probe_copy_guards(stub):
    f = stub.dit_probe_copy
    for flags in range(8):                          # bit 2: the flat layout
        assert f(OUT, X, 1024, flags, None) == OK
    assert f(OUT, X, 1024, 8, None) == INVALID
    assert f(OUT, X, 1024, -1, None) == INVALID
    assert f(OUT, X, 24, 7, None) == UNSUPPORTED     # not a multiple of 16 bytes
    assert f(OUT, OUT + 512, 1024, 7, None) == INVALID   # overlapping buffers
    assert f(OUT, X, 0, 7, None) == OK


def test_wan_modulation_table_guards(stub):
    r = Rec(stub)
    f = stub.dit_wan_modulation_table
    n0 = r.calls
    assert f(OUT, W, X, 1, 100, 6, 512, None) == OK
    assert r.calls == n0 + 1 and r.name == "wan_mod_table" and r.vals[:4] == [1, 100, 6, 512]
    for args, status, why in [
            ((OUT, W, X, 1, 100, 6, 516, None), UNSUPPORTED, "multiple of 8"),
            ((OUT, W, X, -1, 100, 6, 512, None), INVALID, "negative"),
            ((0, W, X, 1, 100, 6, 512, None), INVALID, "NULL"),
            ((OUT + 8, W, X, 1, 100, 6, 512, None), UNSUPPORTED, "aligned"),
            ((X, W, X, 1, 100, 6, 512, None), INVALID, "overlaps"),
            ((W - 4096, W, X, 1, 100, 6, 512, None), INVALID, "overlaps")]:
        n0 = r.calls
        assert f(*args) == status, args
        assert r.calls == n0
        assert why.lower() in stub.dit_status_reason().decode().lower(), (args, why)
    assert f(OUT, W, X, 0, 100, 6, 512, None) == OK                   # empty


class Stream(ctypes.Structure):
    _fields_ = [("q", vp), ("k", vp), ("v", vp), ("tok_stride", i64), ("batch_stride", i64),
                ("q_weight", vp), ("k_weight", vp), ("tokens", i64)]


def _qkv(lib, txt, img, qo, ko, vo, ots, obs, batch=2, heads=24, hd=128, cos=A * 40,
         sin=A * 44, mode=0):
    lib.dit_qk_norm_rope.argtypes = [vp, vp, vp, i64, i64, ctypes.POINTER(Stream),
                                     ctypes.POINTER(Stream), vp, vp, i64, i64, i64, f32, cint, vp]
    return lib.dit_qk_norm_rope(qo, ko, vo, ots, obs, ctypes.byref(txt) if txt else None,
                                ctypes.byref(img) if img else None, cos, sin, batch, heads, hd,
                                1e-6, mode, None)


def _streams():
    H, Dh = 24, 128
    W3 = 3 * H * Dh
    img_base, txt_base = A * 64, A * 256
    img = Stream(img_base, img_base + 2 * H * Dh, img_base + 4 * H * Dh, W3, 4096 * W3,
                 A * 48, A * 49, 4096)
    txt = Stream(txt_base, txt_base + 2 * H * Dh, txt_base + 4 * H * Dh, W3, 512 * W3,
                 A * 50, A * 51, 512)
    return txt, img


def test_qkv_guards(stub):
    r = Rec(stub)
    txt, img = _streams()
    H, Dh, S = 24, 128, 4608
    base = A * 512
    # separate contiguous outputs
    assert _qkv(stub, txt, img, base, base + A * 64, base + A * 128, H * Dh, S * H * Dh) == OK
    assert r.name == "qk_norm_rope" and r.vals[:7] == [2, 24, 4608, 3072, S * 3072, 512, 4096]
    # one interleaved [B, S, 3, H, Dh] buffer
    assert _qkv(stub, txt, img, base, base + 2 * H * Dh, base + 4 * H * Dh, 3 * H * Dh,
                S * 3 * H * Dh) == OK
    # outputs overlapping each other
    assert _qkv(stub, txt, img, base, base + 2 * 1024, base + 4 * H * Dh, 3 * H * Dh,
                S * 3 * H * Dh) == INVALID
    # output over an input stream
    assert _qkv(stub, txt, img, txt.q, base + A * 64, base + A * 128, H * Dh, S * H * Dh) \
        == INVALID
    assert _qkv(stub, txt, img, base, base + A * 64, base + A * 128, H * Dh, S * H * Dh,
                hd=64) == UNSUPPORTED
    assert _qkv(stub, txt, img, base, base + A * 64, base + A * 128, H * Dh, S * H * Dh,
                heads=65) == UNSUPPORTED
    assert _qkv(stub, txt, img, base, base + A * 64, base + A * 128, H * Dh, S * H * Dh,
                mode=7) == INVALID
    # empty problems launch nothing
    n0 = r.calls
    assert _qkv(stub, None, None, 0, 0, 0, 0, 0) == OK
    assert _qkv(stub, txt, img, base, base + A * 64, base + A * 128, H * Dh, S * H * Dh,
                batch=0) == OK
    assert r.calls == n0
    # text-only
    assert _qkv(stub, txt, None, base, base + A * 64, base + A * 128, H * Dh, 512 * H * Dh) == OK
    # misaligned table
    assert _qkv(stub, txt, img, base, base + A * 64, base + A * 128, H * Dh, S * H * Dh,
                cos=A * 40 + 4) == UNSUPPORTED


def test_qkv_rejects_outputs_that_overlap_themselves(stub):
    r = Rec(stub)
    txt, img = _streams()
    H, Dh, S, B = 24, 128, 4608, 2
    base = A * 512
    sep = A * 64
    # batch stride = token stride: batch 1 token 0 would be batch 0 token 1
    n0 = r.calls
    assert _qkv(stub, txt, img, base, base + sep, base + 2 * sep, H * Dh, H * Dh) == UNSUPPORTED
    assert "overlap itself" in stub.dit_status_reason().decode()
    # token stride below a token's width
    assert _qkv(stub, txt, img, base, base + sep, base + 2 * sep, H * Dh - 8, S * H * Dh) \
        == UNSUPPORTED
    assert r.calls == n0
    # token-major [S, B, H, Dh] nests the other way round and is accepted
    assert _qkv(stub, txt, img, base, base + sep, base + 2 * sep, B * H * Dh, H * Dh) == OK
    # one token: the token stride is never used
    one = Stream(txt.q, txt.k, txt.v, txt.tok_stride, txt.batch_stride, txt.q_weight,
                 txt.k_weight, 1)
    assert _qkv(stub, one, None, base, base + sep, base + 2 * sep, 0, H * Dh) == OK


def _qkv_dest(lib, txt, img, qo, ko, vo, ots, obs, hpd, ds, batch=2, heads=24, mode=0):
    lib.dit_qk_norm_rope_dest.argtypes = [vp, vp, vp, i64, i64, i64, i64, ctypes.POINTER(Stream),
                                          ctypes.POINTER(Stream), vp, vp, i64, i64, i64, f32,
                                          cint, vp]
    return lib.dit_qk_norm_rope_dest(qo, ko, vo, ots, obs, hpd, ds,
                                     ctypes.byref(txt) if txt else None,
                                     ctypes.byref(img) if img else None, A * 40, A * 44, batch,
                                     heads, 128, 1e-6, mode, None)


def test_qkv_destination_major_guards(stub):
    r = Rec(stub)
    txt, img = _streams()
    H, Dh, S, B = 24, 128, 4608, 2
    base = A * 512
    for P in (1, 2, 4, 8):
        hpd = H // P
        ts = 3 * hpd * Dh
        bs, ds = S * ts, B * S * ts
        assert _qkv_dest(stub, txt, img, base, base + 2 * hpd * Dh, base + 4 * hpd * Dh, ts, bs,
                         hpd, ds) == OK
        assert r.name == "qk_norm_rope"
        assert r.vals[:5] == [B, H, S, ts, bs]
        assert r.vals[9:11] == [hpd, ds if P > 1 else 0]
    # the plain entry point forwards a single destination
    assert _qkv(stub, txt, img, base, base + A * 64, base + A * 128, H * Dh, S * H * Dh) == OK
    assert r.vals[9:11] == [H, 0]
    hpd, ts = 6, 3 * 6 * Dh
    bs, ds = S * ts, B * S * ts
    n0 = r.calls
    for kw, status, why in [
            (dict(hpd=5), INVALID, "heads_per_dest"),
            (dict(hpd=0), INVALID, "heads_per_dest"),
            (dict(ds=-8), INVALID, "negative destination"),
            (dict(ds=ds + 4), UNSUPPORTED, "% 8"),
            (dict(ds=bs), UNSUPPORTED, "overlap itself"),            # destinations collide
            (dict(ds=ds - 8), INVALID, "overlap each other"),        # q of p+1 over v of p
            (dict(ots=hpd * Dh - 8), UNSUPPORTED, "overlap itself"),
            (dict(ko=base + 2 * (hpd * Dh - 8)), INVALID, "overlap each other"),
            (dict(qo=txt.q), INVALID, "overlaps an input"),
    ]:
        args = dict(qo=base, ko=base + 2 * hpd * Dh, vo=base + 4 * hpd * Dh, ots=ts, obs=bs,
                    hpd=hpd, ds=ds)
        args.update(kw)
        assert _qkv_dest(stub, txt, img, **args) == status, kw
        assert why.lower() in stub.dit_status_reason().decode().lower(), kw
    assert r.calls == n0
    # destinations interleaved per token ([B, S, P, 3, hpd, Dh]) also nest
    assert _qkv_dest(stub, txt, img, base, base + 2 * hpd * Dh, base + 4 * hpd * Dh, 4 * ts,
                     S * 4 * ts, hpd, ts) == OK


def mod(lib, out=OUT, out_rs=512, x=X, x_rs=512, sc=SC, sh=SH, mod_rs=512, mod_rows=2, rows=8,
        dim=512, mode=0):
    lib.dit_modulate_scale_shift.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, cint,
                                             vp]
    return lib.dit_modulate_scale_shift(out, out_rs, x, x_rs, sc, sh, mod_rs, mod_rows, rows, dim,
                                        mode, None)


def test_modulate_scale_shift_guards(stub):
    r = Rec(stub)
    n0 = r.calls
    assert mod(stub, x_rs=1024, out_rs=2048) == OK
    assert r.calls == n0 + 1 and r.name == "modulate_scale_shift"
    assert r.vals[:6] == [8, 512, 4, 2048, 1024, 512]
    assert mod(stub, out=X) == OK                                # in place
    assert mod(stub, mode=1) == OK
    assert mod(stub, rows=0, x=0, out=0) == OK
    n1 = r.calls
    for kw, status, why in [
            (dict(out=X + 16), INVALID, "partially overlaps"),
            (dict(out=SC), INVALID, "modulation"),
            (dict(out=SH + 512), INVALID, "modulation"),
            (dict(sh=0), INVALID, "shift is NULL"),
            (dict(mod_rows=3), UNSUPPORTED, "mod_rows"),
            (dict(dim=508, x_rs=512), UNSUPPORTED, "% 8"),
            (dict(dim=8200, x_rs=8200, out_rs=8200, mod_rs=8200), UNSUPPORTED, "8192"),
            (dict(x_rs=500), UNSUPPORTED, "stride"),
            (dict(x=X + 2), UNSUPPORTED, "aligned"),
            (dict(mode=5), INVALID, "mode"),
    ]:
        assert mod(stub, **kw) == status, kw
        assert why.lower() in stub.dit_status_reason().decode().lower(), kw
    assert r.calls == n1


# ---------------------------------------------------------------------------------------
# Extents beyond the address space: rejected before any other stride arithmetic
# ---------------------------------------------------------------------------------------

BIG_ROWS, BIG_RS = 1 << 32, 1 << 40         # (rows - 1) * rs * 2 is about 2^73 bytes
TOP = (1 << 64) - (1 << 20)                  # 1 MiB below the end of the address space


def _all_row_ops(stub, rows, rs, x=X, out=OUT, res=RES, y=Y, mod_rows=1, dim=512):
    """Calls every row-shaped entry point with row tensors of `rows` rows at
    row stride `rs` (modulation per batch, one row)."""
    q8 = Q8
    calls = {
        "ln_modulate": lambda: stub.dit_ln_modulate(out, rs, x, rs, SC, SH, 512, mod_rows, rows,
                                                    dim, 1e-6, 0, None),
        "rmsnorm_scale": lambda: stub.dit_rmsnorm_scale(out, rs, x, rs, W, SC, 512, mod_rows,
                                                        rows, dim, 1e-6, 0, None),
        "rmsnorm_tanh_residual": lambda: stub.dit_rmsnorm_tanh_residual(
            out, rs, x, rs, res, rs, W, G, 512, mod_rows, rows, dim, 1e-6, 0, None),
        "residual_gate_add": lambda: stub.dit_residual_gate_add(out, rs, res, rs, y, rs, G, 512,
                                                                mod_rows, rows, dim, 0, None),
        "modulate_scale_shift": lambda: mod(stub, out=out, out_rs=rs, x=x, x_rs=rs,
                                            mod_rows=mod_rows, rows=rows, dim=dim),
        "gate_add_ln_modulate": lambda: gate_ln(stub, out_res=out, out_res_rs=rs, out=A * 10,
                                                out_rs=rs, res=res, res_rs=rs, y=y, y_rs=rs,
                                                mod_rows=mod_rows, rows=rows, dim=dim),
        "ln_modulate_fp8": lambda: stub.dit_ln_modulate_fp8(out, rs, q8, rs, x, rs, SC, SH, 512,
                                                            mod_rows, rows, dim, 1e-6, FS, 0,
                                                            None),
        "gate_add_ln_modulate_fp8": lambda: stub.dit_gate_add_ln_modulate_fp8(
            out, rs, A * 10, rs, q8, rs, res, rs, y, rs, G, SC, SH, 512, mod_rows, rows, dim,
            1e-6, FS, 0, None),
    }
    return {k: f() for k, f in calls.items()}


def test_huge_row_extent_rejected_by_every_row_entry_point(stub):
    """rows = 2^32 at row stride 2^40 describes about 2^73 bytes: every row
    entry point refuses it (DIT_ERR_INVALID) and launches nothing."""
    r = Rec(stub)
    n0 = r.calls
    for name, st in _all_row_ops(stub, BIG_ROWS, BIG_RS).items():
        assert st == INVALID, name
        assert "extent" in stub.dit_status_reason().decode(), name
    assert r.calls == n0


def test_row_stride_at_int64_limit_rejected(stub):
    r = Rec(stub)
    n0 = r.calls
    for name, st in _all_row_ops(stub, 2, (1 << 63) - 8).items():
        assert st == INVALID, name
    assert r.calls == n0


def test_single_row_ignores_its_stride(stub):
    """With one row the stride never enters an address: any value is fine."""
    r = Rec(stub)
    n0 = r.calls
    for name, st in _all_row_ops(stub, 1, (1 << 63) - 8).items():
        assert st == OK, name
    assert r.calls == n0 + 8


def test_tensor_running_past_the_address_space_rejected(stub):
    r = Rec(stub)
    n0 = r.calls
    for name, st in _all_row_ops(stub, 8, 1 << 17, x=TOP, res=TOP, y=TOP).items():  # 256 KiB rows
        assert st == INVALID, name
    assert r.calls == n0
    assert ln(stub, x=TOP, x_rs=512, rows=8, dim=512) == OK            # 8 KiB fits


def test_qkv_huge_extents_rejected(stub):
    r = Rec(stub)
    txt, img = _streams()
    H, Dh, S = 24, 128, 4608
    base = A * 512
    n0 = r.calls
    big = Stream(img.q, img.k, img.v, 1 << 40, 1 << 60, img.q_weight, img.k_weight, 1 << 32)
    assert _qkv(stub, txt, big, base, base + A * 64, base + A * 128, H * Dh,
                S * H * Dh) in (INVALID, UNSUPPORTED)
    wide = Stream(img.q, img.k, img.v, 1 << 40, 1 << 60, img.q_weight, img.k_weight, 4096)
    assert _qkv(stub, txt, wide, base, base + A * 64, base + A * 128, H * Dh,
                S * H * Dh) == INVALID
    assert "extent" in stub.dit_status_reason().decode()
    assert _qkv(stub, txt, img, base, base + A * 64, base + A * 128, 1 << 40,
                1 << 60) == INVALID                          # output strides
    huge = Stream(img.q, img.k, img.v, img.tok_stride, img.batch_stride, img.q_weight,
                  img.k_weight, (1 << 63) - 1)               # token counts that overflow
    assert _qkv(stub, huge, huge, base, base + A * 64, base + A * 128, H * Dh,
                S * H * Dh) == UNSUPPORTED
    assert _qkv(stub, txt, img, base, base + A * 64, base + A * 128, H * Dh, S * H * Dh,
                batch=1 << 40) == UNSUPPORTED
    assert _qkv_dest(stub, txt, img, base, base + 2 * 6 * Dh, base + 4 * 6 * Dh, 3 * 6 * Dh,
                     S * 3 * 6 * Dh, 6, 1 << 61) == INVALID   # destination stride
    assert r.calls == n0


def test_wan_table_and_probes_past_the_address_space_rejected(stub):
    r = Rec(stub)
    n0 = r.calls
    assert stub.dit_wan_modulation_table(TOP, A * 2, A * 3, 1, 75600, 6, 5120, None) == INVALID
    assert stub.dit_probe_copy(TOP, A * 2, 1 << 21, 0, None) == INVALID
    assert stub.dit_probe_unary(0, TOP, A * 2, 1 << 20, 0, None) == INVALID
    assert stub.dit_probe_fp8(0, A * 2, TOP, 1 << 20, None, None) == INVALID
    assert r.calls == n0


def test_c_abi_check_program_builds_and_links(tmp_path):
    """The C-ABI check program compiles against include/*.h with the host
    compiler alone and links libdit.so and liboracle.so."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "dit_c_check_build", os.path.join(os.path.dirname(__file__), "c_abi", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    if not (os.path.exists(os.path.join(mod.PKG, "libdit.so"))
            and os.path.exists(os.path.join(mod.ORACLE, "liboracle.so"))):
        pytest.skip("libdit.so / liboracle.so not built")
    out = mod.build(out=str(tmp_path / "dit_c_check"))
    res = subprocess.run(["ldd", out], capture_output=True, text=True)
    assert "libdit.so" in res.stdout and "liboracle.so" in res.stdout
    assert "not found" not in res.stdout
