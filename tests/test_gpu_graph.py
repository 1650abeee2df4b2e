"""Prepared calls and HIP-graph replays of the epilogues give the same bits as
eager calls (and the oracle).

The graph test replays a captured step -- the five epilogues, the fused
producers (with their E4M3 copies), the standalone modulate, the
destination-major QKV epilogue and the Wan modulation table, and the row
epilogues again with per-token modulation (the split-row layout, and
tanh-residual's per-token row layout) -- several
times, with eager work and synchronisations in between (inputs and the
E4M3 scale are rewritten in place before each replay, so a replay must read
the new values), and checks every replay against eager results.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bits_equal, dev, host, say
from modulation_bf16_row_amd import synth

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import modulation_bf16_row_amd as m
    assert torch.cuda.is_available()
    m.lib()


def m():
    import modulation_bf16_row_amd as mod
    return mod


def _views(a, H, Dh=128):
    return [a[:, :, i * H * Dh:(i + 1) * H * Dh].view(a.shape[0], a.shape[1], H, Dh)
            for i in range(3)]


class Step:
    """Buffers and calls of one small five-epilogue step."""

    def __init__(self, seed):
        rows, D, B = 512, 1024, 2
        w = synth.qwen_image_block(seed_base=seed, batch=B, tokens=rows // B, dim=D)
        self.h = w
        self.x, self.res = dev(w["x"]), dev(w["residual"])
        self.sc, self.sh, self.g = dev(w["scale"]), dev(w["shift"]), dev(w["gate"])
        self.s2, self.w = dev(w["scale2"]), dev(w["weight"])
        self.out = {k: torch.empty_like(self.x) for k in ("ln", "rms", "tanh", "gate")}
        q = synth.qwen_image_qkv(seed_base=seed + 7, s_img=64, s_txt=8, grid=(8, 8), heads=4)
        self.qh = q
        H = q["heads"]
        self.tq = _views(dev(q["txt_qkv"]), H)
        self.iq = _views(dev(q["img_qkv"]), H)
        self._keep = (self.tq, self.iq)
        self.txt = dict(q=self.tq[0], k=self.tq[1], v=self.tq[2],
                        q_weight=dev(q["txt_q_weight"]), k_weight=dev(q["txt_k_weight"]))
        self.img = dict(q=self.iq[0], k=self.iq[1], v=self.iq[2],
                        q_weight=dev(q["img_q_weight"]), k_weight=dev(q["img_k_weight"]))
        self.cos = torch.from_numpy(q["cos"]).cuda()
        self.sin = torch.from_numpy(q["sin"]).cuda()
        S = q["cos"].shape[0]
        self.qkv_out = tuple(torch.empty((2, S, H, 128), dtype=torch.bfloat16, device="cuda")
                             for _ in range(3))
        # fused producers, standalone modulate, destination-major QKV, modulation table
        self.y = dev(synth.normal_bf16(tuple(self.x.shape), 1.0, seed + 11))
        self.fs = torch.tensor([0.05], dtype=torch.float32, device="cuda")
        for k in ("rp", "gln", "ln8b", "grp8", "gln8", "mod"):
            self.out[k] = torch.empty_like(self.x)
        self.q8 = {k: torch.empty(tuple(self.x.shape), dtype=torch.uint8, device="cuda")
                   for k in ("ln8", "gln8")}
        self.packed = torch.empty((2, 2, S, 3, H // 2, 128), dtype=torch.bfloat16, device="cuda")
        g = torch.Generator(device="cuda").manual_seed(seed + 13)
        self.table = torch.randn((6, 256), device="cuda", generator=g) * 0.05
        self.temb = (torch.randn((2, 40, 6, 256), device="cuda", generator=g) * 0.3).to(
            torch.bfloat16)
        self.mt = torch.empty((6, 2, 40, 256), dtype=torch.float32, device="cuda")
        # per-token modulation rows (the split-row layout)
        self.sct = dev(synth.normal_bf16(tuple(self.x.shape), 0.1, seed + 21))
        self.sht = dev(synth.normal_bf16(tuple(self.x.shape), 0.1, seed + 22))
        self.gt = dev(synth.normal_bf16(tuple(self.x.shape), 0.1, seed + 23))
        for k in ("lnpt", "rmspt", "tanhpt", "rppt", "glnpt"):
            self.out[k] = torch.empty_like(self.x)

    def run(self, prepare=False):
        M = m()
        calls = [
            M.dit_ln_modulate(self.x, self.sc, self.sh, EPS, out=self.out["ln"], prepare=prepare),
            M.dit_rmsnorm_scale(self.x, self.w, self.s2, EPS, out=self.out["rms"],
                                prepare=prepare),
            M.dit_rmsnorm_tanh_residual(self.x, self.res, self.w, self.g, EPS,
                                        out=self.out["tanh"], prepare=prepare),
            M.dit_residual_gate_add(self.res, self.x, self.g, out=self.out["gate"],
                                    prepare=prepare),
            M.dit_qk_norm_rope(self.txt, self.img, self.cos, self.sin, EPS, out=self.qkv_out,
                               prepare=prepare),
            M.dit_gate_add_ln_modulate(self.res, self.y, self.g, self.sc, self.sh, EPS,
                                       out_residual=self.out["rp"], out=self.out["gln"],
                                       prepare=prepare),
            M.dit_ln_modulate_fp8(self.x, self.sc, self.sh, self.fs, EPS, out=self.out["ln8b"],
                                  out_fp8=self.q8["ln8"], prepare=prepare),
            M.dit_gate_add_ln_modulate_fp8(self.res, self.y, self.g, self.sc, self.sh, self.fs,
                                           EPS, out_residual=self.out["grp8"],
                                           out=self.out["gln8"], out_fp8=self.q8["gln8"],
                                           prepare=prepare),
            M.dit_modulate_scale_shift(self.x, self.sc, self.sh, out=self.out["mod"],
                                       prepare=prepare),
            M.dit_qk_norm_rope_packed(self.txt, self.img, self.cos, self.sin, 2, EPS,
                                      out=self.packed, prepare=prepare),
            M.dit_wan_modulation_table(self.table, self.temb, out=self.mt, prepare=prepare),
            M.dit_ln_modulate(self.x, self.sct, self.sht, EPS, out=self.out["lnpt"],
                              prepare=prepare),
            M.dit_rmsnorm_scale(self.x, self.w, self.sct, EPS, out=self.out["rmspt"],
                                prepare=prepare),
            M.dit_rmsnorm_tanh_residual(self.x, self.res, self.w, self.gt, EPS,
                                        out=self.out["tanhpt"], prepare=prepare),
            M.dit_gate_add_ln_modulate(self.res, self.y, self.gt, self.sct, self.sht, EPS,
                                       out_residual=self.out["rppt"], out=self.out["glnpt"],
                                       prepare=prepare),
        ]
        return calls

    def snapshot(self):
        torch.cuda.synchronize()
        return [host(self.out[k]) for k in ("ln", "rms", "tanh", "gate")] + \
            [host(t) for t in self.qkv_out] + \
            [host(self.out[k]) for k in ("rp", "gln", "ln8b", "grp8", "gln8", "mod")] + \
            [self.q8[k].cpu().numpy() for k in ("ln8", "gln8")] + \
            [host(self.packed), self.mt.cpu().numpy().view(np.uint32)] + \
            [host(self.out[k]) for k in ("lnpt", "rmspt", "tanhpt", "rppt", "glnpt")]

    def clear(self):
        for t in list(self.out.values()) + list(self.qkv_out) + list(self.q8.values()) + \
                [self.packed, self.mt]:
            t.zero_()


def test_prepared_calls_match_direct_calls():
    s = Step(6000)
    say("direct calls")
    s.run()
    ref = s.snapshot()
    s.clear()
    say("prepared calls")
    plans = s.run(prepare=True)
    for p in plans:
        p()
    got = s.snapshot()
    for i, (a, b) in enumerate(zip(got, ref)):
        assert_bits_equal(a, b, f"output {i}")
    # and the LN output against the oracle
    w = s.h
    assert_bits_equal(got[0], oracle.ln_modulate(w["x"], w["scale"], w["shift"], EPS), "ln")


def test_graph_replays_match_eager():
    s = Step(6100)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("capture")
    with torch.cuda.graph(g):
        s.run()
    for rep in range(4):
        # eager work between replays: new inputs, written by the default stream
        xn = synth.normal_bf16(tuple(s.x.shape), 1.0, 100 + rep)
        s.x.copy_(dev(xn))
        s.iq[0].copy_(dev(synth.normal_bf16(tuple(s.iq[0].shape), 1.0, 200 + rep)))
        s.fs.fill_(0.05 * (rep + 1))                   # a new static E4M3 scale
        s.temb.normal_(0.0, 0.3)
        torch.cuda.synchronize()
        s.clear()
        say(f"replay {rep}")
        g.replay()
        got = s.snapshot()
        s.clear()
        s.run()
        ref = s.snapshot()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert_bits_equal(a, b, f"replay {rep} output {i}")
        w = s.h
        assert_bits_equal(got[0], oracle.ln_modulate(xn, w["scale"], w["shift"], EPS),
                          f"replay {rep} ln vs oracle")
        ref8 = oracle.ln_modulate_fp8(xn, w["scale"], w["shift"], EPS, 0.05 * (rep + 1))
        assert np.array_equal(got[13], ref8[1]), f"replay {rep} E4M3 copy vs oracle"
        assert_bits_equal(got[17], oracle.ln_modulate(xn, host(s.sct), host(s.sht), EPS),
                          f"replay {rep} per-token ln vs oracle")
