"""Prepared calls and HIP-graph replays of the epilogues give the same bits as
eager calls (and the oracle).

The graph test replays a captured five-epilogue step several times, with
eager work and synchronisations in between (the inputs are rewritten
eagerly before each replay), and checks every replay against eager results.
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
        ]
        return calls

    def snapshot(self):
        torch.cuda.synchronize()
        return [host(self.out[k]) for k in ("ln", "rms", "tanh", "gate")] + \
            [host(t) for t in self.qkv_out]

    def clear(self):
        for t in list(self.out.values()) + list(self.qkv_out):
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
