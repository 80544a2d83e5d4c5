"""The scan with the short conv fused into its loads (gdn_prefill_conv_packed)
against the two launches it replaces: gdn_conv1d_silu_packed writing y, then
gdn_prefill_packed on y's q, k and v column views, with the same conv states,
checkpoints and windows.  The fused path runs the conv in the conv kernel's
operation order and converts its bf16 outputs for the products exactly as
loaded rows are, so every result is compared bit for bit: outputs, final and
checkpoint states, conv states out and the conv windows at checkpoints.  The
two-launch path is checked against the oracle elsewhere (the layer-step and
decode tests); the chat wave here is also compared with the oracle's conv
followed by its recurrence on sampled (prompt, head) pairs.

Cases: prompts of 0 to 3 tokens (windows reaching into the conv state),
lengths on both sides of the 32-token tile, checkpoints on and off the tile
grid (also at a prompt's first and second token), GQA groups of 1 to 4 (all
with the XCD-paired grid order), conv states in or NULL, written in place or
to their own buffer, no windows or states asked for, a padded x row stride,
inputs far from unit scale
(q/k rows scaled into fp16 range), the full chat wave and long prompts."""
import numpy as np
import pytest
import torch

import gated_deltanet_prefill_varlen_amd as gdn
import workloads as W
from gpu_util import (DEV, compare_pairs, f32_tensor, i32_tensor, io_tensor, oracle_pairs, sample_pairs,
                      to_f64)

pytestmark = pytest.mark.gpu


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16)).view(torch.bfloat16).to(DEV)


class Case:
    """One pack's inputs on the GPU and both paths' outputs."""

    def __init__(self, p, ck, state_in=True, pad=0, x_scale=1.0, seed=7):
        self.p, self.ck = p, np.asarray(ck, np.int32)
        T, N, Hqk, Hv, d = p.n_tokens, p.n_seqs, p.Hqk, p.Hv, p.dk
        self.C = C = 2 * Hqk * d + Hv * d
        rng = np.random.default_rng(seed)
        x = p.x
        if x_scale != 1.0:   # bf16 bits of x * x_scale (a power of two: exact)
            x = W.f32_to_bf16_bits(W.bf16_bits_to_f32(x) * np.float32(x_scale))
        xp = np.zeros((T, C + pad), np.uint16)
        xp[:, :C] = x
        self.xs = C + pad
        self.x = _bf16(xp)                     # [T, C + pad]; rows of C channels used
        self.w = f32_tensor(p.conv_w)
        self.st_in = (_bf16(W.f32_to_bf16_bits(rng.standard_normal((N, 3, C)).astype(np.float32)))
                      if state_in else None)
        self.cu = i32_tensor(p.cu_seqlens)
        self.ck_d = i32_tensor(self.ck) if len(self.ck) else None
        self.g, self.beta = f32_tensor(p.g), f32_tensor(p.beta)
        self.init = f32_tensor(p.init) if p.init is not None else None

    def buffers(self):
        p = self.p
        T, N, n_ck, C = p.n_tokens, p.n_seqs, len(self.ck), self.C
        return dict(
            out=torch.full((T, p.Hv, p.dv), 7.0, dtype=torch.bfloat16, device=DEV),
            final=torch.full((N, p.Hv, p.dv, p.dk), 7.0, dtype=torch.float32, device=DEV),
            ckbuf=(torch.full((n_ck, p.Hv, p.dv, p.dk), 7.0, dtype=torch.float32, device=DEV)
                   if n_ck else None),
            st_out=torch.full((N, 3, C), 7.0, dtype=torch.bfloat16, device=DEV),
            conv_ck=torch.full((max(n_ck, 1), 3, C), 7.0, dtype=torch.bfloat16, device=DEV))

    def shape(self, strided=False):
        p = self.p
        st = self.xs if strided else 0
        return gdn.make_shape(p.Hqk, p.Hv, p.dk, p.dv, p.chunk, q_tok_stride=st, k_tok_stride=st,
                              v_tok_stride=st)

    def two_launches(self, st_out=True, windows=True, in_place=False):
        p, b = self.p, self.buffers()
        Hd = p.Hqk * p.dk
        y = torch.full((p.n_tokens, self.xs), 7.0, dtype=torch.bfloat16, device=DEV)
        so = self.st_in if in_place else (b["st_out"] if st_out else None)
        ck_h = self.ck if len(self.ck) else None
        gdn.gdn_conv1d_silu_packed(self.shape(), self.cu, p.cu_seqlens, self.x, self.w, y, self.st_in, so,
                                   self.ck_d, ck_h, b["conv_ck"] if (windows and len(self.ck)) else None,
                                   x_tok_stride=self.xs, y_tok_stride=self.xs)
        gdn.gdn_prefill_packed(self.shape(strided=True), self.cu, p.cu_seqlens, y[:, :Hd], y[:, Hd:2 * Hd],
                               y[:, 2 * Hd:], self.g, self.beta, self.init, self.ck_d, ck_h, b["out"],
                               b["final"], b["ckbuf"])
        b["st_out"] = so
        return b

    def fused(self, st_out=True, windows=True, in_place=False):
        p, b = self.p, self.buffers()
        so = self.st_in if in_place else (b["st_out"] if st_out else None)
        gdn.gdn_prefill_conv_packed(self.shape(), self.cu, p.cu_seqlens, self.x, self.w, self.g, self.beta,
                                    self.init, self.ck_d, self.ck if len(self.ck) else None, b["out"],
                                    b["final"], b["ckbuf"], conv_state_in=self.st_in, conv_state_out=so,
                                    conv_ckpt=b["conv_ck"] if (windows and len(self.ck)) else None,
                                    x_tok_stride=self.xs)
        b["st_out"] = so
        return b


def assert_same(a, b, what=""):
    for key in ("out", "final", "ckbuf", "st_out", "conv_ck"):
        if a[key] is None and b[key] is None:
            continue
        assert torch.equal(a[key], b[key]), f"{what}: {key} differs"


def small_pack(lengths, Hqk=2, Hv=4, seed=0, init_std=0.1):
    return W.make_pack("fused_conv_small", lengths, Hqk, Hv, 128, 128, 64, 16, seed=seed,
                       init_std=init_std, with_conv=True, conv_std=0.5)


LENGTHS = [1, 2, 3, 0, 5, 31, 32, 33, 64, 100, 257, 7]


def mixed_ckpts(p):
    """The planner's every-16 list plus positions off the tile grid: a
    prompt's first and second token, and odd offsets."""
    cu = p.cu_seqlens
    ck = set(int(x) for x in gdn.gdn_plan_checkpoints(cu, 16))
    for s in range(p.n_seqs):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        for off in (1, 2, 19, 45, 111):
            if c0 + off <= c1:
                ck.add(c0 + off)
    return np.array(sorted(ck), np.int32)


@pytest.mark.parametrize("Hqk,Hv", [(2, 4), (2, 2), (2, 8), (2, 6)])
def test_fused_equals_two_launches_ragged(Hqk, Hv):
    p = small_pack(LENGTHS, Hqk, Hv)
    ck = mixed_ckpts(p)
    print(f"ragged fused: Hqk {Hqk} Hv {Hv} T {p.n_tokens} ckpts {len(ck)}", flush=True)
    c = Case(p, ck)
    ref = c.two_launches()
    torch.cuda.synchronize()
    assert not torch.equal(ref["out"], torch.full_like(ref["out"], 7.0))
    for rep in range(3):   # every run the same bits
        assert_same(ref, c.fused(), f"ragged, run {rep}")


def test_fused_equals_two_launches_variants():
    p = small_pack(LENGTHS, seed=3)
    ck = mixed_ckpts(p)
    # no conv state in; a padded x row stride
    c = Case(p, ck, state_in=False, pad=64)
    print("fused variants: no state in, padded rows", flush=True)
    assert_same(c.two_launches(), c.fused(), "no state in, padded")
    # no conv state out, no windows
    c = Case(p, ck)
    print("fused variants: no state out, no windows", flush=True)
    assert_same(c.two_launches(st_out=False, windows=False), c.fused(st_out=False, windows=False),
                "no state out")
    # conv states written in place (a launch of their own after the scan)
    print("fused variants: conv state in place", flush=True)
    c1, c2 = Case(p, ck), Case(p, ck)
    ref, got = c1.two_launches(in_place=True), c2.fused(in_place=True)
    torch.cuda.synchronize()
    assert_same(ref, got, "in place")
    # without checkpoints
    print("fused variants: no checkpoints", flush=True)
    c = Case(p, [])
    assert_same(c.two_launches(), c.fused(), "no checkpoints")


@pytest.mark.parametrize("x_scale", [2.0 ** -8, 2.0 ** 8])
def test_fused_equals_two_launches_far_from_unit_scale(x_scale):
    p = small_pack([40, 97, 3, 130], seed=5)
    ck = mixed_ckpts(p)
    print(f"fused range: x * {x_scale}", flush=True)
    c = Case(p, ck, x_scale=x_scale)
    assert_same(c.two_launches(), c.fused(), f"x scale {x_scale}")


def test_fused_chat_wave_bitwise_and_sampled_oracle():
    p = W.chat_wave(seed=0, with_conv=True)
    ck = gdn.gdn_plan_checkpoints(p.cu_seqlens, p.block)
    print(f"chat wave fused: T {p.n_tokens} ckpts {len(ck)}", flush=True)
    c = Case(p, ck, state_in=False)
    ref = c.two_launches()
    got = c.fused()
    torch.cuda.synchronize()
    assert_same(ref, got, "chat wave")
    pairs = sample_pairs(p, 64, seed=11)
    refs = oracle_pairs(p, pairs, ck, conv=True)
    wo, ws = compare_pairs(p, pairs, refs, to_f64(got["out"]), to_f64(got["final"]), to_f64(got["ckbuf"]), ck)
    print(f"chat wave fused vs oracle: out {wo:.2e} state {ws:.2e}")


def test_fused_long_prompts_bitwise():
    p = W.make_pack("long_conv", [8192, 8192, 3000, 5000], 16, 32, 128, 128, 64, 1024, seed=2,
                    with_conv=True, conv_std=0.5)
    ck = gdn.gdn_plan_checkpoints(p.cu_seqlens, p.block)
    print(f"long fused: T {p.n_tokens} ckpts {len(ck)}", flush=True)
    c = Case(p, ck)
    assert_same(c.two_launches(), c.fused(), "long")
