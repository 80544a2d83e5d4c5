"""GPU parity at input scales far from unit length, and checkpoints at any
position inside a prompt, against the fp64 oracle, through the C ABI.

The scan's products run on fp16 operands (normal range about 6e-5 .. 65504).
q/k rows far from unit length are scaled by a power of two before conversion
and each state wave holds its columns as 2^E S, so the relative errors stay
those of unit-scale inputs whatever the scale.  Tolerances as everywhere:
states and checkpoints 1e-3 relative Frobenius per (sequence or checkpoint,
head), bf16 outputs 2e-2 max-relative per (token, head) row.

A chunk of the scan also ends at every checkpoint, so checkpoints need not
sit on the chunk grid: a prompt resumed from an absolute position p0 that is
not a multiple of the chunk (cut by a pass's token budget, sparkinfer release
v0.6.4 "What changed") gets its planned checkpoints, and a run resumed from
any checkpoint is bit-identical to the unbroken run (sparkinfer release
v0.6.28, "Measured": checkpoints identical alone or packed)."""
import numpy as np
import pytest
import torch

import gated_deltanet_prefill_varlen_amd as gdn
import oracle as O
import workloads as W
from gpu_util import DEV, DevPack, all_pairs, assert_parity, sample_pairs

pytestmark = pytest.mark.gpu

# (d, chunk): d = 128 with chunk 64 runs the pipelined scan, d = 64 and
# chunk 16 the chunked scan
KERNELS = [(128, 64), (64, 32), (128, 16)]


def _scaled_pack(d, chunk, qk_mul, v_mul, gate_scale=1.0, seed=41, lengths=(130, 64, 33, 300)):
    p = W.make_pack("scales", list(lengths), 2, 4, d, d, chunk, 64, seed=seed, init_std=0.1,
                    unit_qk=False, gate_scale=gate_scale)
    p.init = (p.init.astype(np.float64) * v_mul).astype(np.float32)
    for name, mul in (("q", qk_mul), ("k", qk_mul), ("v", v_mul)):
        x = O.to_f64(getattr(p, name), "bf16") * mul
        setattr(p, name, W.f32_to_bf16_bits(x.astype(np.float32)))
    return p


@pytest.mark.parametrize("d,chunk", KERNELS)
@pytest.mark.parametrize("qk_mul,v_mul", [
    (1.0, 2.0 ** -10), (1.0, 2.0 ** -14), (1.0, 2.0 ** -24),   # small values: fp16 subnormals
    (1.0, 2.0 ** 14),                                           # large values: past fp16's range in S
    (2.0 ** 16, 1.0), (2.0 ** -16, 1.0),                        # q/k past fp16's range / subnormal
    (2.0 ** 20, 2.0 ** -14),
])
def test_input_scales_far_from_unit(d, chunk, qk_mul, v_mul):
    p = _scaled_pack(d, chunk, qk_mul, v_mul)
    dp = DevPack(p, gdn.gdn_plan_checkpoints(p.cu_seqlens, p.block)).run()
    torch.cuda.synchronize()
    eo, es = assert_parity(dp, all_pairs(p))
    print(f"d {d} chunk {chunk} q,k x{qk_mul:g} v x{v_mul:g}: out {eo:.2e} state {es:.2e}")


@pytest.mark.parametrize("d,chunk", KERNELS)
def test_slow_decay_state_grows_large(d, chunk):
    """Little decay and large values: the state's entries reach about 2^17,
    past fp16's largest finite value, and are held scaled."""
    p = _scaled_pack(d, chunk, 1.0, 2.0 ** 15, gate_scale=0.001, lengths=(900, 257))
    p.beta[:] = 1.0
    dp = DevPack(p, gdn.gdn_plan_checkpoints(p.cu_seqlens, p.block)).run()
    torch.cuda.synchronize()
    assert float(dp.final.abs().max()) > 65504.0, "the state did not leave fp16's range"
    eo, es = assert_parity(dp, all_pairs(p))
    print(f"d {d} chunk {chunk} slow decay, large state: out {eo:.2e} state {es:.2e}")


@pytest.mark.parametrize("d,chunk", KERNELS)
def test_value_scale_jumps_between_chunks(d, chunk):
    """v at unit scale, then 2^-16, then 2^12 within one prompt, the jumps on
    chunk boundaries, and a 2^8 step inside a chunk: the state's scale is
    chosen again at every chunk.  (One chunk's rows share one scale, so rows
    more than about 2^14 below the chunk's largest lose precision to fp16
    subnormals; that is the operand domain.)"""
    p = W.make_pack("jumps", [400, 250], 2, 4, d, d, chunk, 64, seed=7, init_std=0.1, gate_scale=0.05)
    v = O.to_f64(p.v, "bf16")
    v[96:224] *= 2.0 ** -16
    v[224:] *= 2.0 ** 12
    v[300:310] *= 2.0 ** -8
    p.v = W.f32_to_bf16_bits(v.astype(np.float32))
    dp = DevPack(p, gdn.gdn_plan_checkpoints(p.cu_seqlens, p.block)).run()
    torch.cuda.synchronize()
    assert_parity(dp, all_pairs(p))


# ------------------------------------------------ checkpoints off the grid --

def _random_ckpts(p, rng, per_prompt=3):
    """Checkpoints at random positions inside each prompt (1 token in, mid-
    chunk, the prompt end), strictly increasing."""
    out = []
    for s in range(p.n_seqs):
        c0, c1 = int(p.cu_seqlens[s]), int(p.cu_seqlens[s + 1])
        L = c1 - c0
        if L == 0:
            continue
        cand = set(int(x) for x in rng.integers(1, L + 1, size=per_prompt))
        cand |= {1, L} if L > 2 else {L}
        out += [c0 + c for c in sorted(cand)]
    return np.array(out, np.int32)


@pytest.mark.parametrize("d,chunk", KERNELS)
def test_checkpoints_anywhere_vs_oracle(d, chunk):
    p = W.make_pack("anywhere", [1, 31, 33, 100, 129, 0, 257], 2, 4, d, d, chunk, 64, seed=d + chunk,
                    init_std=0.1, gate_scale=0.1)
    ck = _random_ckpts(p, np.random.default_rng(chunk))
    assert any((c - p.cu_seqlens[np.searchsorted(p.cu_seqlens, c, "right") - 1]) % 32 for c in ck)
    dp = DevPack(p, ck).run()
    torch.cuda.synchronize()
    eo, es = assert_parity(dp, all_pairs(p))
    print(f"d {d} chunk {chunk}: {len(ck)} checkpoints anywhere: out {eo:.2e} state {es:.2e}")


@pytest.mark.parametrize("d,chunk", KERNELS)
def test_resume_from_off_grid_checkpoint_is_bitwise(d, chunk):
    """Prefill [0, L) with checkpoints at c1 < c2 (neither on the chunk
    grid), then [c1, L) from the checkpoint at c1 with the later checkpoint:
    outputs, the later checkpoint and the final state are bit-identical."""
    L, c1, c2 = 333, 45, 200
    p = W.make_pack("resume", [L], 2, 4, d, d, chunk, 64, seed=3, init_std=0.1, gate_scale=0.05)
    full = DevPack(p, [c1, c2]).run()
    torch.cuda.synchronize()
    sub = W.Pack(name="tail", cu_seqlens=np.array([0, L - c1], np.int32), Hqk=p.Hqk, Hv=p.Hv, dk=p.dk,
                 dv=p.dv, chunk=p.chunk, block=p.block, dtype=p.dtype, q=p.q[c1:], k=p.k[c1:],
                 v=p.v[c1:], g=p.g[c1:], beta=p.beta[c1:], init=None)
    cont = DevPack(sub, [c2 - c1])
    cont.init = full.ckpt_buf[0:1].clone()
    cont.run()
    torch.cuda.synchronize()
    assert torch.equal(cont.out, full.out[c1:])
    assert torch.equal(cont.ckpt_buf[0], full.ckpt_buf[1])
    assert torch.equal(cont.final, full.final)
    assert_parity(full, all_pairs(p))


@pytest.mark.parametrize("d,chunk", KERNELS)
def test_off_grid_checkpoints_packed_equals_alone(d, chunk):
    p = W.make_pack("alone", [77, 300, 5, 190], 2, 4, d, d, chunk, 64, seed=11, init_std=0.1)
    ck = _random_ckpts(p, np.random.default_rng(4))
    dp = DevPack(p, ck).run()
    torch.cuda.synchronize()
    for s in range(p.n_seqs):
        c0, c1 = int(p.cu_seqlens[s]), int(p.cu_seqlens[s + 1])
        sub = W.Pack(name="one", cu_seqlens=np.array([0, c1 - c0], np.int32), Hqk=p.Hqk, Hv=p.Hv,
                     dk=p.dk, dv=p.dv, chunk=p.chunk, block=p.block, dtype=p.dtype, q=p.q[c0:c1],
                     k=p.k[c0:c1], v=p.v[c0:c1], g=p.g[c0:c1], beta=p.beta[c0:c1],
                     init=p.init[s:s + 1])
        mine = [int(x) - c0 for x in ck if c0 < x <= c1]
        one = DevPack(sub, mine).run()
        torch.cuda.synchronize()
        assert torch.equal(one.out, dp.out[c0:c1])
        assert torch.equal(one.final[0], dp.final[s])
        idx = [i for i, x in enumerate(ck) if c0 < x <= c1]
        assert torch.equal(one.ckpt_buf, dp.ckpt_buf[idx])


def test_mixed_pass_continuation_with_planned_checkpoints():
    """A prompt cut by a mixed pass's 1,024-token budget is continued in the
    next pass from absolute position p0 (not a multiple of the chunk); its
    planned checkpoints there fall off the chunk grid.  The continuation's
    checkpoints, outputs and final state match the oracle's run of the whole
    prompt at the same absolute positions."""
    rng = np.random.default_rng(0)
    lens = W.mixed_fill(rng)                     # the last prompt is cut to the budget
    full_len = 1500
    cut = lens[-1]
    assert cut % 64 != 0
    p = W.make_pack("whole", [full_len], 16, 32, 128, 128, 64, 256, seed=9)
    # first pass: the cut prompt's first `cut` tokens, checkpoints from p0 = 0
    first = W.Pack(name="first", cu_seqlens=np.array([0, cut], np.int32), Hqk=16, Hv=32, dk=128, dv=128,
                   chunk=64, block=256, dtype="bf16", q=p.q[:cut], k=p.k[:cut], v=p.v[:cut],
                   g=p.g[:cut], beta=p.beta[:cut], init=None)
    ck1 = gdn.gdn_plan_checkpoints(first.cu_seqlens, 256)
    a = DevPack(first, ck1).run()
    # second pass: the rest, resumed at p0 = cut from the first pass's final state
    rest = W.Pack(name="rest", cu_seqlens=np.array([0, full_len - cut], np.int32), Hqk=16, Hv=32,
                  dk=128, dv=128, chunk=64, block=256, dtype="bf16", q=p.q[cut:], k=p.k[cut:],
                  v=p.v[cut:], g=p.g[cut:], beta=p.beta[cut:], init=None)
    ck2 = gdn.gdn_plan_checkpoints(rest.cu_seqlens, 256, p0_host=np.array([cut], np.int32))
    assert len(ck2) and all((c % 64) != 0 for c in ck2)
    b = DevPack(rest, ck2)
    b.init = a.final.clone()
    b.run()
    torch.cuda.synchronize()
    absolute = [int(c) for c in ck1] + [cut + int(c) for c in ck2]
    assert absolute == list(O.plan_checkpoints(np.array([0, full_len], np.int32), 256))
    # the oracle on the whole prompt, at the absolute positions
    for h in sample_pairs(p, 6, seed=1):
        hh = h[1]
        j = hh // 2
        ro, rf, rc = O.prefill_recurrent(O.to_f64(p.q[:, j:j + 1], "bf16"), O.to_f64(p.k[:, j:j + 1], "bf16"),
                                         O.to_f64(p.v[:, hh:hh + 1], "bf16"),
                                         p.g[:, hh:hh + 1].astype(np.float64),
                                         p.beta[:, hh:hh + 1].astype(np.float64), [0, full_len],
                                         ckpt_positions=absolute)
        got_ck = [a.ckpt_buf[i, hh] for i in range(len(ck1))] + [b.ckpt_buf[i, hh] for i in range(len(ck2))]
        for i, t in enumerate(got_ck):
            assert O.rel_frobenius(t.double().cpu().numpy(), rc[i, 0]) <= 1e-3
        assert O.rel_frobenius(b.final[0, hh].double().cpu().numpy(), rf[0, 0]) <= 1e-3
        out = np.concatenate([a.out[:, hh].float().cpu().numpy(), b.out[:, hh].float().cpu().numpy()])
        assert float(np.max(O.max_rel_rows(out.astype(np.float64), ro[:, 0]))) <= 2e-2
