"""GPU parity of gdn_prefill_packed against the fp64 oracle, through the C ABI.

Tolerances: states and checkpoints 1e-3 relative Frobenius per (sequence or
checkpoint, head); outputs max-relative per (token, head) row 2e-2 for bf16,
1e-3 for fp32; checkpoint positions and packed-vs-alone results bit-exact."""
import numpy as np
import pytest
import torch

import gated_deltanet_prefill_varlen_amd as gdn
import oracle as O
import workloads as W
from gpu_util import (DevPack, all_pairs, assert_parity, compare_pairs, oracle_pairs, sample_pairs,
                      shape_of, to_f64, io_tensor, f32_tensor, i32_tensor, DEV)

pytestmark = pytest.mark.gpu


def _ckpt(p, block=None):
    return gdn.gdn_plan_checkpoints(p.cu_seqlens, block or p.block)


def test_tiny_pack_fp32():
    p = W.tiny_pack()
    ck = _ckpt(p)
    assert list(ck) == [16]
    dp = DevPack(p, ck).run()
    torch.cuda.synchronize()
    eo, es = assert_parity(dp, all_pairs(p))
    print(f"tiny fp32: out {eo:.2e} state {es:.2e}")


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 64), (128, 128)])
def test_every_residue_bf16(dk, dv):
    p = W.make_pack("residue", list(range(1, 131)), 2, 4, dk, dv, 16, 16, seed=dk + dv, init_std=0.1)
    dp = DevPack(p, _ckpt(p)).run()
    torch.cuda.synchronize()
    assert_parity(dp, sample_pairs(p, 60, seed=dk))


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunk_sizes_and_slow_decay(chunk):
    p = W.make_pack("slow", [200, 64, 129, 1, 300], 2, 4, 128, 128, chunk, 64, seed=chunk,
                    init_std=0.1, gate_scale=0.01)
    dp = DevPack(p, _ckpt(p, 64)).run()
    torch.cuda.synchronize()
    assert_parity(dp, all_pairs(p))


def test_unnormalised_qk_and_scale():
    p = W.make_pack("raw", [77, 190], 2, 4, 128, 128, 64, 64, seed=5, init_std=0.1, unit_qk=False,
                    scale=128 ** -0.5)
    dp = DevPack(p, _ckpt(p)).run()
    torch.cuda.synchronize()
    assert_parity(dp, all_pairs(p))


def test_strided_views_of_one_row():
    """q, k, v as column views of one [T, conv_dim] tensor (token strides)."""
    p = W.make_pack("views", [100, 37], 2, 4, 64, 64, 32, 32, seed=9, init_std=0.1)
    T = p.n_tokens
    row = np.concatenate([p.q.reshape(T, -1), p.k.reshape(T, -1), p.v.reshape(T, -1)], axis=1)
    big = io_tensor(row, "bf16")
    nq = p.Hqk * p.dk
    dp = DevPack(p, _ckpt(p))
    dp.q, dp.k, dp.v = big[:, :nq], big[:, nq:2 * nq], big[:, 2 * nq:]
    cd = row.shape[1]
    dp.run(shape_of(p, q_tok_stride=cd, k_tok_stride=cd, v_tok_stride=cd))
    torch.cuda.synchronize()
    assert_parity(dp, all_pairs(p))


def test_empty_prompts_keep_their_state():
    p = W.make_pack("empty", [0, 50, 0, 0, 70, 0], 2, 4, 32, 32, 16, 16, seed=3, init_std=0.1)
    dp = DevPack(p, _ckpt(p)).run()
    torch.cuda.synchronize()
    fin = to_f64(dp.final)
    for s in (0, 2, 3, 5):
        np.testing.assert_array_equal(fin[s], p.init[s].astype(np.float64))
    assert_parity(dp, all_pairs(p))


# d_k = d_v = 128 with chunk 32 or 64 runs the pipelined kernel (state,
# loader and factor waves, up to three chunks ahead); the cases below cover
# its pipeline fill and drain on short prompts, empty prompts, strided views
# and GQA ratios.
@pytest.mark.parametrize("chunk", [32, 64])
def test_pipelined_every_residue(chunk):
    """Prompts of every length 1..130 (one to five 32-token chunks, most
    shorter than the pipeline's depth), checkpoints every `chunk` tokens."""
    p = W.make_pack("residue_pipe", list(range(1, 131)), 2, 4, 128, 128, chunk, chunk, seed=chunk + 7,
                    init_std=0.1)
    dp = DevPack(p, _ckpt(p)).run()
    torch.cuda.synchronize()
    eo, es = assert_parity(dp, sample_pairs(p, 60, seed=chunk))
    print(f"pipelined residues chunk {chunk}: out {eo:.2e} state {es:.2e}")


def test_pipelined_empty_prompts_and_strided_views():
    """Empty prompts keep their state bit for bit; q, k, v as column views of
    one [T, conv_dim] tensor."""
    p = W.make_pack("empty_views", [0, 70, 0, 0, 129, 0, 33], 2, 4, 128, 128, 64, 64, seed=13, init_std=0.1)
    T = p.n_tokens
    row = np.concatenate([p.q.reshape(T, -1), p.k.reshape(T, -1), p.v.reshape(T, -1)], axis=1)
    big = io_tensor(row, "bf16")
    nq = p.Hqk * p.dk
    dp = DevPack(p, _ckpt(p))
    dp.q, dp.k, dp.v = big[:, :nq], big[:, nq:2 * nq], big[:, 2 * nq:]
    cd = row.shape[1]
    dp.run(shape_of(p, q_tok_stride=cd, k_tok_stride=cd, v_tok_stride=cd))
    torch.cuda.synchronize()
    fin = to_f64(dp.final)
    for s in (0, 2, 3, 5):
        np.testing.assert_array_equal(fin[s], p.init[s].astype(np.float64))
    assert_parity(dp, all_pairs(p))


@pytest.mark.parametrize("hqk,hv", [(4, 4), (1, 4), (2, 8), (2, 6)])
def test_pipelined_gqa_ratios(hqk, hv):
    p = W.make_pack("gqa", [150, 1, 95, 64], hqk, hv, 128, 128, 64, 64, seed=10 * hqk + hv, init_std=0.1)
    dp = DevPack(p, _ckpt(p)).run()
    torch.cuda.synchronize()
    assert_parity(dp, all_pairs(p))


def test_zero_init_equals_null_init():
    p = W.make_pack("z", [90, 33], 2, 4, 64, 64, 32, 32, seed=4)
    a = DevPack(p, _ckpt(p)).run()
    p.init = np.zeros((p.n_seqs, p.Hv, p.dv, p.dk), np.float32)
    b = DevPack(p, _ckpt(p)).run()
    torch.cuda.synchronize()
    assert torch.equal(a.out, b.out) and torch.equal(a.final, b.final)


def test_deterministic_run_twice():
    p = W.ragged_pack(seed=2)
    dp = DevPack(p, _ckpt(p)).run()
    o1, f1, c1 = dp.out.clone(), dp.final.clone(), dp.ckpt_buf.clone()
    dp.run()
    torch.cuda.synchronize()
    assert torch.equal(o1, dp.out) and torch.equal(f1, dp.final) and torch.equal(c1, dp.ckpt_buf)


@pytest.mark.parametrize("seed", [0, 1])
def test_ragged_packed_equals_alone_bitwise(seed):
    """Checkpoints, outputs and final states are bit-identical whether each
    prompt is prefilled alone or packed (the pages' alone-vs-packed check)."""
    p = W.ragged_pack(seed=seed)
    ck = _ckpt(p)
    np.testing.assert_array_equal(ck, O.plan_checkpoints(p.cu_seqlens, p.block))
    dp = DevPack(p, ck).run()
    torch.cuda.synchronize()
    for s in range(p.n_seqs):
        c0, c1 = int(p.cu_seqlens[s]), int(p.cu_seqlens[s + 1])
        sub = W.Pack(name="alone", cu_seqlens=np.array([0, c1 - c0], np.int32), Hqk=p.Hqk, Hv=p.Hv,
                     dk=p.dk, dv=p.dv, chunk=p.chunk, block=p.block, dtype=p.dtype,
                     q=p.q[c0:c1], k=p.k[c0:c1], v=p.v[c0:c1], g=p.g[c0:c1], beta=p.beta[c0:c1],
                     init=p.init[s:s + 1])
        mine = [int(x) - c0 for x in ck if c0 < x <= c1]
        alone = DevPack(sub, mine).run()
        torch.cuda.synchronize()
        assert torch.equal(alone.out, dp.out[c0:c1])
        assert torch.equal(alone.final[0], dp.final[s])
        idx = [i for i, x in enumerate(ck) if c0 < x <= c1]
        if idx:
            assert torch.equal(alone.ckpt_buf, dp.ckpt_buf[idx])
    assert_parity(dp, sample_pairs(p, 24, seed=seed))


def _full_size(p, pairs):
    ck = _ckpt(p)
    dp = DevPack(p, ck).run()
    torch.cuda.synchronize()
    refs = oracle_pairs(p, pairs, ck)
    ck_np = to_f64(dp.ckpt_buf) if dp.ckpt_buf is not None else None
    return ck, compare_pairs(p, pairs, refs, to_f64(dp.out), to_f64(dp.final), ck_np, ck)


@pytest.mark.slow
def test_chat_wave_full_size_all_pairs():
    """All 1,024 (prompt, head) pairs, every output row and checkpoint of
    each, in the launch configuration the benchmark times."""
    p = W.chat_wave()
    ck, (eo, es) = _full_size(p, all_pairs(p))
    assert len(ck) == 96
    print(f"chat wave: out {eo:.2e} state {es:.2e}")


@pytest.mark.slow
def test_long_prompts_full_size_all_pairs():
    """All 128 (prompt, head) pairs of the 4 x 8,192-token pack."""
    p = W.long_prompts()
    ck, (eo, es) = _full_size(p, all_pairs(p))
    assert len(ck) == 28
    print(f"long prompts: out {eo:.2e} state {es:.2e}")


def test_slow_decay_ragged_init_visible():
    """With slow decay the initial state still shapes the final state, so a
    dropped or misplaced init would fail here (it need not at fast decay)."""
    p = W.slow_decay(W.ragged_pack, seed=3)
    dp = DevPack(p, _ckpt(p)).run()
    torch.cuda.synchronize()
    assert_parity(dp, sample_pairs(p, 12, seed=3))


def _degenerate_pack(case):
    """A small ragged pack with one of the method's degenerate inputs."""
    p = W.make_pack(case, [130, 64, 33], 2, 4, 128, 128, 64, 64, seed=31, init_std=0.1)
    T = p.n_tokens
    if case == "beta0_g0":            # no write and no decay: the state is carried unchanged
        p.beta[:] = 0.0
        p.g[:] = 0.0
    elif case == "no_decay":          # g = 0: pure delta rule, nothing forgets
        p.g[:] = 0.0
    elif case == "beta1_repeated_keys":   # beta = 1, runs of 8 tokens with one key: overwrites
        p.beta[:] = 1.0
        for t in range(T):
            p.k[t] = p.k[t - t % 8]
    elif case == "strong_decay":      # e^G underflows inside a chunk
        p.g[:] = -30.0
    elif case == "zero_rows":         # all-zero k, q or v rows (the L2 norm gives zero vectors)
        p.k[::5] = 0
        p.q[::3] = 0
        p.v[::7] = 0
    else:
        raise ValueError(case)
    return p


@pytest.mark.parametrize("case", ["beta0_g0", "no_decay", "beta1_repeated_keys", "strong_decay",
                                  "zero_rows"])
def test_degenerate_inputs(case):
    p = _degenerate_pack(case)
    dp = DevPack(p, _ckpt(p)).run()
    torch.cuda.synchronize()
    if case == "beta0_g0":
        np.testing.assert_array_equal(to_f64(dp.final), p.init.astype(np.float64))
    eo, es = assert_parity(dp, all_pairs(p))
    print(f"{case}: out {eo:.2e} state {es:.2e}")


@pytest.mark.parametrize("qk_mul,v_mul", [(256.0, 64.0), (1.0 / 64, 1.0 / 64)])
def test_input_scales(qk_mul, v_mul):
    """Raw q/k and v scaled by powers of two (exact in bf16): the L2 norms
    undo the q/k scale and the state follows v's, so the relative errors stay
    those of unit-scale inputs while the fp16 operands sit far from 1.  (With
    v at 1/1024 of unit scale the state's entries reach fp16's subnormal
    range and the state error rises to 1.2e-3: the fp16 operand domain.)"""
    p = W.make_pack("scales", [130, 64, 33], 2, 4, 128, 128, 64, 64, seed=41, init_std=0.1,
                    unit_qk=False)
    p.init = (p.init * v_mul).astype(np.float32)
    for name, mul in (("q", qk_mul), ("k", qk_mul), ("v", v_mul)):
        x = O.to_f64(getattr(p, name), "bf16") * mul
        setattr(p, name, W.f32_to_bf16_bits(x.astype(np.float32)))
    dp = DevPack(p, _ckpt(p)).run()
    torch.cuda.synchronize()
    eo, es = assert_parity(dp, all_pairs(p))
    print(f"scales q,k x{qk_mul} v x{v_mul}: out {eo:.2e} state {es:.2e}")
