"""GPU parity of gdn_decode_step, gdn_conv1d_silu_packed and
gdn_snapshot_copy, and the mixed prefill + decode pass, through the C ABI."""
import numpy as np
import pytest
import torch

import gated_deltanet_prefill_varlen_amd as gdn
import oracle as O
import workloads as W
from gpu_util import (DevPack, all_pairs, assert_parity, f32_tensor, i32_tensor, io_tensor,
                      shape_of, to_f64, DEV, OUT_TOL, STATE_TOL)

pytestmark = pytest.mark.gpu


def _decode_dev(d: W.DecodeBatch):
    q, k, v = (io_tensor(a, d.dtype) for a in (d.q, d.k, d.v))
    st = f32_tensor(d.state)
    out = torch.empty((d.batch, d.Hv, d.dv), dtype=torch.bfloat16 if d.dtype == "bf16" else torch.float32,
                      device=DEV)
    return q, k, v, f32_tensor(d.g), f32_tensor(d.beta), st, i32_tensor(d.slot), out


def _decode_shape(d, **kw):
    return gdn.make_shape(d.Hqk, d.Hv, d.dk, d.dv, 64, gdn.GDN_BF16 if d.dtype == "bf16" else gdn.GDN_F32,
                          scale=d.scale, **kw)


@pytest.mark.parametrize("dtype,pool", [("bf16", None), ("bf16", 50), ("f32", 40)])
def test_decode_step_vs_oracle(dtype, pool):
    d = W.decode_batch(seed=3, batch=32, dtype=dtype, pool=pool)
    q, k, v, g, b, st, slot, out = _decode_dev(d)
    gdn.gdn_decode_step(_decode_shape(d), q, k, v, g, b, st, slot, d.slot, out)
    torch.cuda.synchronize()
    ro, rs = O.decode_step(O.to_f64(d.q, dtype), O.to_f64(d.k, dtype), O.to_f64(d.v, dtype),
                           d.g.astype(np.float64), d.beta.astype(np.float64), d.state.astype(np.float64),
                           d.slot, scale=d.scale)
    got_s = to_f64(st)
    assert np.max(O.rel_frobenius(got_s[d.slot], rs[d.slot])) <= STATE_TOL
    untouched = np.setdiff1d(np.arange(d.state.shape[0]), d.slot)
    np.testing.assert_array_equal(got_s[untouched], d.state[untouched].astype(np.float64))
    assert np.max(O.max_rel_rows(to_f64(out), ro)) <= OUT_TOL[dtype]


def _token_rows(a, n_tok, batch):
    """Rows of a [batch, ...] array drawn per token: [batch * n_tok, ...]."""
    return a.reshape((batch * n_tok,) + a.shape[2:]) if a.ndim > 1 else a


def test_decode_tokens_vs_oracle_and_successive_steps():
    """Speculative verification: 4 tokens per sequence with the state after
    each kept.  Against the oracle (tolerance) and bitwise against 4 calls of
    gdn_decode_step (same per-token arithmetic)."""
    B, n, Hqk, Hv, d = 16, 4, 4, 8, 128
    rng = np.random.default_rng(21)
    P = 24
    q = W.f32_to_bf16_bits(_unit(rng.standard_normal((B * n, Hqk, d))))
    k = W.f32_to_bf16_bits(_unit(rng.standard_normal((B * n, Hqk, d))))
    v = W.f32_to_bf16_bits(rng.standard_normal((B * n, Hv, d)))
    g = (-np.log1p(np.exp(rng.standard_normal((B * n, Hv))))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((B * n, Hv))))).astype(np.float32)
    state = (0.1 * rng.standard_normal((P, Hv, d, d))).astype(np.float32)
    slot = rng.permutation(P)[:B].astype(np.int32)
    shape = gdn.make_shape(Hqk, Hv, d, d, 64)
    st = f32_tensor(state)
    out = torch.empty((B * n, Hv, d), dtype=torch.bfloat16, device=DEV)
    snaps = torch.empty((B, n, Hv, d, d), dtype=torch.float32, device=DEV)
    gdn.gdn_decode_tokens(shape, n, io_tensor(q, "bf16"), io_tensor(k, "bf16"), io_tensor(v, "bf16"),
                          f32_tensor(g), f32_tensor(beta), st, i32_tensor(slot), slot, out, snaps)
    # the same tokens as n one-token steps
    st2 = f32_tensor(state)
    outs = []
    for i in range(n):
        rows = np.arange(B) * n + i
        o = torch.empty((B, Hv, d), dtype=torch.bfloat16, device=DEV)
        gdn.gdn_decode_step(shape, io_tensor(q[rows], "bf16"), io_tensor(k[rows], "bf16"),
                            io_tensor(v[rows], "bf16"), f32_tensor(g[rows]), f32_tensor(beta[rows]), st2,
                            i32_tensor(slot), slot, o)
        torch.cuda.synchronize()
        outs.append(o)
        assert torch.equal(snaps[:, i], st2[torch.from_numpy(slot).long().to(DEV)])
    torch.cuda.synchronize()
    assert torch.equal(st, st2)
    for i in range(n):
        assert torch.equal(out[torch.from_numpy(np.arange(B) * n + i).to(DEV)], outs[i])
    ro, rs, rsn = O.decode_tokens(O.to_f64(q, "bf16"), O.to_f64(k, "bf16"), O.to_f64(v, "bf16"),
                                  g.astype(np.float64), beta.astype(np.float64), state.astype(np.float64),
                                  n, slot)
    assert np.max(O.max_rel_rows(to_f64(out), ro)) <= OUT_TOL["bf16"]
    assert np.max(O.rel_frobenius(to_f64(st)[slot], rs[slot])) <= STATE_TOL
    assert np.max(O.rel_frobenius(to_f64(snaps).reshape(B * n, Hv, d, d),
                                  rsn.reshape(B * n, Hv, d, d))) <= STATE_TOL


def _unit(x):
    return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)


@pytest.mark.parametrize("n,d,dtype", [(1, 128, "bf16"), (4, 128, "bf16"), (2, 64, "bf16"), (3, 32, "f32")])
def test_decode_with_conv_window_shift(n, d, dtype):
    """Decode with the short convolution applied per token: q, k, v are the
    conv's inputs, each slot's conv window supplies the history and moves on
    by the call's tokens.  Against the oracle's conv (history = the slot's
    window, output rounded to the io dtype) followed by its decode, with a
    permuted slot pool; and bitwise against gdn_conv1d_silu_packed followed by
    gdn_decode_tokens without the conv (same operation order)."""
    B, Hqk, Hv, P = 6, 2, 4, 11
    rng = np.random.default_rng(100 + n + d)
    C = 2 * Hqk * d + Hv * d
    enc = (lambda a: W.f32_to_bf16_bits(a.astype(np.float32))) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    x = enc(rng.standard_normal((B * n, C)))                   # pre-conv rows, channels q | k | v
    w = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    cstate = enc(rng.standard_normal((P, 3, C)))
    g = (-np.log1p(np.exp(rng.standard_normal((B * n, Hv))))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((B * n, Hv))))).astype(np.float32)
    state = (0.1 * rng.standard_normal((P, Hv, d, d))).astype(np.float32)
    slot = rng.permutation(P)[:B].astype(np.int32)
    nq = Hqk * d
    io = gdn.GDN_BF16 if dtype == "bf16" else gdn.GDN_F32
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xt = io_tensor(x, dtype)
    shape = gdn.make_shape(Hqk, Hv, d, d, 64, io, q_tok_stride=C, k_tok_stride=C, v_tok_stride=C)
    st, cs = f32_tensor(state), io_tensor(cstate, dtype)
    out = torch.empty((B * n, Hv, d), dtype=tdt, device=DEV)
    snaps = torch.empty((B, n, Hv, d, d), dtype=torch.float32, device=DEV)
    wt = f32_tensor(w)
    gdn.gdn_decode_tokens(shape, n, xt[:, :nq], xt[:, nq:2 * nq], xt[:, 2 * nq:], f32_tensor(g),
                          f32_tensor(beta), st, i32_tensor(slot), slot, out, snaps, conv_w=wt, conv_state=cs)
    torch.cuda.synchronize()

    # oracle: conv per sequence from its slot's window, rounded as stored, then decode
    xf = O.to_f64(x, dtype)
    cu = np.arange(B + 1) * n
    y, cs_out, _ = O.conv1d_silu_packed(xf, w.astype(np.float64), cu, O.to_f64(cstate, dtype)[slot])
    if dtype == "bf16":
        y = O.round_bf16(y)
    qf = y[:, :nq].reshape(B * n, Hqk, d)
    kf = y[:, nq:2 * nq].reshape(B * n, Hqk, d)
    vf = y[:, 2 * nq:].reshape(B * n, Hv, d)
    ro, rs, rsn = O.decode_tokens(qf, kf, vf, g.astype(np.float64), beta.astype(np.float64),
                                  state.astype(np.float64), n, slot)
    assert np.max(O.max_rel_rows(to_f64(out), ro)) <= OUT_TOL[dtype]
    assert np.max(O.rel_frobenius(to_f64(st)[slot], rs[slot])) <= STATE_TOL
    assert np.max(O.rel_frobenius(to_f64(snaps).reshape(B * n, Hv, d, d), rsn.reshape(B * n, Hv, d, d))) <= STATE_TOL
    got_cs = to_f64(cs)
    np.testing.assert_array_equal(got_cs[slot], cs_out)          # the windows moved on exactly
    untouched = np.setdiff1d(np.arange(P), slot)
    np.testing.assert_array_equal(got_cs[untouched], O.to_f64(cstate, dtype)[untouched])
    np.testing.assert_array_equal(to_f64(st)[untouched], state[untouched].astype(np.float64))

    # the two-call path: the packed conv, then the decode on its outputs
    yt = torch.empty_like(xt)
    cs_in = io_tensor(cstate, dtype)[torch.from_numpy(slot).long().to(DEV)].contiguous()
    gdn.gdn_conv1d_silu_packed(shape, i32_tensor(cu), cu, xt, wt, yt, conv_state_in=cs_in)
    st2 = f32_tensor(state)
    out2 = torch.empty_like(out)
    snaps2 = torch.empty_like(snaps)
    gdn.gdn_decode_tokens(shape, n, yt[:, :nq], yt[:, nq:2 * nq], yt[:, 2 * nq:], f32_tensor(g),
                          f32_tensor(beta), st2, i32_tensor(slot), slot, out2, snaps2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(st, st2) and torch.equal(snaps, snaps2)


def test_decode_identity_slots_and_small_heads():
    d = W.decode_batch(seed=4, batch=5, Hqk=2, Hv=4, dk=32, dv=64)
    q, k, v, g, b, st, _, out = _decode_dev(d)
    # without slots the pool rows 0..B-1 are used in order
    order = np.arange(5)
    gdn.gdn_decode_step(_decode_shape(d), q, k, v, g, b, st, None, None, out)
    torch.cuda.synchronize()
    ro, rs = O.decode_step(O.to_f64(d.q, "bf16"), O.to_f64(d.k, "bf16"), O.to_f64(d.v, "bf16"),
                           d.g.astype(np.float64), d.beta.astype(np.float64), d.state.astype(np.float64),
                           order)
    assert np.max(O.rel_frobenius(to_f64(st), rs)) <= STATE_TOL
    assert np.max(O.max_rel_rows(to_f64(out), ro)) <= OUT_TOL["bf16"]


def test_decode_after_prefill_continues_the_prompt():
    """Prefill L tokens, then decode token L+1 from the final state: equals a
    prefill of L+1 tokens (tolerance; different kernels)."""
    p = W.make_pack("cont", [65, 130], 2, 4, 128, 128, 64, 64, seed=8, init_std=0.1)
    L = [64, 129]
    head = W.Pack(name="head", cu_seqlens=np.array([0, 64, 193], np.int32), Hqk=2, Hv=4, dk=128, dv=128,
                  chunk=64, block=64, dtype="bf16",
                  q=np.concatenate([p.q[0:64], p.q[65:194]]), k=np.concatenate([p.k[0:64], p.k[65:194]]),
                  v=np.concatenate([p.v[0:64], p.v[65:194]]), g=np.concatenate([p.g[0:64], p.g[65:194]]),
                  beta=np.concatenate([p.beta[0:64], p.beta[65:194]]), init=p.init)
    dh = DevPack(head).run()
    last = [64, 194]
    q = io_tensor(p.q[last], "bf16"); k = io_tensor(p.k[last], "bf16"); v = io_tensor(p.v[last], "bf16")
    out = torch.empty((2, 4, 128), dtype=torch.bfloat16, device=DEV)
    gdn.gdn_decode_step(shape_of(p), q, k, v, f32_tensor(p.g[last]), f32_tensor(p.beta[last]), dh.final,
                        None, None, out)
    torch.cuda.synchronize()
    full = DevPack(p).run()
    torch.cuda.synchronize()
    assert np.max(O.rel_frobenius(to_f64(dh.final), to_f64(full.final))) <= 2 * STATE_TOL
    assert np.max(O.max_rel_rows(to_f64(out), to_f64(full.out[last]))) <= OUT_TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_vs_oracle_with_history_and_windows(dtype):
    p = W.make_pack("conv", [40, 24, 2, 0, 57], 2, 2, 32, 32, 16, 16, dtype=dtype, seed=11,
                    with_conv=True, conv_std=0.5)
    T, C = p.x.shape
    rng = np.random.default_rng(12)
    hist = W._normal(rng, (p.n_seqs, 3, C))
    if dtype == "bf16":
        hist = W.f32_to_bf16_bits(hist)
    ck = gdn.gdn_plan_checkpoints(p.cu_seqlens, 16)
    x = io_tensor(p.x, dtype)
    hist_d = io_tensor(hist, dtype)
    y = torch.empty_like(x)
    st_out = torch.empty_like(hist_d)
    win = torch.empty((len(ck), 3, C), dtype=x.dtype, device=DEV)
    gdn.gdn_conv1d_silu_packed(shape_of(p), i32_tensor(p.cu_seqlens), p.cu_seqlens, x,
                               f32_tensor(p.conv_w), y, hist_d, st_out, i32_tensor(ck), ck, win)
    torch.cuda.synchronize()
    ry, rst, rwin = O.conv1d_silu_packed(O.to_f64(p.x, dtype), p.conv_w.astype(np.float64), p.cu_seqlens,
                                         conv_state=O.to_f64(hist, dtype), ckpt_positions=ck)
    assert np.max(O.max_rel_rows(to_f64(y), ry)) <= OUT_TOL[dtype]
    np.testing.assert_array_equal(to_f64(st_out), rst)       # pure copies: exact
    np.testing.assert_array_equal(to_f64(win), rwin)


def test_conv_in_place_state_and_no_history():
    p = W.make_pack("conv2", [5, 1, 33], 2, 2, 32, 32, 16, 16, dtype="bf16", seed=13, with_conv=True)
    x = io_tensor(p.x, "bf16")
    y = torch.empty_like(x)
    C = p.x.shape[1]
    state = torch.zeros((3, 3, C), dtype=torch.bfloat16, device=DEV)
    gdn.gdn_conv1d_silu_packed(shape_of(p), i32_tensor(p.cu_seqlens), p.cu_seqlens, x,
                               f32_tensor(p.conv_w), y, state, state)
    torch.cuda.synchronize()
    ry, rst, _ = O.conv1d_silu_packed(O.to_f64(p.x, "bf16"), p.conv_w.astype(np.float64), p.cu_seqlens)
    assert np.max(O.max_rel_rows(to_f64(y), ry)) <= OUT_TOL["bf16"]
    np.testing.assert_array_equal(to_f64(state), rst)


def test_conv_large_pack_past_grid_row_limit():
    """A pack of 1.1M tokens (68,752 strips of 16 plus the checkpoint windows
    and conv states, past the 65,535 rows of one grid dimension): sampled rows
    on both sides of row 65,535 * 16 and at the end against the oracle's conv
    of that slice (its three history rows passed as the conv state); conv
    states and checkpoint windows bit-exact (they are copies)."""
    lens = [600_000, 500_017]
    T, C = sum(lens), 96                     # Hqk = Hv = 1, d = 32
    rng = np.random.default_rng(21)
    xb = W.f32_to_bf16_bits(W._normal(rng, (T, C)))
    w = (0.5 * W._normal(rng, (C, 4))).astype(np.float32)
    cu = np.array([0, lens[0], T], dtype=np.int32)
    ck = gdn.gdn_plan_checkpoints(cu, 4096)
    x = io_tensor(xb, "bf16")
    y = torch.empty_like(x)
    st_out = torch.empty((2, 3, C), dtype=torch.bfloat16, device=DEV)
    win = torch.empty((len(ck), 3, C), dtype=torch.bfloat16, device=DEV)
    gdn.gdn_conv1d_silu_packed(gdn.make_shape(1, 1, 32, 32, 64), i32_tensor(cu), cu, x, f32_tensor(w), y,
                               None, st_out, i32_tensor(ck), ck, win)
    torch.cuda.synchronize()
    x64 = O.to_f64(xb, "bf16")
    for r0, r1 in ((65535 * 16 - 200, 65535 * 16 + 200), (T - 4096, T)):
        ry, _, _ = O.conv1d_silu_packed(x64[r0:r1], w.astype(np.float64), [0, r1 - r0],
                                        conv_state=x64[None, r0 - 3:r0])
        assert np.max(O.max_rel_rows(to_f64(y[r0:r1]), ry)) <= OUT_TOL["bf16"], (r0, r1)
    xt = torch.from_numpy(np.ascontiguousarray(xb)).view(torch.bfloat16)
    for s in range(2):
        assert torch.equal(st_out[s].cpu(), xt[int(cu[s + 1]) - 3:int(cu[s + 1])])
    for i, c in enumerate(ck):
        assert torch.equal(win[i].cpu(), xt[int(c) - 3:int(c)])


def test_tiny_pipeline_conv_then_scan():
    """Tiny workload end to end: conv on the drawn q|k|v, then the scan with
    its own L2 norm, against the oracle's conv followed by its scan."""
    p = W.tiny_pack()
    T, C = p.x.shape
    x = io_tensor(p.x, "f32")
    y = torch.empty_like(x)
    gdn.gdn_conv1d_silu_packed(shape_of(p), i32_tensor(p.cu_seqlens), p.cu_seqlens, x,
                               f32_tensor(p.conv_w), y)
    nq = p.Hqk * p.dk
    ck = gdn.gdn_plan_checkpoints(p.cu_seqlens, 16)
    dp = DevPack(p, ck)
    dp.q, dp.k, dp.v = y[:, :nq], y[:, nq:2 * nq], y[:, 2 * nq:]
    dp.run(shape_of(p, q_tok_stride=C, k_tok_stride=C, v_tok_stride=C))
    torch.cuda.synchronize()
    ry, _, _ = O.conv1d_silu_packed(p.x.astype(np.float64), p.conv_w.astype(np.float64), p.cu_seqlens)
    q = ry[:, :nq].reshape(T, p.Hqk, p.dk)
    k = ry[:, nq:2 * nq].reshape(T, p.Hqk, p.dk)
    v = ry[:, 2 * nq:].reshape(T, p.Hv, p.dv)
    ro, rf, rc = O.prefill_recurrent(q, k, v, p.g.astype(np.float64), p.beta.astype(np.float64),
                                     p.cu_seqlens, ckpt_positions=ck)
    assert np.max(O.max_rel_rows(to_f64(dp.out), ro)) <= OUT_TOL["f32"]
    assert np.max(O.rel_frobenius(to_f64(dp.final), rf)) <= STATE_TOL
    assert np.max(O.rel_frobenius(to_f64(dp.ckpt_buf), rc)) <= STATE_TOL


def test_snapshot_copy_device_pool_on_own_stream():
    p = W.ragged_pack(seed=5)
    ck = gdn.gdn_plan_checkpoints(p.cu_seqlens, p.block)
    dp = DevPack(p, ck).run()
    scan_done = torch.cuda.Event()
    scan_done.record()
    n = len(ck)
    each = p.Hv * p.dv * p.dk * 4
    pool = torch.zeros((n + 7, p.Hv, p.dv, p.dk), dtype=torch.float32, device=DEV)
    slots = np.random.default_rng(0).permutation(n + 7)[:n].astype(np.int64)
    copy_stream = torch.cuda.Stream()
    done = torch.cuda.Event()
    gdn.gdn_snapshot_copy(dp.ckpt_buf, n, each, pool, torch.from_numpy(slots).to(DEV), slots, n + 7,
                          wait_event=scan_done, copy_stream=copy_stream, done_event=done)
    assert done.cuda_event, "the copy-done event was left unrecorded"
    done.synchronize()
    assert torch.equal(pool[torch.from_numpy(slots).to(DEV)], dp.ckpt_buf)
    rest = np.setdiff1d(np.arange(n + 7), slots)
    assert torch.count_nonzero(pool[torch.from_numpy(rest).to(DEV)]) == 0


def test_mixed_step_two_streams():
    """A mixed pass: packed prefill of the admitted prompt tokens on one
    stream, the decode batch on another, joined by an event."""
    pack, dec = W.mixed_step(seed=0)
    assert pack.n_tokens == 1024 and pack.n_seqs <= 8
    dp = DevPack(pack)
    q, k, v, g, b, st, slot, out = _decode_dev(dec)
    s1 = torch.cuda.Stream()
    start = torch.cuda.Event()
    start.record()
    s1.wait_event(start)
    dp.run()
    gdn.gdn_decode_step(_decode_shape(dec), q, k, v, g, b, st, slot, dec.slot, out, stream=s1)
    joined = torch.cuda.Event()
    joined.record(s1)
    torch.cuda.current_stream().wait_event(joined)
    torch.cuda.synchronize()
    assert_parity(dp, all_pairs(pack)[:: max(1, len(all_pairs(pack)) // 24)])
    ro, rs = O.decode_step(O.to_f64(dec.q, "bf16"), O.to_f64(dec.k, "bf16"), O.to_f64(dec.v, "bf16"),
                           dec.g.astype(np.float64), dec.beta.astype(np.float64),
                           dec.state.astype(np.float64), dec.slot)
    assert np.max(O.rel_frobenius(to_f64(st)[dec.slot], rs[dec.slot])) <= STATE_TOL
    assert np.max(O.max_rel_rows(to_f64(out), ro)) <= OUT_TOL["bf16"]
