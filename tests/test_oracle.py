"""Pins of the fp64 oracle against closed forms, hand-worked values,
invariants and brute force.  CPU only (no GPU, no HIP library)."""
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng(1234)


def rand_pack(rng, lengths, Hqk=2, Hv=4, dk=8, dv=6, init_std=0.3, gate_scale=1.0):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T, N = int(cu[-1]), len(lengths)
    q = rng.standard_normal((T, Hqk, dk))
    k = rng.standard_normal((T, Hqk, dk))
    v = rng.standard_normal((T, Hv, dv))
    g = -np.log1p(np.exp(rng.standard_normal((T, Hv)))) * gate_scale
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, Hv))))
    init = rng.standard_normal((N, Hv, dv, dk)) * init_std if init_std else None
    return cu, q, k, v, g, beta, init


# ----------------------------------------------------------- recurrence ----

def test_p1_no_write_no_decay_keeps_state():
    rng = np.random.default_rng(1)
    cu, q, k, v, g, beta, init = rand_pack(rng, [7, 5])
    g[:] = 0.0
    beta[:] = 0.0
    out, fin, _ = O.prefill_recurrent(q, k, v, g, beta, cu, init=init, scale=0.7)
    np.testing.assert_array_equal(fin, init)
    qn = q / np.sqrt((q ** 2).sum(-1, keepdims=True) + O.DEFAULT_EPS)
    grp = 2
    for t in range(int(cu[-1])):
        s = 0 if t < cu[1] else 1
        for h in range(4):
            np.testing.assert_allclose(out[t, h], 0.7 * init[s, h] @ qn[t, h // grp], rtol=1e-13, atol=1e-13)


def test_p2_pure_decay_closed_form():
    rng = np.random.default_rng(2)
    cu, q, k, v, g, beta, init = rand_pack(rng, [9, 4, 11])
    beta[:] = 0.0
    _, fin, _ = O.prefill_recurrent(q, k, v, g, beta, cu, init=init)
    for s in range(3):
        decay = np.exp(g[cu[s]:cu[s + 1]].sum(0))
        np.testing.assert_allclose(fin[s], decay[:, None, None] * init[s], rtol=1e-12, atol=1e-300)


def test_p3_orthonormal_keys_overwrite():
    rng = np.random.default_rng(3)
    dk, dv, n = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Qm[:, :n].T                           # n orthonormal keys
    V = rng.standard_normal((n, dv))
    S0 = rng.standard_normal((1, 1, dv, dk))
    q = rng.standard_normal((n, 1, dk))
    out, fin, _ = O.prefill_recurrent(q, K[:, None, :], V[:, None, :], np.zeros((n, 1)), np.ones((n, 1)),
                                      [0, n], init=S0, eps=0.0)
    expect = S0[0, 0] @ (np.eye(dk) - K.T @ K) + V.T @ K
    np.testing.assert_allclose(fin[0, 0], expect, rtol=1e-12, atol=1e-12)
    for i in range(n):                        # each key now reads back its own value
        np.testing.assert_allclose(fin[0, 0] @ K[i], V[i], rtol=1e-12, atol=1e-12)


def test_p4_single_token_from_zero():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 8)) * 3
    k = rng.standard_normal((1, 1, 8)) * 0.2
    v = rng.standard_normal((1, 1, 6))
    g = np.array([[-0.4]])
    beta = np.array([[0.3]])
    out, fin, _ = O.prefill_recurrent(q, k, v, g, beta, [0, 1], scale=0.5)
    kh = k[0, 0] / np.sqrt(k[0, 0] @ k[0, 0] + 1e-6)
    qh = q[0, 0] / np.sqrt(q[0, 0] @ q[0, 0] + 1e-6)
    np.testing.assert_allclose(fin[0, 0], 0.3 * np.outer(v[0, 0], kh), rtol=1e-14)
    np.testing.assert_allclose(out[0, 0], 0.5 * 0.3 * (kh @ qh) * v[0, 0], rtol=1e-13)


def test_p5_scalar_case_by_hand():
    rows = np.loadtxt(os.path.join(GOLDEN, "scalar_recurrence.txt"), comments="#")
    alpha, beta, k, v, q, s_exp, o_exp = rows.T
    n = len(rows)
    out, fin, ck = O.prefill_recurrent(q.reshape(n, 1, 1), k.reshape(n, 1, 1), v.reshape(n, 1, 1),
                                       np.log(alpha).reshape(n, 1), beta.reshape(n, 1), [0, n],
                                       init=np.full((1, 1, 1, 1), 2.0), ckpt_positions=[1, 2],
                                       l2norm=False)
    np.testing.assert_allclose(out[:, 0, 0], o_exp, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(ck[:, 0, 0, 0], s_exp[:2], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(fin[0, 0, 0, 0], s_exp[2], rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 64])
def test_p6_chunked_equals_sequential(chunk):
    rng = np.random.default_rng(6 + chunk)
    lengths = [1, chunk, chunk + 1, 2 * chunk + chunk // 2 + 1, 5] + list(range(2, 2 + min(chunk, 6)))
    cu, q, k, v, g, beta, init = rand_pack(rng, lengths, dk=16, dv=12)
    # checkpoints on chunk boundaries inside the longer prompts
    ck = [int(cu[s]) + m * chunk for s in range(len(lengths))
          for m in range(1, lengths[s] // chunk + 1) if m * chunk <= lengths[s]]
    a = O.prefill_recurrent(q, k, v, g, beta, cu, init=init, ckpt_positions=ck, scale=0.9)
    b = O.prefill_chunked(q, k, v, g, beta, cu, chunk, init=init, ckpt_positions=ck, scale=0.9)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) <= 1e-11 * max(1.0, np.max(np.abs(x)))


def test_p6_chunked_equals_sequential_long_chunk64():
    rng = np.random.default_rng(66)
    cu, q, k, v, g, beta, init = rand_pack(rng, [200, 64, 129], Hqk=1, Hv=2, dk=32, dv=32)
    a = O.prefill_recurrent(q, k, v, g, beta, cu, init=init)
    b = O.prefill_chunked(q, k, v, g, beta, cu, 64, init=init)
    assert np.max(O.rel_frobenius(a[1], b[1])) < 1e-12
    assert np.max(O.max_rel_rows(a[0], b[0])) < 1e-11


def test_p7_linearity_and_row_independence():
    rng = np.random.default_rng(7)
    cu, q, k, v, g, beta, init = rand_pack(rng, [13, 6])
    v2 = rng.standard_normal(v.shape)
    i2 = rng.standard_normal(init.shape)
    a = O.prefill_recurrent(q, k, v, g, beta, cu, init=init)
    b = O.prefill_recurrent(q, k, v2, g, beta, cu, init=i2)
    c = O.prefill_recurrent(q, k, 2 * v - 3 * v2, g, beta, cu, init=2 * init - 3 * i2)
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(z, 2 * x - 3 * y, rtol=1e-10, atol=1e-10)
    # row r of S (value dim) depends only on row r of V and S0
    v3, i3 = v.copy(), init.copy()
    v3[:, :, 2] = 5.0
    i3[:, :, 2, :] = -1.0
    d = O.prefill_recurrent(q, k, v3, g, beta, cu, init=i3)
    keep = [r for r in range(v.shape[2]) if r != 2]
    np.testing.assert_array_equal(a[1][:, :, keep], d[1][:, :, keep])
    np.testing.assert_array_equal(a[0][:, :, keep], d[0][:, :, keep])
    assert not np.allclose(a[1][:, :, 2], d[1][:, :, 2])


def test_p8_prefix_continuation_bitwise():
    rng = np.random.default_rng(8)
    cu, q, k, v, g, beta, init = rand_pack(rng, [37])
    full = O.prefill_recurrent(q, k, v, g, beta, cu, init=init, ckpt_positions=[16])
    head = O.prefill_recurrent(q[:16], k[:16], v[:16], g[:16], beta[:16], [0, 16], init=init)
    np.testing.assert_array_equal(full[2][0], head[1][0])
    tail = O.prefill_recurrent(q[16:], k[16:], v[16:], g[16:], beta[16:], [0, 21], init=head[1])
    np.testing.assert_array_equal(tail[1], full[1])
    np.testing.assert_array_equal(tail[0], full[0][16:])


def test_p9_packed_equals_alone():
    rng = np.random.default_rng(9)
    lengths = [17, 3, 40]
    cu, q, k, v, g, beta, init = rand_pack(rng, lengths)
    ck = O.plan_checkpoints(cu, 16)
    packed = O.prefill_recurrent(q, k, v, g, beta, cu, init=init, ckpt_positions=ck)
    for s in range(3):
        sl = slice(cu[s], cu[s + 1])
        mine = [int(p - cu[s]) for p in ck if cu[s] < p <= cu[s + 1]]
        alone = O.prefill_recurrent(q[sl], k[sl], v[sl], g[sl], beta[sl], [0, lengths[s]],
                                    init=init[s:s + 1], ckpt_positions=mine)
        np.testing.assert_array_equal(alone[0], packed[0][sl])
        np.testing.assert_array_equal(alone[1][0], packed[1][s])
        idx = [i for i, p in enumerate(ck) if cu[s] < p <= cu[s + 1]]
        np.testing.assert_array_equal(alone[2], packed[2][idx])


def test_gqa_mapping_value_head_reads_qk_head_div_group():
    rng = np.random.default_rng(10)
    cu, q, k, v, g, beta, init = rand_pack(rng, [12], Hqk=2, Hv=4)
    k[:, 1, :] = 0.0                 # qk head 1 writes and removes nothing
    g[:] = 0.0
    _, fin, _ = O.prefill_recurrent(q, k, v, g, beta, cu, init=init)
    np.testing.assert_array_equal(fin[0, 2:], init[0, 2:])   # v heads 2, 3 read qk head 1
    assert not np.allclose(fin[0, :2], init[0, :2])


def test_checkpoint_is_state_after_first_c_tokens():
    rng = np.random.default_rng(11)
    cu, q, k, v, g, beta, init = rand_pack(rng, [20, 33])
    ck = [8, 16, 20, 20 + 16, 20 + 32]
    _, _, cks = O.prefill_recurrent(q, k, v, g, beta, cu, init=init, ckpt_positions=ck)
    for i, p in enumerate(ck):
        s = 0 if p <= 20 else 1
        c = p - cu[s]
        sl = slice(cu[s], cu[s] + c)
        _, f, _ = O.prefill_recurrent(q[sl], k[sl], v[sl], g[sl], beta[sl], [0, c], init=init[s:s + 1])
        np.testing.assert_array_equal(cks[i], f[0])


def test_p12_norms_and_contraction():
    x = np.array([[3.0, 4.0]])
    assert O.l2_rnorm(x)[0] == pytest.approx(1 / np.sqrt(25 + 1e-6), rel=1e-15)
    rng = np.random.default_rng(12)
    cu, q, k, v, g, beta, init = rand_pack(rng, [30], Hqk=1, Hv=1)
    prev = init[0, 0]
    for t in range(30):
        _, f, _ = O.prefill_recurrent(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1],
                                      [0, 1], init=prev[None, None])
        cur = f[0, 0]
        bound = np.exp(g[t, 0]) * np.linalg.norm(prev, 2) + beta[t, 0] * np.linalg.norm(v[t, 0])
        assert np.linalg.norm(cur, 2) <= bound * (1 + 1e-12)
        prev = cur


def test_scale_is_linear_on_outputs_only():
    rng = np.random.default_rng(13)
    cu, q, k, v, g, beta, init = rand_pack(rng, [9])
    a = O.prefill_recurrent(q, k, v, g, beta, cu, init=init, scale=1.0)
    b = O.prefill_recurrent(q, k, v, g, beta, cu, init=init, scale=0.25)
    np.testing.assert_allclose(b[0], 0.25 * a[0], rtol=1e-15)
    np.testing.assert_array_equal(a[1], b[1])


def test_decode_is_one_token_step_on_addressed_slots():
    rng = np.random.default_rng(14)
    B, P = 3, 5
    q = rng.standard_normal((B, 2, 8)); k = rng.standard_normal((B, 2, 8))
    v = rng.standard_normal((B, 4, 6)); g = -rng.random((B, 4)); beta = rng.random((B, 4))
    state = rng.standard_normal((P, 4, 6, 8))
    slot = np.array([4, 0, 2])
    out, new = O.decode_step(q, k, v, g, beta, state, slot, scale=0.3)
    np.testing.assert_array_equal(new[[1, 3]], state[[1, 3]])
    for b in range(B):
        o1, f1, _ = O.prefill_recurrent(q[b:b + 1], k[b:b + 1], v[b:b + 1], g[b:b + 1], beta[b:b + 1],
                                        [0, 1], init=state[slot[b]][None], scale=0.3)
        np.testing.assert_array_equal(out[b], o1[0])
        np.testing.assert_array_equal(new[slot[b]], f1[0])


def test_decode_tokens_is_successive_decode_steps():
    """n tokens at once, with the state after each kept, equal n one-token
    steps (up to fp64 rounding order), and the last kept state is the final."""
    rng = np.random.default_rng(15)
    B, n, P = 3, 4, 6
    q = rng.standard_normal((B * n, 2, 8)); k = rng.standard_normal((B * n, 2, 8))
    v = rng.standard_normal((B * n, 4, 6)); g = -rng.random((B * n, 4)); beta = rng.random((B * n, 4))
    state = rng.standard_normal((P, 4, 6, 8))
    slot = np.array([5, 1, 3])
    out, new, snaps = O.decode_tokens(q, k, v, g, beta, state, n, slot, scale=0.7)
    cur = np.array(state)
    for i in range(n):
        rows = np.arange(B) * n + i
        o1, cur = O.decode_step(q[rows], k[rows], v[rows], g[rows], beta[rows], cur, slot, scale=0.7)
        np.testing.assert_allclose(out[rows], o1, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(snaps[:, i], cur[slot], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(new, cur, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(snaps[:, -1], new[slot])
    np.testing.assert_array_equal(new[[0, 2, 4]], state[[0, 2, 4]])
    o1, s1, sn1 = O.decode_tokens(q[::n], k[::n], v[::n], g[::n], beta[::n], state, 1, slot, scale=0.7)
    o2, s2 = O.decode_step(q[::n], k[::n], v[::n], g[::n], beta[::n], state, slot, scale=0.7)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


# -------------------------------------------------------------- planner ----

def _golden_planner():
    cases = []
    for line in open(os.path.join(GOLDEN, "planner_cases.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        lhs, rhs = line.split("->")
        block, tail, p0, L = (int(x) for x in lhs.split())
        rhs = rhs.strip()
        want = [] if rhs == "-" else [int(x) for x in rhs.split(",")]
        cases.append((block, tail, p0, L, want))
    return cases


@pytest.mark.parametrize("case", _golden_planner())
def test_p10_planner_golden(case):
    block, tail, p0, L, want = case
    got = O.plan_checkpoints([0, L], block, tail, p0=[p0])
    assert list(got) == want


def test_p10_planner_closed_form_brute_force():
    for block in (16, 32, 64, 256, 1024):
        for p0 in (0, block, 3 * block):
            for L in range(0, 4 * block + 40):
                got = list(O.plan_checkpoints([0, L], block, 16, p0=[p0]))
                closed = [m * block - p0 for m in range(1, (p0 + L) // block + 1)
                          if p0 < m * block <= p0 + L - 16]
                assert got == closed, (block, p0, L)


def test_p10_planner_packs():
    t = W.tiny_pack()
    assert list(O.plan_checkpoints(t.cu_seqlens, 16)) == [16]
    c = W.chat_wave()
    ck = O.plan_checkpoints(c.cu_seqlens, 256)
    assert len(ck) == 96 and list(ck[:4]) == [256, 512, 768, 1024 + 256]
    cu = np.array([0, 100, 100, 420])          # an empty prompt in the middle
    assert list(O.plan_checkpoints(cu, 64)) == [64, 100 + 64, 100 + 128, 100 + 192, 100 + 256]


# ----------------------------------------------------------------- conv ----

def test_p11_conv_tap_selection():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((20, 5))
    cu = [0, 12, 20]
    silu = lambda z: z / (1 + np.exp(-z))
    for j in range(4):
        w = np.zeros((5, 4)); w[:, j] = 1.0
        y, st, _ = O.conv1d_silu_packed(x, w, cu)
        shift = 3 - j
        for s in range(2):
            for i in range(cu[s + 1] - cu[s]):
                src = x[cu[s] + i - shift] if i >= shift else np.zeros(5)
                np.testing.assert_allclose(y[cu[s] + i], silu(src), rtol=1e-15, atol=0)
        np.testing.assert_array_equal(st[1], x[17:20])


def test_p11_conv_matches_numpy_convolve_with_history():
    rng = np.random.default_rng(16)
    C = 6
    x = rng.standard_normal((30, C)); w = rng.standard_normal((C, 4))
    cu = [0, 2, 19, 30]
    hist = rng.standard_normal((3, 3, C))
    ck = [16, 2 + 16]
    y, st, win = O.conv1d_silu_packed(x, w, cu, conv_state=hist, ckpt_positions=ck)
    for s in range(3):
        ext = np.concatenate([hist[s], x[cu[s]:cu[s + 1]]])
        for c in range(C):
            full = np.convolve(ext[:, c], w[c, ::-1], mode="valid")   # correlation with taps 0..3
            z = full
            np.testing.assert_allclose(y[cu[s]:cu[s + 1], c], z / (1 + np.exp(-z)), rtol=1e-12, atol=1e-14)
        np.testing.assert_array_equal(st[s], ext[-3:])
    assert st[0][0].tolist() == hist[0][2].tolist()    # a 2-token prompt keeps one history row
    np.testing.assert_array_equal(win[0], x[13:16])
    np.testing.assert_array_equal(win[1], x[15:18])


def test_p11_conv_packed_first_tokens_equal_alone():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((25, 4)); w = rng.standard_normal((4, 4))
    cu = [0, 10, 25]
    y, _, _ = O.conv1d_silu_packed(x, w, cu)
    y1, _, _ = O.conv1d_silu_packed(x[10:], w, [0, 15])
    np.testing.assert_array_equal(y[10:], y1)


# ------------------------------------------------------------ encodings ----

def test_bf16_rounding_ties_to_even():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 2 ** -7 + 2 ** -8, -3.140625, 1e-40])
    r = O.round_bf16(vals)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1 + 2 ** -6 and r[3] == -3.140625
    bits = W.f32_to_bf16_bits(vals.astype(np.float32))
    np.testing.assert_array_equal(O.bf16_to_f64(bits), r)


def test_comparators():
    ref = np.array([[1.0, -2.0], [0.0, 0.0]])
    x = np.array([[1.0, -1.9], [0.0, 1e-3]])
    np.testing.assert_allclose(O.max_rel_rows(x, ref), [0.05, 1e-3])
    assert O.rel_frobenius(np.zeros((2, 2)), np.zeros((2, 2))) == 0.0
