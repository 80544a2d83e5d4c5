"""Helpers for the GPU tests: move seeded packs to the device, run libgdn
through its C ABI, run the oracle on the same inputs, compare."""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np
import torch

import gated_deltanet_prefill_varlen_amd as gdn
import oracle as O
import workloads as W

DEV = "cuda:0"
STATE_TOL = 1e-3          # relative Frobenius per (sequence or checkpoint, head)
OUT_TOL = {"bf16": 2e-2, "f32": 1e-3}   # max-relative per (token, head) row


def io_tensor(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def f32_tensor(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i32_tensor(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def shape_of(p: W.Pack, l2norm=True, **kw) -> gdn.gdn_shape:
    return gdn.make_shape(p.Hqk, p.Hv, p.dk, p.dv, p.chunk,
                          gdn.GDN_BF16 if p.dtype == "bf16" else gdn.GDN_F32,
                          l2norm=l2norm, scale=p.scale, **kw)


class DevPack:
    """A pack's inputs resident on the GPU, with output buffers."""

    def __init__(self, p: W.Pack, ckpt=None, with_init=True):
        self.p = p
        self.ckpt = np.zeros(0, np.int32) if ckpt is None else np.asarray(ckpt, np.int32)
        self.cu = i32_tensor(p.cu_seqlens)
        self.q, self.k, self.v = (io_tensor(a, p.dtype) for a in (p.q, p.k, p.v))
        self.g, self.beta = f32_tensor(p.g), f32_tensor(p.beta)
        self.init = f32_tensor(p.init) if (with_init and p.init is not None) else None
        self.ckpt_d = i32_tensor(self.ckpt) if len(self.ckpt) else None
        T, N = p.n_tokens, p.n_seqs
        odt = torch.bfloat16 if p.dtype == "bf16" else torch.float32
        self.out = torch.empty((T, p.Hv, p.dv), dtype=odt, device=DEV)
        self.final = torch.empty((N, p.Hv, p.dv, p.dk), dtype=torch.float32, device=DEV)
        self.ckpt_buf = (torch.empty((len(self.ckpt), p.Hv, p.dv, p.dk), dtype=torch.float32, device=DEV)
                         if len(self.ckpt) else None)

    def run(self, shape=None, stream=None):
        gdn.gdn_prefill_packed(shape or shape_of(self.p), self.cu, self.p.cu_seqlens, self.q, self.k,
                               self.v, self.g, self.beta, self.init, self.ckpt_d,
                               self.ckpt if len(self.ckpt) else None, self.out, self.final,
                               self.ckpt_buf, stream=stream)
        return self


def oracle_inputs(p: W.Pack):
    return (O.to_f64(p.q, p.dtype), O.to_f64(p.k, p.dtype), O.to_f64(p.v, p.dtype),
            p.g.astype(np.float64), p.beta.astype(np.float64))


def oracle_seq_head(p: W.Pack, s: int, h: int, ckpt=(), l2norm=True):
    """Oracle on one (prompt, value head) of a pack: (out [L, dv], final
    [dv, dk], ckpts [n, dv, dk]) with n the checkpoints inside prompt s."""
    c0, c1 = int(p.cu_seqlens[s]), int(p.cu_seqlens[s + 1])
    j = h // (p.Hv // p.Hqk)
    sl = slice(c0, c1)
    q = O.to_f64(p.q[sl, j:j + 1], p.dtype)
    k = O.to_f64(p.k[sl, j:j + 1], p.dtype)
    v = O.to_f64(p.v[sl, h:h + 1], p.dtype)
    init = None if p.init is None else p.init[s:s + 1, h:h + 1].astype(np.float64)
    mine = [int(x) - c0 for x in ckpt if c0 < x <= c1]
    out, fin, ck = O.prefill_recurrent(q, k, v, p.g[sl, h:h + 1].astype(np.float64),
                                       p.beta[sl, h:h + 1].astype(np.float64), [0, c1 - c0],
                                       init=init, ckpt_positions=mine, scale=p.scale, l2norm=l2norm)
    return out[:, 0], fin[0, 0], ck[:, 0]


def check_seq_head(dp: DevPack, s: int, h: int, out_np=None, final_np=None, ck_np=None, l2norm=True):
    """Compare one (prompt, head) of a GPU run with the oracle; returns the
    worst (output, state) errors."""
    p = dp.p
    ro, rf, rc = oracle_seq_head(p, s, h, dp.ckpt, l2norm=l2norm)
    c0, c1 = int(p.cu_seqlens[s]), int(p.cu_seqlens[s + 1])
    out = to_f64(dp.out[c0:c1, h]) if out_np is None else out_np[c0:c1, h]
    fin = to_f64(dp.final[s, h]) if final_np is None else final_np[s, h]
    eo = float(np.max(O.max_rel_rows(out, ro))) if c1 > c0 else 0.0
    es = float(O.rel_frobenius(fin, rf))
    idx = [i for i, x in enumerate(dp.ckpt) if c0 < x <= c1]
    for n, i in enumerate(idx):
        got = to_f64(dp.ckpt_buf[i, h]) if ck_np is None else ck_np[i, h]
        es = max(es, float(O.rel_frobenius(got, rc[n])))
    return eo, es


def assert_parity(dp: DevPack, pairs, l2norm=True):
    tol_o = OUT_TOL[dp.p.dtype]
    worst_o = worst_s = 0.0
    out_np = to_f64(dp.out)
    fin_np = to_f64(dp.final)
    ck_np = to_f64(dp.ckpt_buf) if dp.ckpt_buf is not None else None
    for s, h in pairs:
        eo, es = check_seq_head(dp, s, h, out_np, fin_np, ck_np, l2norm=l2norm)
        assert eo <= tol_o, f"output rel err {eo:.3e} > {tol_o} at seq {s} head {h}"
        assert es <= STATE_TOL, f"state rel err {es:.3e} > {STATE_TOL} at seq {s} head {h}"
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
    return worst_o, worst_s


def all_pairs(p: W.Pack):
    return [(s, h) for s in range(p.n_seqs) for h in range(p.Hv)]


def sample_pairs(p: W.Pack, n: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    pairs = {(p.n_seqs - 1, p.Hv - 1), (0, 0)}
    while len(pairs) < min(n, p.n_seqs * p.Hv):
        pairs.add((int(rng.integers(p.n_seqs)), int(rng.integers(p.Hv))))
    return sorted(pairs)


# ------------------------------------------- many pairs in a process pool --

def _oracle_job(job):
    """One (prompt, head) on the oracle: optional conv (its output rounded to
    bf16 as the GPU tensor stores it), then the token-by-token recurrence."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        q, k, v, g, b, init, mine, scale, xs, w, d = job
        if xs is not None:
            ys = O.round_bf16(O.conv1d_silu_packed(xs, w, [0, xs.shape[0]])[0])
            q, k, v = ys[:, None, :d], ys[:, None, d:2 * d], ys[:, None, 2 * d:]
        out, fin, ck = O.prefill_recurrent(q, k, v, g, b, [0, q.shape[0]], init=init,
                                           ckpt_positions=mine, scale=scale)
        return out[:, 0], fin[0, 0], ck[:, 0]


def oracle_pairs(p: W.Pack, pairs, ckpt=(), conv=False, g=None, beta=None, procs=None):
    """The oracle on many (prompt, head) pairs of a pack, one process per host
    core (at most 16), each job holding only its prompt's slices.  With conv,
    q, k, v come from the pack's pre-conv rows x and conv weights.  Returns a
    list of (out [L, dv], final [dv, dk], ckpts [n, dv, dk])."""
    g = p.g if g is None else g
    beta = p.beta if beta is None else beta
    cu = p.cu_seqlens
    d = p.dk
    jobs = []
    for s, h in pairs:
        c0, c1 = int(cu[s]), int(cu[s + 1])
        j = h // (p.Hv // p.Hqk)
        init = None if p.init is None else p.init[s:s + 1, h:h + 1].astype(np.float64)
        mine = [int(x) - c0 for x in ckpt if c0 < x <= c1]
        gb = (g[c0:c1, h:h + 1].astype(np.float64), beta[c0:c1, h:h + 1].astype(np.float64))
        if conv:
            chans = np.r_[j * d:(j + 1) * d, p.Hqk * d + j * d:p.Hqk * d + (j + 1) * d,
                          2 * p.Hqk * d + h * p.dv:2 * p.Hqk * d + (h + 1) * p.dv]
            jobs.append((None, None, None) + gb + (init, mine, p.scale, O.to_f64(p.x[c0:c1][:, chans], p.dtype),
                                                   p.conv_w[chans].astype(np.float64), d))
        else:
            jobs.append((O.to_f64(p.q[c0:c1, j:j + 1], p.dtype), O.to_f64(p.k[c0:c1, j:j + 1], p.dtype),
                         O.to_f64(p.v[c0:c1, h:h + 1], p.dtype)) + gb + (init, mine, p.scale, None, None, d))
    procs = procs or max(1, min(16, len(os.sched_getaffinity(0)), len(jobs)))
    if procs == 1:
        return [_oracle_job(j) for j in jobs]
    with mp.get_context("spawn").Pool(procs) as pool:
        res = pool.map(_oracle_job, jobs)
        pool.close()
        pool.join()
    return res


def compare_pairs(p: W.Pack, pairs, refs, out, final, ckpt_buf, ckpt=()):
    """Element-by-element comparison of GPU results (host fp64 arrays: out
    [T, Hv, dv], final [N, Hv, dv, dk], ckpt_buf [n, Hv, dv, dk]) with oracle
    results for the pairs; asserts the tolerances, returns the worst errors."""
    tol_o = OUT_TOL[p.dtype]
    cu = p.cu_seqlens
    worst_o = worst_s = 0.0
    for (s, h), (ro, rf, rc) in zip(pairs, refs):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        eo = float(np.max(O.max_rel_rows(out[c0:c1, h], ro))) if c1 > c0 else 0.0
        es = float(O.rel_frobenius(final[s, h], rf))
        idx = [i for i, x in enumerate(ckpt) if c0 < x <= c1]
        for n, i in enumerate(idx):
            es = max(es, float(O.rel_frobenius(ckpt_buf[i, h], rc[n])))
        assert eo <= tol_o, f"output rel err {eo:.3e} > {tol_o} at seq {s} head {h}"
        assert es <= STATE_TOL, f"state rel err {es:.3e} > {STATE_TOL} at seq {s} head {h}"
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
    return worst_o, worst_s
