"""fp64 CPU oracle of the packed gated-delta-rule prefill path.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing) and
imports nothing from it.

What is computed, and where it comes from
-----------------------------------------
* The recurrence is the gated delta rule (Yang, Kautz & Hatamizadeh, "Gated
  Delta Networks: Improving Mamba2 with Delta Rule", ICLR 2025, the gated
  delta rule equation): per sequence and value head, with alpha_t = exp(g_t),

      S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
      o_t = scale * S_t q_t,

  S is dv x dk (v k^T orientation), q and k are L2-normalised per token and
  qk head with 1/sqrt(sum x^2 + eps), value head h reads qk head
  h // (Hv / Hqk).  ``prefill_recurrent`` runs it token by token.
* ``prefill_chunked`` is an independent fp64 rewrite of the same map in the
  chunked WY/UT form (Yang et al., "Parallelizing Linear Transformers with the
  Delta Rule over Sequence Length", NeurIPS 2024, the UT transform section),
  extended with the per-token decay: inside a chunk with G = cumsum(g),
  A = strict_tril(diag(beta) (exp(G_t - G_i)) o K K^T), T = (I + A)^-1 (a
  library triangular solve), U = T diag(beta) V - T diag(beta e^G) K S0^T,
  O = scale [diag(e^G) Q S0^T + (tril(exp(G_t - G_i)) o Q K^T) U],
  S_C = e^{G_C} S0 + U^T diag(exp(G_C - G)) K.
* Packing: several prompts share one pass, each prompt's scan starting from
  its own initial state (sparkinfer release v0.6.28, intro: a wave of prompts
  prefilled in shared packed passes).  Checkpoints are the recurrent state
  after the first c tokens of a prompt, and must not depend on whether the
  prompt ran alone or packed (same release, "Measured": the checkpoint check
  alone vs packed).
* Checkpoint planning: every multiple of the block inside the prompt, except
  that one landing in the prompt's last 16 tokens moves back by one block so
  the prompt can stay in the pack (same release, the bullet on checkpoints in
  a prompt's last 16 tokens).  Reading: "in the last 16 tokens" means
  L - c < 16, the move happens once, a moved checkpoint that lands at or
  before the prompt start or on an existing one is dropped, and the prompt
  end is never a checkpoint (the final state covers it).
* Short convolution: width-4 causal depthwise conv over each prompt's own
  tokens followed by SiLU, ahead of the L2 norm and the scan (Gated Delta
  Networks, the block design with short convolution on q, k, v).  History
  before a prompt's first token comes from its conv state (the last three
  pre-conv inputs), zeros when none is given.
* Decode: one step of the recurrence per sequence on a state addressed by
  slot; mixed passes carry such decodes beside a packed prefill (sparkinfer
  release v0.6.4, "What changed").

Every function is pinned by tests against closed forms, invariants and brute
force (tests/test_oracle.py); see each docstring for the pin that covers it.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import scipy.linalg

DEFAULT_EPS = 1e-6


# ------------------------------------------------------------------ inputs --

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor -> float64 (bf16 bit patterns or fp32 values)."""
    if dtype == "bf16":
        return bf16_to_f64(a)
    return np.asarray(a, dtype=np.float64)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as
    float64.  Used where a tensor crosses an exported call in bf16."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------- pieces --

def l2_rnorm(x: np.ndarray, eps: float = DEFAULT_EPS) -> np.ndarray:
    """1 / sqrt(sum_d x^2 + eps) over the last axis."""
    return 1.0 / np.sqrt(np.sum(x * x, axis=-1) + eps)


def plan_checkpoints(cu_seqlens: Sequence[int], block: int, tail: int = 16,
                     p0: Optional[Sequence[int]] = None) -> np.ndarray:
    """Checkpoint positions (global offsets into the pack) for every prompt.

    For a prompt of length L at pack offset cu[s] whose first token is
    absolute position p0 (0 unless it resumes from a cached prefix), take each
    multiple c of ``block`` with p0 < c <= p0 + L; if it falls in the last
    ``tail`` tokens (p0 + L - c < tail) move it back one block; keep it only if
    it is still after p0 and not already taken.  Returned as cu[s] + (c - p0),
    sorted.  Pinned by the closed form {m*block : p0 < m*block <= p0+L-tail}
    and hand-worked spot values (tests/golden/planner_cases.txt).
    """
    cu = [int(x) for x in cu_seqlens]
    out = []
    for s in range(len(cu) - 1):
        L = cu[s + 1] - cu[s]
        start = 0 if p0 is None else int(p0[s])
        taken = []
        c = block * (start // block + 1)
        while c <= start + L:
            pos = c
            if start + L - pos < tail:
                pos -= block
            if pos > start and pos not in taken:
                taken.append(pos)
            c += block
        out.extend(cu[s] + (p - start) for p in sorted(taken))
    return np.asarray(out, dtype=np.int32)


def _silu(x):
    return x / (1.0 + np.exp(-x))


def conv1d_silu_packed(x: np.ndarray, w: np.ndarray, cu_seqlens: Sequence[int],
                       conv_state: Optional[np.ndarray] = None,
                       ckpt_positions: Sequence[int] = ()):
    """Width-4 causal depthwise conv + SiLU over each prompt of a pack.

    x: [T, C] pre-conv inputs (float64); w: [C, 4], tap 3 on the current token;
    conv_state: [N, 3, C] the three inputs before each prompt (oldest first),
    zeros if None.  Returns (y [T, C], state_out [N, 3, C], windows
    [n_ckpt, 3, C]) where state_out holds each prompt's last three inputs
    (reaching into its history when L < 3) and windows[i] the three inputs
    before checkpoint position i.  Pinned by tap-selection closed forms and by
    numpy.convolve per channel.
    """
    cu = [int(v) for v in cu_seqlens]
    T, C = x.shape
    N = len(cu) - 1
    y = np.zeros((T, C))
    state_out = np.zeros((N, 3, C))
    ext_all = []
    for s in range(N):
        hist = np.zeros((3, C)) if conv_state is None else np.asarray(conv_state[s], dtype=np.float64)
        ext = np.concatenate([hist, x[cu[s]:cu[s + 1]]], axis=0)  # ext[3 + i] = token i
        for i in range(cu[s + 1] - cu[s]):
            acc = np.zeros(C)
            for j in range(4):
                acc += w[:, j] * ext[i + j]
            y[cu[s] + i] = _silu(acc)
        state_out[s] = ext[-3:]
        ext_all.append(ext)
    windows = np.zeros((len(ckpt_positions), 3, C))
    for i, p in enumerate(ckpt_positions):
        s = next(s for s in range(N) if cu[s] < p <= cu[s + 1])
        loc = int(p) - cu[s]
        windows[i] = ext_all[s][loc:loc + 3]
    return y, state_out, windows


def _seq_of_positions(cu, positions):
    """Map each checkpoint position p to (sequence s, local count p - cu[s])
    with cu[s] < p <= cu[s+1]."""
    res = {}
    for i, p in enumerate(positions):
        p = int(p)
        s = next(s for s in range(len(cu) - 1) if cu[s] < p <= cu[s + 1])
        res.setdefault(s, []).append((p - cu[s], i))
    return res


# -------------------------------------------------------- recurrent oracle --

def prefill_recurrent(q, k, v, g, beta, cu_seqlens, init=None, ckpt_positions=(),
                      scale: float = 1.0, l2norm: bool = True, eps: float = DEFAULT_EPS):
    """Token-by-token gated delta rule over a pack (the definition).

    q, k: [T, Hqk, dk]; v: [T, Hv, dv]; g (log-gate), beta: [T, Hv]; all
    float64.  init: [N, Hv, dv, dk] or None.  Returns (out [T, Hv, dv],
    final [N, Hv, dv, dk], ckpt [n_ckpt, Hv, dv, dk]).  Pinned by the
    beta = 0 / g = 0 closed forms, orthonormal-key overwrite, the scalar case
    worked by hand, linearity, row independence and prefix continuation.
    """
    cu = [int(x) for x in cu_seqlens]
    T, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    grp = Hv // Hqk
    N = len(cu) - 1
    out = np.zeros((T, Hv, dv))
    final = np.zeros((N, Hv, dv, dk))
    ckpt = np.zeros((len(ckpt_positions), Hv, dv, dk))
    where = _seq_of_positions(cu, ckpt_positions)
    for s in range(N):
        S = np.zeros((Hv, dv, dk)) if init is None else np.array(init[s], dtype=np.float64)
        marks = dict(where.get(s, []))
        for t in range(cu[s], cu[s + 1]):
            kt, qt = k[t], q[t]
            if l2norm:
                kt = kt * l2_rnorm(kt, eps)[:, None]
                qt = qt * l2_rnorm(qt, eps)[:, None]
            kh = np.repeat(kt, grp, axis=0)          # value head h reads qk head h // grp
            qh = np.repeat(qt, grp, axis=0)
            alpha = np.exp(g[t])[:, None, None]
            b = beta[t][:, None, None]
            Sk = np.matmul(S, kh[:, :, None])        # S k          [Hv, dv, 1]
            S = alpha * (S - b * Sk * kh[:, None, :]) + b * v[t][:, :, None] * kh[:, None, :]
            out[t] = scale * np.matmul(S, qh[:, :, None])[:, :, 0]
            loc = t + 1 - cu[s]
            if loc in marks:
                ckpt[marks[loc]] = S
        final[s] = S
    return out, final, ckpt


def decode_step(q, k, v, g, beta, state, slot=None, scale: float = 1.0,
                l2norm: bool = True, eps: float = DEFAULT_EPS):
    """One recurrent step for each of B sequences on state[slot[b]].

    q, k: [B, Hqk, dk]; v: [B, Hv, dv]; g, beta: [B, Hv]; state: [P, Hv, dv, dk].
    Returns (out [B, Hv, dv], new_state) with new_state a copy of the pool
    where the addressed rows advanced one token.  Defined as a one-token
    prefill from the slot's state (pinned against ``prefill_recurrent``).
    """
    B = q.shape[0]
    slot = np.arange(B) if slot is None else np.asarray(slot)
    new_state = np.array(state, dtype=np.float64)
    cu = np.arange(B + 1)
    out, fin, _ = prefill_recurrent(q, k, v, g, beta, cu, init=new_state[slot], scale=scale,
                                    l2norm=l2norm, eps=eps)
    new_state[slot] = fin
    return out, new_state


def decode_tokens(q, k, v, g, beta, state, n_tok: int, slot=None, scale: float = 1.0,
                  l2norm: bool = True, eps: float = DEFAULT_EPS):
    """n_tok recurrent steps for each of B sequences on state[slot[b]], with
    the state after every token kept (speculative or multi-token-prediction
    verification, rolled back by restoring a kept state).

    q, k: [B * n_tok, Hqk, dk]; v: [B * n_tok, Hv, dv]; g, beta: [B * n_tok,
    Hv], sequence-major (row b * n_tok + i).  Returns (out [B * n_tok, Hv, dv],
    new_state, snapshots [B, n_tok, Hv, dv, dk]) with snapshot i the state
    after token i + 1 and the addressed pool rows at the state after the last
    token.  Defined as a prefill of each sequence's n_tok tokens from its slot
    state with a checkpoint after every token.
    """
    B = q.shape[0] // n_tok
    slot = np.arange(B) if slot is None else np.asarray(slot)
    new_state = np.array(state, dtype=np.float64)
    cu = np.arange(B + 1) * n_tok
    marks = [int(cu[b] + i) for b in range(B) for i in range(1, n_tok + 1) if i < n_tok]
    out, fin, ck = prefill_recurrent(q, k, v, g, beta, cu, init=new_state[slot], ckpt_positions=marks,
                                     scale=scale, l2norm=l2norm, eps=eps)
    Hv, dv, dk = fin.shape[1:]
    snaps = np.zeros((B, n_tok, Hv, dv, dk))
    if n_tok > 1:
        snaps[:, :n_tok - 1] = ck.reshape(B, n_tok - 1, Hv, dv, dk)
    snaps[:, n_tok - 1] = fin
    new_state[slot] = fin
    return out, new_state, snaps


# ---------------------------------------------------------- chunked oracle --

def prefill_chunked(q, k, v, g, beta, cu_seqlens, chunk, init=None, ckpt_positions=(),
                    scale: float = 1.0, l2norm: bool = True, eps: float = DEFAULT_EPS):
    """The same map in chunked WY/UT form, chunks restarting at every prompt.

    Independent of ``prefill_recurrent`` (no shared code beyond the L2 norm
    scalars); agrees with it to ~1e-14 in fp64 (pin P-6).  Checkpoints must
    sit on chunk boundaries of their prompt.
    """
    cu = [int(x) for x in cu_seqlens]
    T, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    grp = Hv // Hqk
    N = len(cu) - 1
    if l2norm:
        qn = q * l2_rnorm(q, eps)[..., None]
        kn = k * l2_rnorm(k, eps)[..., None]
    else:
        qn, kn = q, k
    out = np.zeros((T, Hv, dv))
    final = np.zeros((N, Hv, dv, dk))
    ckpt = np.zeros((len(ckpt_positions), Hv, dv, dk))
    where = _seq_of_positions(cu, ckpt_positions)
    for s in range(N):
        marks = dict(where.get(s, []))
        L = cu[s + 1] - cu[s]
        if any(m % chunk != 0 and m != L for m in marks):
            raise ValueError("checkpoint not on a chunk boundary of its prompt")
        for h in range(Hv):
            j = h // grp
            S = np.zeros((dv, dk)) if init is None else np.array(init[s, h], dtype=np.float64)
            for c0 in range(cu[s], cu[s + 1], chunk):
                c1 = min(c0 + chunk, cu[s + 1])
                n = c1 - c0
                K, Q, V = kn[c0:c1, j], qn[c0:c1, j], v[c0:c1, h]
                bt = beta[c0:c1, h]
                G = np.cumsum(g[c0:c1, h])
                D = np.exp(G[:, None] - G[None, :])
                A = np.tril(bt[:, None] * D * (K @ K.T), -1)
                Tm = scipy.linalg.solve_triangular(np.eye(n) + A, np.eye(n), lower=True,
                                                   unit_diagonal=True)
                W = Tm @ ((bt * np.exp(G))[:, None] * K)
                U = Tm @ (bt[:, None] * V) - W @ S.T
                out[c0:c1, h] = scale * (np.exp(G)[:, None] * (Q @ S.T)
                                         + (np.tril(D) * (Q @ K.T)) @ U)
                S = np.exp(G[-1]) * S + U.T @ (np.exp(G[-1] - G)[:, None] * K)
                loc = c1 - cu[s]
                if loc in marks:
                    ckpt[marks[loc], h] = S
            final[s, h] = S
    return out, final, ckpt


# ------------------------------------------------------------- comparators --

def rel_frobenius(x: np.ndarray, ref: np.ndarray, axes=(-2, -1)) -> np.ndarray:
    """||x - ref||_F / ||ref||_F over ``axes`` (absolute norm where ref = 0)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(np.sum((x - ref) ** 2, axis=axes))
    den = np.sqrt(np.sum(ref ** 2, axis=axes))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def max_rel_rows(x: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per row (last axis): max |x - ref| / max |ref| (absolute if ref row = 0)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(x - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


__all__ = [
    "DEFAULT_EPS", "bf16_to_f64", "to_f64", "round_bf16", "l2_rnorm", "plan_checkpoints",
    "conv1d_silu_packed", "prefill_recurrent", "prefill_chunked", "decode_step", "decode_tokens",
    "rel_frobenius", "max_rel_rows",
]
