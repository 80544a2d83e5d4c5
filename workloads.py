"""Seeded synthetic inputs for packed gated-delta-rule prefill and decode.

The shapes follow the serving workloads the sources describe: waves of about
32 chat prompts of 1,024 tokens prefilled in shared packed passes, 8K-token
prompts, ragged packs that save prefix-cache checkpoints, and mixed passes that
carry up to 1,024 prompt tokens from at most 8 waiting prompts (oldest first)
beside a batch of decoding requests (sparkinfer release v0.6.28, intro and
"Measured"; sparkinfer release v0.6.4, "What changed").  No public dataset is
involved: the layer only ever sees tensor shapes, so every value is drawn here.

This module is shared by the tests, the benchmark and the oracle-side checks.
It holds none of the method's arithmetic: it draws numbers, encodes them in the
storage dtype (bf16 round-to-nearest-even bit patterns) and lays out packs.
The q/k directions of the bf16 workloads are drawn uniformly on the unit
sphere (a normal vector divided by its length) because the workloads specify
unit-length q and k; the layer's own L2 normalisation is not done here.

Draw order inside one workload (one ``numpy.random.default_rng(seed)``):
lengths, q, k, v, z_g, z_beta, init, conv weight, x.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


# ---------------------------------------------------------------- encoding --

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the fp32 values they encode (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------- packs --

@dataclass
class Pack:
    """One packed pass: N prompts laid end to end, ``cu_seqlens`` marks them.

    q, k: [T, Hqk, dk]; v: [T, Hv, dv]; g, beta: [T, Hv] fp32.  For
    ``dtype == "bf16"`` q/k/v hold uint16 bf16 bit patterns, otherwise fp32.
    init: [N, Hv, dv, dk] fp32 or None (zero state).  x: [T, conv_dim] pre-conv
    inputs (channels ordered q | k | v) and conv_w: [conv_dim, 4] when the
    workload includes the short convolution.
    """
    name: str
    cu_seqlens: np.ndarray
    Hqk: int
    Hv: int
    dk: int
    dv: int
    chunk: int
    block: int
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    init: Optional[np.ndarray] = None
    conv_w: Optional[np.ndarray] = None
    x: Optional[np.ndarray] = None
    p0: Optional[np.ndarray] = None
    scale: float = 1.0
    extra: dict = field(default_factory=dict)

    @property
    def n_seqs(self) -> int:
        return int(len(self.cu_seqlens) - 1)

    @property
    def n_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens)

    @property
    def conv_dim(self) -> int:
        return 2 * self.Hqk * self.dk + self.Hv * self.dv


@dataclass
class DecodeBatch:
    """B sequences each advancing one token from a carried fp32 state.

    q, k: [B, Hqk, dk]; v: [B, Hv, dv] (bf16 bits or fp32); g, beta: [B, Hv];
    state: [P, Hv, dv, dk] pool; slot: [B] int32 rows of the pool (distinct).
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    state: np.ndarray
    slot: np.ndarray
    Hqk: int
    Hv: int
    dk: int
    dv: int
    dtype: str
    scale: float = 1.0

    @property
    def batch(self) -> int:
        return int(self.slot.shape[0])


def _cu(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def _normal(rng, shape, std=1.0):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _unit_rows(a: np.ndarray) -> np.ndarray:
    """Rows scaled to length one: a normal draw divided by its length is
    uniform on the sphere (distribution recipe, computed in fp32)."""
    n = np.sqrt(np.sum(a.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (a / n).astype(np.float32)


def _log_gate(z: np.ndarray) -> np.ndarray:
    """Log-gate draw: minus a softplus of a standard normal (always <= 0)."""
    z = z.astype(np.float32)
    return (-(np.maximum(z, 0) + np.log1p(np.exp(-np.abs(z))))).astype(np.float32)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float32)
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def make_pack(name, lengths, Hqk, Hv, dk, dv, chunk, block, dtype="bf16", seed=0,
              init_std=0.0, unit_qk=True, gate_scale=1.0, with_conv=False,
              conv_std=0.5, scale=1.0, p0=None) -> Pack:
    """Draw one pack in the fixed order lengths, q, k, v, z_g, z_beta, init,
    conv weight, x.  ``lengths`` is a list or a callable(rng) -> list."""
    rng = np.random.default_rng(seed)
    if callable(lengths):
        lengths = lengths(rng)
    lengths = [int(x) for x in lengths]
    cu = _cu(lengths)
    T, N = int(cu[-1]), len(lengths)
    q = _normal(rng, (T, Hqk, dk))
    k = _normal(rng, (T, Hqk, dk))
    v = _normal(rng, (T, Hv, dv))
    zg = _normal(rng, (T, Hv))
    zb = _normal(rng, (T, Hv))
    init = _normal(rng, (N, Hv, dv, dk), init_std) if init_std > 0 else None
    conv_w = x = None
    if with_conv:
        conv_dim = 2 * Hqk * dk + Hv * dv
        conv_w = _normal(rng, (conv_dim, 4), conv_std)
        # the drawn q | k | v (before any normalisation) are the conv inputs
        x = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)
    if unit_qk:
        q, k = _unit_rows(q), _unit_rows(k)
    g = (_log_gate(zg) * np.float32(gate_scale)).astype(np.float32)
    beta = _sigmoid(zb)
    if dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
        if x is not None:
            x = f32_to_bf16_bits(x)
    elif dtype != "f32":
        raise ValueError(dtype)
    return Pack(name=name, cu_seqlens=cu, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, chunk=chunk,
                block=block, dtype=dtype, q=q, k=k, v=v, g=g, beta=beta, init=init,
                conv_w=conv_w, x=x, scale=scale,
                p0=None if p0 is None else np.asarray(p0, dtype=np.int32))


# --------------------------------------------------------- named workloads --

def tiny_pack(seed=0) -> Pack:
    """2 prompts (40 and 24 tokens), 2 qk / 2 v heads, dk = dv = 32, fp32,
    chunk 16, checkpoint block 16, width-4 conv with std-0.5 weights."""
    return make_pack("tiny", [40, 24], 2, 2, 32, 32, 16, 16, dtype="f32", seed=seed,
                     with_conv=True, conv_std=0.5)


def chat_wave(seed=0, n_prompts=32, prompt_len=1024, with_conv=False) -> Pack:
    """32 x 1,024-token chat prompts, 16 qk / 32 v heads, d = 128, bf16,
    zero initial state, chunk 64, checkpoint every 256 tokens; with_conv adds
    the pre-conv rows x (q | k | v as drawn) and std-0.5 conv weights."""
    return make_pack("chat_wave_32x1024", [prompt_len] * n_prompts, 16, 32, 128, 128, 64, 256,
                     seed=seed, with_conv=with_conv, conv_std=0.5)


def _ragged_lengths(n=8, lo=17, hi=2048, cap=8192):
    def draw(rng):
        while True:  # redraw the whole vector until the pack fits the cap
            ls = rng.integers(lo, hi + 1, size=n)
            if int(ls.sum()) <= cap:
                return [int(x) for x in ls]
    return draw


def ragged_pack(seed=0) -> Pack:
    """8 prompts with lengths uniform in [17, 2048] (total <= 8,192), non-zero
    fp32 initial states (std 0.1) from a prefix cache, checkpoint every 256."""
    return make_pack("ragged_8_prefix_cache", _ragged_lengths(), 16, 32, 128, 128, 64, 256,
                     seed=seed, init_std=0.1)


def long_prompts(seed=0) -> Pack:
    """4 x 8,192-token prompts, checkpoint every 1,024 tokens."""
    return make_pack("long_4x8192", [8192] * 4, 16, 32, 128, 128, 64, 1024, seed=seed)


def mixed_fill(rng, budget=1024, max_prompts=8, lo=64, hi=512):
    """Waiting prompts in arrival order fill the prompt-token budget, oldest
    first; the last one admitted is cut to what is left of the budget."""
    waiting = [int(x) for x in rng.integers(lo, hi + 1, size=max_prompts)]
    taken, left = [], budget
    for L in waiting:
        if left == 0 or len(taken) == max_prompts:
            break
        taken.append(min(L, left))
        left -= taken[-1]
    return taken


def mixed_step(seed=0, n_decode=32):
    """A mixed pass: a 1,024-token prefill pack (<= 8 prompts, lengths uniform
    in [64, 512]) plus ``n_decode`` sequences advancing one token each from
    carried fp32 states (std 0.1).  Returns (Pack, DecodeBatch)."""
    pack = make_pack("mixed_1024_plus_32_decode", mixed_fill, 16, 32, 128, 128, 64, 256, seed=seed)
    dec = decode_batch(seed=seed + 1000, batch=n_decode)
    return pack, dec


def decode_batch(seed=0, batch=32, Hqk=16, Hv=32, dk=128, dv=128, dtype="bf16", pool=None,
                 state_std=0.1, unit_qk=True, scale=1.0) -> DecodeBatch:
    """One decode token for each of ``batch`` sequences, states in a pool of
    ``pool`` slots (default: exactly ``batch``) addressed by a permutation."""
    rng = np.random.default_rng(seed)
    P = batch if pool is None else pool
    q = _normal(rng, (batch, Hqk, dk))
    k = _normal(rng, (batch, Hqk, dk))
    v = _normal(rng, (batch, Hv, dv))
    zg = _normal(rng, (batch, Hv))
    zb = _normal(rng, (batch, Hv))
    state = _normal(rng, (P, Hv, dv, dk), state_std)
    slot = rng.permutation(P)[:batch].astype(np.int32)
    if unit_qk:
        q, k = _unit_rows(q), _unit_rows(k)
    if dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return DecodeBatch(q=q, k=k, v=v, g=_log_gate(zg), beta=_sigmoid(zb), state=state,
                       slot=slot, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv, dtype=dtype, scale=scale)


def every_residue_pack(seed=0, max_len=130, Hqk=2, Hv=4, d=32, chunk=16, dtype="bf16",
                       init_std=0.1, gate_scale=1.0) -> Pack:
    """Prompts of lengths 1 .. max_len packed together: every partial-chunk
    residue occurs, and many prompts start mid-way into a 16-token row."""
    return make_pack("every_residue", list(range(1, max_len + 1)), Hqk, Hv, d, d, chunk, chunk,
                     dtype=dtype, seed=seed, init_std=init_std, gate_scale=gate_scale)


def slow_decay(pack_fn, seed=0, **kw) -> Pack:
    """Same shapes with the log-gates scaled by 0.01 (slow decay), which keeps
    the initial state and the inter-chunk hand-off visible in the outputs."""
    p = pack_fn(seed=seed, **kw)
    p.g = (p.g * np.float32(0.01)).astype(np.float32)
    p.name += "_slow_decay"
    return p
