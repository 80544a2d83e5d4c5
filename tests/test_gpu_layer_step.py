"""The whole hot path in the launch configuration the benchmark times, at the
chat wave's full size: the packed conv1d + SiLU from the pre-conv rows into
one [T, conv_dim] tensor (conv states, conv windows at the checkpoints), the
scan reading q, k, v as column views of it, and the checkpoint copy into a
device pool on its own stream.  Two steps run as consecutive layers: each
step's copy waits for an event from its scan and runs beside the next step's
work, the two steps writing alternate checkpoint buffers (the second with
other gates, so that a copy of the wrong buffer shows).  The second step is checked against the oracle's conv followed by
its token-by-token recurrence on 64 sampled (prompt, head) pairs (the conv
output rounded to bf16 as the tensor stores it); conv states, windows and
both pools are bit-exact (they are copies).

Tolerances: as the prefill tests (states 1e-3 relative Frobenius, bf16
outputs 2e-2 max-relative per row)."""
import numpy as np
import pytest
import torch

import gated_deltanet_prefill_varlen_amd as gdn
import workloads as W
from gpu_util import (DEV, compare_pairs, io_tensor, f32_tensor, i32_tensor, oracle_pairs, sample_pairs,
                      to_f64)

pytestmark = pytest.mark.gpu


def test_layer_step_chat_wave_sampled():
    p = W.chat_wave(seed=0, with_conv=True)
    T, N, Hqk, Hv, d = p.n_tokens, p.n_seqs, p.Hqk, p.Hv, p.dk
    C = 2 * Hqk * d + Hv * d
    ck = gdn.gdn_plan_checkpoints(p.cu_seqlens, p.block)
    n_ck = len(ck)
    x = io_tensor(p.x, "bf16")
    w = f32_tensor(p.conv_w)
    y = torch.empty_like(x)
    conv_state = torch.empty((N, 3, C), dtype=torch.bfloat16, device=DEV)
    conv_ckpt = torch.empty((n_ck, 3, C), dtype=torch.bfloat16, device=DEV)
    cu_d, ck_d = i32_tensor(p.cu_seqlens), i32_tensor(ck)
    out = torch.empty((T, Hv, d), dtype=torch.bfloat16, device=DEV)
    final = torch.empty((N, Hv, d, d), dtype=torch.float32, device=DEV)
    ckbufs = [torch.empty((n_ck, Hv, d, d), dtype=torch.float32, device=DEV) for _ in range(2)]
    pools = [torch.zeros((n_ck + 7, Hv, d, d), dtype=torch.float32, device=DEV) for _ in range(2)]
    slots = np.random.default_rng(3).permutation(n_ck + 7)[:n_ck].astype(np.int64)
    slots_d = torch.from_numpy(slots).to(DEV)
    shape = gdn.make_shape(Hqk, Hv, d, d, p.chunk, q_tok_stride=C, k_tok_stride=C, v_tok_stride=C)
    stream, cstream = torch.cuda.Stream(), torch.cuda.Stream()
    scan_done = [torch.cuda.Event(), torch.cuda.Event()]
    copy_done = [torch.cuda.Event(), torch.cuda.Event()]
    other = W.chat_wave(seed=1)
    gates = [(f32_tensor(p.g), f32_tensor(p.beta)), (f32_tensor(other.g), f32_tensor(other.beta))]

    def copy(b):
        gdn.gdn_snapshot_copy(ckbufs[b], n_ck, Hv * d * d * 4, pools[b], slots_d, slots, n_ck + 7,
                              wait_event=scan_done[b], copy_stream=cstream, done_event=copy_done[b])

    for b in range(2):
        gdn.gdn_conv1d_silu_packed(shape, cu_d, p.cu_seqlens, x, w, y, None, conv_state, ck_d, ck,
                                   conv_ckpt, stream=stream)
        gdn.gdn_prefill_packed(shape, cu_d, p.cu_seqlens, y[:, :Hqk * d], y[:, Hqk * d:2 * Hqk * d],
                               y[:, 2 * Hqk * d:], gates[b][0], gates[b][1], None, ck_d, ck, out,
                               final, ckbufs[b], stream=stream)
        scan_done[b].record(stream)
        copy(b)                            # beside the next step's conv
    stream.wait_event(copy_done[1])
    assert copy_done[0].cuda_event and copy_done[1].cuda_event, "copy-done events left unrecorded"
    torch.cuda.synchronize()

    for b in range(2):
        assert torch.equal(pools[b][slots_d], ckbufs[b])
    assert not torch.equal(ckbufs[0], ckbufs[1])
    ckbuf = ckbufs[1]
    g_np, beta_np = other.g, other.beta
    xb = torch.from_numpy(np.ascontiguousarray(p.x)).view(torch.bfloat16)
    cu = p.cu_seqlens
    for s in range(N):   # conv states: each prompt's last three inputs, copies of x
        assert torch.equal(conv_state[s].cpu(), xb[int(cu[s + 1]) - 3:int(cu[s + 1])])
    for i, c in enumerate(ck):   # conv windows: the three inputs before each checkpoint
        assert torch.equal(conv_ckpt[i].cpu(), xb[int(c) - 3:int(c)])

    pairs = sample_pairs(p, 64, seed=5)
    refs = oracle_pairs(p, pairs, ck, conv=True, g=g_np, beta=beta_np)
    worst_o, worst_s = compare_pairs(p, pairs, refs, to_f64(out), to_f64(final), to_f64(ckbuf), ck)
    print(f"layer step: out {worst_o:.2e} state {worst_s:.2e}")
