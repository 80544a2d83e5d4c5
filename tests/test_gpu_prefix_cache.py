"""Prefix-cache restore through the C ABI: checkpoints gathered on their own
stream into a pinned host pool allocated once, restored into init_state, and
the prompts continued from there.  A continuation from a checkpoint on the
chunk grid is bit-identical to the unbroken prefill: same chunk boundaries,
same inputs, and the state crosses the cut as the exact fp32 bits the
unbroken run carried (sparkinfer v0.6.28: pinned checkpoint buffers created
with the prefix cache, the alone-vs-packed check)."""
import ctypes

import numpy as np
import pytest
import torch

import gated_deltanet_prefill_varlen_amd as gdn
import workloads as W
from gpu_util import DevPack, DEV, assert_parity, sample_pairs

pytestmark = pytest.mark.gpu


def _device_address(pinned: torch.Tensor) -> int:
    """Device address of a pinned host tensor (hipHostGetDevicePointer); fails
    on the host, before any kernel runs, if the memory is not pinned."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                            ctypes.c_uint]
    d = ctypes.c_void_p()
    rc = hip.hipHostGetDevicePointer(ctypes.byref(d), ctypes.c_void_p(pinned.data_ptr()), 0)
    assert rc == 0 and d.value, f"hipHostGetDevicePointer returned {rc}"
    return d.value


def _suffix_pack(p, cuts):
    """The prompts of p continued from local offsets cuts (one per prompt)."""
    cu = p.cu_seqlens
    parts = [np.arange(cu[s] + cuts[s], cu[s + 1]) for s in range(p.n_seqs)]
    idx = np.concatenate(parts)
    lens = [len(x) for x in parts]
    return W.Pack(name="suffix", cu_seqlens=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
                  Hqk=p.Hqk, Hv=p.Hv, dk=p.dk, dv=p.dv, chunk=p.chunk, block=p.block, dtype=p.dtype,
                  q=p.q[idx], k=p.k[idx], v=p.v[idx], g=p.g[idx], beta=p.beta[idx],
                  init=None), idx


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_restore_from_pinned_pool_continues_bitwise(dk, dv):
    p = W.make_pack("prefix", [700, 513, 1024, 300], 2, 4, dk, dv, 64, 256, seed=21, init_std=0.1)
    ck = gdn.gdn_plan_checkpoints(p.cu_seqlens, p.block)
    dp = DevPack(p, ck).run()
    scan_done = torch.cuda.Event()
    scan_done.record()

    # pinned host pool, allocated once, more slots than checkpoints
    n = len(ck)
    each = p.Hv * p.dv * p.dk * 4
    pool = torch.zeros((n + 5, p.Hv, p.dv, p.dk), dtype=torch.float32, pin_memory=True)
    assert pool.is_pinned()
    slots = np.random.default_rng(1).permutation(n + 5)[:n].astype(np.int64)
    copy_stream = torch.cuda.Stream()
    done = torch.cuda.Event()
    gdn.gdn_snapshot_copy(dp.ckpt_buf, n, each, _device_address(pool), torch.from_numpy(slots).to(DEV),
                          slots, n + 5, wait_event=scan_done, copy_stream=copy_stream, done_event=done)
    assert done.cuda_event, "the copy-done event was left unrecorded"
    done.synchronize()
    ckpt_host = dp.ckpt_buf.cpu()
    assert torch.equal(pool[torch.from_numpy(slots)], ckpt_host)

    # continue every prompt from its first checkpoint, state restored from the pool
    cu = p.cu_seqlens
    first = {}
    for i, c in enumerate(ck):
        s = int(np.searchsorted(cu, c, side="right") - 1)
        first.setdefault(s, (i, int(c - cu[s])))
    assert sorted(first) == list(range(p.n_seqs))
    cuts = [first[s][1] for s in range(p.n_seqs)]
    sub, idx = _suffix_pack(p, cuts)
    sub_ck = gdn.gdn_plan_checkpoints(sub.cu_seqlens, p.block, p0_host=cuts)
    cont = DevPack(sub, sub_ck)
    cont.init = torch.empty((p.n_seqs, p.Hv, p.dv, p.dk), dtype=torch.float32, device=DEV)
    for s in range(p.n_seqs):                        # H2D from views of the pinned pool
        cont.init[s].copy_(pool[int(slots[first[s][0]])], non_blocking=True)
    cont.run()
    torch.cuda.synchronize()

    assert torch.equal(cont.out, dp.out[torch.from_numpy(idx).to(DEV)])
    assert torch.equal(cont.final, dp.final)
    # the continuation's checkpoints are the unbroken run's later ones
    later = [i for i, c in enumerate(ck)
             if c - cu[int(np.searchsorted(cu, c, side="right") - 1)] > cuts[
                 int(np.searchsorted(cu, c, side="right") - 1)]]
    assert len(sub_ck) == len(later)
    if later:
        assert torch.equal(cont.ckpt_buf, dp.ckpt_buf[later])
    assert_parity(dp, sample_pairs(p, 8, seed=2))
