"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, its planner equals the oracle's, and every validation error
is returned from the host before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import gated_deltanet_prefill_varlen_amd as gdn
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

# Fake device addresses (16-byte aligned) used only in calls that must fail
# validation; never run where a GPU is present.
FAKE = 0x100000
no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="host-validation probes with fake device pointers run only without a GPU")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"GDN_API\s+[\w\s\*]+?\b(gdn_\w+)\s*\(", text)))


def test_header_declares_exactly_the_exported_symbols():
    assert declared_symbols() == sorted(gdn.EXPORTED)


def test_library_loads_and_exports_every_declared_symbol():
    lib = gdn.load()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert gdn.gdn_status_string(0) == "GDN_OK"
    for code in range(1, 8):
        assert gdn.gdn_status_string(code).startswith(gdn.STATUS[code])
    assert "unknown" in gdn.gdn_status_string(99)


def test_planner_matches_oracle_planner():
    rng = np.random.default_rng(0)
    for block in (16, 32, 64, 256, 1024):
        for trial in range(40):
            n = int(rng.integers(0, 9))
            lens = rng.integers(0, 5 * block + 40, size=n)
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            p0 = (rng.integers(0, 4, size=n) * block).astype(np.int32)
            for pz in (None, p0):
                got = gdn.gdn_plan_checkpoints(cu, block, 16, pz)
                want = O.plan_checkpoints(cu, block, 16, p0=pz)
                np.testing.assert_array_equal(got, want)


@no_gpu
def test_planner_output_passes_validation_with_p0_off_the_chunk_grid():
    """A prompt continued from an absolute position p0 that is not a
    multiple of the chunk (a prompt cut by the pass's token budget and
    resumed in the next pass) gets checkpoints off its chunk grid; the
    planner's list is accepted as it is."""
    cu = np.array([0, 300], np.int32)
    ck = gdn.gdn_plan_checkpoints(cu, 256, 16, np.array([137], np.int32))
    np.testing.assert_array_equal(ck, [119])
    assert 119 % 16 != 0
    sh = gdn.make_shape(2, 2, 32, 32, 16, gdn.GDN_F32)
    assert _prefill_call(sh, cu=tuple(cu), ck=tuple(ck)) == 7   # validated; no device to launch on
    rng = np.random.default_rng(5)
    for trial in range(50):
        lens = rng.integers(0, 700, size=int(rng.integers(1, 6)))
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        p0 = rng.integers(0, 2000, size=len(lens)).astype(np.int32)
        ck = gdn.gdn_plan_checkpoints(cu, 256, 16, p0)
        np.testing.assert_array_equal(ck, O.plan_checkpoints(cu, 256, 16, p0=p0))
        if len(ck):
            assert _prefill_call(sh, cu=tuple(cu), ck=tuple(ck)) == 7


def test_planner_errors_and_capacity():
    lib = gdn.load()
    cu = np.array([0, 1024, 2048], np.int32)
    n = ctypes.c_int32(-1)
    out = np.zeros(2, np.int32)
    st = lib.gdn_plan_checkpoints(cu.ctypes.data, 2, None, 256, 16, out.ctypes.data, 2, ctypes.byref(n))
    assert st == 6 and n.value == 6 and list(out) == [256, 512]
    assert lib.gdn_plan_checkpoints(cu.ctypes.data, 2, None, 0, 16, None, 0, ctypes.byref(n)) == 2
    bad = np.array([0, 10, 5], np.int32)
    assert lib.gdn_plan_checkpoints(bad.ctypes.data, 2, None, 16, 16, None, 0, ctypes.byref(n)) == 4
    assert lib.gdn_plan_checkpoints(None, 2, None, 16, 16, None, 0, ctypes.byref(n)) == 1


def _prefill_call(shape=None, cu=(0, 40, 64), T=None, ck=(), ptr=FAKE, ckbuf=True, q=None, out=None):
    lib = gdn.load()
    shape = shape if shape is not None else gdn.make_shape(2, 2, 32, 32, 16, gdn.GDN_F32)
    cu = np.asarray(cu, np.int32)
    T = int(cu[-1]) if T is None else T
    ck = np.asarray(ck, np.int32)
    q = ptr if q is None else q
    return lib.gdn_prefill_packed(ctypes.byref(shape) if shape is not False else None, ptr,
                                  cu.ctypes.data, len(cu) - 1, T, q, ptr, ptr, ptr, ptr, None,
                                  ptr if len(ck) else None, ck.ctypes.data if len(ck) else None,
                                  len(ck), ptr if out is None else out, ptr,
                                  ptr if (ckbuf and len(ck)) else None, None)


@no_gpu
def test_prefill_validation_errors():
    S = lambda **kw: gdn.make_shape(**{**dict(Hqk=2, Hv=2, dk=32, dv=32, chunk=16,
                                              io_dtype=gdn.GDN_F32), **kw})
    assert _prefill_call(shape=False) == 1
    assert _prefill_call(S(Hqk=2, Hv=3)) == 3
    assert _prefill_call(S(dk=48)) == 3
    assert _prefill_call(S(dv=256)) == 3
    assert _prefill_call(S(chunk=128)) == 3
    assert _prefill_call(S(io_dtype=5)) == 3
    sh = S(); sh.flags = 2
    assert _prefill_call(sh) == 3
    sh = S(); sh.l2_eps = -1.0
    assert _prefill_call(sh) == 2
    assert _prefill_call(S(Hqk=0)) == 2
    assert _prefill_call(cu=(1, 40, 64)) == 4
    assert _prefill_call(cu=(0, 40, 30)) == 4
    assert _prefill_call(cu=(0, 40, 64), T=65) == 4
    assert _prefill_call(q=0) == 1
    assert _prefill_call(ck=(32, 16)) == 5          # not increasing
    # any position inside a prompt passes validation (the scan ends a chunk
    # there); without a GPU the call then fails at its launch (GDN_ERR_HIP)
    assert _prefill_call(ck=(8,)) == 7
    assert _prefill_call(ck=(40, 41)) == 7
    assert _prefill_call(ck=(0,)) == 5              # not inside a prompt
    assert _prefill_call(ck=(80,)) == 5             # past the pack
    assert _prefill_call(ck=(16,), ckbuf=False) == 1
    assert _prefill_call(out=FAKE + 4) == 2         # misaligned
    assert _prefill_call(S(q_tok_stride=32)) == 2   # shorter than one token row
    assert _prefill_call(S(k_tok_stride=65)) == 2   # rows not 16-byte aligned
    assert _prefill_call(S(v_tok_stride=1 << 23)) == 2   # past the 32-bit row offsets


def test_empty_pack_is_ok_without_any_launch():
    assert _prefill_call(cu=(0,)) == 0


@no_gpu
def test_decode_validation_errors():
    lib = gdn.load()
    sh = gdn.make_shape(2, 4, 32, 32, 16)
    def call(batch=3, pool=5, slot=None, cw=None, cs=None):
        sl = None if slot is None else np.asarray(slot, np.int32)
        return lib.gdn_decode_step(ctypes.byref(sh), batch, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, pool,
                                   FAKE if sl is not None else None,
                                   sl.ctypes.data if sl is not None else None, FAKE, cw, cs, None)
    assert call(batch=0) == 0
    assert call(batch=6, pool=5) == 6
    assert call(slot=[0, 1, 1]) == 6
    assert call(slot=[0, 1, 5]) == 6
    assert call(slot=[0, -1, 2]) == 6
    assert call(pool=1 << 40, slot=[0, 7, 7]) == 6   # a huge pool: the check is O(batch) on the host
    assert call(cw=FAKE) == 1                       # conv weights without conv states
    assert call(cs=FAKE) == 1                       # and the other way round
    assert call(cw=FAKE, cs=FAKE + 4) == 2          # misaligned conv state
    assert lib.gdn_decode_step(ctypes.byref(sh), 3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 5, FAKE, None,
                               FAKE, None, None, None) == 1
    assert lib.gdn_decode_step(ctypes.byref(sh), 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, 5, None, None,
                               FAKE, None, None, None) == 1
    assert lib.gdn_decode_tokens(ctypes.byref(sh), 3, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 5, None,
                                 None, FAKE, None, None, None, None) == 2


@no_gpu
def test_snapshot_and_conv_validation_errors():
    lib = gdn.load()
    sl = np.array([0, 2, 2], np.int64)
    assert lib.gdn_snapshot_copy(FAKE, 3, 64, FAKE, 4, FAKE, sl.ctypes.data, None, None, None) == 6
    sl = np.array([0, 2, 4], np.int64)
    assert lib.gdn_snapshot_copy(FAKE, 3, 64, FAKE, 4, FAKE, sl.ctypes.data, None, None, None) == 6
    sl = np.array([0, 2, 3], np.int64)
    assert lib.gdn_snapshot_copy(FAKE, 3, 60, FAKE, 4, FAKE, sl.ctypes.data, None, None, None) == 2
    assert lib.gdn_snapshot_copy(FAKE, 3, 64, None, 4, FAKE, sl.ctypes.data, None, None, None) == 1
    assert lib.gdn_snapshot_copy(FAKE, 0, 64, None, 4, None, None, None, None, None) == 0
    sl = np.array([5, 5], np.int64)   # a huge pool: the slot check needs no pool-sized memory
    assert lib.gdn_snapshot_copy(FAKE, 2, 64, FAKE, 1 << 40, FAKE, sl.ctypes.data, None, None, None) == 6
    sh = gdn.make_shape(2, 2, 32, 32, 16, gdn.GDN_F32)
    cu = np.array([0, 40, 64], np.int32)
    # y overlapping x
    assert lib.gdn_conv1d_silu_packed(ctypes.byref(sh), FAKE, cu.ctypes.data, 2, 64, FAKE, 0, FAKE, None,
                                      FAKE + 192 * 4, 0, None, None, None, 0, None, None) == 2
    bad = np.array([0, 40, 63], np.int32)
    assert lib.gdn_conv1d_silu_packed(ctypes.byref(sh), FAKE, bad.ctypes.data, 2, 64, FAKE, 0, FAKE, None,
                                      FAKE * 64, 0, None, None, None, 0, None, None) == 4


@no_gpu
def test_fused_conv_prefill_validation_errors():
    lib = gdn.load()
    cu = np.array([0, 40, 64], np.int32)
    C = 2 * 2 * 128 + 4 * 128          # conv_dim at Hqk 2, Hv 4, d 128
    def call(sh=None, cu=cu, T=64, x=FAKE, w=FAKE, out=1 << 32, ck=(), ckbuf=True, xs=0, st_in=None,
             st_out=None):
        sh = sh if sh is not None else gdn.make_shape(2, 4, 128, 128, 64)
        ck = np.asarray(ck, np.int32)
        return lib.gdn_prefill_conv_packed(
            ctypes.byref(sh), FAKE, cu.ctypes.data, len(cu) - 1, T, x, xs, w, st_in, st_out, FAKE, FAKE,
            None, FAKE if len(ck) else None, ck.ctypes.data if len(ck) else None, len(ck), None, out,
            None, FAKE if (ckbuf and len(ck)) else None, None)
    # only the fused kernel's shape: bf16, d_k = d_v = 128, 32-token tiles
    assert call(gdn.make_shape(2, 4, 64, 64, 64)) == 3
    assert call(gdn.make_shape(2, 4, 128, 64, 64)) == 3
    assert call(gdn.make_shape(2, 4, 128, 128, 16)) == 3
    assert call(gdn.make_shape(2, 4, 128, 128, 64, gdn.GDN_F32)) == 3
    assert call(gdn.make_shape(2, 3, 128, 128, 64)) == 3
    assert call(x=None) == 1
    assert call(w=None) == 1
    assert call(out=None) == 1
    assert call(cu=np.array([0, 40, 63], np.int32)) == 4
    assert call(ck=(40, 40)) == 5
    assert call(ck=(16,), ckbuf=False) == 1
    assert call(xs=C - 8) == 2                      # shorter than a row
    assert call(xs=C + 4) == 2                      # rows not 16-byte aligned
    assert call(x=FAKE + 8) == 2                    # misaligned
    assert call(st_in=FAKE + 4) == 2
    assert call(out=FAKE + 64 * C) == 2             # out overlapping x's last row
    assert call(cu=np.array([0], np.int32), T=0) == 0   # an empty pack: nothing to do


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(gdn, "_lib", None)
    monkeypatch.setattr(gdn, "LIB_PATH", "/nonexistent/libgdn.so")
    with pytest.raises(RuntimeError, match="not built"):
        gdn.load()
