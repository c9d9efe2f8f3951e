"""C-ABI checks that need no GPU: the library loads, exports every function
include/la.h declares, and rejects bad arguments with the documented status
before touching the device."""
import ctypes
import os
import re

import pytest

import long_context_attention_chunkwise_amd as la
from long_context_attention_chunkwise_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la.h")

OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, WORKSPACE, TOO_LARGE = 0, 1, 2, 3, 4, 5, 6, 8
F32, BF16 = la.LA_F32, la.LA_BF16

# Fake, widely spaced, 16-byte aligned device addresses: validation only
# compares them, it never dereferences them.
GB = 1 << 40
Q, K, V, O, S_IN, S_OUT, WS, DO, DQ, DK, DV, DS = (ctypes.c_void_p(GB * i) for i in range(1, 13))


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return la.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == sorted(_lib.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    for code in range(9):
        s = lib.la_status_str(code).decode()
        assert s and (code == 0) == (s == "ok")
    assert lib.la_status_str(99).decode() == "unknown status"


def fwd(lib, q=Q, k=K, v=V, o=O, B=1, Hq=4, Hkv=1, N=1000, d=128, dv=128, block=64, i=BF16, out=BF16,
        s_in=None, s_out=None, ws=WS, ws_bytes=1 << 32):
    return lib.la_forward_ex(q, k, v, o, B, Hq, Hkv, N, d, dv, block, i, out, s_in, s_out, ws, ws_bytes, None)


def test_forward_validation(lib):
    assert fwd(lib, q=None) == NULL
    assert fwd(lib, o=None) == NULL
    assert fwd(lib, Hq=6, Hkv=4) == SHAPE
    assert fwd(lib, B=0) == SHAPE
    assert fwd(lib, N=-1) == SHAPE
    assert fwd(lib, d=64, dv=48) == UNSUP                # scalar kernels: dv a multiple of 32
    assert fwd(lib, d=256) == UNSUP                      # head sizes up to 128
    assert fwd(lib, block=96) == UNSUP                   # above 64 tokens, multiples of 64 only
    assert fwd(lib, block=(1 << 20) + 64) == UNSUP       # blocks of up to 2^20 tokens
    assert fwd(lib, B=1 << 12, Hq=1 << 12, Hkv=1 << 12, N=1 << 30) == UNSUP   # byte counts would overflow
    assert fwd(lib, B=1 << 40, Hq=1 << 40, Hkv=1 << 40, N=1) == UNSUP          # B * Hq itself would overflow
    assert fwd(lib, i=BF16, out=2) == UNSUP
    assert fwd(lib, i=F32, out=BF16) == UNSUP
    assert fwd(lib, i=F32, out=F32, dv=48) == UNSUP       # fp32 path: dv multiple of 32
    assert fwd(lib, i=F32, out=F32, block=65) == UNSUP
    assert fwd(lib, q=ctypes.c_void_p(GB + 8)) == ALIGN
    assert fwd(lib, s_out=ctypes.c_void_p(GB * 6 + 4)) == ALIGN
    assert fwd(lib, o=ctypes.c_void_p(GB + 4096)) == ALIAS    # o inside q
    # o == q (in place) only on the four-head matrix-core kernel, bf16 in and out
    assert fwd(lib, o=Q, i=F32, out=F32) == ALIAS
    assert fwd(lib, o=Q, out=F32) == ALIAS
    assert fwd(lib, o=Q, Hq=2, Hkv=1) == ALIAS
    assert fwd(lib, o=Q, d=64, dv=64, Hq=2, Hkv=1) == ALIAS   # head size 64: groups of four only
    assert fwd(lib, s_out=ctypes.c_void_p(GB * 3 + 64)) == ALIAS  # s_out inside v
    assert fwd(lib, ws=None) == WORKSPACE
    assert fwd(lib, ws_bytes=1024) == WORKSPACE
    assert fwd(lib, ws=ctypes.c_void_p(GB * 2 + 256)) == ALIAS  # workspace inside k


def test_decode_validation(lib):
    def dec(S=S_IN, q=Q, k=K, v=V, o=O, B=2, Hq=8, Hkv=2, d=128, dv=128, i=BF16, out=F32):
        return lib.la_decode_step(S, q, k, v, o, B, Hq, Hkv, d, dv, i, out, None)
    assert dec(S=None) == NULL
    assert dec(Hq=6, Hkv=4) == SHAPE
    assert dec(dv=126) == UNSUP
    assert dec(Hq=2050, Hkv=2) == UNSUP                   # more than 1024 query heads per KV head
    assert dec(B=1 << 40, Hq=1 << 40, Hkv=1 << 40) == UNSUP   # no overflow in the size checks
    assert dec(o=ctypes.c_void_p(GB * 4 + 2)) == ALIGN
    assert dec(o=ctypes.c_void_p(GB * 5 + 16)) == ALIAS   # o inside S


def bwd(lib, q=Q, k=K, v=V, do=DO, dq=DQ, dk=DK, dv=DV, B=1, Hq=4, Hkv=1, N=1000, d=128, dvs=128, block=64,
        i=BF16, g=BF16, s_in=S_IN, ds_out=S_OUT, ds_in=DS, ws=WS, ws_bytes=1 << 32):
    return lib.la_backward(q, k, v, do, dq, dk, dv, B, Hq, Hkv, N, d, dvs, block, i, g, s_in, ds_out, ds_in, ws,
                           ws_bytes, None)


def test_backward_validation(lib):
    assert bwd(lib, do=None) == NULL
    assert bwd(lib, dk=None) == NULL
    assert bwd(lib, Hq=6, Hkv=4) == SHAPE
    assert bwd(lib, N=-1) == SHAPE
    assert bwd(lib, i=F32, g=BF16) == UNSUP                # float32 inputs take float32 gradients
    assert bwd(lib, i=F32, g=F32, d=48, dvs=64) == UNSUP   # float32: d a multiple of 32
    assert bwd(lib, i=F32, g=F32, d=64, dvs=64, block=96) == UNSUP    # float32: above 64, multiples of 64 only
    assert bwd(lib, i=F32, g=F32, d=64, dvs=64, ws=None) == WORKSPACE
    assert bwd(lib, d=48) == UNSUP                         # scalar kernels: d a multiple of 32
    assert bwd(lib, g=2) == UNSUP
    assert bwd(lib, dq=ctypes.c_void_p(GB * 9 + 8)) == ALIGN
    assert bwd(lib, dq=ctypes.c_void_p(GB * 1 + 4096)) == ALIAS       # dq inside q
    assert bwd(lib, dv=ctypes.c_void_p(GB * 9 + 4096)) == ALIAS       # dv inside dq
    assert bwd(lib, ds_in=ctypes.c_void_p(GB * 6 + 64)) == ALIAS      # partial overlap with ds_out
    assert bwd(lib, ds_in=ctypes.c_void_p(GB * 8 + 64)) == ALIAS      # ds_in inside dO
    assert bwd(lib, ws=None) == WORKSPACE
    assert bwd(lib, ws_bytes=1024) == WORKSPACE
    assert bwd(lib, ws=ctypes.c_void_p(GB * 10 + 256)) == ALIAS       # workspace inside dk


def var(lib, q=Q, k=K, v=V, o=O, B=1, Hq=4, Hkv=1, N=1000, d=128, dv=128, block=64, i=BF16, out=BF16, causal=1,
        fmap=1, norm=1, eps=1e-6, s_in=None, s_out=None, z_in=None, z_out=None, ws=WS, ws_bytes=1 << 32):
    return lib.la_forward_variant(q, k, v, o, B, Hq, Hkv, N, d, dv, block, i, out, causal, fmap, norm, eps, s_in,
                                  s_out, z_in, z_out, ws, ws_bytes, None)


def test_variant_validation(lib):
    assert var(lib, q=None) == NULL
    assert var(lib, Hq=6, Hkv=4) == SHAPE
    assert var(lib, d=64, dv=48) == UNSUP                 # scalar kernels: dv a multiple of 32
    assert var(lib, i=F32, out=BF16) == UNSUP             # float32 inputs give float32 outputs
    assert var(lib, i=F32, out=F32, d=64, dv=48) == UNSUP  # float32: dv a multiple of 32
    assert lib.la_forward_variant_workspace_bytes(1, 4, 1, 1000, 64, 64, 64, F32, 0, 1) == 0   # float32: none
    assert var(lib, fmap=2) == UNSUP
    assert var(lib, causal=2) == UNSUP
    assert var(lib, eps=-1.0) == UNSUP
    assert var(lib, eps=float("nan")) == UNSUP
    assert var(lib, norm=0, z_out=DS) == UNSUP            # normaliser sums only when normalising
    assert var(lib, z_out=ctypes.c_void_p(GB * 12 + 4)) == ALIGN
    assert var(lib, z_out=ctypes.c_void_p(GB * 3 + 512)) == ALIAS    # z_out inside v
    assert var(lib, s_out=ctypes.c_void_p(GB * 4 + 64)) == ALIAS     # s_out inside o
    assert var(lib, ws=None) == WORKSPACE
    assert var(lib, ws=ctypes.c_void_p(GB * 1 + 256)) == ALIAS       # workspace inside q


def test_workspace_plan(lib):
    # Host planning with the default 256 compute units (no device here): the
    # 1M-token GQA problem splits each of the 32 chains into 8 segments and
    # every segment but the last into 2 pre-pass parts (448 pre-pass
    # workgroups: one round at two per compute unit at head size 128).
    n = lib.la_forward_workspace_bytes(1, 128, 32, 1 << 20, 128, 128, 64, BF16)
    assert n == (32 * 7 * 2 + 32 * 8) * 128 * 128 * 4
    assert lib.la_forward_workspace_bytes(1, 1, 1, 256, 64, 64, 64, F32) == 0
    # a block that is a multiple of 64 tokens is computed as 64-token blocks: same plan
    for blk in (128, 4096):
        assert lib.la_forward_workspace_bytes(1, 128, 32, 1 << 20, 128, 128, blk, BF16) == n
        assert lib.la_backward_workspace_bytes(1, 128, 32, 1 << 20, 128, 128, blk, BF16) == \
            lib.la_backward_workspace_bytes(1, 128, 32, 1 << 20, 128, 128, 64, BF16)
    assert lib.la_forward_workspace_bytes(1, 128, 32, 1 << 20, 128, 128, 96, BF16) == 0   # unsupported -> 0
    # head size 64 on the matrix cores for every group size (three pre-pass workgroups per compute unit,
    # so 3 parts): groups of four and of two (one workgroup per KV head either way) give the same split; groups of three take one workgroup per query head (96
    # chains: 3 segments, the first two summed in 12 parts)
    assert lib.la_forward_workspace_bytes(1, 128, 32, 1 << 20, 64, 64, 64, BF16) == (32 * 7 * 3 + 32 * 8) * 64 * 64 * 4
    assert lib.la_forward_workspace_bytes(1, 64, 32, 1 << 20, 64, 64, 64, BF16) == (32 * 7 * 3 + 32 * 8) * 64 * 64 * 4
    assert lib.la_forward_workspace_bytes(1, 96, 32, 1 << 20, 64, 64, 64, BF16) == (32 * 2 * 12 + 32 * 3) * 64 * 64 * 4
    # variants at head size 64 on the matrix cores too: causal = the forward's split, non-causal sums
    # all 8 segments of each chain (3 parts each) and scans 9 entries
    assert lib.la_forward_variant_workspace_bytes(1, 128, 32, 1 << 20, 64, 64, 64, BF16, 1, 0) == \
        (32 * 7 * 3 + 32 * 8) * 64 * 64 * 4
    assert lib.la_forward_variant_workspace_bytes(1, 128, 32, 1 << 20, 64, 64, 64, BF16, 0, 0) == \
        (32 * 8 * 3 + 32 * 9) * 64 * 64 * 4
    assert lib.la_forward_variant_workspace_bytes(1, 64, 32, 1 << 20, 64, 64, 64, BF16, 0, 0) == \
        (32 * 8 * 3 + 32 * 9) * 64 * 64 * 4
    assert lib.la_forward_workspace_bytes(256, 128, 32, 8192, 128, 128, 64, BF16) == 0
    assert lib.la_forward_workspace_bytes(1, 128, 32, 0, 128, 128, 64, BF16) == 0
    assert lib.la_forward_workspace_bytes(1, 6, 4, 64, 128, 128, 64, BF16) == 0   # invalid -> 0
    # Backward at 1M tokens: the dQ forward's workspace, the transposed
    # initial states, and for dK/dV 8 segments per chain whose 7 later
    # segments' sums of q^T dO the dQ pass writes (one per chain and segment:
    # its segments are the same), plus 8 start states per chain.
    n = lib.la_backward_workspace_bytes(1, 128, 32, 1 << 20, 128, 128, 64, BF16)
    assert n == ((32 * 7 * 2 + 32 * 8) + 32 + 32 * 7 + 32 * 8) * 128 * 128 * 4
    # Eight query heads per KV head: the dQ pass splits each group in two and
    # runs 4 segments per chain (its pre-pass: 3 segments of the 32 KV heads
    # in 5 parts), the dK/dV kernel 8, so the pre-pass over (Q, dO) sums the
    # 7 later segments of 256 query heads (2 parts each: 3584 workgroups,
    # seven rounds at two per compute unit).
    n8 = lib.la_backward_workspace_bytes(1, 256, 32, 1 << 20, 128, 128, 64, BF16)
    assert n8 == ((32 * 3 * 5 + 32 * 4) + 32 + 256 * 7 * 2 + 32 * 8) * 128 * 128 * 4
    assert lib.la_backward_workspace_bytes(1, 128, 32, 0, 128, 128, 64, BF16) == 0
    # Head size 64 (groups of four): states of 64 x 64, and two dK/dV workgroups per compute unit, so
    # 16 segments per chain whose 15 later segments are summed in 2 parts each (3840 pre-pass
    # workgroups: five rounds); with groups of two, 64 query heads' partials in 4 parts each.
    n64 = lib.la_backward_workspace_bytes(1, 128, 32, 1 << 20, 64, 64, 64, BF16)
    assert n64 == ((32 * 7 * 3 + 32 * 8) + 32 + 128 * 15 * 2 + 32 * 16) * 64 * 64 * 4
    assert lib.la_backward_workspace_bytes(1, 64, 32, 1 << 20, 64, 64, 64, BF16) == \
        ((32 * 7 * 3 + 32 * 8) + 32 + 64 * 15 * 4 + 32 * 16) * 64 * 64 * 4
    assert lib.la_backward_workspace_bytes(1, 4, 2, 64, 128, 96, 64, F32) == 2 * 128 * 96 * 4   # s_in^T
    assert lib.la_backward_workspace_bytes(1, 4, 2, 64, 48, 96, 64, F32) == 0                  # d not a multiple of 32
    # bf16 at other head sizes runs on the scalar kernels: no forward workspace, s_in^T for the backward
    assert lib.la_forward_workspace_bytes(1, 4, 1, 1000, 96, 96, 64, BF16) == 0
    assert lib.la_backward_workspace_bytes(1, 4, 2, 64, 64, 96, 64, BF16) == 2 * 64 * 96 * 4
    # Variants at 1M tokens: causal = the forward's split (+ normaliser sums);
    # non-causal sums all 8 segments of each chain (2 parts each) and scans
    # 9 entries, the last being the total.
    DD, d = 128 * 128, 128
    causal = lib.la_forward_variant_workspace_bytes(1, 128, 32, 1 << 20, 128, 128, 64, BF16, 1, 1)
    assert causal == ((32 * 7 * 2 + 32 * 8) * DD + (32 * 7 * 2 + 32 * 8) * d) * 4
    nonc = lib.la_forward_variant_workspace_bytes(1, 128, 32, 1 << 20, 128, 128, 64, BF16, 0, 0)
    assert nonc == (32 * 8 * 2 + 32 * 9) * DD * 4
    assert lib.la_forward_variant_workspace_bytes(1, 8, 2, 256, 128, 128, 64, BF16, 0, 1) > 0  # one segment still sums
    assert lib.la_forward_variant_workspace_bytes(1, 2, 1, 256, 128, 128, 64, BF16, 1, 0) == 0  # unsupported -> 0


def test_binding_requires_gpu_tensors():
    import torch
    x = torch.zeros((1, 1, 4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        la.forward(x, x, x)


def test_forward_state_validation(lib):
    """la_forward_state (state only, no outputs): argument errors before any
    launch, and the workspace of its parts (one round of two pre-pass
    workgroups per compute unit at head size 128, three at 64, planned here
    for 256 compute units)."""
    def st(k=K, v=V, B=1, Hkv=4, N=1000, d=128, dv=128, i=BF16, s_in=None, s_out=S_OUT, ws=WS, ws_bytes=1 << 32):
        return lib.la_forward_state(k, v, B, Hkv, N, d, dv, i, s_in, s_out, ws, ws_bytes, None)

    assert st(k=None) == NULL
    assert st(s_out=None) == NULL
    assert st(B=0) == SHAPE
    assert st(N=-1) == SHAPE
    assert st(d=256) == UNSUP
    assert st(i=7) == UNSUP
    assert st(v=ctypes.c_void_p(GB * 3 + 8)) == ALIGN
    assert st(s_out=ctypes.c_void_p(GB * 2 + 4096)) == ALIAS                  # inside k
    assert st(s_in=S_IN, s_out=ctypes.c_void_p(GB * 5 + 1024)) == ALIAS      # partly over s_in
    assert st(ws=None) == WORKSPACE
    assert st(ws_bytes=16) == WORKSPACE
    assert st(ws=ctypes.c_void_p(GB * 2 + 64)) == ALIAS                       # workspace inside k
    # 1M tokens, 32 KV heads: 16 parts per chain (1024 blocks each) at 128, 24 at 64
    assert lib.la_forward_state_workspace_bytes(1, 32, 1 << 20, 128, 128, BF16) == 32 * 16 * 128 * 128 * 4
    assert lib.la_forward_state_workspace_bytes(1, 32, 1 << 20, 64, 64, BF16) == 32 * 24 * 64 * 64 * 4
    assert lib.la_forward_state_workspace_bytes(1, 32, 100, 128, 128, BF16) == 32 * 128 * 128 * 4   # one part
    assert lib.la_forward_state_workspace_bytes(1, 32, 1 << 20, 128, 128, F32) == 0   # float32 FMA path
    assert lib.la_forward_state_workspace_bytes(1, 32, 0, 128, 128, BF16) == 0
    assert lib.la_forward_state_workspace_bytes(1, 32, 1000, 256, 256, BF16) == 0     # invalid


def test_backward_state_validation(lib):
    """la_backward_state (the initial-state gradient alone): argument errors
    before any launch; its parts run over the query heads (128 chains at 1M
    tokens: 4 parts each on 256 compute units)."""
    def bs(q=Q, do=DO, B=1, Hq=8, Hkv=2, N=1000, d=128, dv=128, i=BF16, gso=None, gsi=DS, ws=WS, ws_bytes=1 << 32):
        return lib.la_backward_state(q, do, B, Hq, Hkv, N, d, dv, i, gso, gsi, ws, ws_bytes, None)

    assert bs(q=None) == NULL
    assert bs(do=None) == NULL
    assert bs(gsi=None) == NULL
    assert bs(Hq=6, Hkv=4) == SHAPE
    assert bs(d=256) == UNSUP
    assert bs(do=ctypes.c_void_p(GB * 8 + 2)) == ALIGN
    assert bs(gsi=ctypes.c_void_p(GB + 4096)) == ALIAS                        # inside q
    assert bs(gso=S_OUT, gsi=ctypes.c_void_p(GB * 6 + 1024)) == ALIAS         # partly over grad_s_out
    assert bs(ws=None) == WORKSPACE
    assert bs(ws=ctypes.c_void_p(GB * 8 + 64)) == ALIAS                       # workspace inside grad_o
    assert lib.la_backward_state_workspace_bytes(1, 128, 32, 1 << 20, 128, 128, BF16) == 128 * 4 * 128 * 128 * 4
    assert lib.la_backward_state_workspace_bytes(1, 128, 32, 1 << 20, 128, 128, F32) == 0
    assert lib.la_backward_state_workspace_bytes(1, 6, 4, 1000, 128, 128, BF16) == 0   # invalid


def test_noalloc_rejects_before_touching_the_device(lib):
    """la_forward_noalloc: argument errors come back as from la_forward_ex, and
    a problem whose workspace exceeds the fixed scratch is LA_ERR_TOO_LARGE,
    both decided before any device call.  1100 (batch, KV head) pairs with two
    four-head subgroups each need one 64 KiB start state per pair (68.75 MiB)."""
    assert _lib.LA_NOALLOC_SCRATCH_BYTES == 64 << 20

    def na(q=Q, k=K, v=V, o=O, B=1, Hq=4, Hkv=1, N=1000, d=128, dv=128, block=64, i=BF16, out=BF16):
        return lib.la_forward_noalloc(q, k, v, o, B, Hq, Hkv, N, d, dv, block, i, out, None, None, None)

    assert na(q=None) == NULL
    assert na(Hq=6, Hkv=4) == SHAPE
    assert na(d=256) == UNSUP
    assert na(B=1100, Hq=8, Hkv=1, N=64) == TOO_LARGE
    assert lib.la_forward_workspace_bytes(1100, 8, 1, 64, 128, 128, 64, BF16) == 1100 * 128 * 128 * 4
    # the 1M-token, 128/32-head workload fits (planned here for 256 compute units)
    assert lib.la_forward_workspace_bytes(1, 128, 32, 1 << 20, 128, 128, 64, BF16) == (32 * 7 * 2 + 32 * 8) * 65536


def test_stream_library_exports_its_header():
    """libla_stream.so (the benchmark's HBM streaming references) exports what
    include/la_stream.h declares and refuses bad arguments without launching."""
    from long_context_attention_chunkwise_amd import build
    names = declared_functions(os.path.join(ROOT, "include", "la_stream.h"))
    assert names == ["la_stream_bytes_moved", "la_stream_run"]
    slib = ctypes.CDLL(build.STREAM_LIB_PATH)
    for n in names:
        assert getattr(slib, n) is not None
    slib.la_stream_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    slib.la_stream_bytes_moved.argtypes = [ctypes.c_int, ctypes.c_size_t]
    slib.la_stream_bytes_moved.restype = ctypes.c_size_t
    assert slib.la_stream_run(4, 0, Q, K, 1 << 30, S_IN, 256, None) == 1       # no such mode
    assert slib.la_stream_run(1, 0, Q, None, 1 << 30, S_IN, 256, None) == 1    # copy needs dst
    assert slib.la_stream_run(0, 0, ctypes.c_void_p(GB + 4), None, 1 << 30, S_IN, 256, None) == 1   # misaligned
    assert slib.la_stream_bytes_moved(0, 1 << 30) == 1 << 30
    assert slib.la_stream_bytes_moved(1, 1 << 30) == 2 << 30
    assert slib.la_stream_bytes_moved(3, 1 << 30) == 2 << 30                 # in place: read + write
    assert slib.la_stream_bytes_moved(4, 1 << 30) == 0
    # 3:2 mix: 60 KiB steps, 2/3 of what is read is written
    steps = (1 << 30) // (256 * 15 * 16)
    assert slib.la_stream_bytes_moved(2, 1 << 30) == steps * 256 * 15 * 16 + steps * 256 * 10 * 16
