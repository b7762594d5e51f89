"""The C-ABI library loads without a GPU, exports every function that
include/kda.h declares, and rejects bad arguments on the host before any
launch (these calls never reach the HIP runtime).  CPU only."""
import ctypes
import os
import re

import pytest

import kimi_delta_attention_kda_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    txt = open(HDR).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        pytest.fail("libkda.so is not built: run __graft_entry__.build()")
    return kda.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(kda.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert lib.kda_status_str(code)
    assert lib.kda_status_str(0) == b"ok"


A = ctypes.c_void_p(0x10000)   # 16-byte aligned fake addresses: never dereferenced,
B = ctypes.c_void_p(0x20000)   # every call below fails validation first
MIS = ctypes.c_void_p(0x20004)


def chunk(lib, **kw):
    args = dict(q=A, k=A, v=A, g=A, b=A, A_log=B, dt=B, h0=None, cu=None, chunk=16, o=A,
                hT=None, B=1, T=16, H=1, dk=128, dv=128, n_seq=1, scale=0.1, dtype=1, ws=None, wsb=0)
    args.update(kw)
    return lib.kda_chunk_fwd(args["q"], args["k"], args["v"], args["g"], args["b"],
                             args["A_log"], args["dt"], args["h0"], args["cu"], args["chunk"],
                             args["o"], args["hT"], args["B"], args["T"], args["H"], args["dk"],
                             args["dv"], args["n_seq"], args["scale"], args["dtype"], args["ws"], args["wsb"],
                             None)


def test_chunk_validation(lib):
    assert chunk(lib, chunk=32) == -3
    assert chunk(lib, dk=96) == -3
    assert chunk(lib, dtype=0, dk=128) == -3       # fp32 activations built for dk = 64
    assert chunk(lib, dtype=7) == -3
    assert chunk(lib, H=0) == -2
    assert chunk(lib, n_seq=2) == -2                # dense input needs n_seq == B
    assert chunk(lib, cu=A, B=2, n_seq=2) == -2     # packed input needs B == 1
    assert chunk(lib, A_log=None) == -1
    assert chunk(lib, q=None) == -1
    assert chunk(lib, o=MIS) == -4
    assert chunk(lib, ws=MIS, wsb=1 << 20) == -4    # a workspace must be aligned too
    assert chunk(lib, n_seq=0, B=0) == 0            # nothing to do, no launch


def chunk_noalloc(lib, **kw):
    args = dict(q=A, k=A, v=A, g=A, b=A, A_log=B, dt=B, h0=None, cu=None, chunk=16, o=A,
                hT=None, B=1, T=16, H=1, dk=128, dv=128, n_seq=1, scale=0.1, dtype=1)
    args.update(kw)
    return lib.kda_chunk_fwd_noalloc(*(args[k_] for k_ in ("q", "k", "v", "g", "b", "A_log", "dt", "h0", "cu",
                                                          "chunk", "o", "hT", "B", "T", "H", "dk", "dv", "n_seq",
                                                          "scale", "dtype")), None)


def test_chunk_noalloc_validation(lib):
    """The allocation-free variant rejects what kda_chunk_fwd rejects, before
    it touches the GPU (its scratch-size check needs the device)."""
    assert chunk_noalloc(lib, chunk=32) == -3
    assert chunk_noalloc(lib, dk=96) == -3
    assert chunk_noalloc(lib, H=0) == -2
    assert chunk_noalloc(lib, n_seq=2) == -2
    assert chunk_noalloc(lib, q=None) == -1
    assert chunk_noalloc(lib, o=MIS) == -4
    assert chunk_noalloc(lib, n_seq=0, B=0) == 0


def test_chunk_workspace_bytes(lib):
    """13,824 bytes per chunk row and head at dk = 128 (7,424 at dk = 64):
    B * ceil(T/16) rows for dense input, ceil(T/16) + n_seq for packed."""
    f = lib.kda_chunk_fwd_workspace_bytes
    assert f(4, 4096, 16, 128, 128, 4, 0) == 13824 * 4 * 256 * 16
    assert f(1, 17, 2, 64, 64, 1, 0) == 7424 * 2 * 2
    assert f(1, 129830, 32, 128, 128, 32, 1) == 13824 * 32 * ((129830 + 15) // 16 + 32)
    assert f(1, 16, 0, 128, 128, 1, 0) == 0
    assert f(1, 16, 1, 96, 128, 1, 0) == 0


def chunk_states(lib, **kw):
    args = dict(q=A, k=A, v=A, g=A, b=A, A_log=B, dt=B, h0=None, cu=None, chunk=16, o=A,
                hT=None, hc=A, B=1, T=16, H=1, dk=128, dv=128, n_seq=1, scale=0.1, dtype=1)
    args.update(kw)
    return lib.kda_chunk_fwd_states(args["q"], args["k"], args["v"], args["g"], args["b"],
                                    args["A_log"], args["dt"], args["h0"], args["cu"], args["chunk"],
                                    args["o"], args["hT"], args["hc"], args["B"], args["T"], args["H"],
                                    args["dk"], args["dv"], args["n_seq"], args["scale"], args["dtype"],
                                    None, 0, None)


def test_chunk_states_validation(lib):
    assert chunk_states(lib, hc=None) == -1
    assert chunk_states(lib, hc=MIS) == -4
    assert chunk_states(lib, chunk=64) == -3
    assert chunk_states(lib, n_seq=0, B=0) == 0


def chunk_pool(lib, **kw):
    args = dict(q=A, k=A, v=A, g=A, b=A, A_log=B, dt=B, pool=A, idx=B, cu=None, chunk=16, o=A,
                B=1, T=16, H=1, dk=128, dv=128, n_seq=1, P=4, scale=0.1, dtype=1)
    args.update(kw)
    return lib.kda_chunk_fwd_pool(args["q"], args["k"], args["v"], args["g"], args["b"],
                                  args["A_log"], args["dt"], args["pool"], args["idx"], args["cu"],
                                  args["chunk"], args["o"], args["B"], args["T"], args["H"],
                                  args["dk"], args["dv"], args["n_seq"], args["P"], args["scale"],
                                  args["dtype"], None, 0, None)


def test_chunk_pool_validation(lib):
    assert chunk_pool(lib, P=0) == -2
    assert chunk_pool(lib, pool=None) == -1
    assert chunk_pool(lib, idx=None) == -1
    assert chunk_pool(lib, idx=MIS) == -4
    assert chunk_pool(lib, chunk=8) == -3
    assert chunk_pool(lib, n_seq=2) == -2            # dense input needs n_seq == B
    assert chunk_pool(lib, n_seq=0, B=0) == 0        # nothing to do, no launch


def decode(lib, **kw):
    args = dict(qkv=A, a=A, b=A, A_log=B, dt=B, pool=A, idx=A, o=A, B=4, H=2, HV=4, K=128,
                V=128, P=8, scale=0.1, flags=1)
    args.update(kw)
    return lib.kda_decode_step(args["qkv"], args["a"], args["b"], args["A_log"], args["dt"],
                               args["pool"], args["idx"], args["o"], args["B"], args["H"],
                               args["HV"], args["K"], args["V"], args["P"], args["scale"],
                               args["flags"], None)


def test_decode_validation(lib):
    assert decode(lib, K=64) == -3
    assert decode(lib, HV=3) == -2                   # HV % H != 0
    assert decode(lib, pool=None) == -1
    assert decode(lib, idx=MIS) == -4
    assert decode(lib, B=0) == 0


def extend(lib, **kw):
    args = dict(qkv=A, a=A, b=A, A_log=B, dt=B, pool=A, idx=A, o=A, B=4, T=3, H=2, HV=4, K=128,
                V=128, P=8, scale=0.1, flags=1)
    args.update(kw)
    return lib.kda_decode_extend(args["qkv"], args["a"], args["b"], args["A_log"], args["dt"],
                                 args["pool"], args["idx"], args["o"], args["B"], args["T"],
                                 args["H"], args["HV"], args["K"], args["V"], args["P"],
                                 args["scale"], args["flags"], None)


def test_decode_extend_validation(lib):
    assert extend(lib, V=64) == -3
    assert extend(lib, T=-1) == -2
    assert extend(lib, HV=6, H=4) == -2              # HV % H != 0
    assert extend(lib, o=None) == -1
    assert extend(lib, qkv=MIS) == -4
    assert extend(lib, T=0) == 0                     # nothing to do, no launch
    assert extend(lib, B=0) == 0


def conv_decode(lib, **kw):
    args = dict(x=A, cs=A, cw=A, cb=None, a=A, b=A, A_log=B, dt=B, pool=A, idx=A, o=A, B=4, H=2, HV=4,
                K=128, V=128, W=4, P=8, scale=0.1, flags=1)
    args.update(kw)
    return lib.kda_conv_decode_step(args["x"], args["cs"], args["cw"], args["cb"], args["a"], args["b"],
                                    args["A_log"], args["dt"], args["pool"], args["idx"], args["o"],
                                    args["B"], args["H"], args["HV"], args["K"], args["V"], args["W"],
                                    args["P"], args["scale"], args["flags"], None)


def test_conv_decode_validation(lib):
    assert conv_decode(lib, W=5) == -3
    assert conv_decode(lib, W=1) == -3
    assert conv_decode(lib, K=64) == -3
    assert conv_decode(lib, H=1, HV=127) == -3        # conv outputs of a workgroup exceed 64 KiB of LDS
    assert conv_decode(lib, HV=3) == -2               # HV % H != 0
    assert conv_decode(lib, cs=None) == -1
    assert conv_decode(lib, cw=None) == -1
    assert conv_decode(lib, cb=MIS) == -4
    assert conv_decode(lib, B=0) == 0


def chunk_o(lib, **kw):
    args = dict(q=A, k=A, v=A, g=A, b=A, A_log=B, dt=B, hc=A, cu=None, o=A, B=2, T=20, H=1, dk=128, dv=128,
                n_seq=2, nc=4, scale=0.1, dtype=1)
    args.update(kw)
    return lib.kda_chunk_o(*(args[k_] for k_ in ("q", "k", "v", "g", "b", "A_log", "dt", "hc", "cu", "o", "B",
                                                 "T", "H", "dk", "dv", "n_seq", "nc", "scale", "dtype")), None)


def test_chunk_o_validation(lib):
    assert chunk_o(lib, dtype=0) == -3
    assert chunk_o(lib, dk=64) == -3
    assert chunk_o(lib, nc=3) == -2                   # dense: B * ceil(T / 16) rows
    assert chunk_o(lib, hc=None) == -1
    assert chunk_o(lib, o=MIS) == -4
    assert chunk_o(lib, B=0, n_seq=0, nc=0) == 0


def backward(lib, **kw):
    args = dict(q=A, k=A, v=A, g=A, b=A, A_log=B, dt=B, hc=A, cu=None, do=A, dhT=None, dq=A, dk=A, dv=A,
                dg=A, db=A, dA=None, ddt=None, dh0=None, ws=A, wsb=1 << 30, B=1, T=16, H=1, dk_=128, dv_=128,
                n_seq=1, scale=0.1, dtype=1)
    args.update(kw)
    return lib.kda_backward(*(args[k_] for k_ in ("q", "k", "v", "g", "b", "A_log", "dt", "hc", "cu", "do",
                                                  "dhT", "dq", "dk", "dv", "dg", "db", "dA", "ddt", "dh0",
                                                  "ws", "wsb", "B", "T", "H", "dk_", "dv_", "n_seq", "scale",
                                                  "dtype")), None)


def test_backward_validation(lib):
    # per (chunk row, head), for ceil(100 / 16) + 2 rows (at most one partial chunk per
    # sequence): the chunk's operands (14,336 bytes, rounded up to 256 in all), a
    # gradient row (40,960 bytes) and the parameter sums (129 floats); per head, 64
    # slices of those sums
    items = (7 + 2) * 3
    assert lib.kda_backward_workspace_bytes(2, 3, 128, 128, 100) == \
        ((items * 14336 + 255) // 256) * 256 + items * 40960 + items * 129 * 4 + 3 * 64 * 129 * 4
    assert lib.kda_backward_workspace_bytes(2, 3, 64, 128, 100) == 0
    assert backward(lib, dtype=0) == -3               # float32 activations: no d = 128 forward to pair with
    assert backward(lib, dk_=64) == -3
    assert backward(lib, wsb=1024) == -2              # workspace too small
    assert backward(lib, ws=None) == -1
    assert backward(lib, hc=None) == -1
    assert backward(lib, do=MIS) == -4
    assert backward(lib, n_seq=2) == -2               # dense input needs n_seq == B
    assert backward(lib, n_seq=0, B=0) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 16, 1, 64)
    with pytest.raises(kda.KDAError):
        kda.chunk_fwd(x, x, x, x, torch.zeros(1, 16, 1), torch.zeros(1), torch.zeros(1, 64))
