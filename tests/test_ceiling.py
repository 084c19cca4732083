"""The plain-read ceiling (libqgemv_ceiling.so, the benchmark's bandwidth
reference): every mapping, depth and load policy must read every byte once,
so the XOR it folds the bytes into equals the host's fold of the same bytes;
and bad arguments are refused before anything is launched."""
import ctypes as C
import os

import numpy as np
import pytest

from gpu_util import torch_cuda

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "quantized_weight_decode_amd", "libqgemv_ceiling.so")


def _lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built: run quantized_weight_decode_amd.build")
    L = C.CDLL(LIB)
    L.qgemv_ceiling_read.restype = C.c_int
    L.qgemv_ceiling_read.argtypes = [C.c_void_p, C.c_size_t, C.c_int, C.c_int, C.c_int, C.c_int,
                                     C.c_void_p, C.c_size_t, C.c_void_p]
    return L


def test_refusals():
    # every call here is refused on the host, before any pointer is used
    L = _lib()
    buf, out = C.c_void_p(1 << 20), C.c_void_p(1 << 21)
    ok = dict(buf=buf, bytes=1 << 16, pattern=0, wpb=8, u=2, wgs=0, out=out, out_len=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return L.qgemv_ceiling_read(a["buf"], a["bytes"], a["pattern"], a["wpb"], a["u"],
                                    a["wgs"], a["out"], a["out_len"], None)

    assert call(buf=None) == 1
    assert call(out=None) == 1
    assert call(wpb=3) == 1
    assert call(u=3) == 1
    assert call(wgs=-1) == 1
    assert call(wgs=4, u=1) == 1          # the slab mapping needs a ring
    assert call(pattern=4) == 1
    assert call(pattern=-1) == 1
    assert call(bytes=17) == 1            # contiguous: whole 16-byte chunks
    assert call(pattern=1, bytes=135) == 1    # MQ4: whole 136-byte groups
    assert call(pattern=3, bytes=137) == 1
    assert call(buf=C.c_void_p((1 << 20) + 8)) == 1              # contiguous: 16-byte aligned
    assert call(pattern=1, bytes=136, buf=C.c_void_p((1 << 20) + 4)) == 1   # MQ4: 8-byte aligned
    assert call(out_len=1) == 1           # more waves than out holds


@pytest.mark.gpu
@pytest.mark.parametrize("pattern", [0, 1, 2, 3])
@pytest.mark.parametrize("wpb,u,wgs", [(4, 1, 0), (8, 4, 0), (16, 8, 0), (8, 2, 37), (16, 4, 256),
                                       (4, 8, 256)])
def test_reads_every_byte(pattern, wpb, u, wgs):
    torch = torch_cuda()
    L = _lib()
    mq4 = pattern & 1
    nbytes = 136 * 7777 if mq4 else (1 << 20) + 48
    rng = np.random.default_rng(pattern * 100 + wpb * 10 + u)
    host = rng.integers(0, 256, nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).to("cuda:0")
    out = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")
    st = L.qgemv_ceiling_read(buf.data_ptr(), nbytes, pattern, wpb, u, wgs, out.data_ptr(),
                              out.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    if mq4:
        # each group's two header dwords are folded in four times each (cancel)
        want = np.bitwise_xor.reduce(host.reshape(-1, 136)[:, 8:].copy().view(np.uint32).ravel())
    else:
        want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert got == want
