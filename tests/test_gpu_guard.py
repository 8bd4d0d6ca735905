"""Guard bands around every output the library writes: each output lives in
the middle of a buffer whose 4 KB on either side (and, for strided y, the
columns between rows) are filled with 0xA5 beforehand and must still hold
0xA5 after the call -- pack (planes, meta), the exception list (offsets,
entries), unpack (w_out), and the GEMMs with fp32 and BF16 output, split K
included.  The values themselves are checked against the oracle as in the
parity tests."""
import numpy as np
import pytest
import torch

from lossless_bit_weight_amd import inputs, w12
from tests.gpu_util import assert_gemm_close, require_gpu, to_dev, to_host_u16

pytestmark = pytest.mark.gpu

GUARD = 4096
FILL = 0xA5


class Guarded:
    """`nbytes` of device memory with GUARD bytes of 0xA5 on either side."""

    def __init__(self, nbytes: int):
        self.nbytes = nbytes
        self.buf = torch.full((GUARD + nbytes + GUARD,), FILL, dtype=torch.uint8, device="cuda")

    def view(self, dtype=torch.uint8, shape=None):
        t = self.buf[GUARD:GUARD + self.nbytes].view(dtype)
        return t if shape is None else t.view(shape)

    def check(self, what: str):
        torch.cuda.synchronize()
        lo = self.buf[:GUARD].cpu().numpy()
        hi = self.buf[GUARD + self.nbytes:].cpu().numpy()
        assert (lo == FILL).all(), what + ": write below the buffer"
        assert (hi == FILL).all(), what + ": write past the buffer"


def _raw(N, K, seed):
    return inputs.inject_zeros(inputs.gaussian_bf16((N, K), 0.02, seed), 0.01, seed + 1)


def _guarded_pack(bits):
    N, K = bits.shape
    pb, mb = w12.w12_plane_bytes(N, K), w12.w12_meta_bytes(N, K)
    g = [Guarded(pb) for _ in range(3)] + [Guarded(mb)]
    wt = w12.W12Weight(g[0].view(), g[1].view(), g[2].view(), g[3].view(), N, K)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    w12.w12_pack(to_dev(bits), out=wt, bad_groups=bad)
    for gi, name in zip(g, ("p0", "p1", "p2", "meta")):
        gi.check("pack " + name)
    return wt, int(bad.item()), g


@pytest.mark.parametrize("shape", [(37, 384), (16, 128), (130, 1152)])
def test_pack_unpack_list_stay_inside(oracle, shape):
    require_gpu()
    N, K = shape
    bits = _raw(N, K, 3 * N + K)
    print("guard: pack/unpack/list", shape, flush=True)
    wt, bad, _ = _guarded_pack(bits)
    r0, r1, r2, rmeta, rbad = oracle.pack(bits)
    for got, ref, name in ((wt.p0, r0, "p0"), (wt.p1, r1, "p1"), (wt.p2, r2, "p2"),
                           (wt.meta, rmeta, "meta")):
        assert np.array_equal(got.cpu().numpy(), ref), name
    assert bad == rbad and bad > 0
    # unpack into a guarded BF16 tensor
    gw = Guarded(2 * N * K)
    out = gw.view(torch.bfloat16, (N, K))
    w12.w12_unpack(wt, out=out)
    gw.check("unpack w_out")
    assert np.array_equal(to_host_u16(out), oracle.unpack(r0, r1, r2, rmeta, N, K))
    # the exception list into guarded offsets / entries
    off_ref, ent_ref = oracle.exceptions(bits)
    L = w12.lib()
    wd = to_dev(bits)
    wsb = int(L.w12_exceptions_workspace_bytes(N, K))
    gws, goff, gent, gtot = Guarded(wsb), Guarded(4 * off_ref.size), Guarded(8 * len(ent_ref)), Guarded(4)
    stream = torch.cuda.current_stream().cuda_stream
    rc = L.w12_exceptions(wd.data_ptr(), N, K, gws.view().data_ptr(), wsb, goff.view().data_ptr(),
                          gent.view().data_ptr(), len(ent_ref), gtot.view().data_ptr(), stream)
    assert rc == 0
    for gi, name in ((gws, "workspace"), (goff, "offsets"), (gent, "entries"), (gtot, "total")):
        gi.check("exceptions " + name)
    assert np.array_equal(goff.view(torch.int32).cpu().numpy().view(np.uint32), off_ref)
    assert np.array_equal(gent.view(torch.int32).cpu().numpy().view(np.uint32).reshape(-1, 2),
                          ent_ref)
    # unpack with the list: lossless, still inside w_out
    wt.exc_offsets = goff.view(torch.int32)
    wt.exc_entries = gent.view(torch.int32, (-1, 2))
    gw2 = Guarded(2 * N * K)
    out2 = gw2.view(torch.bfloat16, (N, K))
    w12.w12_unpack(wt, out=out2)
    gw2.check("unpack with list")
    assert np.array_equal(to_host_u16(out2), bits)


@pytest.mark.parametrize("shape,M", [((37, 384), 1), ((37, 384), 17), ((1000, 640), 9),
                                     ((130, 1152), 32), ((896, 5120), 16), ((300, 2560), 64),
                                     ((1024, 17408), 2)])
@pytest.mark.parametrize("ytype", ["f32", "bf16"])
def test_gemm_stays_inside_y(oracle, shape, M, ytype):
    require_gpu()
    N, K = shape
    print("guard: gemm", shape, M, ytype, flush=True)
    first, _ = w12.pack(to_dev(_raw(N, K, 5 * N + K)))
    wc = w12.w12_unpack(first)
    wt, bad = w12.pack(wc)
    assert bad == 0
    bt = w12.w12_bf16_tile(wc)
    x_bits = inputs.gaussian_bf16((M, K), 1.0, 7 * M + N)
    x = to_dev(x_bits)
    ldy = N + 13          # columns N..ldy-1 of every row must stay untouched
    dt, esz = (torch.float32, 4) if ytype == "f32" else (torch.bfloat16, 2)
    w_ref = to_host_u16(wc)
    y_ref = oracle.gemm_bf16_f64(x_bits, w_ref)
    tol = oracle.tolerance(x_bits, w_ref)
    results = []
    for name, call in (("w12_gemm_ws", lambda y: w12.w12_gemm(x, wt, y=y)),
                       ("w12_gemm", lambda y: w12.w12_gemm(x, wt, y=y, split_k=False)),
                       ("bf16_gemm_ws", lambda y: w12.bf16_gemm(x, bt, y=y)),
                       ("w12_gemm_noalloc", lambda y: w12.w12_gemm_noalloc(x, wt, y=y))):
        g = Guarded(esz * M * ldy)
        full = g.view(dt, (M, ldy))
        call(full[:, :N])
        g.check("%s y" % name)
        raw = full.view(torch.uint8).cpu().numpy().reshape(M, ldy * esz)
        assert (raw[:, N * esz:] == 0xA5).all(), name + ": wrote between rows of y"
        y = full[:, :N].float().cpu().numpy() if ytype == "bf16" else full[:, :N].cpu().numpy()
        results.append(full[:, :N].clone())
        if ytype == "f32":
            assert_gemm_close(y, y_ref, tol, "%s %s M=%d" % (name, shape, M))
    # the _ws, bf16 _ws and no-alloc calls share one tiling: bitwise equal
    iv = torch.int16 if ytype == "bf16" else torch.int32
    for r in (results[2], results[3]):
        assert torch.equal(r.view(iv), results[0].view(iv))
