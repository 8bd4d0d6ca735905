"""The C-ABI library without a GPU: it loads, exports every function the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import re

import pytest

from lossless_bit_weight_amd import w12

P = ctypes.c_void_p
A16 = P(4096)       # a non-null, 16-byte aligned stand-in (never dereferenced:
MIS = P(4098)       # every call below fails validation before any launch)


def test_loads_and_exports_every_declared_symbol():
    L = w12.lib()
    names = w12.header_functions()
    assert set(names) >= {"w12_pack", "w12_unpack", "w12_gemm", "bf16_gemm", "w12_bf16_tile",
                          "w12_plane_bytes", "w12_meta_bytes", "w12_status_string",
                          "w12_abi_version", "w12_gemm_variant", "w12_gemm_ws", "bf16_gemm_ws",
                          "w12_gemm_workspace_bytes", "w12_gemm_ex", "bf16_gemm_ex",
                          "w12_exceptions", "w12_exceptions_workspace_bytes",
                          "w12_gemm_noalloc"}
    for n in names:
        assert hasattr(L, n), n
    assert w12.w12_abi_version() == 8


def test_sizes():
    assert w12.w12_plane_bytes(7168, 5120) == 7168 * 5120 // 2
    assert w12.w12_meta_bytes(7168, 5120) == 7168 * 40
    assert w12.w12_padded_rows(1) == 16 and w12.w12_padded_rows(32) == 32
    assert w12.w12_plane_bytes(3, 128) == 16 * 64
    assert w12.w12_meta_bytes(17, 256) == 32 * 2
    assert w12.w12_bf16_tiled_bytes(17, 256) == 32 * 256 * 2
    assert w12.w12_plane_bytes(3, 100) == 0
    assert w12.w12_plane_bytes(1, (1 << 24) - 128) == 16 * ((1 << 24) - 128) // 2
    assert w12.w12_plane_bytes(1, 1 << 24) == 0
    assert w12.w12_meta_bytes(0, 128) == 0


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -6, -7, -8, -9, 99):
        assert isinstance(w12.w12_status_string(s), str) and w12.w12_status_string(s)


def _gemm(**kw):
    a = dict(x=A16, M=1, ldx=512, p0=A16, p1=A16, p2=A16, meta=A16, N=64, K=512, y=A16,
             ldy=64, yt=0)
    a.update(kw)
    return w12.lib().w12_gemm(a["x"], a["M"], a["ldx"], a["p0"], a["p1"], a["p2"], a["meta"],
                              a.get("eo"), a.get("ee"), a["N"], a["K"], a["y"], a["ldy"], a["yt"],
                              None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), -1), (dict(p1=None), -1), (dict(meta=None), -1), (dict(y=None), -1),
    (dict(K=500), -2), (dict(K=0), -2), (dict(N=0), -2), (dict(M=0), -2),
    (dict(K=1 << 24, ldx=1 << 24), -2), (dict(N=1 << 26, K=1 << 14, ldx=1 << 14, ldy=1 << 26), -2),
    (dict(ldx=256), -2), (dict(ldy=63), -2),
    (dict(M=129), -6), (dict(yt=2), -4),
    (dict(x=MIS), -3), (dict(ldx=516), -3), (dict(p2=MIS), -3),
    (dict(yt=1, y=P(4098)), -3),
    (dict(eo=A16), -1), (dict(ee=A16), -1), (dict(eo=P(4098), ee=A16), -3),
    (dict(eo=A16, ee=A16, K=1 << 24, ldx=1 << 24), -2),
])
def test_gemm_rejects(kw, status):
    assert _gemm(**kw) == status


def test_bf16_gemm_rejects():
    L = w12.lib()
    assert L.bf16_gemm(A16, 1, 512, None, 64, 512, A16, 64, 0, None) == -1
    assert L.bf16_gemm(A16, 1, 512, MIS, 64, 512, A16, 64, 0, None) == -3
    assert L.bf16_gemm(A16, 129, 512, A16, 64, 512, A16, 64, 0, None) == -6
    assert L.bf16_gemm(A16, 1, 512, A16, 64, 384 + 1, A16, 64, 0, None) == -2


def test_pack_unpack_reject():
    L = w12.lib()
    assert L.w12_bf16_tile(None, 4, 128, A16, None) == -1
    assert L.w12_bf16_tile(A16, 4, 100, A16, None) == -2
    assert L.w12_bf16_tile(A16, 4, 128, MIS, None) == -3
    assert L.w12_pack(None, 4, 128, A16, A16, A16, A16, None, None) == -1
    assert L.w12_pack(A16, 4, 130, A16, A16, A16, A16, None, None) == -2
    assert L.w12_pack(MIS, 4, 128, A16, A16, A16, A16, None, None) == -3
    assert L.w12_pack(A16, 4, 128, A16, A16, A16, A16, P(4097), None) == -3
    assert L.w12_unpack(A16, A16, A16, None, None, None, 4, 128, A16, None) == -1
    assert L.w12_unpack(A16, A16, A16, A16, None, None, -1, 128, A16, None) == -2
    assert L.w12_unpack(A16, A16, A16, A16, None, None, 4, 128, MIS, None) == -3
    assert L.w12_unpack(A16, A16, A16, A16, A16, None, 4, 128, A16, None) == -1
    assert L.w12_unpack(A16, A16, A16, A16, A16, P(4098), 4, 128, A16, None) == -3
    assert L.w12_unpack(A16, A16, A16, A16, A16, A16, 4, 1 << 24, A16, None) == -2


def test_exceptions_rejects():
    L = w12.lib()
    assert w12.lib().w12_exceptions_workspace_bytes(17, 256) == 2 * 2 * 4
    assert w12.lib().w12_exceptions_workspace_bytes(17, 200) == 0
    ws = 16
    ok = (A16, 17, 256, A16, ws, A16, A16, 4, A16, None)
    bad = [((None,) + ok[1:], -1),
           (ok[:2] + (200,) + ok[3:], -2),
           (ok[:2] + (1 << 24,) + ok[3:], -2),                 # k does not fit 24 bits
           (ok[:1] + (1 << 20,) + (4096,) + ok[3:], -2),       # N*K not below 2^32
           (ok[:5] + (None,) + ok[6:], -1),                     # offsets
           (ok[:8] + (None,) + ok[9:], -1),                     # total
           (ok[:6] + (None,) + ok[7:], -1),                     # capacity without room
           (ok[:7] + (-1,) + ok[8:], -1),
           ((MIS,) + ok[1:], -3),
           (ok[:5] + (P(4098),) + ok[6:], -3),
           (ok[:3] + (None,) + ok[4:], -8),                     # workspace
           (ok[:4] + (15,) + ok[5:], -8)]
    for args, status in bad:
        assert L.w12_exceptions(*args) == status, args


def test_variant_selection():
    assert w12.w12_gemm_variant(1, 7168, 5120).startswith("w12_gemv_m1_")
    assert w12.w12_gemm_variant(4, 7168, 5120, False).startswith("bf16_mfma_mt16_")
    assert w12.w12_gemm_variant(2, 7168, 5120).startswith("w12_mfma_mt16_r2_kw4_d2_xdirect")
    assert w12.w12_gemm_variant(8, 7168, 5120).startswith("w12_mfma_mt16_")
    assert w12.w12_gemm_variant(9, 7168, 5120).startswith("w12_mfma_mt16_")
    assert w12.w12_gemm_variant(16, 34816, 5120).startswith("w12_mfma_mt16_")
    assert w12.w12_gemm_variant(1, 34816, 5120) == "w12_gemv_m1_r1_kw4_d2_xdirect"
    assert w12.w12_gemm_variant(1, 5120, 17408) == "w12_gemv_m1_r1_kw2_d4_xdirect"
    assert w12.w12_gemm_variant(17, 5120, 17408).startswith("w12_mfma_mt32_")
    assert w12.w12_gemm_variant(33, 5120, 17408).startswith("w12_mfma_mt64_r1_kw1_d2_chunked_w8_s6")
    assert w12.w12_gemm_variant(33, 2048, 5120).startswith("w12_mfma_mt64_r1_kw2_d2_chunked_w8")
    assert w12.w12_gemm_variant(65, 7168, 5120).startswith("w12_mfma_mt128_r1_kw1_d2_chunked_w8")
    assert w12.w12_gemm_variant(128, 896, 5120).startswith("w12_mfma_mt128_")
    assert w12.w12_gemm_variant(129, 5120, 17408) is None


def test_variant_with_exception_list():
    """With an exception list the x-direct MFMA defaults run one tile per
    wave below 6 rows and give way to the LDS-staged kernel (corrections in
    its main loop) from 6 rows, or with K split three ways or more, with the
    same split; the GEMV at M = 1 and the LDS-staged defaults are
    unchanged."""
    V = w12.w12_gemm_variant
    assert V(1, 7168, 5120, 3) == V(1, 7168, 5120)
    assert V(2, 7168, 5120, 3) == "w12_mfma_mt16_r1_kw4_d2_xdirect"
    assert V(4, 7168, 5120, 3) == "w12_mfma_mt16_r1_kw4_d2_xdirect"
    assert V(6, 7168, 5120, 3) == "w12_mfma_mt16_r1_kw4_d2_chunked_w8"
    assert V(8, 7168, 5120, 3) == "w12_mfma_mt16_r1_kw4_d2_chunked_w8"
    assert V(6, 34816, 5120, 3) == "w12_mfma_mt16_r1_kw4_d2_chunked_w8"
    assert V(2, 5120, 17408) == "w12_mfma_mt16_r2_kw4_d2_xdirect_s3"
    assert V(2, 5120, 17408, 3) == "w12_mfma_mt16_r1_kw2_d2_chunked_w8_s3"
    for M in (16, 32, 64):
        assert V(M, 7168, 5120, 3) == V(M, 7168, 5120)
    # the split (and so the workspace a default call needs) never changes
    split = lambda name: re.search(r"_s(\d+)$", name).group(1) if re.search(r"_s(\d+)$", name) else "1"
    for M in range(1, 33):
        for N, K in ((7168, 5120), (896, 5120), (5120, 2176), (5120, 17408), (5120, 640)):
            a, b = V(M, N, K), V(M, N, K, 3)
            assert split(a) == split(b), (M, N, K, a, b)
    assert w12.w12_gemm_variant(1, 5120, 100) is None


def test_explicit_tiling_rejects():
    L = w12.lib()
    args = (A16, 17, 512, A16, A16, A16, A16, None, None, 64, 512, A16, 64, 0)
    assert L.w12_gemm_ex(A16, 5, 512, A16, A16, A16, A16, None, None, 64, 512, A16, 64, 0,
                         w12._tiling_arg(w12.Tiling(0, 1, 1, 2, 1)), None, 0, None) == -6  # x_direct: M <= 4
    bad = [w12.Tiling(0, 1, 1, 4),      # GEMV needs M <= 8
           w12.Tiling(2, 1, 1, 4),      # unknown kind
           w12.Tiling(1, 3, 1, 2),      # r not built
           w12.Tiling(1, 1, 3, 2),      # kw not built
           w12.Tiling(1, 2, 1, 8),      # (r, depth) pair not built
           w12.Tiling(1, 1, 1, 8, 1),   # MFMA direct x: ring too large
           w12.Tiling(1, 2, 1, 4, 1),   # (32-row A: 2 tiles -> 4 * 16 * 4 > 192)
           w12.Tiling(0, 1, 1, 2, 2)]   # x_direct is 0 or 1
    bad += [w12.Tiling(1, 1, 1, 2, 0, 65),   # split-K factor above 64
            w12.Tiling(1, 1, 1, 2, 0, -1)]
    for t in bad:
        assert L.w12_gemm_ex(*args, w12._tiling_arg(t), None, 0, None) == -6, t
    assert L.bf16_gemm_ex(A16, 9, 512, A16, 64, 512, A16, 64, 0,
                          w12._tiling_arg(w12.Tiling(0, 1, 1, 2)), None, 0, None) == -6


def test_workspace_bytes():
    # M=4, N=100 (Np=112, 7 tiles), K=1024 (G=8): a 64 KB counter area, then
    # the partial sums of every slice.
    C = 65536
    t = lambda s: (0, 1, 4, 2, 0, s)
    assert w12.w12_gemm_workspace_bytes(4, 100, 1024, t(1)) == 0
    assert w12.w12_gemm_workspace_bytes(4, 100, 1024, t(0)) == 0
    assert w12.w12_gemm_workspace_bytes(4, 100, 1024, t(4)) == C + 4 * 4 * 112 * 4
    assert w12.w12_gemm_workspace_bytes(4, 100, 1024, t(3)) == C + 3 * 4 * 112 * 4  # 3+3+2
    assert w12.w12_gemm_workspace_bytes(4, 100, 1024, t(5)) == C + 4 * 4 * 112 * 4  # 2 each
    assert w12.w12_gemm_workspace_bytes(4, 100, 1024, t(64)) == C + 8 * 4 * 112 * 4
    assert w12.w12_gemm_workspace_bytes(4, 100, 1024, (1, 1, 1, 2, 0, 2)) == C + 2 * 4 * 112 * 4
    with pytest.raises(w12.W12Error):
        w12.w12_gemm_workspace_bytes(4, 100, 1000)
    with pytest.raises(w12.W12Error):
        w12.w12_gemm_workspace_bytes(4, 100, 1024, (0, 1, 4, 2, 0, 65))
    # at most 16384 row blocks may split K (one tile per workgroup with kw=4)
    assert w12.w12_gemm_workspace_bytes(1, 16384 * 16, 256, t(2)) == C + 2 * 16384 * 16 * 4
    with pytest.raises(w12.W12Error):
        w12.w12_gemm_workspace_bytes(1, 16384 * 16 + 1, 256, t(2))
    assert w12.w12_gemm_workspace_bytes(1, 16384 * 16 + 1, 256, t(1)) == 0
    assert w12.w12_default_tiling(1, 16384 * 16 + 1, 256).splitk == 1


def test_workspace_rejects():
    L = w12.lib()
    args = (A16, 4, 1024, A16, A16, A16, A16, None, None, 100, 1024, A16, 100, 0)
    t = w12._tiling_arg(w12.Tiling(0, 1, 4, 2, 0, 4))
    need = 65536 + 4 * 4 * 112 * 4
    assert L.w12_gemm_ex(*args, t, None, 0, None) == -8
    assert L.w12_gemm_ex(*args, t, A16, need - 1, None) == -8
    assert L.w12_gemm_ex(*args, t, P(4096 + 16), need, None) == -8   # not 256-byte aligned
    assert L.bf16_gemm_ex(A16, 4, 1024, A16, 100, 1024, A16, 100, 0, t, None, 0, None) == -8
    # a shape whose default splits K (M = 4): 4 tiles, 136 groups
    K = 17408
    assert w12.w12_default_tiling(4, 64, K).splitk == 3
    assert w12.w12_default_tiling(4, 64, K, allow_splitk=False).splitk == 1
    assert w12.w12_gemm_variant(4, 64, K).endswith("_s3")
    assert L.w12_gemm_ws(A16, 4, K, A16, A16, A16, A16, None, None, 64, K, A16, 64, 0, None, 0, None) == -8
    assert L.bf16_gemm_ws(A16, 4, K, A16, 64, K, A16, 64, 0, None, 0, None) == -8
    # argument errors still come first
    assert L.w12_gemm_ws(None, 4, K, A16, A16, A16, A16, None, None, 64, K, A16, 64, 0, None, 0, None) == -1
    assert L.w12_gemm_ws(A16, 129, K, A16, A16, A16, A16, None, None, 64, K, A16, 64, 0, None, 0, None) == -6


def test_default_split_rule():
    """MFMA: slices of at least 40 groups, and none once ~2048 workgroups
    fill the grid: the 40-group shapes never split, the 136-group down shape
    splits in three, a very tall long-K weight does not.  Small weights (at
    most 128 tiles, at least 20 groups) split in two at every M, the GEMV
    included; short rows (10-20 groups) on 257-512 tiles split in two up to
    8 rows; the LDS path above 16 rows takes at most two slices for
    filling the grid."""
    assert w12.w12_default_tiling(1, 7168, 5120).splitk == 1
    assert w12.w12_default_tiling(32, 34816, 5120).splitk == 1
    for M in (4, 8, 16, 32):
        assert w12.w12_default_tiling(M, 5120, 17408).splitk == 3
    # the M = 1 GEMV splits K only on small weights
    assert w12.w12_default_tiling(1, 5120, 17408).splitk == 1
    assert w12.w12_default_tiling(1, 640, 17408).splitk == 1     # 136 groups
    for N, K in ((896, 5120), (640, 2560)):
        for M in (1, 2, 8, 16, 32):
            t = w12.w12_default_tiling(M, N, K)
            assert t.splitk == 2 and t.x_direct == 1
    for M in (2, 4, 8):
        t = w12.w12_default_tiling(M, 5120, 2176)
        assert (t.kind, t.splitk, t.x_direct) == (1, 2, 1)
    assert w12.w12_default_tiling(16, 5120, 2176).splitk == 1
    for M in (24, 32):
        assert w12.w12_default_tiling(M, 4352, 5120).splitk == 2
    assert w12.w12_default_tiling(32, 5120 * 64, 17408).splitk == 1


def test_default_tiling():
    for split in (False, True):
        t = w12.w12_default_tiling(1, 7168, 5120, split)
        assert t.kind == 0 and t.astuple()[:5] in w12.GEMV_TILINGS and t.splitk >= 1
        t = w12.w12_default_tiling(16, 34816, 5120, split)
        assert t.kind == 1 and t.astuple()[:5] in w12.MFMA_TILINGS and t.splitk >= 1
        assert t.waves in (4, 8)
        if not split:
            assert t.splitk == 1
    with pytest.raises(w12.W12Error):
        w12.w12_default_tiling(129, 64, 512)


def test_default_waves_rule():
    """M = 2-8 (2-3 on 257-384 tiles with >= 40 groups, 2-6 above 1024
    tiles), M <= 32 on weights of <= 256 tiles, and M = 9-10 on weights of
    385-1024 tiles and <= 64 groups per row, read x directly in 256-thread
    workgroups (one tile per wave on <= 256 tiles, two above); otherwise x
    is staged in LDS for 512-thread workgroups: four K-waves when K is not
    split and M <= 16 (or the weight has < 128 row blocks), else two."""
    for M in (1, 2, 3):
        assert w12.w12_default_tiling(M, 5120, 17408).waves == 4
    # from 4 rows on 257-384 tiles with >= 40 groups x is staged in LDS
    for M in (4, 6):
        t = w12.w12_default_tiling(M, 5120, 17408)
        assert (t.waves, t.kw, t.x_direct, t.splitk) == (8, 2, 0, 3)
        t = w12.w12_default_tiling(M, 5120, 5120)
        assert (t.waves, t.kw, t.x_direct, t.splitk) == (8, 4, 0, 1)
    # 7-8 rows on 257-384 tiles with >= 40 groups stage x in LDS
    for M in (7, 8):
        assert w12.w12_default_tiling(M, 7168, 5120).waves == 4
        assert w12.w12_default_tiling(M, 5120, 5120).waves == 8
    # rows of <= 8 groups: two K-waves, x read directly, up to 32 rows
    for M in (2, 8, 16, 24, 32):
        t = w12.w12_default_tiling(M, 5120, 640)
        assert (t.waves, t.kw, t.x_direct, t.splitk) == (4, 2, 1, 1)
    # rows of 10-20 groups on 257-512 tiles: the same at 9-12 rows, x in LDS above
    for M in (9, 12):
        t = w12.w12_default_tiling(M, 5120, 2176)
        assert (t.waves, t.r, t.kw, t.x_direct, t.splitk) == (4, 1, 2, 1, 1)
    assert w12.w12_default_tiling(13, 5120, 2176).x_direct == 0
    t = w12.w12_default_tiling(8, 5120, 17408)
    assert (t.waves, t.kw, t.x_direct, t.splitk) == (8, 2, 0, 3)
    # 9-32 rows on long rows of 257-512 tiles: sixteen waves, four K-waves
    for M in (9, 16, 24, 32):
        t = w12.w12_default_tiling(M, 5120, 17408)
        assert (t.waves, t.kw, t.x_direct, t.splitk) == (16, 4, 0, 3)
    # above 1024 tiles from 7 rows, on 385-1024 tiles from 11 rows
    assert w12.w12_default_tiling(6, 34816, 5120).waves == 4
    assert w12.w12_default_tiling(7, 34816, 5120).waves == 8
    assert w12.w12_default_tiling(10, 7168, 5120).waves == 4
    assert w12.w12_default_tiling(11, 7168, 5120).waves == 8
    for M in (9, 16, 24, 32):
        t = w12.w12_default_tiling(M, 34816, 5120)
        assert (t.waves, t.kw, t.x_direct, t.splitk) == (8, 4 if M <= 16 else 2, 0, 1)
    for M in (9, 10):
        t = w12.w12_default_tiling(M, 7168, 5120)
        assert (t.waves, t.x_direct) == (4, 1)
        t = w12.w12_default_tiling(M, 5120, 5120)
        assert (t.waves, t.kw, t.x_direct, t.splitk) == (8, 4, 0, 1)
    t = w12.w12_default_tiling(16, 7168, 5120)
    assert (t.waves, t.kw, t.x_direct, t.splitk) == (8, 4, 0, 1)
    for M in (24, 32):
        for N in (7168, 5120):
            t = w12.w12_default_tiling(M, N, 5120)
            assert (t.waves, t.kw, t.splitk) == (8, 2, 2)
        t = w12.w12_default_tiling(M, 2048, 5120)
        assert (t.waves, t.r, t.kw, t.x_direct, t.splitk) == (4, 1, 4, 1, 2)
        t = w12.w12_default_tiling(M, 7168, 5120, False)
        assert (t.waves, t.kw, t.x_direct, t.splitk) == (8, 4, 0, 1)
        t = w12.w12_default_tiling(M, 5120, 17408, False)
        assert (t.waves, t.kw, t.splitk) == (8, 4, 1)


def test_default_small_weights():
    """Weights of <= 256 tiles: x direct, one tile per wave, four K-waves;
    at most 128 tiles with 20-64 groups split K in two at every M; otherwise
    from M = 9 K is split into up to 256 / tiles slices of >= 10 groups.
    Up to M = 6 weights of more than 512 tiles also take one tile per wave."""
    for M in (2, 4, 8):
        t = w12.w12_default_tiling(M, 896, 5120)
        assert (t.kind, t.r, t.kw, t.x_direct, t.waves, t.splitk) == (1, 1, 4, 1, 4, 2)
    for M in (9, 16, 32):
        assert w12.w12_default_tiling(M, 896, 5120).splitk == 2
        assert w12.w12_default_tiling(M, 896, 5120, False).splitk == 1
        assert w12.w12_default_tiling(M, 1536, 5120).splitk == 2
        assert w12.w12_default_tiling(M, 4096, 5120).splitk == 1
        assert w12.w12_default_tiling(M, 896, 2176).splitk == 1    # 17 groups
        assert w12.w12_default_tiling(M, 1024, 17408).splitk == 4
    # 257-512 tiles: two tiles per wave (at most 256 workgroups); above 512
    # tiles one again up to M = 6
    assert w12.w12_default_tiling(3, 4112, 5120).r == 2
    assert w12.w12_default_tiling(3, 4096, 5120).r == 1
    assert w12.w12_default_tiling(4, 8192, 5120).r == 2
    assert w12.w12_default_tiling(4, 8208, 5120).r == 1
    assert w12.w12_default_tiling(6, 34816, 5120).r == 1
    assert w12.w12_default_tiling(7, 16384, 5120).r == 2


def test_default_large_m():
    """M = 33-128: 64 or 128 padded rows in 512-thread workgroups with x in
    LDS.  On weights of >= 256 tiles one K-wave, K split into as many slices
    of >= 10 groups as fill 256 workgroups; a grid of >= 512 row blocks that
    K does not split takes two tiles per wave; smaller weights split K as
    above 16 rows."""
    t = w12.w12_default_tiling(64, 34816, 5120)
    assert (t.kind, t.waves, t.r, t.kw, t.x_direct, t.splitk) == (1, 8, 2, 1, 0, 1)
    t = w12.w12_default_tiling(64, 7168, 5120)
    assert (t.waves, t.kw, t.splitk) == (8, 1, 4)
    t = w12.w12_default_tiling(48, 5120, 17408)
    assert (t.waves, t.kw, t.splitk) == (8, 1, 6)
    t = w12.w12_default_tiling(64, 2048, 5120)
    assert (t.waves, t.kw, t.splitk) == (8, 2, 3)
    t = w12.w12_default_tiling(128, 34816, 5120)
    assert (t.waves, t.r, t.kw, t.splitk) == (8, 2, 1, 1)
    # without a workspace K is never split
    t = w12.w12_default_tiling(128, 7168, 5120, False)
    assert (t.waves, t.splitk) == (8, 1)
    for N, K in ((34816, 5120), (7168, 5120), (5120, 17408), (896, 5120)):
        t = w12.w12_default_tiling(128, N, K)
        assert (t.waves, t.kw, t.x_direct) == (8, 1, 0)
        assert t.r == (2 if N == 34816 else 1)
        assert w12.w12_gemm_variant(100, N, K).startswith("w12_mfma_mt128_")


def test_tiling_waves_rejects():
    """512-thread workgroups are built only for the MFMA with x in LDS, r = 1,
    depth 2 and kw <= 8; 1024-thread ones for the same with 2 <= kw <= 8 and
    at most 32 rows; 4 and 0 (= 4) are the other wave counts."""
    L = w12.lib()
    nbytes = ctypes.c_size_t()
    ok = (1, 1, 2, 2, 0, 1, 8)
    assert L.w12_gemm_workspace_bytes(16, 5120, 5120, w12._tiling_arg(ok), ctypes.byref(nbytes)) == 0
    for bad in ((0, 1, 2, 2, 0, 1, 8), (1, 2, 2, 2, 0, 1, 8), (1, 2, 1, 2, 0, 1, 8), (1, 1, 2, 4, 0, 1, 8),
                (1, 1, 2, 2, 1, 1, 8), (1, 1, 8, 2, 0, 1, 4), (1, 1, 2, 2, 0, 1, 6),
                (1, 1, 16, 2, 0, 1, 8), (1, 1, 1, 2, 0, 1, 16), (1, 2, 4, 2, 0, 1, 16),
                (1, 1, 4, 2, 1, 1, 16), (0, 1, 4, 2, 0, 1, 16), (1, 1, 4, 4, 0, 1, 16),
                (1, 1, 16, 2, 0, 1, 16), (1, 1, 4, 2, 0, 1, 12)):
        rc = L.w12_gemm_workspace_bytes(16, 5120, 5120, w12._tiling_arg(bad), ctypes.byref(nbytes))
        assert rc == -6, bad
    for ok16 in ((1, 1, 2, 2, 0, 1, 16), (1, 1, 4, 2, 0, 3, 16), (1, 1, 8, 2, 0, 1, 16)):
        assert L.w12_gemm_workspace_bytes(16, 5120, 5120, w12._tiling_arg(ok16),
                                          ctypes.byref(nbytes)) == 0, ok16
    # above 32 rows only 256- and 512-thread workgroups
    assert L.w12_gemm_workspace_bytes(33, 5120, 5120, w12._tiling_arg((1, 1, 4, 2, 0, 1, 16)),
                                      ctypes.byref(nbytes)) == -6


def test_read_probe_rejects():
    L = w12.lib()
    assert L.w12_read_probe(None, 16, A16, None) == -1
    assert L.w12_read_probe(A16, 16, None, None) == -1
    assert L.w12_read_probe(MIS, 16, A16, None) == -3
    assert L.w12_read_probe(A16, 24, A16, None) == -3
    assert L.w12_read_probe(A16, 16, P(4097), None) == -3
    assert L.w12_read_probe(A16, 0, A16, None) == -2


def test_w12b_entry_points_and_routing():
    """Every W12-v1 container call has its W12-b twin with the same
    signature, and the binding routes a W12-b container to it."""
    L = w12.lib()
    for name in ("pack", "unpack", "exceptions", "gemm", "gemm_ws", "gemm_ex"):
        fb, fv = getattr(L, "w12b_" + name), getattr(L, "w12_" + name)
        assert fb.argtypes == fv.argtypes and fb.restype == fv.restype
        assert w12._fmt_fn("b", "w12_" + name)[1] == "w12b_" + name
        assert w12._fmt_fn("v1", "w12_" + name)[1] == "w12_" + name
    with pytest.raises(ValueError):
        w12._fmt_fn("v2", "w12_gemm")
    # argument errors of the W12-b calls are the W12-v1 ones
    assert L.w12b_pack(None, 4, 128, A16, A16, A16, A16, None, None) == -1
    assert L.w12b_pack(A16, 4, 100, A16, A16, A16, A16, None, None) == -2
    assert L.w12b_unpack(A16, A16, A16, A16, None, None, 4, 128, MIS, None) == -3
    assert L.w12b_gemm(A16, 129, 512, A16, A16, A16, A16, None, None, 64, 512, A16, 64, 0,
                       None) == -6
    assert w12.w12_gemm_variant(1, 7168, 5120, 2).startswith("w12b_gemv_m1_")


def _noalloc(**kw):
    a = dict(x=A16, M=1, ldx=512, p0=A16, p1=A16, p2=A16, meta=A16, N=64, K=512, y=A16,
             ldy=64, yt=0)
    a.update(kw)
    return w12.lib().w12_gemm_noalloc(a["x"], a["M"], a["ldx"], a["p0"], a["p1"], a["p2"],
                                      a["meta"], a.get("eo"), a.get("ee"), a["N"], a["K"], a["y"],
                                      a["ldy"], a["yt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), -1), (dict(meta=None), -1), (dict(K=500), -2), (dict(M=0), -2),
    (dict(M=129), -6), (dict(yt=2), -4), (dict(x=MIS), -3), (dict(eo=A16), -1),
    # a default tiling whose split-K partial sums exceed the fixed 16 MiB
    # scratch: M = 32, N = 64000, K = 15360 splits K in three,
    # 3 * 32 * 64000 * 4 bytes = 23.4 MiB
    (dict(M=32, N=64000, K=15360, ldx=15360, ldy=64000), -9),
])
def test_noalloc_rejects_before_any_launch(kw, status):
    assert _noalloc(**kw) == status


def test_noalloc_scratch_covers_the_workloads():
    """Every M up to 128 on the four layer shapes fits the 16 MiB scratch
    (the default split-K partial sums, without the 64 KB counter area)."""
    for N, K in ((7168, 5120), (5120, 5120), (34816, 5120), (5120, 17408)):
        for M in (1, 2, 4, 8, 16, 32, 64, 128):
            need = w12.w12_gemm_workspace_bytes(M, N, K)
            assert need == 0 or need - 65536 <= 16 << 20, (N, K, M, need)
    assert w12.w12_gemm_workspace_bytes(128, 16384, 5120) - 65536 == 16 << 20   # fits exactly
    assert w12.w12_gemm_workspace_bytes(32, 64000, 15360) - 65536 > 16 << 20


def test_tiling_variant_names():
    """An explicit tiling's kernel name (for profiles of one variant): the
    same scheme as the defaults, None for a tiling the library rejects."""
    T = w12.w12_tiling_variant
    assert T(4, 7168, 5120, (0, 1, 2, 4, 1)) == "w12_gemv_m4_r1_kw2_d4_xdirect"
    assert T(4, 7168, 5120, (0, 1, 2, 4, 1), False) == "bf16_gemv_m4_r1_kw2_d4_xdirect"
    assert T(4, 7168, 5120, (0, 1, 2, 4, 1), 2) == "w12b_gemv_m4_r1_kw2_d4_xdirect"
    assert T(2, 7168, 5120, (1, 2, 4, 2, 1)) == w12.w12_gemm_variant(2, 7168, 5120)
    assert T(16, 7168, 5120, (1, 1, 4, 2, 0, 1, 8)) == w12.w12_gemm_variant(16, 7168, 5120)
    assert T(4, 7168, 5120, (0, 1, 2, 4, 1, 1, 8)) is None        # eight waves: MFMA only
    assert T(9, 7168, 5120, (0, 1, 2, 4, 1)) is None              # GEMV up to 8 rows
    assert T(4, 7168, 5000, (0, 1, 2, 4, 1)) is None              # K not a multiple of 128
