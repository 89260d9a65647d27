"""Host-side tests of the C ABI (no GPU): the library loads, exports every
declared symbol, and rejects bad arguments with the documented codes before
launching anything."""
import ctypes

import pytest

from dense_half_precision_amd import hgemm


@pytest.fixture(scope="module")
def lib():
    return hgemm.lib()


def test_exports_every_declared_symbol(lib):
    names = hgemm.declared_functions()
    assert {"hgemm_tn", "hgemm_nn", "hgemm_tn_ex", "hgemm_nn_ex"} <= set(names)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"declared but not exported: {missing}"


def test_version_and_status_strings(lib):
    assert lib.hgemm_version().decode().startswith("hgemm-gfx950")
    for code, text in ((0, "ok"), (1, "invalid argument"), (3, "HIP runtime error")):
        assert lib.hgemm_status_string(code).decode() == text
    assert lib.hgemm_status_string(99).decode() == "unknown status"
    assert lib.hgemm_last_hip_error() == 0


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails or the call is a no-op


@pytest.mark.parametrize("fn", [hgemm.hgemm_tn, hgemm.hgemm_nn])
def test_validation_codes(fn):
    inv, uns = hgemm.ERR_INVALID_ARG, hgemm.ERR_UNSUPPORTED
    assert fn(-1, 8, 8, 0, FAKE, FAKE, FAKE) == inv
    assert fn(8, -8, 8, 0, FAKE, FAKE, FAKE) == inv
    assert fn(8, 8, -8, 0, FAKE, FAKE, FAKE) == inv
    assert fn(8, 8, 8, 7, FAKE, FAKE, FAKE) == inv          # unknown dtype
    assert fn(8, 8, 8, 0, FAKE, FAKE, 0) == inv             # NULL C
    assert fn(8, 8, 8, 0, 0, FAKE, FAKE) == inv             # NULL A
    assert fn(8, 8, 8, 1, FAKE, 0, FAKE) == inv             # NULL B
    assert fn(8, 12, 8, 0, FAKE, FAKE, FAKE) == uns         # N % 8
    assert fn(8, 8, 12, 0, FAKE, FAKE, FAKE) == uns         # K % 8
    assert fn(8, 8, 8, 0, FAKE + 2, FAKE, FAKE) == uns      # misaligned A
    assert fn(8, 8, 8, 0, FAKE, FAKE + 8, FAKE) == uns      # misaligned B
    assert fn(8, 8, 8, 0, FAKE, FAKE, FAKE + 4) == uns      # misaligned C
    assert fn((1 << 30) + 1, 8, 8, 0, FAKE, FAKE, FAKE) == uns
    assert fn(8, (1 << 23) + 8, 8, 0, FAKE, FAKE, FAKE) == uns
    assert fn(8, 8, (1 << 21) + 8, 0, FAKE, FAKE, FAKE) == uns
    # empty outputs are no-ops and launch nothing, even with NULL pointers
    assert fn(0, 8, 8, 0, 0, 0, 0) == hgemm.OK
    assert fn(8, 0, 8, 1, 0, 0, 0) == hgemm.OK


def test_general_validation_codes():
    """hgemm_gemm: operation flags, leading dimensions, limits (nothing launches)."""
    g = hgemm.hgemm_gemm
    inv, uns, ok = hgemm.ERR_INVALID_ARG, hgemm.ERR_UNSUPPORTED, hgemm.OK
    N_, T_ = hgemm.OP_N, hgemm.OP_T
    M, N, K = 16, 24, 32
    # minimum leading dimensions per flag
    assert g(N_, N_, M, N, K, 0, 1, FAKE, K - 8, FAKE, N, 0, FAKE, N) == inv   # lda < K
    assert g(T_, N_, M, N, K, 0, 1, FAKE, M - 8, FAKE, N, 0, FAKE, N) == inv   # lda < M
    assert g(N_, N_, M, N, K, 0, 1, FAKE, K, FAKE, N - 8, 0, FAKE, N) == inv   # ldb < N
    assert g(N_, T_, M, N, K, 0, 1, FAKE, K, FAKE, K - 8, 0, FAKE, N) == inv   # ldb < K
    assert g(N_, N_, M, N, K, 0, 1, FAKE, K, FAKE, N, 0, FAKE, N - 8) == inv   # ldc < N
    assert g(2, N_, M, N, K, 0, 1, FAKE, K, FAKE, N, 0, FAKE, N) == inv        # bad flag
    assert g(N_, -1, M, N, K, 0, 1, FAKE, K, FAKE, N, 0, FAKE, N) == inv
    # multiples of 8 and limits
    assert g(N_, N_, M, N, K, 0, 1, FAKE, K + 4, FAKE, N, 0, FAKE, N) == uns   # lda % 8
    assert g(N_, N_, M, N, K, 0, 1, FAKE, K, FAKE, N, 0, FAKE, N + 4) == uns   # ldc % 8
    assert g(T_, N_, 12, N, K, 0, 1, FAKE, 16, FAKE, N, 0, FAKE, N) == uns     # M % 8, A^T
    assert g(N_, T_, M, N, K, 0, 1, FAKE, (1 << 22) + 8, FAKE, K, 0, FAKE, N) == uns
    assert g(T_, N_, M, N, K, 0, 1, FAKE, (1 << 23) + 8, FAKE, N, 0, FAKE, N) == uns
    assert g(N_, N_, M, N, K, 0, 1, FAKE, K, FAKE, (1 << 23) + 8, 0, FAKE, N) == uns
    assert g(N_, N_, M, N, K, 0, 1, FAKE, K, FAKE, N, 0, FAKE + 8, N) == uns   # misaligned C
    # empty output: a no-op even with NULL pointers
    assert g(T_, T_, 0, N, K, 0, 1, 0, K, 0, K, 0, 0, N) == ok
    # the register-staged baseline only takes packed operands, alpha 1, beta 0
    rs = hgemm.kernel_index("rs_tn_f16_256x256x64_xor")
    assert g(N_, T_, M, N, K, 0, 1, FAKE, K + 8, FAKE, K, 0, FAKE, N, kernel=rs) == uns
    assert g(N_, T_, M, N, K, 0, 2.0, FAKE, K, FAKE, K, 0, FAKE, N, kernel=rs) == uns
    # a kernel of another layout
    nn = hgemm.kernel_index("nn_f16_256x256x64")
    assert g(N_, T_, M, N, K, 0, 1, FAKE, K, FAKE, K, 0, FAKE, N, kernel=nn) == inv


def test_ex_config_validation():
    inv = hgemm.ERR_INVALID_ARG
    tab = hgemm.kernel_table()
    tn16 = next(k["index"] for k in tab if k["layout"] == hgemm.TN and k["dtype"] == hgemm.F16)
    nn16 = next(k["index"] for k in tab if k["layout"] == hgemm.NN and k["dtype"] == hgemm.F16)
    assert hgemm.hgemm_tn_ex(8, 8, 8, 0, FAKE, FAKE, FAKE, kernel=nn16) == inv  # wrong layout
    assert hgemm.hgemm_tn_ex(8, 8, 8, 1, FAKE, FAKE, FAKE, kernel=tn16) == inv  # wrong dtype
    assert hgemm.hgemm_tn_ex(8, 8, 8, 0, FAKE, FAKE, FAKE, kernel=len(tab)) == inv
    assert hgemm.hgemm_tn_ex(8, 8, 8, 0, FAKE, FAKE, FAKE, group_m=-1) == inv
    assert hgemm.hgemm_tn_ex(8, 8, 8, 0, FAKE, FAKE, FAKE, xcd_remap=2) == inv
    cfg = hgemm.Config(-1, 0, -1, 5)  # a K split needs a workspace
    st = hgemm.lib().hgemm_tn_ex(8, 8, 8, 0, FAKE, FAKE, FAKE, 0, ctypes.byref(cfg))
    assert st == inv


def test_split_workspace_size_and_validation():
    """The workspace the automatic K split asks for, and the refusals of a
    forced split, all decided on the host before any launch."""
    inv, uns = hgemm.ERR_INVALID_ARG, hgemm.ERR_UNSUPPORTED
    size = hgemm.gemm_ws_size
    # 7168^3: 28 x 28 = 784 tiles of 256 x 256 = 3 rounds of 256 CUs + a tail
    # of 16 tiles of 112 K steps; the estimate is least at 14 segments (224
    # of them, one wave), 256 KiB of partial sums each
    assert size(0, 1, 7168, 7168, 7168, "f16") == 16 * 14 * 256 * 256 * 4
    assert size(0, 0, 7168, 7168, 7168, "bf16") == 16 * 14 * 256 * 256 * 4
    # 6144^3: 576 tiles = 2 rounds + a tail of 64, but 192 x 256 tiles fill
    # three whole rounds and run unsplit as fast as the best split: no split,
    # no workspace
    assert size(0, 1, 6144, 6144, 6144, "f16") == 0
    assert size(0, 1, 8192, 8192, 8192, "f16") == 0      # 1024 tiles: whole rounds
    assert size(0, 1, 2048, 2048, 64, "f16") == 0        # one K step: nothing to split
    # 512 x 512 x 65536: 4 tiles, 1024 K steps: 64 segments each fill the CUs
    assert size(0, 1, 512, 512, 65536, "f16") == 4 * 64 * 256 * 256 * 4
    # 4352 x 4352 x 1024: a tail of 33 tiles of 16 steps; the 128 x 128 tile
    # without a split is estimated faster
    assert size(0, 1, 4352, 4352, 1024, "f16") == 0
    assert size(2, 1, 6144, 6144, 6144, "f16") == 0      # bad operation flag
    assert size(0, 1, 0, 6144, 6144, "f16") == 0
    assert size(0, 1, 6144, 6144, 6144, 5) == 0

    g = hgemm.hgemm_gemm_ws
    M = N = K = 6144
    need = 64 * 4 * 256 * 256 * 4  # a forced split in 4: the 64 tail tiles' partial sums

    def call(split, ws=FAKE, nbytes=need, kernel=None, m=M, n=N, k=K):
        return g(0, 1, m, n, k, "f16", 1.0, FAKE, k, FAKE, k, 0.0, FAKE, n, ws, nbytes,
                 kernel=kernel, split=split)
    assert call(1) == inv                       # one segment is no split
    assert call(-2) == inv
    assert call(4, ws=0, nbytes=0) == inv       # a forced split needs a workspace
    assert call(4, ws=FAKE + 8) == uns          # workspace not 16-byte aligned
    assert call(4, nbytes=need - 1) == uns      # too small for the forced split
    assert call(97, nbytes=1 << 40) == uns      # more segments than the 96 K steps
    assert call(4, m=8192, n=8192, k=8192) == uns  # no tail to split
    k128 = hgemm.kernel_index("tn_f16_128x128x64")
    assert call(4, kernel=k128) == uns          # the split runs the 256 x 256 kernels only
    kp = hgemm.kernel_index("tn_f16_256x256x64_persist")
    assert call(4, kernel=kp) == uns            # ... that have K-segment launches
    kws = hgemm.kernel_index("ws_tn_f16_128x256x64")
    assert call(4, kernel=kws) == uns


def test_noalloc_refusals_on_the_host():
    """hgemm_gemm_noalloc validates like hgemm_gemm and refuses, before any
    HIP call, a shape whose automatic K split needs more partial-sum bytes
    than the library's static scratch holds."""
    f = hgemm.lib().hgemm_gemm_noalloc
    lim = hgemm.NOALLOC_SCRATCH_BYTES
    size = hgemm.gemm_ws_size

    def call(m, n, k, opA=0, opB=1, dt=0, lda=None, ldb=None, ldc=None, ptr=FAKE):
        lda = lda if lda is not None else (m if opA else k)
        ldb = ldb if ldb is not None else (k if opB else n)
        return f(opA, opB, m, n, k, dt, 1.0, ptr, lda, ptr, ldb, 0.0, ptr,
                 ldc if ldc is not None else n, 0)
    assert hgemm.lib().hgemm_status_string(hgemm.ERR_SCRATCH).decode().startswith("the K split")
    # over the limit: 2560^2 x 16384 is 100 tiles of 256 K steps, split in 5
    over = [(m, n, k) for (m, n, k) in ((2560, 2560, 16384), (2048, 3072, 16384))
            if size(0, 1, m, n, k, "f16") > lim]
    assert over, "no shape over the scratch limit among the candidates"
    for m, n, k in over:
        assert call(m, n, k) == hgemm.ERR_SCRATCH
    assert size(0, 1, 4096, 4608, 6144, "f16") == lim  # exactly the limit: accepted (GPU test)
    assert call(-1, 8, 8) == hgemm.ERR_INVALID_ARG
    assert call(8, 8, 8, opA=2) == hgemm.ERR_INVALID_ARG
    assert call(8, 8, 8, dt=7) == hgemm.ERR_INVALID_ARG
    assert call(8, 12, 8) == hgemm.ERR_UNSUPPORTED       # N % 8
    assert call(8, 8, 8, ptr=FAKE + 2) == hgemm.ERR_UNSUPPORTED
    assert call(0, 8, 8) == hgemm.OK                      # empty: nothing to do


def test_kernel_table_and_auto_choice():
    tab = hgemm.kernel_table()
    assert len(tab) == hgemm.lib().hgemm_kernel_count() > 0
    assert hgemm.lib().hgemm_kernel_info(len(tab), None, None, None, None, None) is None
    for k in tab:
        assert k["layout"] in (0, 1, 2, 3) and k["dtype"] in (0, 1) and k["bk"] == 64
        lay = ("tn", "nn", "at_tn", "at_nn")[k["layout"]]
        stem = k["name"][3:] if k["name"][:3] in ("rs_", "ws_") else k["name"]
        assert stem.startswith(f"{lay}_{'f16' if k['dtype'] == 0 else 'bf16'}_")
    # every layout/dtype has an automatic choice, matching layout and dtype
    for lay in (0, 1, 2, 3):
        for dt in (0, 1):
            for M, N in ((1, 8), (512, 512), (2048, 2048), (8192, 8192)):
                i = hgemm.auto_kernel(lay, dt, M, N, 64)
                assert 0 <= i < len(tab)
                assert tab[i]["layout"] == lay and tab[i]["dtype"] == dt
    assert hgemm.auto_kernel(4, 0, 8, 8, 8) == -1
    assert hgemm.auto_kernel(0, 0, 0, 8, 8) == -1
    # the large configurations get the 256 x 256 tile, the square 2048 the 128 one
    assert tab[hgemm.auto_kernel(0, 0, 8192, 8192, 8192)]["bm"] == 256
    assert tab[hgemm.auto_kernel(1, 1, 4096, 4096, 4096)]["bm"] == 256
    assert tab[hgemm.auto_kernel(0, 0, 2048, 2048, 2048)]["bm"] == 128
    # one round of 128 x 128 tiles (at most 256) over 24 or more K steps takes
    # the ring with one more stage per operand; more rounds, or fewer steps, not
    assert tab[hgemm.auto_kernel(0, 0, 2048, 2048, 2048)]["name"] == "tn_f16_128x128x64_r3"
    assert tab[hgemm.auto_kernel(3, 1, 1536, 1536, 1536)]["name"] == "at_nn_bf16_128x128x64_r3"
    assert tab[hgemm.auto_kernel(1, 1, 2048, 2048, 1472)]["name"] == "nn_bf16_128x128x64"
    # tiles that share CUs (more tiles than CUs) run at the measured shared
    # rates: 1024^3 stays 64 x 64; 2048 x 2048 x 8192 takes one round of the
    # deeper-ring 128 x 128 kernel (28 % faster than 256 x 128)
    assert tab[hgemm.auto_kernel(0, 0, 1024, 1024, 1024)]["name"] == "tn_f16_64x64x64"
    # four 64 x 64 workgroups sharing a CU overlap their prologues and
    # epilogues: 468 of them beat 117 tiles of 128 x 128 (14 % measured)
    assert tab[hgemm.auto_kernel(0, 0, 1152, 1664, 1472)]["name"] == "tn_f16_64x64x64"
    # a single round of 64 x 64 tiles whose A and B pass 6 MiB takes the ring
    # with 5 A + 4 B stages (1.5-1.8x faster measured there); under it, or with
    # more tiles than CUs, the default ring
    assert tab[hgemm.auto_kernel(0, 0, 512, 512, 8192)]["name"] == "tn_f16_64x64x64_r4"
    assert tab[hgemm.auto_kernel(0, 0, 640, 640, 3072)]["name"] == "tn_f16_64x64x64_r4"
    assert tab[hgemm.auto_kernel(1, 1, 1024, 1024, 16384)]["name"] == "nn_bf16_64x64x64_r4"
    assert tab[hgemm.auto_kernel(3, 0, 512, 512, 65536)]["name"] == "at_nn_f16_64x64x64_r4"
    assert tab[hgemm.auto_kernel(0, 0, 512, 512, 2048)]["name"] == "tn_f16_64x64x64"
    assert tab[hgemm.auto_kernel(0, 0, 768, 768, 2048)]["name"] == "tn_f16_64x64x64"
    assert tab[hgemm.auto_kernel(0, 0, 2048, 2048, 8192)]["name"] == "tn_f16_128x128x64_r3"
    # one round of 256 x 128 tiles where 128 x 128 tiles would take two: the
    # measured sweeps put it 6-15 % ahead of every square tile on these
    assert tab[hgemm.auto_kernel(0, 0, 1024, 8192, 8192)]["name"] == "tn_f16_256x128x64"
    assert tab[hgemm.auto_kernel(0, 0, 8192, 1024, 8192)]["name"] == "tn_f16_256x128x64"
    assert tab[hgemm.auto_kernel(1, 1, 1024, 8192, 8192)]["name"] == "nn_bf16_256x128x64"
    for s in (2304, 2560, 2816):
        assert tab[hgemm.auto_kernel(0, 0, s, s, s)]["name"] == "tn_f16_256x128x64", s
    # tiles of 192 rows or columns where they fill the CUs better than 256 x 256
    # ones (3-27 % ahead of every other tile on the sweeps), in every layout:
    # 256 x 192, and 192 x 192 where it fills whole rounds (3072^2: 256 tiles)
    for M, N, K in ((6144, 6144, 6144), (4608, 4608, 4608), (6000, 6000, 3000),
                    (7000, 5000, 4000)):
        assert tab[hgemm.auto_kernel(0, 0, M, N, K)]["name"] == "tn_f16_256x192x64", (M, N, K)
        assert tab[hgemm.auto_kernel(1, 1, M, N, K)]["name"] == "nn_bf16_256x192x64", (M, N, K)
        assert tab[hgemm.auto_kernel(3, 0, M, N, K)]["name"] == "at_nn_f16_256x192x64", (M, N, K)
    for layout, prefix in ((0, "tn_f16"), (1, "nn_f16"), (2, "at_tn_f16"), (3, "at_nn_f16")):
        assert tab[hgemm.auto_kernel(layout, 0, 3072, 3072, 3072)]["name"] == f"{prefix}_192x192x64"
    assert tab[hgemm.auto_kernel(0, 1, 1536, 12288, 4096)]["name"] == "tn_bf16_192x192x64"
    assert tab[hgemm.auto_kernel(1, 1, 1536, 12288, 4096)]["name"] == "nn_bf16_192x192x64"
    # and not where the 256 x 256 tile was faster on the same sweeps
    for s in (4096, 5120, 8192):
        assert tab[hgemm.auto_kernel(0, 0, s, s, s)]["name"] == "tn_f16_256x256x64", s
    assert tab[hgemm.auto_kernel(0, 0, 256, 16384, 4096)]["name"] == "tn_f16_128x128x64_r3"
    # two 128 x 128 workgroups sharing a CU: (KT - 1) steps a round at rate 0.56,
    # which wins at a few K steps and loses to one round of 192 x 192 tiles at
    # many (the six choices the refit moved, each to the faster kernel measured)
    assert tab[hgemm.auto_kernel(0, 0, 4096, 4096, 256)]["name"] == "tn_f16_128x128x64"
    assert tab[hgemm.auto_kernel(1, 1, 4096, 4096, 256)]["name"] == "nn_bf16_128x128x64"
    assert tab[hgemm.auto_kernel(1, 1, 8000, 1280, 576)]["name"] == "nn_bf16_128x128x64"
    assert tab[hgemm.auto_kernel(1, 1, 10688, 5248, 512)]["name"] == "nn_bf16_128x128x64"
    assert tab[hgemm.auto_kernel(1, 1, 1344, 11584, 4416)]["name"] == "nn_bf16_192x192x64"
    assert tab[hgemm.auto_kernel(1, 1, 1152, 7168, 9664)]["name"] == "nn_bf16_192x192x64"
    # and K = 1024 on the same 4096^2 stays with 256 x 256 (14 % ahead there)
    assert tab[hgemm.auto_kernel(0, 0, 4096, 4096, 1024)]["name"] == "tn_f16_256x256x64"


@pytest.mark.parametrize("tiles_m,tiles_n", [(1, 1), (2, 2), (3, 5), (32, 32), (16, 16), (8, 8),
                                              (5, 33), (33, 7), (4, 64), (128, 2)])
@pytest.mark.parametrize("group_m", [1, 3, 8, 16])
@pytest.mark.parametrize("xcd", [0, 1])
def test_tile_order_is_a_bijection(tiles_m, tiles_n, group_m, xcd):
    """Every workgroup computes a distinct in-range tile and every tile is
    computed (the kernels' own mapping, run on the host)."""
    tm, tn = hgemm.tile_order(tiles_m, tiles_n, group_m, xcd)
    assert all(0 <= a < tiles_m for a in tm) and all(0 <= b < tiles_n for b in tn)
    assert len(set(zip(tm, tn))) == tiles_m * tiles_n


def test_tile_order_locality():
    """With the XCD remap, the 32 workgroups an XCD runs at once (ids x, x+8,
    x+16, ...) cover a compact block of tiles: at most 8 tile rows and 4 tile
    columns for an 8192^2 output of 256^2 tiles and group_m = 8."""
    tm, tn = hgemm.tile_order(32, 32, 8, 1)
    for x in range(8):
        ids = [x + 8 * j for j in range(32)]
        rows = {tm[i] for i in ids}
        cols = {tn[i] for i in ids}
        assert len(rows) <= 8 and len(cols) <= 4, (x, sorted(rows), sorted(cols))
