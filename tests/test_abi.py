"""C-ABI checks that need no GPU: exports, status codes, argument validation,
plan registry and the workgroup -> tile schedule (the kernels' own map, evaluated on the host)."""
import ctypes
import os
import re

import pytest

import attention_scores_amd as asl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_scores.h")


def _declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"AS_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)))


def test_header_declares_binding_names():
    assert _declared_functions() == sorted(asl.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = asl.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    # and nothing else is exported with C linkage beyond the header's names
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", asl.LIB_PATH], capture_output=True, text=True).stdout
    text_syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert text_syms == set(_declared_functions())


def test_status_strings():
    assert asl.as_status_str(0) == "AS_OK"
    assert asl.as_status_str(1) == "AS_ERR_INVALID"
    assert asl.as_status_str(2) == "AS_ERR_UNSUPPORTED"
    assert asl.as_status_str(3) == "AS_ERR_HIP"
    assert asl.as_status_str(4) == "AS_ERR_NOMEM"
    assert asl.as_status_str(99) == "AS_UNKNOWN_STATUS"


def _status(fn, *args):
    try:
        fn(*args)
    except asl.AsError as e:
        return e.status
    return asl.AS_OK


RM = lambda r, c: (c, 1, 0)   # row-major r x c


@pytest.mark.parametrize("M,N,K,batch", [(0, 512, 512, 1), (512, -1, 512, 1), (512, 512, 0, 1), (512, 512, 512, 0)])
def test_create_rejects_bad_sizes(M, N, K, batch):
    st = _status(asl.gemm_create, M, N, K, batch, (max(K, 8), 1, 0), (max(N, 8), 1, 0), (max(N, 8), 1, 0))
    assert st == asl.AS_ERR_INVALID


def test_create_rejects_bad_flags_and_dtypes():
    args = (512, 512, 512, 1, RM(512, 512), RM(512, 512), RM(512, 512))
    assert _status(asl.gemm_create, *args, asl.AS_BF16, asl.AS_BF16, asl.AS_F32, 0x1000) == asl.AS_ERR_INVALID
    assert _status(asl.gemm_create, *args, asl.AS_BF16, asl.AS_BF16, asl.AS_F32,
                   asl.AS_FLAG_TILE_128 | asl.AS_FLAG_TILE_256) == asl.AS_ERR_INVALID
    assert _status(asl.gemm_create, *args, asl.AS_BF16, asl.AS_BF16, asl.AS_F32,
                   asl.AS_FLAG_NT_A | asl.AS_FLAG_NO_NT_A) == asl.AS_ERR_INVALID
    assert _status(asl.gemm_create, *args, asl.AS_BF16, asl.AS_BF16, asl.AS_F32,
                   asl.AS_FLAG_ROTATE_K | asl.AS_FLAG_NO_ROTATE_K) == asl.AS_ERR_INVALID
    assert _status(asl.gemm_create, *args, asl.AS_BF16, asl.AS_BF16, 7, 0) == asl.AS_ERR_INVALID
    assert _status(asl.gemm_create, *args, asl.AS_F32, asl.AS_BF16, asl.AS_F32, 0) == asl.AS_ERR_UNSUPPORTED
    assert _status(asl.gemm_create, *args, asl.AS_BF16, asl.AS_F32, asl.AS_F32, 0) == asl.AS_ERR_UNSUPPORTED


def test_create_rejects_bad_strides():
    base = dict(M=512, N=512, K=512, batch=1)
    mk = lambda a, b, c, batch=1: _status(asl.gemm_create, 512, 512, 512, batch, a, b, c)
    assert mk((-512, 1, 0), RM(512, 512), RM(512, 512)) == asl.AS_ERR_INVALID        # negative
    assert mk((512, 2, 0), RM(512, 512), RM(512, 512)) == asl.AS_ERR_UNSUPPORTED      # no unit stride
    assert mk((516, 1, 0), RM(512, 512), RM(512, 512)) == asl.AS_ERR_UNSUPPORTED      # ld % 8
    assert mk(RM(512, 512), (512, 2, 0), RM(512, 512)) == asl.AS_ERR_UNSUPPORTED
    assert mk(RM(512, 512), RM(512, 512), (512, 2, 0)) == asl.AS_ERR_UNSUPPORTED      # C col stride
    assert mk(RM(512, 512), RM(512, 512), (256, 1, 0)) == asl.AS_ERR_INVALID          # C rows overlap
    assert mk(RM(512, 512), RM(512, 512), (512, 1, 0), batch=2) == asl.AS_ERR_INVALID  # C batches overlap
    assert mk(RM(512, 512), RM(512, 512), (514, 1, 0)) == asl.AS_ERR_UNSUPPORTED      # C row alignment
    del base


@pytest.mark.parametrize("M,N,K", [(512, 512, 100), (384, 384, 4), (1, 1, 12)])
def test_create_refuses_k_not_a_multiple_of_8(M, N, K):
    st = _status(asl.gemm_create, M, N, K, 1, (K + (-K) % 8, 1, 0), (N + (-N) % 8, 1, 0), (N + (-N) % 8, 1, 0))
    assert st == asl.AS_ERR_UNSUPPORTED
    assert "multiple of 8" in asl.as_last_error()


@pytest.mark.parametrize("M,N,K,tile", [(500, 512, 512, 64), (512, 520, 512, 64), (512, 512, 80, 64),
                                        (1, 1, 8, 64), (8000, 8000, 8000, 256), (8100, 8000, 4096, 256),
                                        (4224, 4224, 4096, 128), (2048, 1024, 512, 128)])
def test_ragged_shapes_plan_partial_tiles(M, N, K, tile):
    # M and N need not be multiples of the tile nor K of the 64-deep stage:
    # edge tiles are partial, the tile count rounds up.
    p = asl.gemm_create(M, N, K, 1, (K + (-K) % 8, 1, 0), (N + (-N) % 8, 1, 0), (N + (-N) % 8, 1, 0))
    tm, tn, tk, tiles, _ = asl.gemm_plan_info(p)
    assert (tm, tn, tk) == (tile, tile, 64)
    assert tiles == -(-M // tm) * -(-N // tn)
    asl.gemm_destroy(p)


def test_create_refuses_huge_leading_stride():
    # 256 rows of a K-major tile at ld = 2^23 elements overflow 32-bit offsets
    st = _status(asl.gemm_create, 8192, 8192, 8192, 1, (1 << 23, 1, 0), RM(8192, 8192), RM(8192, 8192))
    assert st == asl.AS_ERR_UNSUPPORTED


def test_plan_registry_and_run_argument_checks():
    p = asl.gemm_create(512, 512, 512, 1, RM(512, 512), RM(512, 512), RM(512, 512))
    assert asl.gemm_plan_info(p) == (64, 64, 64, 64, 64)
    assert _status(asl.gemm_run, p, 0, 0, 0) == asl.AS_ERR_INVALID
    assert _status(asl.gemm_run, p, 16, 32, 0) == asl.AS_ERR_INVALID
    assert _status(asl.gemm_run, p, 8, 16, 32) == asl.AS_ERR_UNSUPPORTED          # misaligned
    assert _status(asl.gemm_run, p + 8, 16, 32, 48) == asl.AS_ERR_INVALID         # unknown plan
    assert _status(asl.gemm_run, 0, 16, 32, 48) == asl.AS_ERR_INVALID
    asl.gemm_destroy(p)
    assert _status(asl.gemm_destroy, p) == asl.AS_ERR_INVALID                     # double destroy
    assert _status(asl.gemm_run, p, 16, 32, 48) == asl.AS_ERR_INVALID             # destroyed plan
    assert _status(asl.gemm_destroy, 0) == asl.AS_ERR_INVALID
    L = asl.lib()
    assert L.gemm_create(None, 512, 512, 512, 1, asl.Strides(512, 1, 0), asl.Strides(512, 1, 0),
                         asl.Strides(512, 1, 0), 0, 0, 1, 0) == asl.AS_ERR_INVALID


def test_last_error_is_per_call():
    _status(asl.gemm_create, 0, 1, 1, 1, (8, 1, 0), (8, 1, 0), (8, 1, 0))
    assert "positive" in asl.as_last_error()
    p = asl.gemm_create(512, 512, 512, 1, RM(512, 512), RM(512, 512), RM(512, 512))
    assert asl.as_last_error() == ""
    asl.gemm_destroy(p)


def test_tile_choice():
    p = asl.gemm_create(8192, 8192, 8192, 1, RM(8192, 8192), RM(8192, 8192), RM(8192, 8192), c_t=asl.AS_BF16)
    assert asl.gemm_plan_info(p) == (256, 256, 64, 1024, 256)   # one resident workgroup per CU
    asl.gemm_destroy(p)
    p = asl.gemm_create(8192, 8192, 8192, 1, RM(8192, 8192), RM(8192, 8192), RM(8192, 8192), c_t=asl.AS_BF16,
                        flags=asl.AS_FLAG_ONE_TILE_PER_WORKGROUP)
    assert asl.gemm_plan_info(p) == (256, 256, 64, 1024, 1024)
    asl.gemm_destroy(p)
    p = asl.gemm_create(512, 512, 512, 1, RM(512, 512), RM(512, 512), RM(512, 512), flags=asl.AS_FLAG_TILE_256)
    assert asl.gemm_plan_info(p)[0] == 256
    asl.gemm_destroy(p)
    p = asl.gemm_create(65536, 256, 4096, 1, RM(65536, 4096), RM(4096, 256), RM(65536, 256))
    assert asl.gemm_plan_info(p) == (256, 256, 64, 256, 256)
    asl.gemm_destroy(p)
    # small grids that cannot split K: 64 tiles, as many as the CUs at most
    for (M, N, K, batch), want in (((512, 512, 512, 1), (64, 64, 64, 64, 64)),
                                   ((512, 512, 512, 3), (64, 64, 64, 192, 192)),
                                   ((1024, 1024, 1024, 1), (64, 64, 64, 256, 256)),
                                   ((1024, 1152, 1024, 1), (128, 128, 64, 72, 72)),     # 288 tiles of 64
                                   ((1024, 1024, 4096, 1), (128, 128, 64, 64, 256))):   # splits K in 4
        p = asl.gemm_create(M, N, K, batch, (K, 1, M * K), (N, 1, K * N), (N, 1, M * N))
        assert asl.gemm_plan_info(p) == want, (M, N, K, batch)
        asl.gemm_destroy(p)
    assert _status(asl.gemm_create, 512, 512, 512, 1, RM(512, 512), RM(512, 512), RM(512, 512), asl.AS_BF16,
                   asl.AS_BF16, asl.AS_F32, asl.AS_FLAG_TILE_64 | asl.AS_FLAG_TILE_128) == asl.AS_ERR_INVALID


SHAPES = [  # (M, N, K, batch, flags)
    (8192, 8192, 8192, 1, 0),                             # 1024 tiles over 256 workgroups
    (2048, 2048, 128, 32, 0),                             # 8192 tiles of 128 over 512
    (65536, 256, 4096, 1, 0),
    (16384, 8192, 2048, 1, 0),
    (640, 384, 64, 1, 0),          # 15 tiles: not a multiple of the 8 XCDs
    (512, 512, 512, 3, asl.AS_FLAG_TILE_128),
    (1024, 768, 256, 5, 0),
    (8192, 8192, 8256 - 64, 1, asl.AS_FLAG_ONE_TILE_PER_WORKGROUP),
    (4096, 6144, 1024, 3, 0),                             # 1152 tiles over 256 (not a multiple)
    (2048, 2048, 128, 7, 0),                              # 1792 tiles of 128 over 512 workgroups
    (2048, 2048, 128, 7, asl.AS_FLAG_ONE_TILE_PER_WORKGROUP),
    (8192, 8192, 8192, 1, asl.AS_FLAG_NO_GROUPING),
    (8192, 8192, 8192, 1, asl.AS_FLAG_NO_XCD_SPLIT),
    (2048, 2048, 128, 7, asl.AS_FLAG_NO_XCD_SPLIT),
    (1000, 3000, 96, 3, 0),                               # ragged: partial edge tiles
    (4100, 4104, 520, 2, asl.AS_FLAG_TILE_256),
]


@pytest.mark.parametrize("M,N,K,batch,flags", SHAPES)
def test_schedule_is_a_bijection(M, N, K, batch, flags):
    p = asl.gemm_create(M, N, K, batch, (K, 1, M * K), (N, 1, K * N), (N, 1, M * N), flags=flags)
    tm, tn, _, wg, grid = asl.gemm_plan_info(p)
    tiles_m, tiles_n = -(-M // tm), -(-N // tn)
    assert wg == batch * tiles_m * tiles_n
    assert grid == (wg if flags & asl.AS_FLAG_ONE_TILE_PER_WORKGROUP else min(wg, 256 if tm == 256 else 512))
    seen = set()
    for h in range(wg):
        b, r, c = asl.gemm_plan_tile_of(p, h)
        assert 0 <= b < batch and 0 <= r < tiles_m and 0 <= c < tiles_n
        seen.add((b, r, c))
    assert len(seen) == wg
    assert _status(asl.gemm_plan_tile_of, p, wg) == asl.AS_ERR_INVALID
    asl.gemm_destroy(p)


def _slot_model(slot, P, tiles, tiles_m, tiles_n, gm, grouped, xcd_split):
    """Execution slot -> (batch, tile row, tile column) written out with plain
    integer division: XCD x owns the contiguous range [x*q + min(x, r), ...)
    of q or q+1 logical tiles and its workgroups stride through it; logical
    tiles walk bands of gm tile rows column by column (a partial last band
    keeps its own height)."""
    h, j = slot % P, slot // P
    if xcd_split:
        x, s = h % 8, h // 8
        q, r = divmod(tiles, 8)
        start, count = x * q + min(x, r), q + (1 if x < r else 0)
        first, stride, end = start + s, P // 8 + (1 if x < P % 8 else 0), start + count
    else:
        first, stride, end = h, P, tiles
    L = first + j * stride
    if L >= end:
        return None
    b, t = divmod(L, tiles_m * tiles_n)
    if not grouped:
        return b, t // tiles_n, t % tiles_n
    band, inn = divmod(t, gm * tiles_n)
    top = band * gm
    height = min(tiles_m - top, gm)
    return b, top + inn % height, inn // height


@pytest.mark.parametrize("M,N,K,batch,flags,nsample", [
    (1000, 3000, 96, 3, 0, None),                         # 8 x 24 tiles of 128, batch 3, bands of 8
    (7680, 8192, 8192, 1, 0, None),                       # 30 x 32 tiles of 256, bands of 4: last band 2
    (7936, 6144, 4096, 1, 0, None),                       # 31 x 24, bands of 4: last band 3
    (2600, 4096, 128, 3, 0, None),                        # 21 x 32 tiles of 128 x 3, bands of 16: last band 5
    (2000, 9000, 1024, 1, asl.AS_FLAG_TILE_128, None),    # 16 x 71
    (2048, 2048, 128, 7, asl.AS_FLAG_NO_XCD_SPLIT, None),
    (3000, 3000, 1024, 2, asl.AS_FLAG_NO_GROUPING, None),
    (1000000, 999936, 1024, 1, 0, 4000),                  # 3907 x 3906 tiles: a divisor near 2^24, last band 3
    (1000000, 2000, 512, 700, asl.AS_FLAG_TILE_128, 4000),  # 7813 x 16 x 700 tiles: dividends near 2^26
])
def test_tile_map_equals_the_plain_division_definition(M, N, K, batch, flags, nsample):
    # The kernels map a logical tile to its coordinates with multiply-high
    # division by divisors prepared on the host; gemm_plan_tile_of evaluates
    # that same map.  Compare it with the definition written with plain
    # integer division, for the plan's group size (one of 1, 2, 4, ..., 64).
    import random
    p = asl.gemm_create(M, N, K, batch, (K, 1, M * K), (N, 1, K * N), (N, 1, M * N), flags=flags)
    tm, tn, _, wg, grid = asl.gemm_plan_info(p)
    assert asl.gemm_plan_split_k(p)[0] == 1
    tiles_m, tiles_n = -(-M // tm), -(-N // tn)
    rng = random.Random(M ^ N ^ batch)
    slots = range(wg) if nsample is None else sorted({0, wg - 1, *(rng.randrange(wg) for _ in range(nsample))})
    got = {h: asl.gemm_plan_tile_of(p, h) for h in slots}
    asl.gemm_destroy(p)
    grouped = not flags & asl.AS_FLAG_NO_GROUPING
    xcd_split = grouped and not flags & asl.AS_FLAG_NO_XCD_SPLIT
    matches = [gm for gm in (1, 2, 4, 8, 16, 32, 64) if gm <= tiles_m and all(
        _slot_model(h, grid, wg, tiles_m, tiles_n, gm, grouped, xcd_split) == got[h] for h in slots)]
    assert matches, (M, N, K, batch, flags)


def _wave_panels(p, wg, cus_per_xcd=32):
    """Largest number of (batch, tile row) + (batch, tile col) panels that the
    workgroups of one XCD running together (32 consecutive slots) touch."""
    worst = 0
    for x in range(8):
        hs = list(range(x, wg, 8))
        for w0 in range(0, len(hs), cus_per_xcd):
            rows, cols = set(), set()
            for h in hs[w0:w0 + cus_per_xcd]:
                b, r, c = asl.gemm_plan_tile_of(p, h)
                rows.add((b, r))
                cols.add((b, c))
            worst = max(worst, len(rows) + len(cols))
    return worst


@pytest.mark.parametrize("M,N,K,sa", [(8192, 8192, 8192, (8192, 1, 0)), (16384, 8192, 2048, (1, 16384, 0))])
def test_concurrent_tiles_touch_few_panels(M, N, K, sa):
    # 32 tiles that run at once on an XCD can touch as few as 4 A + 8 B (or
    # 8 + 4) panels; the plan's group size must reach that minimum.
    p = asl.gemm_create(M, N, K, 1, sa, (N, 1, 0), (N, 1, 0), c_t=asl.AS_BF16)
    assert asl.gemm_plan_info(p)[0] == 256
    assert _wave_panels(p, asl.gemm_plan_info(p)[3]) <= 12
    asl.gemm_destroy(p)


def test_xcd_split_is_what_keeps_a_wave_of_tiles_on_few_panels():
    # 8192^3: 32 tiles running together on an XCD touch 12 panels under the
    # default order and under the identity (whose row-major walk happens to
    # give each XCD four whole tile columns, 32 being a multiple of 8), but
    # 18 under the band order without the XCD split: a 4-row band's
    # consecutive tiles run on 8 different XCDs, so XCD 0 takes row 0 and row
    # 4 of two bands at every other column (2 A + 16 B panels).
    got = {}
    for flags in (0, asl.AS_FLAG_NO_GROUPING, asl.AS_FLAG_NO_XCD_SPLIT):
        p = asl.gemm_create(8192, 8192, 8192, 1, (8192, 1, 0), (8192, 1, 0), (8192, 1, 0), c_t=asl.AS_BF16,
                            flags=flags)
        got[flags] = _wave_panels(p, asl.gemm_plan_info(p)[3])
        asl.gemm_destroy(p)
    assert got[0] == 12 and got[asl.AS_FLAG_NO_GROUPING] == 12
    assert got[asl.AS_FLAG_NO_XCD_SPLIT] == 18


def test_grouping_keeps_slices_on_one_xcd_identity_spreads_them():
    args = (2048, 2048, 128, 32, (128, 1, 2048 * 128), (1, 128, 2048 * 128), (2048, 1, 2048 * 2048))
    for flags, want in ((0, 4), (asl.AS_FLAG_NO_GROUPING, 32)):
        p = asl.gemm_create(*args, flags=flags)
        wg = asl.gemm_plan_info(p)[3]
        per_xcd = [set() for _ in range(8)]
        for h in range(wg):
            per_xcd[h % 8].add(asl.gemm_plan_tile_of(p, h)[0])
        assert all(len(sl) == want for sl in per_xcd), (flags, [len(sl) for sl in per_xcd])
        asl.gemm_destroy(p)


def test_attention_scores_share_whole_slices_per_xcd():
    # 32 slices of 2048x2048 scores, 256 tiles of 128x128 per slice: every
    # XCD computes 4 whole slices, so each slice's Q and K are fetched by one
    # XCD only.
    p = asl.gemm_create(2048, 2048, 128, 32, (128, 1, 2048 * 128), (1, 128, 2048 * 128), (2048, 1, 2048 * 2048))
    assert asl.gemm_plan_info(p) == (128, 128, 64, 8192, 512)
    slices = [set() for _ in range(8)]
    for h in range(8192):
        b, _, _ = asl.gemm_plan_tile_of(p, h)
        slices[h % 8].add(b)
    assert all(len(s) == 4 for s in slices)
    assert len(set().union(*slices)) == 32
    asl.gemm_destroy(p)


def test_sscore_argument_checks():
    q = (128, 1, 2048 * 128)
    s = (2048, 1, 2048 * 2048)
    assert _status(asl.sscore_run, 16, 32, 48, 32, 2048, 2048, 128, (128, 2, 0), q, s) == asl.AS_ERR_UNSUPPORTED
    assert _status(asl.sscore_run, 16, 32, 48, 0, 2048, 2048, 128, q, q, s) == asl.AS_ERR_INVALID
    assert _status(asl.sscore_run, 0, 32, 48, 32, 2048, 2048, 128, q, q, s) == asl.AS_ERR_INVALID
    assert _status(asl.sscore_run, 16, 32, 48, 32, 2048, 2048, 100, (100, 1, 0), (100, 1, 0), s) \
        == asl.AS_ERR_UNSUPPORTED
    assert _status(asl.sscore_run, 16, 32, 48, 32, 2048, 2048, 128, q, q, s, asl.AS_F32) == asl.AS_ERR_UNSUPPORTED


def test_tilecast_argument_checks():
    ok = dict(buf=16, rows=4096, cols=4096, tile_m=128, tile_n=64, consumers=256, group=2, grouped=True,
              iters=10, warmup=0, stride=0, out_checksum=32)

    def st(**kw):
        a = dict(ok)
        a.update(kw)
        return _status(asl.tilecast_run, *a.values())

    assert st(buf=0) == asl.AS_ERR_INVALID
    assert st(out_checksum=0) == asl.AS_ERR_INVALID
    assert st(consumers=100) == asl.AS_ERR_INVALID
    assert st(consumers=8192) == asl.AS_ERR_INVALID
    assert st(group=3) == asl.AS_ERR_INVALID
    assert st(group=64) == asl.AS_ERR_INVALID              # grouped: 32 workgroups per XCD
    assert st(iters=-1) == asl.AS_ERR_INVALID
    assert st(tile_n=60) == asl.AS_ERR_UNSUPPORTED
    assert st(tile_m=1024) == asl.AS_ERR_UNSUPPORTED       # 128 KiB tile
    assert st(rows=4000) == asl.AS_ERR_UNSUPPORTED
    assert st(buf=24) == asl.AS_ERR_UNSUPPORTED


def test_attn_fwd_argument_checks():
    q = (128, 1, 2048 * 128)
    o = (128, 1, 2048 * 128)
    ok = dict(batch=2, Lq=2048, Lk=2048, d=128, dv=128)

    def st(Q=16, K=32, V=48, O=64, q=q, k=q, v=q, o=o, scale=0.1, qkv_t=asl.AS_BF16, o_t=asl.AS_BF16, flags=0,
           **kw):
        a = dict(ok)
        a.update(kw)
        return _status(asl.attn_fwd_run, Q, K, V, O, a["batch"], a["Lq"], a["Lk"], a["d"], a["dv"], q, k, v, o,
                       scale, qkv_t, o_t, flags)

    assert st(batch=0) == asl.AS_ERR_INVALID
    assert st(Lk=0) == asl.AS_ERR_INVALID
    assert st(O=0) == asl.AS_ERR_INVALID                                   # null
    assert st(scale=float("inf")) == asl.AS_ERR_INVALID
    assert st(o_t=7) == asl.AS_ERR_INVALID
    assert st(flags=0x20) == asl.AS_ERR_INVALID                             # unknown flag
    assert st(flags=asl.AS_ATTN_SCHED_STATIC | asl.AS_ATTN_SCHED_QUEUE) == asl.AS_ERR_INVALID  # exclusive
    assert st(flags=asl.AS_ATTN_QUERIES_256 | asl.AS_ATTN_QUERIES_128) == asl.AS_ERR_INVALID   # exclusive

    assert st(flags=asl.AS_ATTN_CAUSAL, Lk=1024) == asl.AS_ERR_INVALID      # causal needs Lk >= Lq
    assert st(q=(-128, 1, 0)) == asl.AS_ERR_INVALID
    assert st(o=(64, 1, 2048 * 64)) == asl.AS_ERR_INVALID                  # O rows overlap
    assert st(o=(128, 1, 1000)) == asl.AS_ERR_INVALID                      # O batches overlap
    assert st(d=96, dv=96, q=(96, 1, 0), k=(96, 1, 0), v=(96, 1, 0), o=(96, 1, 2048 * 96)) == asl.AS_ERR_UNSUPPORTED
    assert st(dv=64) == asl.AS_ERR_UNSUPPORTED                             # d != dv
    assert st(qkv_t=asl.AS_F32) == asl.AS_ERR_UNSUPPORTED
    assert st(k=(128, 2, 0)) == asl.AS_ERR_UNSUPPORTED                     # non-contiguous last dim
    assert st(v=(132, 1, 0)) == asl.AS_ERR_UNSUPPORTED                     # row stride % 8
    assert st(Q=24) == asl.AS_ERR_UNSUPPORTED                              # misaligned
    assert st(k=(1 << 24, 1, 0)) == asl.AS_ERR_UNSUPPORTED                 # 32-bit tile offsets
    assert "16-byte" not in asl.as_last_error()


def test_attention_work_items():
    # 256-query items fill whole rounds of the 256 CUs; 128-query items when
    # they fill the rounds better, and always under the causal mask
    info = asl.attn_fwd_plan_info
    assert info(32, 2048) == (256, 64, 256)
    assert info(64, 2048) == (256, 64, 512)
    assert info(4, 8192) == (128, 128, 256)                    # 128 items of 256 would leave half the CUs idle
    assert info(48, 2048) == (128, 128, 768)                   # 1.5 rounds of 256-query items
    assert info(32, 2048, asl.AS_ATTN_CAUSAL) == (128, 128, 512)
    assert info(32, 2048, asl.AS_ATTN_QUERIES_128) == (128, 128, 512)
    assert info(4, 8192, asl.AS_ATTN_QUERIES_256) == (256, 64, 128)
    assert info(3, 129, asl.AS_ATTN_QUERIES_256 | asl.AS_ATTN_CAUSAL) == (256, 64, 3)
    assert info(32, 2048, asl.AS_ATTN_CAUSAL | asl.AS_ATTN_SCHED_QUEUE) == (128, 128, 256)   # persistent
    assert info(3, 129, asl.AS_ATTN_SCHED_STATIC) == (128, 128, 6)
    for bad in ((0, 10, 0), (1, 0, 0), (1, 10, 0x20), (1, 10, 0x6), (1, 10, 0x18)):
        with pytest.raises(asl.AsError):
            info(*bad)


def test_split_k_plans():
    # K is split only for a single product with fewer tiles than CUs, into
    # chunks that are multiples of 64 and >= 1024 deep
    def plan(M, N, K, batch=1, flags=0):
        p = asl.gemm_create(M, N, K, batch, (K, 1, M * K), (N, 1, K * N), (N, 1, M * N), flags=flags)
        try:
            return asl.gemm_plan_info(p), asl.gemm_plan_split_k(p)
        finally:
            asl.gemm_destroy(p)
    assert plan(1024, 1024, 8192) == ((128, 128, 64, 64, 512), (8, 8 * 1024 * 1024 * 4))
    assert plan(4096, 2048, 8192) == ((256, 256, 64, 128, 256), (2, 2 * 4096 * 2048 * 4))
    assert plan(1000, 3000, 4096)[1] == (2, 2 * 1000 * 3000 * 4)       # ragged tiles
    assert plan(256, 256, 65536)[1][0] == 16                          # at most 16 chunks
    assert plan(512, 512, 512)[1] == (1, 0)                           # chunks would be < 1024 deep
    assert plan(8192, 8192, 8192)[1] == (1, 0)                        # the tiles fill the grid
    assert plan(2048, 2048, 4096)[1] == (1, 0)                        # 256 tiles of 128: one per CU
    assert plan(1024, 1024, 8192, batch=2)[1] == (1, 0)               # batched: no split
    assert plan(1024, 1024, 8200)[1] == (1, 0)                        # K not a multiple of 128
    # without a split, 64 tiles of 128 would fill a quarter of the CUs: 256 tiles of 64 instead
    assert plan(1024, 1024, 8192, flags=asl.AS_FLAG_NO_SPLIT_K) == ((64, 64, 64, 256, 256), (1, 0))
    assert plan(1024, 1024, 8192, flags=asl.AS_FLAG_NO_SPLIT_K | asl.AS_FLAG_TILE_128) == \
        ((128, 128, 64, 64, 64), (1, 0))


def test_split_plan_slots_cover_every_chunk_and_tile():
    M, N, K = 1000, 700, 4096
    p = asl.gemm_create(M, N, K, 1, (K, 1, M * K), (1, K, K * N), (N, 1, M * N))     # K-major B
    try:
        tm, _, _, tiles, grid = asl.gemm_plan_info(p)
        splits, _ = asl.gemm_plan_split_k(p)
        assert splits == 4 and grid == tiles * splits
        seen = {asl.gemm_plan_tile_of(p, h) for h in range(grid)}   # (chunk, tile row, tile column)
        assert seen == {(s, r, c) for s in range(splits) for r in range(-(-M // tm)) for c in range(-(-N // tm))}
        assert _status(asl.gemm_plan_tile_of, p, grid) == asl.AS_ERR_INVALID
    finally:
        asl.gemm_destroy(p)


def test_python_plan_cache_is_bounded_and_keyed_by_stream():
    # the cache keeps the last 64 plans and destroys the rest; a different
    # stream gets its own plan
    asl._plan_cache.clear()
    first = asl.plan_for(256, 256, 64, 1, (64, 1, 0), (256, 1, 0), (256, 1, 0), 0, 0, 1)
    assert asl.plan_for(256, 256, 64, 1, (64, 1, 0), (256, 1, 0), (256, 1, 0), 0, 0, 1, stream=1) != first
    destroyed = []
    real_destroy = asl.gemm_destroy
    asl.gemm_destroy = lambda p: (destroyed.append(p), real_destroy(p))
    try:
        for i in range(1, 70):
            asl.plan_for(256 + 8 * i, 256, 64, 1, (64, 1, 0), (256, 1, 0), (256, 1, 0), 0, 0, 1)
    finally:
        asl.gemm_destroy = real_destroy
    assert len(asl._plan_cache) == asl._PLAN_CACHE_SIZE
    assert destroyed[0] == first and len(destroyed) == 70 + 1 - asl._PLAN_CACHE_SIZE   # oldest first


def test_attn_gqa_argument_checks():
    q = (128, 1, 128 * 256)
    def st(batch=4, kv_group=2):
        return _status(asl.attn_fwd_run_gqa, 16, 32, 48, 64, batch, kv_group, 256, 256, 128, 128, q, q, q, q, 0.1,
                       asl.AS_BF16, asl.AS_BF16, 0)
    assert st(kv_group=0) == asl.AS_ERR_INVALID
    assert st(kv_group=-2) == asl.AS_ERR_INVALID
    assert st(batch=6, kv_group=4) == asl.AS_ERR_INVALID     # must divide batch


def test_python_plan_cache_keeps_evicted_split_plans():
    # A graph may have recorded a run of an evicted split plan, and replays
    # write into that plan's workspace: split plans are set aside, never
    # destroyed, while plans without a split are destroyed.
    asl._plan_cache.clear()
    del asl._retired_split_plans[:]
    split = asl.plan_for(1024, 1024, 8192, 1, (8192, 1, 0), (1024, 1, 0), (1024, 1, 0), 0, 0, 1)
    assert asl.gemm_plan_split_k(split)[0] > 1
    plain = asl.plan_for(256, 256, 64, 1, (64, 1, 0), (256, 1, 0), (256, 1, 0), 0, 0, 1)
    destroyed = []
    real_destroy = asl.gemm_destroy
    asl.gemm_destroy = lambda p: (destroyed.append(p), real_destroy(p))
    try:
        for i in range(1, asl._PLAN_CACHE_SIZE + 1):
            asl.plan_for(256 + 8 * i, 256, 64, 1, (64, 1, 0), (256, 1, 0), (256, 1, 0), 0, 0, 1)
    finally:
        asl.gemm_destroy = real_destroy
    assert destroyed == [plain]
    assert asl._retired_split_plans == [split]
    assert asl.gemm_plan_split_k(split)[0] > 1          # still a live plan


def test_batch_strides_must_start_16_byte_chunks():
    # Each batch origin is read (and C written) in 16-byte pieces, so a batch
    # stride that is used must be a multiple of 8 elements (fp32 C: 4).
    mk = lambda a, b, c, batch=2, c_t=asl.AS_F32: _status(asl.gemm_create, 64, 64, 64, batch, a, b, c,
                                                          asl.AS_BF16, asl.AS_BF16, c_t)
    good_a, good_b, good_c = (64, 1, 64 * 64), (64, 1, 64 * 64), (64, 1, 64 * 64)
    assert mk(good_a, good_b, good_c) == asl.AS_OK
    assert mk((64, 1, 64 * 64 + 4), good_b, good_c) == asl.AS_ERR_UNSUPPORTED
    assert "batch strides" in asl.as_last_error()
    assert mk(good_a, (64, 1, 64 * 64 + 1), good_c) == asl.AS_ERR_UNSUPPORTED
    assert mk(good_a, good_b, (64, 1, 64 * 64 + 4)) == asl.AS_OK                       # fp32 C: 4 suffices
    assert mk(good_a, good_b, (64, 1, 64 * 64 + 2)) == asl.AS_ERR_UNSUPPORTED
    assert mk(good_a, good_b, (64, 1, 64 * 64 + 4), c_t=asl.AS_BF16) == asl.AS_ERR_UNSUPPORTED
    assert mk((64, 1, 4), good_b, good_c, batch=1) == asl.AS_OK                        # unused with one batch
    assert mk((64, 1, 0), (64, 1, 0), good_c) == asl.AS_OK                             # broadcast
    # attention scores: the same rule through sscore_run
    d = 128
    st = lambda q, k, s: _status(asl.sscore_run, 16, 32, 48, 2, 64, 64, d, q, k, s)
    assert st((d, 1, 64 * d + 4), (d, 1, 64 * d), (64, 1, 64 * 64)) == asl.AS_ERR_UNSUPPORTED
    assert st((d, 1, 64 * d), (d, 1, 64 * d + 2), (64, 1, 64 * 64)) == asl.AS_ERR_UNSUPPORTED
    assert st((d, 1, 64 * d), (d, 1, 64 * d), (64, 1, 64 * 64 + 2)) == asl.AS_ERR_UNSUPPORTED
    # fused attention: Q, K, V by 8 elements, O by 4, K and V only when several K/V slices are used
    q = (d, 1, 256 * d)

    def at(batch=4, kv_group=1, qs=q, ks=q, vs=q, os_=q, Q=16):
        return _status(asl.attn_fwd_run_gqa, Q, 32, 48, 64, batch, kv_group, 256, 256, d, d, qs, ks, vs, os_, 0.1,
                       asl.AS_BF16, asl.AS_BF16, 0)
    odd = (d, 1, 256 * d + 4)
    assert at(qs=odd) == asl.AS_ERR_UNSUPPORTED
    assert at(ks=odd) == asl.AS_ERR_UNSUPPORTED
    assert at(vs=(d, 1, 256 * d + 2)) == asl.AS_ERR_UNSUPPORTED
    assert at(os_=(d, 1, 256 * d + 2)) == asl.AS_ERR_UNSUPPORTED
    assert "batch strides" in asl.as_last_error()
    # one shared K/V slice (kv_group == batch): its batch stride is never used,
    # so the call passes that check and stops at the next one (a misaligned
    # Q pointer; no call here may pass every check with these fake pointers)
    assert at(kv_group=4, ks=odd, vs=odd, Q=24) == asl.AS_ERR_UNSUPPORTED
    assert "16-byte aligned" in asl.as_last_error()


def test_plans_survive_concurrent_destroy():
    # Threads create plans, run them (null device pointers: the run reads
    # the plan, then rejects the pointers before any HIP call) and destroy
    # them, while other threads run and destroy the same handles.  Every call
    # must return a status -- a run sees either a live plan (null-pointer
    # error) or an unknown one -- and nothing may crash.
    import threading
    L = asl.lib()
    shared, lock, errors = [], threading.Lock(), []
    S = asl.Strides

    def creator(n):
        for i in range(n):
            h = ctypes.c_void_p()
            K = 8192 if i % 3 == 0 else 512                  # every third plan splits K
            rc = L.gemm_create(ctypes.byref(h), 1024, 1024, K, 1, S(K, 1, 0), S(1024, 1, 0), S(1024, 1, 0),
                               0, 0, 1, 0)
            if rc != asl.AS_OK:
                errors.append(("create", rc))
                continue
            with lock:
                shared.append(h.value)
            if L.gemm_run(h.value, None, None, None, None) != asl.AS_ERR_INVALID:
                errors.append(("run own", rc))

    def runner(n):
        for _ in range(n):
            with lock:
                h = shared[-1] if shared else None
            if h is not None and L.gemm_run(h, None, None, None, None) != asl.AS_ERR_INVALID:
                errors.append(("run shared",))

    def destroyer(n):
        done = 0
        while done < n:
            with lock:
                h = shared.pop(0) if shared else None
            if h is None:
                continue
            if L.gemm_destroy(h) != asl.AS_OK:
                errors.append(("destroy",))
            done += 1

    n = 400
    threads = [threading.Thread(target=creator, args=(n,)) for _ in range(2)] + \
              [threading.Thread(target=runner, args=(2 * n,)) for _ in range(3)] + \
              [threading.Thread(target=destroyer, args=(n,)) for _ in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:5]
    assert not shared
