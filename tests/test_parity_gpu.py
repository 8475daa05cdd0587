"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: bit-exact where the arithmetic is exact (integer-valued data, identity
operands, checksums); otherwise |C_gpu - C_ref| <= 1e-3 * sum_k|a*b| + 1e-5
per element.  Every element is compared: at sizes the oracle finishes in
seconds (several tiles, odd tile counts, the 256 x 256 kernel at full K
depth), and at the five workloads' full sizes, where the oracle computes the
whole product in row blocks on the host's cores.  Only the 8 GiB-output and
one-workgroup-per-tile ablation cases compare seeded samples.
"""
import os

import numpy as np
import pytest
import torch

import attention_scores_amd as asl
import oracle
from workloads import WORKLOADS, bits, draw, operands, sample_points

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    asl.lib()  # fails loudly if the HIP library is missing


def _say(msg):
    print("[case] " + msg, flush=True)


# Oracle threads: a one-GPU job's share of its host is 16 cores, whatever the
# machine reports in all.
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _decode(out: torch.Tensor) -> np.ndarray:
    return out.detach().float().double().cpu().numpy() if out.dtype == torch.bfloat16 else \
        out.detach().double().cpu().numpy()


def _run_gemm(A, B, M, N, K, batch, sa, sb, out_dtype, flags=0):
    """Plan + run through the raw C ABI; A, B are CPU bf16 storage tensors."""
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.empty((batch, M, N), dtype=out_dtype, device=DEV)
    sc = (N, 1, M * N)
    plan = asl.gemm_create(M, N, K, batch, sa, sb, sc, asl.AS_BF16, asl.AS_BF16,
                           asl.AS_BF16 if out_dtype == torch.bfloat16 else asl.AS_F32, flags)
    try:
        asl.gemm_run(plan, Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    finally:
        asl.gemm_destroy(plan)
    return C


def _layout(M, N, K, batch, a_k, b_k):
    """Storage shapes and (row, col, batch) strides for A [M,K] and B [K,N]."""
    if a_k:
        a_shape, sa = (batch, M, K), (K, 1, M * K)
    else:
        a_shape, sa = (batch, K, M), (1, M, M * K)
    if b_k:
        b_shape, sb = (batch, N, K), (1, K, N * K)
    else:
        b_shape, sb = (batch, K, N), (N, 1, K * N)
    return a_shape, sa, b_shape, sb


# ------------------------------------------------------- exact integer pins --

LAYOUTS = [(ak, bk) for ak in (True, False) for bk in (True, False)]


TILE_FLAG = {64: asl.AS_FLAG_TILE_64, 128: asl.AS_FLAG_TILE_128, 256: asl.AS_FLAG_TILE_256}


@pytest.mark.parametrize("tile", [64, 128, 256])
@pytest.mark.parametrize("a_k,b_k", LAYOUTS, ids=lambda v: str(v))
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_integer_data_bit_exact(tile, a_k, b_k, out):
    # integers in [-4, 4]: every fp32 partial sum is exact in any order, so the
    # fp32 output must equal the oracle exactly and the bf16 output must be its
    # round-to-nearest-even.  512 x 768 x 320: several tiles, 5 K steps (odd).
    M, N, K, batch = 512, 768, 320, 2
    _say("int exact tile=%d a_k=%s b_k=%s out=%s" % (tile, a_k, b_k, out))
    a_shape, sa, b_shape, sb = _layout(M, N, K, batch, a_k, b_k)
    A = draw(a_shape, "int", -4, 4, 11 + tile)
    B = draw(b_shape, "int", -4, 4, 12 + tile)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    C = _run_gemm(A, B, M, N, K, batch, sa, sb, od, TILE_FLAG[tile])
    Cref, _ = oracle.gemm(bits(A), bits(B), batch, M, N, K, sa, sb, want_T=False)
    if out == "f32":
        assert np.array_equal(_decode(C), Cref)
    else:
        want = oracle.f64_to_bf16_rne_array(Cref)
        assert np.array_equal(bits(C), want)


def test_identity_operand_bit_exact():
    M = N = K = 512
    for b_k in (True, False):
        _say("identity A, b_k=%s" % b_k)
        a_shape, sa, b_shape, sb = _layout(M, N, K, 1, True, b_k)
        A = torch.eye(M, dtype=torch.bfloat16).reshape(a_shape)
        B = draw(b_shape, "normal", 0, 1, 31)
        C = _run_gemm(A, B, M, N, K, 1, sa, sb, torch.float32)
        Bv = B[0] if not b_k else B[0].t()
        assert torch.equal(C[0].cpu(), Bv.float())


def test_odd_tile_count_and_single_k_step():
    # 640 x 384 with 128 tiles = 15 workgroups (not a multiple of the 8 XCDs), K = 64.
    M, N, K = 640, 384, 64
    _say("odd tile count")
    a_shape, sa, b_shape, sb = _layout(M, N, K, 1, True, False)
    A = draw(a_shape, "int", -4, 4, 41)
    B = draw(b_shape, "int", -4, 4, 42)
    C = _run_gemm(A, B, M, N, K, 1, sa, sb, torch.float32)
    Cref, _ = oracle.gemm(bits(A), bits(B), 1, M, N, K, sa, sb, want_T=False)
    assert np.array_equal(_decode(C), Cref)


def test_batch_broadcast_of_B():
    M, N, K, batch = 256, 256, 128, 3
    _say("batch broadcast")
    A = draw((batch, M, K), "int", -4, 4, 51)
    B = draw((K, N), "int", -4, 4, 52)
    sa, sb = (K, 1, M * K), (N, 1, 0)
    C = _run_gemm(A, B, M, N, K, batch, sa, sb, torch.float32)
    Cref, _ = oracle.gemm(bits(A), bits(B), batch, M, N, K, sa, sb, want_T=False)
    assert np.array_equal(_decode(C), Cref)


# ------------------------------------------------------------ split K --

SPLIT = [  # (M, N, K, a_k, b_k): tiles fill at most half the grid, K deep enough to split
    (512, 768, 4096, True, False),      # 24 tiles of 128, 4 chunks
    (1000, 696, 4096, True, True),      # ragged M and N (696 = 5 x 128 + 56), K-major B
    (768, 512, 4096, False, False),     # column-major A
]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K,a_k,b_k", SPLIT)
def test_split_k_integer_data_bit_exact(M, N, K, a_k, b_k, out):
    # integer data: every partial sum, chunk sum and their total is exact in
    # fp32, so the split product equals the oracle bit for bit (bf16: its RNE)
    _say("split-K int exact %dx%dx%d a_k=%s b_k=%s out=%s" % (M, N, K, a_k, b_k, out))
    a_shape, sa, b_shape, sb = _layout(M, N, K, 1, a_k, b_k)
    A = draw(a_shape, "int", -4, 4, 61 + M)
    B = draw(b_shape, "int", -4, 4, 62 + N)
    plan = asl.gemm_create(M, N, K, 1, sa, sb, (N, 1, M * N))
    assert asl.gemm_plan_split_k(plan)[0] > 1
    asl.gemm_destroy(plan)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    C = _run_gemm(A, B, M, N, K, 1, sa, sb, od)
    Cref, _ = oracle.gemm(bits(A), bits(B), 1, M, N, K, sa, sb, want_T=False)
    if out == "f32":
        assert np.array_equal(_decode(C), Cref)
    else:
        assert np.array_equal(bits(C), oracle.f64_to_bf16_rne_array(Cref))


def test_split_k_on_concurrent_streams():
    # A split plan's runs share its workspace, so the binding keeps one plan
    # per stream: split products enqueued on three streams with no
    # synchronization between them must each equal a lone run bit for bit.
    M, N, K, rounds = 1024, 1024, 8192, 6
    _say("split-K %dx%dx%d on 3 concurrent streams, %d rounds" % (M, N, K, rounds))
    data = [(draw((M, K), "uniform", -1.0, 1.0, 4200 + 2 * i).to(DEV),
             draw((K, N), "uniform", -1.0, 1.0, 4201 + 2 * i).to(DEV)) for i in range(3)]
    refs = [asl.gemm(A, B, out_dtype=torch.float32) for A, B in data]
    torch.cuda.synchronize()
    outs = [[torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV) for _ in range(rounds)]
            for _ in range(3)]
    streams = [torch.cuda.Stream(device=DEV) for _ in range(3)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for r in range(rounds):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                asl.gemm(data[i][0], data[i][1], out=outs[i][r])
    torch.cuda.synchronize()
    bad = [(i, r) for i in range(3) for r in range(rounds) if not torch.equal(outs[i][r], refs[i])]
    assert not bad, "stream/round %s differ from the lone run" % bad[:10]


@pytest.mark.parametrize("M,N,K,a_k,b_k", SPLIT[:2])
def test_split_k_random_data_within_tolerance_and_deterministic(M, N, K, a_k, b_k):
    _say("split-K random %dx%dx%d" % (M, N, K))
    a_shape, sa, b_shape, sb = _layout(M, N, K, 1, a_k, b_k)
    A = draw(a_shape, "uniform", -1, 1, 71 + M)
    B = draw(b_shape, "uniform", -1, 1, 72 + N)
    Ad, Bd = A.to(DEV), B.to(DEV)
    plan = asl.gemm_create(M, N, K, 1, sa, sb, (N, 1, M * N))
    C1 = torch.empty((1, M, N), dtype=torch.float32, device=DEV)
    C2 = torch.full((1, M, N), float("nan"), dtype=torch.float32, device=DEV)
    try:
        st = torch.cuda.current_stream().cuda_stream
        asl.gemm_run(plan, Ad.data_ptr(), Bd.data_ptr(), C1.data_ptr(), st)
        asl.gemm_run(plan, Ad.data_ptr(), Bd.data_ptr(), C2.data_ptr(), st)    # workspace reused
        torch.cuda.synchronize()
    finally:
        asl.gemm_destroy(plan)
    assert torch.equal(C1, C2)
    Cref, T = oracle.gemm(bits(A), bits(B), 1, M, N, K, sa, sb)
    _check_full(C1, Cref, T)
    unsplit = _run_gemm(A, B, M, N, K, 1, sa, sb, torch.float32, asl.AS_FLAG_NO_SPLIT_K)
    _check_full(unsplit, Cref, T)


# -------------------------------------------------- workloads, full checks --

def _check_full(C, Cref, T):
    nfail, util = oracle.check(_decode(C).reshape(Cref.shape), Cref, T)
    assert nfail == 0, "%d elements outside tolerance (max util %.3g)" % (nfail, util)
    return util


def test_gemm512_full():
    w = WORKLOADS["gemm512"]
    _say(w.name)
    A, B = operands(w)
    C = _run_gemm(A, B, w.M, w.N, w.K, 1, w.a_strides(), w.b_strides(), torch.float32)
    Cref, T = oracle.gemm(bits(A), bits(B), 1, w.M, w.N, w.K, w.a_strides(), w.b_strides())
    util = _check_full(C, Cref, T)
    _say("%s max tolerance use %.3g" % (w.name, util))


@pytest.mark.parametrize("name,M,N,K", [
    ("gemm8192", 1024, 1024, 8192),             # 16 tiles, 128 K stages each
    ("gemm65536x256x4096", 8192, 256, 4096),    # one tile column: rotated K loop, non-temporal A
    ("gemm16384x8192x2048_colA", 2048, 1024, 2048),
])
def test_workload_kernel_reduced_full(name, M, N, K):
    """The full workload's kernel -- 256 x 256 tiles, 8 waves of 16x16x32
    MFMAs, its operand layouts, value distribution and output type, the
    workload's full K depth -- on fewer tiles, every element against the
    oracle.  K is not split, so the tile's whole K loop runs as it does at
    full size."""
    w = WORKLOADS[name]
    _say("%s kernel at %dx%dx%d" % (name, M, N, K))
    a_k = w.a_major == "row"
    a_shape, sa, b_shape, sb = _layout(M, N, K, 1, a_k, False)
    A = draw(a_shape, w.dist, w.lo, w.hi, w.seeds[0] + 1000)
    B = draw(b_shape, w.dist, w.lo, w.hi, w.seeds[1] + 1000)
    flags = asl.AS_FLAG_TILE_256 | asl.AS_FLAG_NO_SPLIT_K
    plan = asl.gemm_create(M, N, K, 1, sa, sb, (N, 1, M * N), asl.AS_BF16, asl.AS_BF16,
                           asl.AS_BF16 if w.out == "bf16" else asl.AS_F32, flags)
    try:
        assert asl.gemm_plan_info(plan)[:3] == (256, 256, 64)
        assert asl.gemm_plan_split_k(plan)[0] == 1
    finally:
        asl.gemm_destroy(plan)
    # the full workload plans the same tile
    full = asl.gemm_create(w.M, w.N, w.K, 1, w.a_strides(), w.b_strides(), (w.N, 1, w.M * w.N), asl.AS_BF16,
                           asl.AS_BF16, asl.AS_BF16 if w.out == "bf16" else asl.AS_F32)
    try:
        assert asl.gemm_plan_info(full)[:3] == (256, 256, 64) and asl.gemm_plan_split_k(full)[0] == 1
    finally:
        asl.gemm_destroy(full)
    od = torch.bfloat16 if w.out == "bf16" else torch.float32
    C = _run_gemm(A, B, M, N, K, 1, sa, sb, od, flags)
    Cref, T = oracle.gemm(bits(A), bits(B), 1, M, N, K, sa, sb, nthreads=ORACLE_THREADS)
    _check_full(C, Cref, T)


@pytest.mark.parametrize("batch,Lq,Lk,d", [(4, 512, 512, 128), (3, 768, 512, 128), (2, 256, 384, 64)])
def test_sscore_reduced_full(batch, Lq, Lk, d):
    _say("sscore %dx%dx%dx%d" % (batch, Lq, Lk, d))
    Q = draw((batch, Lq, d), "normal", 0, 1, 201 + Lq)
    K = draw((batch, Lk, d), "normal", 0, 1, 202 + Lk)
    S = asl.sscore(Q.to(DEV), K.to(DEV))
    torch.cuda.synchronize()
    Sref, T = oracle.sscore(bits(Q), bits(K), batch, Lq, Lk, d, (d, 1, Lq * d), (d, 1, Lk * d))
    _check_full(S, Sref, T)


def test_sscore_symmetric_when_Q_is_K():
    b, L, d = 2, 512, 128
    _say("sscore symmetry")
    Q = draw((b, L, d), "normal", 0, 1, 211).to(DEV)
    S = asl.sscore(Q, Q)
    torch.cuda.synchronize()
    Sref, T = oracle.sscore(bits(Q), bits(Q), b, L, L, d, (d, 1, L * d), (d, 1, L * d))
    _check_full(S, Sref, T)
    s = _decode(S)
    assert np.all(np.abs(s - np.transpose(s, (0, 2, 1))) <= 2 * (1e-3 * T + 1e-5))


# ---------------------------------------------- full sizes, every element --

N_SAMPLES = 4000
ROW_BLOCK = 1024      # output rows per oracle call (bounds host memory)


def _gemm_on_gpu(w, A, B, flags=0):
    od = torch.bfloat16 if w.out == "bf16" else torch.float32
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.empty((w.batch, w.M, w.N), dtype=od, device=DEV)
    plan = asl.gemm_create(w.M, w.N, w.K, w.batch, w.a_strides(), w.b_strides(), (w.N, 1, w.M * w.N),
                           asl.AS_BF16, asl.AS_BF16, asl.AS_BF16 if w.out == "bf16" else asl.AS_F32, flags)
    try:
        asl.gemm_run(plan, Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    finally:
        asl.gemm_destroy(plan)
    del Ad, Bd
    return C


def _full_compare(w, C, A, B):
    """Every element of C against the oracle, ROW_BLOCK output rows at a
    time (a row block of A is a view into its storage: a row offset with the
    workload's own strides)."""
    a = bits(A).reshape(-1)
    b = bits(B)
    sa, sb = w.a_strides(), w.b_strides()
    row_step = sa[0]                     # elements from one row of A to the next
    worst, checked = 0.0, 0
    for bi in range(w.batch):
        for r0 in range(0, w.M, ROW_BLOCK):
            r1 = min(w.M, r0 + ROW_BLOCK)
            sub = a[bi * sa[2] + r0 * row_step:]
            Cref, T = oracle.gemm(sub, b[bi * sb[2]:] if sb[2] else b, 1, r1 - r0, w.N, w.K, sa, sb,
                                  nthreads=ORACLE_THREADS)
            got = _decode(C[bi, r0:r1])
            nfail, util = oracle.check(got, Cref[0], T[0])
            assert nfail == 0, "batch %d rows %d..%d: %d elements outside tolerance (max util %.3g)" % (
                bi, r0, r1, nfail, util)
            worst = max(worst, util)
            checked += got.size
    assert checked == w.batch * w.M * w.N
    return worst


@pytest.mark.timeout(900)     # the oracle takes tens of seconds for 8192^3 on 16 cores
@pytest.mark.parametrize("name", ["gemm8192", "gemm65536x256x4096", "gemm16384x8192x2048_colA",
                                  "gemm4096x2048x8192"])
def test_full_size_every_element(name):
    """The workload as the benchmark runs it (default plan, inputs of the
    benchmark's seeds), every output element against the oracle."""
    w = WORKLOADS[name]
    _say("%s full size, every element (oracle on %d threads)" % (name, ORACLE_THREADS))
    A, B = operands(w)
    C = _gemm_on_gpu(w, A, B)
    util = _full_compare(w, C, A, B)
    _say("%s max tolerance use %.3g" % (name, util))


def _sampled_gemm(w, flags=0):
    A, B = operands(w)
    C = _gemm_on_gpu(w, A, B, flags)
    pts = sample_points(w.batch, w.M, w.N, N_SAMPLES, seed=w.seeds[0] * 7)
    idx = torch.from_numpy(pts).to(DEV)
    got = _decode(C[idx[:, 0], idx[:, 1], idx[:, 2]])
    Cref, T = oracle.gemm_points(bits(A), bits(B), pts, w.K, w.a_strides(), w.b_strides(),
                                 dims=(w.batch, w.M, w.N), nthreads=ORACLE_THREADS)
    nfail, util = oracle.check(got, Cref, T)
    assert nfail == 0, "%d sampled elements outside tolerance (max util %.3g)" % (nfail, util)
    return C


@pytest.mark.timeout(600)
def test_sscore_full_size_every_element_and_deterministic():
    w = WORKLOADS["sscore32x2048"]
    _say("sscore full size, every element")
    Q, K = operands(w)
    Qd, Kd = Q.to(DEV), K.to(DEV)
    S1 = asl.sscore(Qd, Kd)
    S2 = asl.sscore(Qd, Kd)
    torch.cuda.synchronize()
    assert torch.equal(S1, S2)
    q, k = bits(Q).reshape(w.batch, -1), bits(K).reshape(w.batch, -1)
    sq, sk = w.a_strides(), w.b_strides()
    worst = 0.0
    for b in range(w.batch):
        Sref, T = oracle.sscore(q[b], k[b], 1, w.M, w.N, w.K, sq, sk, nthreads=ORACLE_THREADS)
        nfail, util = oracle.check(_decode(S1[b]), Sref[0], T[0])
        assert nfail == 0, "slice %d: %d elements outside tolerance (max util %.3g)" % (b, nfail, util)
        worst = max(worst, util)
    _say("%s max tolerance use %.3g" % (w.name, worst))


def test_grouping_ablation_is_bitwise_identical():
    # The schedule changes which workgroup computes a tile, never the
    # arithmetic of the tile: grouped and identity orders agree bit for bit.
    M = N = K = 2048
    _say("grouping ablation")
    A = draw((M, K), "uniform", -1, 1, 61)
    B = draw((K, N), "uniform", -1, 1, 62)
    sa, sb = (K, 1, 0), (N, 1, 0)
    C1 = _run_gemm(A, B, M, N, K, 1, sa, sb, torch.bfloat16, 0)
    C2 = _run_gemm(A, B, M, N, K, 1, sa, sb, torch.bfloat16, asl.AS_FLAG_NO_GROUPING)
    C3 = _run_gemm(A, B, M, N, K, 1, sa, sb, torch.bfloat16, asl.AS_FLAG_NO_XCD_SPLIT)
    assert torch.equal(C1, C2)
    assert torch.equal(C1, C3)


# ------------------------------------------------------ tile fan-out bench --

@pytest.mark.parametrize("group", [1, 2, 8, 32])
@pytest.mark.parametrize("grouped", [True, False])
@pytest.mark.parametrize("streaming", [False, True])
def test_tilecast_checksums(group, grouped, streaming):
    rows, cols, tm, tn, consumers, iters = 4096, 4096, 128, 64, 256, 12
    _say("tilecast G=%d grouped=%s streaming=%s" % (group, grouped, streaming))
    g = torch.Generator().manual_seed(601)
    buf = torch.randint(-32768, 32768, (rows, cols), generator=g, dtype=torch.int32).to(torch.int16)
    stride = consumers // group if streaming else 0
    out = asl.tilecast(buf.to(DEV).view(torch.bfloat16), tm, tn, consumers, group, grouped, iters, 0, stride)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32).reshape(consumers, 2)
    b = buf.numpy().view(np.uint16)
    for w in range(consumers):
        tot, last = oracle.tilecast_checksum(b, rows, cols, tm, tn, w, consumers, group, grouped, iters, stride)
        assert (int(got[w, 0]), int(got[w, 1])) == (tot, last), w


def test_output_beyond_4gib_sampled():
    # 65536 x 65536 bf16 output (8 GiB): element offsets pass 2^32, so every
    # address in the epilogue must be 64-bit.  K = 64: a single stage.
    M = N = 65536
    K = 64
    _say("8 GiB output")
    A = draw((M, K), "uniform", -1, 1, 71)
    B = draw((K, N), "uniform", -1, 1, 72)
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    plan = asl.gemm_create(M, N, K, 1, (K, 1, 0), (N, 1, 0), (N, 1, 0), asl.AS_BF16, asl.AS_BF16, asl.AS_BF16, 0)
    try:
        asl.gemm_run(plan, Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    finally:
        asl.gemm_destroy(plan)
    pts = sample_points(1, M, N, N_SAMPLES, seed=77)
    pts = np.concatenate([pts, np.array([[0, M - 1, N - 1], [0, M - 1, 0], [0, 40000, 50000]])], axis=0)
    idx = torch.from_numpy(pts).to(DEV)
    got = _decode(C[idx[:, 1], idx[:, 2]])
    Cref, T = oracle.gemm_points(bits(A), bits(B), pts, K, (K, 1, 0), (N, 1, 0), dims=(1, M, N))
    # K = 64 of same-scale data: |C| is close to T, and rounding a correct
    # result to bf16 (half an ulp, at most 2^-8 |C|) can exceed 1e-3 T on its
    # own; the bf16-output allowance adds exactly that rounding.
    extra = 2.0 ** -8 * np.abs(Cref)
    nfail, util = oracle.check(got, Cref, T, extra=extra)
    bad = np.nonzero(~(np.abs(got - Cref) <= 1e-3 * T + 1e-5 + extra))[0][:8]
    assert nfail == 0, "%d sampled elements outside tolerance (max util %.3g); first: %s" % (
        nfail, util, [(tuple(pts[i]), float(got[i]), float(Cref[i])) for i in bad])
    del C
    torch.cuda.empty_cache()


@pytest.mark.parametrize("K", [64, 128, 192])
@pytest.mark.parametrize("flags", [0, asl.AS_FLAG_ONE_TILE_PER_WORKGROUP])
def test_grid_kinds_bit_exact(K, flags):
    # 576 tiles of 128 x 128: the resident grid has 512 workgroups, some of
    # which take two tiles, so the LDS ring streams across a tile boundary
    # after 1, 2 or 3 stages; the ablation launches one workgroup per tile.
    # Integer data, so the result must equal the oracle exactly.
    M = N = 3072
    _say("grid kinds, 576 tiles, K=%d flags=%d" % (K, flags))
    A = draw((M, K), "int", -4, 4, 81)
    B = draw((K, N), "int", -4, 4, 82)
    sa, sb = (K, 1, 0), (N, 1, 0)
    C = _run_gemm(A, B, M, N, K, 1, sa, sb, torch.float32, flags | asl.AS_FLAG_TILE_128)
    Cref, _ = oracle.gemm(bits(A), bits(B), 1, M, N, K, sa, sb, want_T=False)
    assert np.array_equal(_decode(C), Cref)


@pytest.mark.parametrize("K,out,a_k,b_k", [(64, "f32", True, True), (192, "f32", False, False),
                                           (128, "bf16", True, False)])
def test_resident_grid_256_tiles_bit_exact(K, out, a_k, b_k):
    # 17 x 16 = 272 tiles of 256 x 256 over 256 resident workgroups: 16 of
    # them write two tiles, the first through the 8-row epilogue region while
    # the next tile's stages load, with that epilogue's stores still in
    # flight at the next stage wait.
    M, N, batch = 4352, 4096, 1
    _say("resident grid 256 tiles K=%d out=%s a_k=%s b_k=%s" % (K, out, a_k, b_k))
    a_shape, sa, b_shape, sb = _layout(M, N, K, batch, a_k, b_k)
    A = draw(a_shape, "int", -4, 4, 91 + K)
    B = draw(b_shape, "int", -4, 4, 92 + K)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    C = _run_gemm(A, B, M, N, K, batch, sa, sb, od, asl.AS_FLAG_TILE_256)
    Cref, _ = oracle.gemm(bits(A), bits(B), batch, M, N, K, sa, sb, want_T=False)
    if out == "f32":
        assert np.array_equal(_decode(C), Cref)
    else:
        assert np.array_equal(bits(C), oracle.f64_to_bf16_rne_array(Cref))


@pytest.mark.parametrize("K,out,a_k,b_k", [(64, "f32", True, False), (576, "bf16", True, False),
                                           (200, "f32", False, True), (192, "bf16", False, False)])
def test_resident_grid_64_tiles_bit_exact(K, out, a_k, b_k):
    # 40 x 36 = 1440 tiles of 64 x 64 over 256 resident workgroups: every
    # workgroup walks several tiles through the 8-stage ring (K = 576: the
    # ring wraps within a tile; K = 200: a partial last stage), with the
    # 8-row (fp32) or 16-row (bf16) epilogue chunks between tiles.
    M, N, batch = 2560, 2300, 1
    _say("resident grid 64 tiles K=%d out=%s a_k=%s b_k=%s" % (K, out, a_k, b_k))
    _ragged(M, N, K, batch, a_k, b_k, out, asl.AS_FLAG_TILE_64, 3300 + K)


@pytest.mark.parametrize("K,out,rotate", [(512, "f32", False), (200, "bf16", False), (448, "f32", True)])
def test_64_tile_short_product_paths_agree(K, out, rotate):
    # On 64 x 64 tiles, a product whose workgroups each get one tile with all
    # its K stages in the 8-stage ring runs the short-product kernel (stage
    # loads by separate waves, released in two halves); with several tiles
    # per workgroup the general ring loop runs.  Both issue the same MFMAs in
    # the same order: slice 0 of an 8-slice product (512 tiles over 256
    # workgroups: the general loop) must equal the 1-slice product (64 tiles:
    # one each) bit for bit, on random data, and lie within tolerance.
    M = N = 512
    _say("64 tile short product paths K=%d out=%s rotate=%s" % (K, out, rotate))
    flags = asl.AS_FLAG_TILE_64 | (asl.AS_FLAG_ROTATE_K if rotate else asl.AS_FLAG_NO_ROTATE_K)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    A1 = draw((1, M, K), "normal", 0, 1, 4101 + K)
    B1 = draw((1, K, N), "normal", 0, 1, 4102 + K)
    A8, B8 = A1.repeat(8, 1, 1), B1.repeat(8, 1, 1)
    sa, sb = (K, 1, M * K), (N, 1, K * N)
    one = _run_gemm(A1, B1, M, N, K, 1, sa, sb, od, flags)
    many = _run_gemm(A8, B8, M, N, K, 8, sa, sb, od, flags)
    assert torch.equal(one[0], many[0]) and torch.equal(many[0], many[7])
    Cref, T = oracle.gemm(bits(A1), bits(B1), 1, M, N, K, sa, sb)
    # With K = 200, |C| reaches 1/4 of T on this data, where rounding a
    # correct result to bf16 (up to 2^-8 |C|) exceeds 1e-3 T by itself: the
    # bf16-output allowance adds exactly that rounding.
    extra = 2.0 ** -8 * np.abs(Cref[0]) if out == "bf16" else None
    nfail, util = oracle.check(one[0].double().cpu().numpy(), Cref[0], T[0], extra=extra)
    assert nfail == 0, util


@pytest.mark.parametrize("M,N,K,batch,a_k,b_k,out,extra", [
    (200, 136, 320, 3, True, False, "f32", 0),                                         # ragged M, N; 5 stages
    (130, 250, 456, 2, False, True, "bf16", 0),                                        # partial last K stage
    (256, 192, 512, 1, True, False, "bf16", "rotate_nt"),                             # rotated, non-temporal A
    (64, 64, 8, 1, True, True, "f32", 0),                                              # one partial stage
])
def test_short_product_kernel_bit_exact(M, N, K, batch, a_k, b_k, out, extra):
    # 64 x 64 tiles with every workgroup holding one tile and K <= 512: the
    # short-product kernel (separate loader waves, stage offsets in the lane
    # offsets).  Integer data, NaN-padded operands, sentinel-filled C:
    # bit-exact against the oracle and nothing stored outside C.
    flags = asl.AS_FLAG_TILE_64
    if extra == "rotate_nt":
        flags |= asl.AS_FLAG_ROTATE_K | asl.AS_FLAG_NT_A
    _say("short product %dx%dx%d batch=%d a_k=%s b_k=%s out=%s %s" % (M, N, K, batch, a_k, b_k, out, extra))
    _ragged(M, N, K, batch, a_k, b_k, out, flags, 5100 + K)


def test_short_product_kernel_broadcast_B_bit_exact():
    # the same kernel with B shared by all slices (batch stride 0)
    M, N, K, batch = 192, 128, 384, 3
    _say("short product, broadcast B")
    A = draw((batch, M, K), "int", -4, 4, 5201)
    B = draw((K, N), "int", -4, 4, 5202)
    sa, sb = (K, 1, M * K), (N, 1, 0)
    C = _run_gemm(A, B, M, N, K, batch, sa, sb, torch.float32, asl.AS_FLAG_TILE_64)
    Cref, _ = oracle.gemm(bits(A), bits(B), batch, M, N, K, sa, sb, want_T=False)
    assert np.array_equal(_decode(C), Cref)


def test_one_tile_per_workgroup_full_size_sampled():
    w = WORKLOADS["gemm8192"]
    _say("gemm8192 one tile per workgroup, sampled")
    _sampled_gemm(w, flags=asl.AS_FLAG_ONE_TILE_PER_WORKGROUP)


# ------------------------------------------------------------ ragged shapes --
# M and N need not be multiples of the tile, nor K of the 64-deep stage (K a
# multiple of 8).  Operands live in padded storage whose padding holds NaN
# bit patterns: a chunk read past K inside a row would turn the result into
# NaN.  C lives in a larger buffer filled with a sentinel: every element
# outside [0, M) x [0, N) of every batch must keep it.

_NAN_BF16 = 0x7FC1
_SENT_F32 = 0x7FC00123
_SENT_BF16 = 0x7FC3


def _padded(rows, cols, batch, ld, seed):
    """[batch, rows, ld] bf16 storage: integers in [-4, 4] in the first `cols`
    columns, NaN bit patterns in the padding; also one spare row of NaN."""
    vals = bits(draw((batch, rows, cols), "int", -4, 4, seed)).astype(np.uint16)
    st = np.full((batch, rows + 1, ld), _NAN_BF16, dtype=np.uint16)
    st[:, :rows, :cols] = vals
    return st, (rows + 1) * ld


def _ragged(M, N, K, batch, a_k, b_k, out, flags, seed):
    lda = (K if a_k else M) + (-(K if a_k else M)) % 8 + 8
    ldb = (K if b_k else N) + (-(K if b_k else N)) % 8 + 8
    if a_k:
        A, abs_ = _padded(M, K, batch, lda, seed)
        sa = (lda, 1, abs_)
    else:
        A, abs_ = _padded(K, M, batch, lda, seed)
        sa = (1, lda, abs_)
    if b_k:
        B, bbs = _padded(N, K, batch, ldb, seed + 1)
        sb = (1, ldb, bbs)
    else:
        B, bbs = _padded(K, N, batch, ldb, seed + 1)
        sb = (ldb, 1, bbs)
    bf = out == "bf16"
    align = 8 if bf else 4
    ldc = N + (-N) % align + align
    rows_c = M + 3
    sent = _SENT_BF16 if bf else _SENT_F32
    cdt = torch.int16 if bf else torch.int32
    Cst = torch.full((batch, rows_c, ldc), sent - (1 << 16 if bf and sent >= 1 << 15 else 0), dtype=cdt, device=DEV)
    Ad = torch.from_numpy(A.view(np.int16)).to(DEV)
    Bd = torch.from_numpy(B.view(np.int16)).to(DEV)
    plan = asl.gemm_create(M, N, K, batch, sa, sb, (ldc, 1, rows_c * ldc), asl.AS_BF16, asl.AS_BF16,
                           asl.AS_BF16 if bf else asl.AS_F32, flags)
    try:
        asl.gemm_run(plan, Ad.data_ptr(), Bd.data_ptr(), Cst.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    finally:
        asl.gemm_destroy(plan)
    got = Cst.cpu().numpy().view(np.uint16 if bf else np.uint32)
    Cref, _ = oracle.gemm(A, B, batch, M, N, K, sa, sb, want_T=False)
    if bf:
        want = oracle.f64_to_bf16_rne_array(Cref)
        assert np.array_equal(got[:, :M, :N], want), "bf16 output differs from RNE(oracle)"
    else:
        assert np.array_equal(np.ascontiguousarray(got[:, :M, :N]).view(np.float32).astype(np.float64), Cref), \
            "fp32 output differs"
    outside = np.ones(got.shape, dtype=bool)
    outside[:, :M, :N] = False
    assert np.all(got[outside] == sent), "stores outside the M x N output"


RAGGED = [  # (M, N, K, batch, tile flag)
    (1, 1, 8, 1, asl.AS_FLAG_TILE_128),          # one element, one partial stage
    (7, 13, 24, 2, asl.AS_FLAG_TILE_128),
    (129, 130, 72, 1, asl.AS_FLAG_TILE_128),      # 2x2 tiles, one full + one 8-deep stage
    (300, 517, 200, 2, asl.AS_FLAG_TILE_128),     # N not a multiple of 8: element stores at the edge
    (257, 300, 136, 1, asl.AS_FLAG_TILE_256),
    (513, 260, 8, 1, asl.AS_FLAG_TILE_256),
    (256, 256, 520, 1, asl.AS_FLAG_TILE_256),     # full tiles, partial last stage only
    (65, 200, 1032, 2, asl.AS_FLAG_TILE_64),      # 17 stages through the 8-stage ring, partial last
    (100, 37, 40, 1, asl.AS_FLAG_TILE_64),
]


@pytest.mark.parametrize("M,N,K,batch,tflag", RAGGED)
@pytest.mark.parametrize("a_k,b_k", LAYOUTS, ids=lambda v: str(v))
def test_ragged_shapes_bit_exact_fp32(M, N, K, batch, tflag, a_k, b_k):
    _say("ragged fp32 M=%d N=%d K=%d b=%d flags=%d a_k=%s b_k=%s" % (M, N, K, batch, tflag, a_k, b_k))
    _ragged(M, N, K, batch, a_k, b_k, "f32", tflag, 1000 + M + K)


@pytest.mark.parametrize("M,N,K,batch,tflag", RAGGED[1:5])
@pytest.mark.parametrize("a_k,b_k", [(True, False), (False, True)], ids=lambda v: str(v))
def test_ragged_shapes_bit_exact_bf16(M, N, K, batch, tflag, a_k, b_k):
    _say("ragged bf16 M=%d N=%d K=%d b=%d flags=%d a_k=%s b_k=%s" % (M, N, K, batch, tflag, a_k, b_k))
    _ragged(M, N, K, batch, a_k, b_k, "bf16", tflag, 2000 + M + K)


@pytest.mark.parametrize("flags", [0, asl.AS_FLAG_ONE_TILE_PER_WORKGROUP])
def test_ragged_resident_grid_walks_edge_and_interior_tiles(flags):
    # 17 x 17 x 4 = 1156 tiles of 128 over 512 resident workgroups: walks mix
    # edge tiles (element stores, full store drain) with interior ones.
    _say("ragged resident grid flags=%d" % flags)
    _ragged(2100, 2050, 136, 4, True, False, "f32", asl.AS_FLAG_TILE_128 | flags, 31)


def test_ragged_attention_scores():
    # 3 slices of Q [1000, 96] . K [77, 96]^T: a 96-deep head (one full and
    # one half stage), 77 keys (N not a multiple of 8), padded S rows.
    batch, Lq, Lk, d = 3, 1000, 77, 96
    _say("ragged sscore %dx%dx%dx%d" % (batch, Lq, Lk, d))
    Q = draw((batch, Lq, d), "int", -4, 4, 41)
    Kt = draw((batch, Lk, d), "int", -4, 4, 42)
    ldc = 80
    S = torch.full((batch, Lq, ldc), float("nan"), dtype=torch.float32, device=DEV)
    Qd, Kd = Q.to(DEV), Kt.to(DEV)      # keep the device copies alive across the call
    asl.sscore_run(Qd.data_ptr(), Kd.data_ptr(), S.data_ptr(), batch, Lq, Lk, d,
                   (d, 1, Lq * d), (d, 1, Lk * d), (ldc, 1, Lq * ldc), asl.AS_BF16, asl.AS_F32,
                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    Sref, _ = oracle.sscore(bits(Q), bits(Kt), batch, Lq, Lk, d, (d, 1, Lq * d), (d, 1, Lk * d))
    got = S.cpu().numpy()
    assert np.array_equal(got[:, :, :Lk].astype(np.float64), Sref)
    assert np.all(np.isnan(got[:, :, Lk:]))


# ------------------------------------------ non-temporal A loads (A streams) --

NT_A = [  # (M, N, K, batch, flags, a_k, b_k), run with the non-temporal hint on A forced on
    (1024, 256, 1024, 1, asl.AS_FLAG_TILE_256, True, False),     # one tile column (the default choice)
    (1024, 512, 576, 2, asl.AS_FLAG_TILE_256, False, True),      # two tile columns, column-major A, batch
    (300, 200, 200, 1, asl.AS_FLAG_TILE_128, True, True),        # ragged, partial last stage
    (512, 256, 8192, 1, asl.AS_FLAG_TILE_256, True, False),      # 2 tiles: split into 8 K chunks
]


@pytest.mark.parametrize("M,N,K,batch,flags,a_k,b_k", NT_A)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_nontemporal_a_bit_exact(M, N, K, batch, flags, a_k, b_k, out):
    """The hint changes only what L2 keeps: integer data give the oracle's
    result bit for bit, and nothing outside C is written."""
    _say("nt_a M=%d N=%d K=%d batch=%d flags=0x%x a_k=%s b_k=%s out=%s" % (M, N, K, batch, flags, a_k, b_k, out))
    _ragged(M, N, K, batch, a_k, b_k, out, flags | asl.AS_FLAG_NT_A | asl.AS_FLAG_NO_ROTATE_K, 4100 + M + K)


# ----------------------------------------------- rotated K loop (A streams) --

ROTATE = [  # (M, N, K, batch, flags, a_k, b_k), run with the K rotation forced on
    (1024, 256, 1024, 1, asl.AS_FLAG_TILE_256, True, False),     # 4 tile rows start at stages 0..3 of 16
    (300, 200, 200, 1, asl.AS_FLAG_TILE_128, True, True),        # the partial stage (8 deep) mid-sequence
    (257, 260, 136, 1, asl.AS_FLAG_TILE_256, False, False),      # column-major A, partial stage
    (512, 256, 8192, 1, asl.AS_FLAG_TILE_256, True, False),      # split into 8 chunks: rotation inside each
    (384, 384, 200, 64, asl.AS_FLAG_TILE_128 | asl.AS_FLAG_NT_A, True, False),  # 576 tiles walked
]


@pytest.mark.parametrize("M,N,K,batch,flags,a_k,b_k", ROTATE)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_rotated_k_bit_exact(M, N, K, batch, flags, a_k, b_k, out):
    """Each tile accumulates every K stage exactly once whatever stage it
    starts at: integer data give the oracle's result bit for bit."""
    _say("rotate M=%d N=%d K=%d batch=%d flags=0x%x a_k=%s b_k=%s out=%s" % (M, N, K, batch, flags, a_k, b_k, out))
    _ragged(M, N, K, batch, a_k, b_k, out, flags | asl.AS_FLAG_ROTATE_K, 5200 + M + K)


def test_rotated_k_random_data_within_tolerance_and_deterministic():
    """The tall-skinny workload's kernel at reduced height with N(0,1) data:
    one 256-wide tile column, so the default plan streams A (rotated K loop,
    non-temporal loads).  Default and forced rotation give the same bits, the
    unrotated ablation sums in another order (different bits), and both are
    within tolerance of the oracle at every element."""
    M, N, K = 8192, 256, 4096
    A = draw((1, M, K), "normal", 0, 1, 411)
    B = draw((1, K, N), "normal", 0, 1, 412)
    sa, sb = (K, 1, M * K), (N, 1, K * N)
    Cref, T = oracle.gemm(bits(A), bits(B), 1, M, N, K, sa, sb, nthreads=ORACLE_THREADS)
    base = asl.AS_FLAG_TILE_256 | asl.AS_FLAG_NO_SPLIT_K
    runs = {}
    for name, flags in (("default", base), ("again", base), ("rotate", base | asl.AS_FLAG_ROTATE_K),
                        ("unrotated", base | asl.AS_FLAG_NO_ROTATE_K)):
        _say("rotate tolerance %s flags=0x%x" % (name, flags))
        C = _run_gemm(A, B, M, N, K, 1, sa, sb, torch.float32, flags)
        _check_full(C, Cref, T)
        runs[name] = C.view(torch.int32)
    assert torch.equal(runs["default"], runs["again"])
    assert torch.equal(runs["default"], runs["rotate"])
    assert not torch.equal(runs["default"], runs["unrotated"])


# ------------------------------------------ deeper A ring (streaming A) --
# With A streaming (one 256-wide tile column, tile-aligned) and one tile per
# workgroup, the kernel gives A a ring of three stages and B one of two.  Its
# MFMA order is the two-stage ring's, which runs when A's loads are ordinary
# (AS_FLAG_NO_NT_A).

_T256 = asl.AS_FLAG_TILE_256
DEEP_A = [  # (M, N, K, flags)
    (65536, 256, 1024, 0),                               # 256 tiles: the resident grid, one tile each
    (8192, 256, 4096, _T256 | asl.AS_FLAG_NO_SPLIT_K),   # 32 tiles of 64 stages
    (4096, 256, 8192, _T256),                            # 16 tiles: split into K chunks, each on the deep ring
    (2048, 256, 64, _T256 | asl.AS_FLAG_NO_SPLIT_K),     # one stage: every later request fetches nothing
    (16384, 256, 2048, _T256 | asl.AS_FLAG_NO_ROTATE_K),  # every tile walks K from stage 0
    (1024, 256, 192, _T256 | asl.AS_FLAG_NO_SPLIT_K),    # three stages: the ring's depth exactly
]


@pytest.mark.parametrize("M,N,K,flags", DEEP_A)
@pytest.mark.parametrize("a_k", [True, False])
def test_deep_a_ring_bitwise_equals_two_stage_ring(M, N, K, flags, a_k):
    _say("deep A ring M=%d N=%d K=%d flags=0x%x a_k=%s" % (M, N, K, flags, a_k))
    A = draw((1, M, K) if a_k else (1, K, M), "normal", 0, 1, 6100 + K)
    B = draw((1, K, N), "normal", 0, 1, 6200 + K)
    sa = (K, 1, M * K) if a_k else (1, M, M * K)
    sb = (N, 1, K * N)
    p = asl.gemm_create(M, N, K, 1, sa, sb, (N, 1, M * N), flags=flags)
    tile, _, _, tiles, grid = asl.gemm_plan_info(p)
    splits = asl.gemm_plan_split_k(p)[0]
    asl.gemm_destroy(p)
    assert tile == 256 and (splits == 1 or K // splits % 64 == 0)
    assert grid >= tiles * splits        # one tile (or K chunk of one) per workgroup
    deep = _run_gemm(A, B, M, N, K, 1, sa, sb, torch.float32, flags)
    two = _run_gemm(A, B, M, N, K, 1, sa, sb, torch.float32, flags | asl.AS_FLAG_NO_NT_A)
    assert torch.equal(deep.view(torch.int32), two.view(torch.int32))
    assert torch.isfinite(deep).all()


DEEP_A_INT = [  # (M, N, K, a_k, b_k)
    (2048, 256, 512, True, False),
    (1024, 256, 64, False, False),
    (1536, 256, 1024, True, True),
    (4096, 256, 4096, False, True),               # split into K chunks
]


@pytest.mark.parametrize("M,N,K,a_k,b_k", DEEP_A_INT)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_deep_a_ring_integer_bit_exact(M, N, K, a_k, b_k, out):
    """Integer data through the deep A ring (padded NaN storage, sentinel C):
    the oracle's result bit for bit, nothing stored outside C."""
    _say("deep A ring integer M=%d N=%d K=%d a_k=%s b_k=%s out=%s" % (M, N, K, a_k, b_k, out))
    _ragged(M, N, K, 1, a_k, b_k, out, _T256, 6300 + M + K)


# --------------------------------------------------- randomized shape sweep --

def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M, N = int(rng.integers(1, 700)), int(rng.integers(1, 600))
        K = 8 * int(rng.integers(1, 80))
        batch = int(rng.integers(1, 3))
        a_k, b_k = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
        out = "bf16" if rng.integers(0, 2) else "f32"
        flags = [asl.AS_FLAG_TILE_256, asl.AS_FLAG_TILE_128, 0, asl.AS_FLAG_TILE_64][i % 4]
        flags |= [0, asl.AS_FLAG_ROTATE_K, asl.AS_FLAG_NT_A, asl.AS_FLAG_ROTATE_K | asl.AS_FLAG_NT_A][(i // 3) % 4]
        cases.append((M, N, K, batch, a_k, b_k, out, flags))
    return cases


@pytest.mark.parametrize("M,N,K,batch,a_k,b_k,out,flags", _random_cases(128, 2026))
def test_random_shapes_bit_exact(M, N, K, batch, a_k, b_k, out, flags):
    """Seeded random shapes, layouts, output types, tiles and streaming
    options on integer data: bit-exact against the oracle, nothing written
    outside C (both MFMA shapes, both wave grids of the 256 tile, edge tiles,
    rotated K loops and split K where the plan chooses it)."""
    _say("random M=%d N=%d K=%d batch=%d a_k=%s b_k=%s out=%s flags=0x%x" % (M, N, K, batch, a_k, b_k, out, flags))
    _ragged(M, N, K, batch, a_k, b_k, out, flags, 7000 + M + N + K)
