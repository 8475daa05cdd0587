"""HIP graph capture of the library's launches (through the C ABI).

The launches clear and synchronize nothing, so each entry point can be
recorded into a graph on a capturing stream (a split plan's first run
allocates its workspace, which is allowed there; the attention work-queue
schedule is refused).  Every case records one step,
checks that recording ran nothing (the outputs still hold their NaN fill), and
replays the graph several times.  Before each replay the outputs are refilled
and unrelated eager work runs.  After each replay the outputs must equal the
eager run bit for bit: every kernel here is deterministic, and the eager path's
parity against the oracle is covered by the other GPU tests.
"""
import pytest
import torch

import attention_scores_amd as asl
from workloads import WORKLOADS, draw, operands

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPLAYS = 4


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    asl.lib()  # fails loudly if the HIP library is missing


def _say(msg):
    print("[case] " + msg, flush=True)


def _fill_nan(outs):
    for o in outs:
        o.fill_(float("nan"))


def _replays_match(launch, outs):
    """launch() enqueues one step on the current stream, writing the tensors `outs`."""
    launch()                                     # eager reference; warms plans and workspaces
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    assert all(not torch.isnan(r.float()).any() for r in ref)

    # unrelated eager work between the replays, through the library and torch
    X = draw((384, 640), "uniform", -1.0, 1.0, 77).to(DEV)
    Y = draw((640, 320), "uniform", -1.0, 1.0, 78).to(DEV)
    Z = torch.empty((384, 320), dtype=torch.float32, device=DEV)

    g = torch.cuda.CUDAGraph()
    _fill_nan(outs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        launch()
    torch.cuda.synchronize()
    assert all(torch.isnan(o.float()).all() for o in outs), "recording must not run the kernels"
    for r in range(REPLAYS):
        _fill_nan(outs)
        asl.gemm(X, Y, out=Z)
        Z.mul_(0.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, want) in enumerate(zip(outs, ref)):
            assert torch.equal(o, want), "replay %d, output %d differs from the eager run" % (r, i)
    del g


def test_gemm_512_graph_replays():
    w = WORKLOADS["gemm512"]
    _say("graph: gemm 512^3 fp32 out")
    A, B = operands(w)
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    _replays_match(lambda: asl.gemm(Ad, Bd, out=C), [C])


def test_ragged_bf16_gemm_graph_replays():
    M, N, K = 1000, 712, 520
    _say("graph: ragged gemm %dx%dx%d bf16 out" % (M, N, K))
    Ad = draw((M, K), "uniform", -1.0, 1.0, 11).to(DEV)
    Bd = draw((K, N), "uniform", -1.0, 1.0, 12).to(DEV)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    _replays_match(lambda: asl.gemm(Ad, Bd, out=C), [C])


def test_split_k_graph_replays_after_an_eager_first_run():
    M, N, K = 1024, 1024, 8192
    _say("graph: split-K gemm %dx%dx%d" % (M, N, K))
    Ad = draw((M, K), "uniform", -1.0, 1.0, 21).to(DEV)
    Bd = draw((K, N), "uniform", -1.0, 1.0, 22).to(DEV)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    plan = asl.gemm_create(M, N, K, 1, (K, 1, M * K), (N, 1, K * N), (N, 1, M * N))
    try:
        assert asl.gemm_plan_split_k(plan)[0] == 8
        run = lambda: asl.gemm_run(plan, Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
        _replays_match(run, [C])                 # its eager first run allocates the workspace
    finally:
        torch.cuda.synchronize()
        asl.gemm_destroy(plan)


def test_split_k_first_run_inside_capture_allocates_and_replays():
    # The plan's first run happens while the stream records: the workspace is
    # allocated then (not a stream operation), the launches are recorded,
    # and every replay computes the eager result.
    M, N, K = 1024, 1024, 8192
    _say("graph: split-K first run inside capture")
    Ad = draw((M, K), "uniform", -1.0, 1.0, 23).to(DEV)
    Bd = draw((K, N), "uniform", -1.0, 1.0, 24).to(DEV)
    ref = torch.empty((M, N), dtype=torch.float32, device=DEV)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    sa, sb, sc = (K, 1, M * K), (N, 1, K * N), (N, 1, M * N)
    eager = asl.gemm_create(M, N, K, 1, sa, sb, sc)
    plan = asl.gemm_create(M, N, K, 1, sa, sb, sc)
    try:
        assert asl.gemm_plan_split_k(plan)[0] > 1
        asl.gemm_run(eager, Ad.data_ptr(), Bd.data_ptr(), ref.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            asl.gemm_run(plan, Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.isnan(C).all(), "recording must not run the kernels"
        for r in range(REPLAYS):
            C.fill_(float("nan"))
            asl.gemm_run(eager, Ad.data_ptr(), Bd.data_ptr(), ref.data_ptr(), torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(C, ref), "replay %d differs from the eager run" % r
        del g
    finally:
        torch.cuda.synchronize()
        asl.gemm_destroy(plan)
        asl.gemm_destroy(eager)


def test_split_k_through_the_binding_on_the_capture_stream():
    # asl.gemm() keeps one plan per stream; a shape warmed on the current
    # stream is planned anew on torch.cuda.graph's capture stream, whose first
    # (split) run then happens inside the capture.
    M, N, K = 512, 768, 4096
    _say("graph: asl.gemm split-K %dx%dx%d on the capture stream" % (M, N, K))
    Ad = draw((M, K), "uniform", -1.0, 1.0, 25).to(DEV)
    Bd = draw((K, N), "uniform", -1.0, 1.0, 26).to(DEV)
    plan = asl.gemm_create(M, N, K, 1, (K, 1, 0), (N, 1, 0), (N, 1, 0))
    try:
        assert asl.gemm_plan_split_k(plan)[0] > 1
    finally:
        asl.gemm_destroy(plan)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    _replays_match(lambda: asl.gemm(Ad, Bd, out=C), [C])


def test_queue_schedule_is_refused_inside_capture():
    # A queue launch's counter slot is chosen at launch time; a replay would
    # reuse it while another launch may hold it, so capture refuses it and
    # records nothing.
    b, L, d = 2, 256, 64
    _say("graph: attention queue schedule inside capture")
    Q = draw((b, L, d), "normal", 0.0, 1.0, 41).to(DEV)
    O = torch.full((b, L, d), float("nan"), dtype=torch.float32, device=DEV)
    st = (d, 1, L * d)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    err = None
    with torch.cuda.graph(g):
        try:
            asl.attn_fwd_run(Q.data_ptr(), Q.data_ptr(), Q.data_ptr(), O.data_ptr(), b, L, L, d, d, st, st, st, st,
                             0.125, asl.AS_BF16, asl.AS_F32, flags=asl.AS_ATTN_SCHED_QUEUE,
                             stream=torch.cuda.current_stream().cuda_stream)
        except asl.AsError as e:
            err = e
        O.add_(0.0)                              # keep the graph non-empty
    assert err is not None and err.status == asl.AS_ERR_UNSUPPORTED
    assert "graph" in str(err)
    g.replay()
    torch.cuda.synchronize()
    assert torch.isnan(O).all()
    del g
    # outside capture the same launch runs
    asl.attn_fwd_run(Q.data_ptr(), Q.data_ptr(), Q.data_ptr(), O.data_ptr(), b, L, L, d, d, st, st, st, st,
                     0.125, asl.AS_BF16, asl.AS_F32, flags=asl.AS_ATTN_SCHED_QUEUE,
                     stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert not torch.isnan(O).any()


def test_scores_and_attention_in_one_graph():
    b, L, d = 4, 512, 128
    _say("graph: scores + attention (default, causal static) b=%d L=%d d=%d" % (b, L, d))
    Q = draw((b, L, d), "normal", 0.0, 1.0, 31).to(DEV)
    K = draw((b, L, d), "normal", 0.0, 1.0, 32).to(DEV)
    V = draw((b, L, d), "normal", 0.0, 1.0, 33).to(DEV)
    S = torch.empty((b, L, L), dtype=torch.float32, device=DEV)
    O = torch.empty((b, L, d), dtype=torch.bfloat16, device=DEV)
    Oq = torch.empty((b, L, d), dtype=torch.float32, device=DEV)
    scale = d ** -0.5

    def step():
        st = torch.cuda.current_stream().cuda_stream
        asl.sscore(Q, K, out=S)
        asl.attention(Q, K, V, scale=scale, out=O)
        asl.attn_fwd_run(Q.data_ptr(), K.data_ptr(), V.data_ptr(), Oq.data_ptr(), b, L, L, d, d,
                         (d, 1, L * d), (d, 1, L * d), (d, 1, L * d), (d, 1, L * d), scale,
                         asl.AS_BF16, asl.AS_F32, flags=asl.AS_ATTN_CAUSAL | asl.AS_ATTN_SCHED_STATIC,
                         stream=st)

    _replays_match(step, [S, O, Oq])
