"""The allocation-free GEMM entry point (gemm_run_no_alloc) through the C ABI.

A split plan run through gemm_run_no_alloc keeps its partial sums in the
library's static per-GPU scratch array instead of its own workspace.  Its
output must equal gemm_run's bit for bit (the same kernels, the same
deterministic chunk order), on two calls in a row -- the second with a
smaller product, so a stale first result left in the array cannot pass --
and the calls must not allocate device memory.
"""
import pytest
import torch

import attention_scores_amd as asl
from workloads import draw

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    asl.lib()  # fails loudly if the HIP library is missing


def _say(msg):
    print("[case] " + msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _set_up():
    # Set-up, before any measurement: the first launches load the library's
    # kernels (and with them the static scratch array) onto the GPU, and the
    # first gemm_run_no_alloc looks up the array's address.
    if not torch.cuda.is_available():
        return
    M, N, K = 256, 256, 2048
    A = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((K, N), dtype=torch.bfloat16, device=DEV)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    plan = _plan(M, N, K, torch.float32)
    try:
        assert asl.gemm_plan_split_k(plan)[0] > 1
        asl.gemm_run(plan, A.data_ptr(), B.data_ptr(), C.data_ptr(), torch.cuda.current_stream().cuda_stream)
        asl.gemm_run_no_alloc(plan, A.data_ptr(), B.data_ptr(), C.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    finally:
        asl.gemm_destroy(plan)


def _plan(M, N, K, out):
    return asl.gemm_create(M, N, K, 1, (K, 1, 0), (N, 1, 0), (N, 1, 0), asl.AS_BF16, asl.AS_BF16,
                           asl.AS_BF16 if out == torch.bfloat16 else asl.AS_F32, 0)


CASES = [  # two calls in a row, the second smaller: (M, N, K, output dtype)
    ((1024, 1024, 8192, torch.float32), (512, 768, 4096, torch.bfloat16)),        # 8 then 4 chunks
    ((4096, 2048, 8192, torch.bfloat16), (1000, 696, 4096, torch.float32)),       # the largest workspace, then ragged
]


@pytest.mark.parametrize("first,second", CASES)
def test_no_alloc_equals_gemm_run_on_two_calls(first, second):
    stream = torch.cuda.current_stream().cuda_stream
    data = []
    for i, (M, N, K, od) in enumerate((first, second)):
        A = draw((M, K), "uniform", -1.0, 1.0, 3100 + 2 * i).to(DEV)
        B = draw((K, N), "uniform", -1.0, 1.0, 3101 + 2 * i).to(DEV)
        want = torch.empty((M, N), dtype=od, device=DEV)
        got = torch.full((M, N), float("nan"), dtype=od, device=DEV)
        data.append((M, N, K, od, A, B, want, got))
    torch.cuda.synchronize()
    for M, N, K, od, A, B, want, got in data:
        _say("no-alloc %dx%dx%d %s" % (M, N, K, od))
        ref_plan, plan = _plan(M, N, K, od), _plan(M, N, K, od)
        try:
            splits, ws_bytes = asl.gemm_plan_split_k(plan)
            assert splits > 1 and 0 < ws_bytes <= 64 << 20
            free0 = torch.cuda.mem_get_info()[0]
            asl.gemm_run_no_alloc(plan, A.data_ptr(), B.data_ptr(), got.data_ptr(), stream)
            torch.cuda.synchronize()
            free1 = torch.cuda.mem_get_info()[0]
            assert free1 == free0, "gemm_run_no_alloc changed free device memory (%d -> %d)" % (free0, free1)
            asl.gemm_run(ref_plan, A.data_ptr(), B.data_ptr(), want.data_ptr(), stream)   # allocates its workspace
            torch.cuda.synchronize()
        finally:
            asl.gemm_destroy(plan)
            asl.gemm_destroy(ref_plan)
        assert torch.equal(got.view(torch.int16 if od == torch.bfloat16 else torch.int32),
                           want.view(torch.int16 if od == torch.bfloat16 else torch.int32))


def test_no_alloc_without_a_split_is_gemm_run():
    M, N, K = 2048, 2048, 1024                    # 256 tiles of 128: no split
    _say("no-alloc without a split")
    stream = torch.cuda.current_stream().cuda_stream
    A = draw((M, K), "uniform", -1.0, 1.0, 3200).to(DEV)
    B = draw((K, N), "uniform", -1.0, 1.0, 3201).to(DEV)
    want = torch.empty((M, N), dtype=torch.float32, device=DEV)
    got = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    plan = _plan(M, N, K, torch.float32)
    try:
        assert asl.gemm_plan_split_k(plan) == (1, 0)
        asl.gemm_run(plan, A.data_ptr(), B.data_ptr(), want.data_ptr(), stream)
        asl.gemm_run_no_alloc(plan, A.data_ptr(), B.data_ptr(), got.data_ptr(), stream)
        torch.cuda.synchronize()
    finally:
        asl.gemm_destroy(plan)
    assert torch.equal(got, want)
