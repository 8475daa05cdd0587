"""GPU parity of the fused attention forward (through the C ABI) against the oracle.

Bars: on data whose every probability is a power of two down to 2^-8
(integer scores in [-4, 4] with scale ln 2) the bf16 probabilities, both
products and every partial sum are exact in fp32; what remains are the
hardware exp2's last-bit errors (in the fp32 sum of probabilities and the
running rescale factors, about 1 ulp each) and the final division, which
together stay far below |O_gpu - O_ref| <= 2^-18 * TO.  A dropped key tile,
a wrong rescale or a key permutation slip moves O by orders of magnitude
more.  On general
data the probabilities pass through bf16: |O_gpu - O_ref| <= 2^-7 * TO + 1e-6
(+ 2^-8 |O_ref| for a bf16 output), TO = sum_j p_j |v_j| / sum_j p_j.
"""
import functools
import math
import os

import numpy as np
import pytest
import torch

import attention_scores_amd as asl
import oracle
from workloads import ATTN_WORKLOADS, attn_operands, bits, draw

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    asl.lib()  # fails loudly if the HIP library is missing


def _say(msg):
    print("[case] " + msg, flush=True)


ITEMS = {None: 0, 256: 0x2, 128: 0x4}   # work-item shape: the library's choice, or forced


SCHED = {"one": 0, "static": 0x8, "queue": 0x10}   # one workgroup per item, or persistent


def _run(Q, K, V, scale, out="bf16", ldo=None, rows_pad=0, causal=False, items=None, sched="one"):
    """Q, K, V: CPU bf16 [b, L, d]; returns the decoded output [b, Lq, dv] and the raw buffer.
    items: None (the library's choice), 256 or 128 queries per work item; sched: one
    workgroup per item, or a persistent grid walking items by a static stride or a queue."""
    b, Lq, d = Q.shape
    Lk, dv = V.shape[1], V.shape[2]
    ldo = ldo or dv
    Qd, Kd, Vd = Q.to(DEV), K.to(DEV), V.to(DEV)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    Ob = torch.full((b, Lq + rows_pad, ldo), float("nan"), dtype=od, device=DEV)
    asl.attn_fwd_run(Qd.data_ptr(), Kd.data_ptr(), Vd.data_ptr(), Ob.data_ptr(), b, Lq, Lk, d, dv,
                     (d, 1, Lq * d), (d, 1, Lk * d), (dv, 1, Lk * dv), (ldo, 1, (Lq + rows_pad) * ldo), scale,
                     asl.AS_BF16, asl.AS_BF16 if out == "bf16" else asl.AS_F32,
                     flags=(asl.AS_ATTN_CAUSAL if causal else 0) | ITEMS[items] | SCHED[sched],
                     stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    raw = Ob.float().cpu().numpy().astype(np.float64)
    return raw[:, :Lq, :dv], raw


def _ref(Q, K, V, scale, rows=None, causal=False):
    b, Lq, d = Q.shape
    Lk, dv = V.shape[1], V.shape[2]
    return oracle.attention(bits(Q), bits(K), bits(V), b, Lq, Lk, d, dv, (d, 1, Lq * d), (d, 1, Lk * d),
                            (dv, 1, Lk * dv), scale, rows=rows, causal=causal)


def _sparse_q(b, Lq, d, seed):
    """Entries in {-1, 0, 1}, exactly four nonzeros per row."""
    g = torch.Generator().manual_seed(seed)
    Q = torch.zeros((b, Lq, d), dtype=torch.float32)
    idx = torch.argsort(torch.rand((b, Lq, d), generator=g), dim=2)[:, :, :4]
    sign = torch.randint(0, 2, (b, Lq, 4), generator=g).float() * 2 - 1
    Q.scatter_(2, idx, sign)
    return Q.to(torch.bfloat16)


EXACT = [  # (batch, Lq, Lk, d)
    (2, 256, 128, 128),
    (1, 512, 640, 64),
    (1, 300, 77, 128),      # ragged queries and keys (last key tile 13 of 64)
    (3, 97, 1, 64),         # a single key
    (1, 1, 200, 128),
]


@pytest.mark.parametrize("items", [256, 128])
@pytest.mark.parametrize("b,Lq,Lk,d", EXACT)
def test_exact_power_of_two_probabilities(b, Lq, Lk, d, items):
    _say("attn exact b=%d Lq=%d Lk=%d d=%d items=%d" % (b, Lq, Lk, d, items))
    Q = _sparse_q(b, Lq, d, 900 + Lq)
    K = draw((b, Lk, d), "int", -1, 1, 901 + Lk)
    V = draw((b, Lk, d), "int", -4, 4, 902 + d)
    got, _ = _run(Q, K, V, math.log(2.0), out="f32", items=items)
    ref, TO = _ref(Q, K, V, math.log(2.0))
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    assert np.all(err <= 2.0 ** -18 * TO), "max err/TO %.3g, max err/|O| %.3g" % (
        (err / TO).max(), (err / np.maximum(np.abs(ref), 1e-30)).max())


RANDOM = [  # (batch, Lq, Lk, d, out)
    (2, 512, 512, 128, "bf16"),
    (2, 512, 512, 128, "f32"),
    (1, 300, 1000, 64, "f32"),
    (3, 129, 77, 128, "bf16"),
    (1, 1024, 2048, 64, "bf16"),
]


@pytest.mark.parametrize("items", [256, 128])
@pytest.mark.parametrize("b,Lq,Lk,d,out", RANDOM)
def test_random_data_within_tolerance(b, Lq, Lk, d, out, items):
    _say("attn random b=%d Lq=%d Lk=%d d=%d out=%s items=%d" % (b, Lq, Lk, d, out, items))
    Q = draw((b, Lq, d), "normal", 0, 1, 910 + Lq)
    K = draw((b, Lk, d), "normal", 0, 1, 911 + Lk)
    V = draw((b, Lk, d), "normal", 0, 1, 912 + d)
    scale = d ** -0.5
    got, _ = _run(Q, K, V, scale, out=out, items=items)
    ref, TO = _ref(Q, K, V, scale)
    nfail, util = oracle.check_attention(got, ref, TO, out_bf16=(out == "bf16"))
    assert nfail == 0, "%d outside tolerance, max util %.3g" % (nfail, util)


def _random_attention_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        causal = bool(rng.integers(0, 2))
        Lq = int(rng.integers(1, 520))
        Lk = Lq + int(rng.integers(0, 300)) if causal else int(rng.integers(1, 700))
        cases.append((int(rng.integers(1, 4)), Lq, Lk, [64, 128][i % 2], causal, [256, 128][(i // 2) % 2],
                      "bf16" if rng.integers(0, 2) else "f32"))
    return cases


@pytest.mark.parametrize("b,Lq,Lk,d,causal,items,out", _random_attention_cases(24, 4242))
def test_random_attention_shapes_within_tolerance(b, Lq, Lk, d, causal, items, out):
    """Seeded random sizes (ragged queries and keys, both head sizes, with and
    without the causal mask, both item shapes, both output types)."""
    _say("attn random shape b=%d Lq=%d Lk=%d d=%d causal=%s items=%d out=%s" % (b, Lq, Lk, d, causal, items, out))
    Q = draw((b, Lq, d), "normal", 0, 1, 930 + Lq)
    K = draw((b, Lk, d), "normal", 0, 1, 931 + Lk)
    V = draw((b, Lk, d), "normal", 0, 1, 932 + d)
    scale = d ** -0.5
    got, _ = _run(Q, K, V, scale, out=out, causal=causal, items=items)
    ref, TO = _ref(Q, K, V, scale, causal=causal)
    nfail, util = oracle.check_attention(got, ref, TO, out_bf16=(out == "bf16"))
    assert nfail == 0, "%d outside tolerance, max util %.3g" % (nfail, util)


def test_padded_output_leaves_the_rest_untouched():
    # O rows of stride 136 with 2 spare rows per slice: only [0, Lq) x [0, dv) is written
    b, Lq, Lk, d = 2, 300, 200, 128
    Q = draw((b, Lq, d), "normal", 0, 1, 920)
    K = draw((b, Lk, d), "normal", 0, 1, 921)
    V = draw((b, Lk, d), "normal", 0, 1, 922)
    got, raw = _run(Q, K, V, 0.1, out="f32", ldo=136, rows_pad=2)
    ref, TO = _ref(Q, K, V, 0.1)
    assert oracle.check_attention(got, ref, TO)[0] == 0
    mask = np.ones(raw.shape, dtype=bool)
    mask[:, :Lq, :d] = False
    assert np.all(np.isnan(raw[mask]))


# Oracle threads: a one-GPU job's share of its host is 16 cores.
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@functools.lru_cache(maxsize=2)
def _workload_ref(name, causal):
    """The oracle's O and TO for every query of workload `name` (computed once per module)."""
    w = ATTN_WORKLOADS[name]
    Q, K, V = attn_operands(w)
    sq, sk, sv, _ = w.strides()
    return oracle.attention(bits(Q), bits(K), bits(V), w.batch, w.Lq, w.Lk, w.d, w.dv, sq, sk, sv, w.scale,
                            nthreads=ORACLE_THREADS, causal=causal)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("items", [None, 128])
def test_workload_every_row_and_determinism(items):
    w = ATTN_WORKLOADS["attn32x2048"]
    _say("attn workload %s every row items=%s" % (w.name, items))
    Q, K, V = attn_operands(w)
    got, _ = _run(Q, K, V, w.scale, out=w.out, items=items)
    again, _ = _run(Q, K, V, w.scale, out=w.out, items=items)
    assert np.array_equal(got, again)
    ref, TO = _workload_ref(w.name, False)
    nfail, util = oracle.check_attention(got, ref, TO, out_bf16=(w.out == "bf16"))
    assert nfail == 0, "%d outside tolerance, max util %.3g" % (nfail, util)


def test_matches_the_unfused_path_on_the_score_workload():
    # softmax of the scores sscore_run writes, times V, agrees with the fused
    # result (both against the oracle's bound) on two slices of the workload
    w = ATTN_WORKLOADS["attn32x2048"]
    Q, K, V = (t[:2].contiguous() for t in attn_operands(w))
    got, _ = _run(Q, K, V, w.scale, out="f32")
    S = asl.sscore(Q.to(DEV), K.to(DEV))
    P = torch.softmax(S.double() * w.scale, dim=2)
    O = (P @ V.to(DEV).double()).cpu().numpy()
    ref, TO = _ref(Q, K, V, w.scale, rows=np.array([[b, i] for b in range(2) for i in range(0, w.Lq, 37)]))
    sel = O[:, ::37].reshape(-1, w.dv)
    assert np.max(np.abs(sel - ref)) < 1e-5       # the unfused fp32-score path is near exact
    nfail, _ = oracle.check_attention(got[:, ::37].reshape(-1, w.dv), ref, TO)
    assert nfail == 0


CAUSAL = [  # (batch, Lq, Lk, d)
    (2, 512, 512, 128),      # diagonal through every wave's tiles
    (1, 300, 1000, 64),      # Lk > Lq: the mask aligned to the last key
    (3, 129, 129, 128),      # ragged queries and keys
    (1, 1, 77, 128),         # one query sees every key
    (1, 640, 700, 64),
]


@pytest.mark.parametrize("items", [256, 128])
@pytest.mark.parametrize("b,Lq,Lk,d", CAUSAL)
def test_causal_exact_power_of_two_probabilities(b, Lq, Lk, d, items):
    _say("attn causal exact b=%d Lq=%d Lk=%d d=%d items=%d" % (b, Lq, Lk, d, items))
    Q = _sparse_q(b, Lq, d, 940 + Lq)
    K = draw((b, Lk, d), "int", -1, 1, 941 + Lk)
    V = draw((b, Lk, d), "int", -4, 4, 942 + d)
    got, _ = _run(Q, K, V, math.log(2.0), out="f32", causal=True, items=items)
    ref, TO = _ref(Q, K, V, math.log(2.0), causal=True)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    assert np.all(err <= 2.0 ** -18 * TO), "max err/TO %.3g" % (err / TO).max()


@pytest.mark.parametrize("items", [256, 128])
@pytest.mark.parametrize("b,Lq,Lk,d", CAUSAL)
def test_causal_random_data_within_tolerance(b, Lq, Lk, d, items):
    _say("attn causal random b=%d Lq=%d Lk=%d d=%d items=%d" % (b, Lq, Lk, d, items))
    Q = draw((b, Lq, d), "normal", 0, 1, 950 + Lq)
    K = draw((b, Lk, d), "normal", 0, 1, 951 + Lk)
    V = draw((b, Lk, d), "normal", 0, 1, 952 + d)
    got, _ = _run(Q, K, V, d ** -0.5, out="bf16", causal=True, items=items)
    ref, TO = _ref(Q, K, V, d ** -0.5, causal=True)
    nfail, util = oracle.check_attention(got, ref, TO, out_bf16=True)
    assert nfail == 0, "%d outside tolerance, max util %.3g" % (nfail, util)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("items", [None, 256])
def test_causal_workload_every_row(items):
    w = ATTN_WORKLOADS["attn32x2048_causal"]
    _say("attn causal workload every row items=%s" % items)
    Q, K, V = attn_operands(w)
    got, _ = _run(Q, K, V, w.scale, out=w.out, causal=True, items=items)
    ref, TO = _workload_ref(w.name, True)
    nfail, util = oracle.check_attention(got, ref, TO, out_bf16=True)
    assert nfail == 0, "%d outside tolerance, max util %.3g" % (nfail, util)


def test_item_shapes_agree_and_each_is_deterministic():
    # the two work-item shapes sum in different orders: equal within the
    # bound, each bitwise repeatable
    b, Lq, Lk, d = 2, 700, 900, 128
    Q = draw((b, Lq, d), "normal", 0, 1, 970)
    K = draw((b, Lk, d), "normal", 0, 1, 971)
    V = draw((b, Lk, d), "normal", 0, 1, 972)
    ref, TO = _ref(Q, K, V, 0.09)
    for items in (256, 128):
        got, _ = _run(Q, K, V, 0.09, out="f32", items=items)
        again, _ = _run(Q, K, V, 0.09, out="f32", items=items)
        assert np.array_equal(got, again)
        assert oracle.check_attention(got, ref, TO)[0] == 0


PERSISTENT = [  # (batch, Lq, Lk, d, items): more items than the 256 resident workgroups
    (300, 128, 128, 64, 128),
    (150, 200, 260, 128, 128),      # ragged: 2 query tiles per slice, partial key stages
    (520, 100, 130, 64, 256),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("b,Lq,Lk,d,items", PERSISTENT)
def test_persistent_schedules_equal_one_workgroup_per_item(b, Lq, Lk, d, items, causal):
    # each item's arithmetic is the same whichever workgroup runs it, so the
    # three schedules agree bit for bit; the exact pin checks the result
    _say("attn persistent b=%d Lq=%d Lk=%d d=%d items=%d causal=%d" % (b, Lq, Lk, d, items, causal))
    Q = _sparse_q(b, Lq, d, 980 + Lq)
    K = draw((b, Lk, d), "int", -1, 1, 981 + Lk)
    V = draw((b, Lk, d), "int", -4, 4, 982 + d)
    one, _ = _run(Q, K, V, math.log(2.0), out="f32", causal=causal, items=items, sched="one")
    ref, TO = _ref(Q, K, V, math.log(2.0), causal=causal)
    assert np.all(np.abs(one - ref) <= 2.0 ** -18 * TO)
    for sched in ("static", "queue", "queue"):
        got, _ = _run(Q, K, V, math.log(2.0), out="f32", causal=causal, items=items, sched=sched)
        assert np.array_equal(got, one), sched


def test_queue_counters_reset_between_launches():
    # back-to-back queue launches of shrinking size: a launch that left its
    # counters behind would make a later one skip items (NaN rows remain)
    w = ATTN_WORKLOADS["attn32x2048"]
    Q, K, V = attn_operands(w)
    full, _ = _run(Q, K, V, w.scale, out="f32", causal=True, sched="one")
    for nb in (32, 31, 9, 32):
        got, _ = _run(Q[:nb].contiguous(), K[:nb].contiguous(), V[:nb].contiguous(), w.scale, out="f32",
                      causal=True, sched="queue")
        assert np.array_equal(got, full[:nb]), nb
    # every launch takes the next of 64 counter slots: 150 more launches reuse
    # each slot at least twice
    Qs, Ks, Vs = Q[:3].contiguous(), K[:3].contiguous(), V[:3].contiguous()
    Qd, Kd, Vd = Qs.to(DEV), Ks.to(DEV), Vs.to(DEV)
    Ob = torch.empty((3, w.Lq, w.dv), dtype=torch.float32, device=DEV)
    ref = torch.from_numpy(full[:3]).float().to(DEV)
    bad = []
    for i in range(150):
        Ob.fill_(float("nan"))
        asl.attn_fwd_run(Qd.data_ptr(), Kd.data_ptr(), Vd.data_ptr(), Ob.data_ptr(), 3, w.Lq, w.Lk, w.d, w.dv,
                         (w.d, 1, w.Lq * w.d), (w.d, 1, w.Lk * w.d), (w.dv, 1, w.Lk * w.dv),
                         (w.dv, 1, w.Lq * w.dv), w.scale, asl.AS_BF16, asl.AS_F32,
                         flags=asl.AS_ATTN_CAUSAL | asl.AS_ATTN_SCHED_QUEUE,
                         stream=torch.cuda.current_stream().cuda_stream)
        if not torch.equal(Ob, ref):
            bad.append(i)
    assert not bad, "launches %s differ" % bad[:10]


def test_queue_launches_overlapping_on_concurrent_streams():
    # Successive launches take successive counter slots, so queue launches
    # that overlap on different streams never share counters.  Three streams
    # each enqueue 12 causal queue launches on their own data, with no
    # synchronization between the streams; every output must equal that
    # data's lone launch bit for bit (the schedule is deterministic).
    b, L, d, rounds = 8, 1024, 128, 12
    _say("queue launches on 3 concurrent streams, b=%d L=%d d=%d, %d rounds" % (b, L, d, rounds))
    scale = d ** -0.5
    data = [tuple(draw((b, L, d), "normal", 0, 1, 4100 + 3 * i + j).to(DEV) for j in range(3)) for i in range(3)]

    def launch(i, O, stream):
        Q, K, V = data[i]
        asl.attn_fwd_run(Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), b, L, L, d, d,
                         (d, 1, L * d), (d, 1, L * d), (d, 1, L * d), (d, 1, L * d), scale,
                         asl.AS_BF16, asl.AS_F32, flags=asl.AS_ATTN_CAUSAL | asl.AS_ATTN_SCHED_QUEUE,
                         stream=stream.cuda_stream)

    refs = []
    for i in range(3):
        O = torch.empty((b, L, d), dtype=torch.float32, device=DEV)
        launch(i, O, torch.cuda.current_stream())
        torch.cuda.synchronize()
        refs.append(O)
    outs = [[torch.full((b, L, d), float("nan"), dtype=torch.float32, device=DEV) for _ in range(rounds)]
            for _ in range(3)]
    streams = [torch.cuda.Stream(device=DEV) for _ in range(3)]
    torch.cuda.synchronize()
    for r in range(rounds):
        for i, st in enumerate(streams):
            launch(i, outs[i][r], st)
    torch.cuda.synchronize()
    bad = [(i, r) for i in range(3) for r in range(rounds) if not torch.equal(outs[i][r], refs[i])]
    assert not bad, "stream/round %s differ from the lone launch" % bad[:10]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("items", [256, 128])
def test_negative_scale_exact_power_of_two_probabilities(items, causal):
    # scale -ln 2: the scale's sign flips the max into a min (the kernel's
    # second specialisation); probabilities are again powers of two
    b, Lq, Lk, d = 2, 300, 333, 128
    _say("attn negative scale items=%d causal=%d" % (items, causal))
    Q = _sparse_q(b, Lq, d, 990)
    K = draw((b, Lk, d), "int", -1, 1, 991)
    V = draw((b, Lk, d), "int", -4, 4, 992)
    got, _ = _run(Q, K, V, -math.log(2.0), out="f32", causal=causal, items=items)
    ref, TO = _ref(Q, K, V, -math.log(2.0), causal=causal)
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= 2.0 ** -18 * TO)


@pytest.mark.parametrize("items", [256, 128])
def test_negative_scale_random_data_within_tolerance(items):
    b, Lq, Lk, d = 2, 512, 640, 64
    Q = draw((b, Lq, d), "normal", 0, 1, 993)
    K = draw((b, Lk, d), "normal", 0, 1, 994)
    V = draw((b, Lk, d), "normal", 0, 1, 995)
    got, _ = _run(Q, K, V, -0.2, out="bf16", items=items)
    ref, TO = _ref(Q, K, V, -0.2)
    assert oracle.check_attention(got, ref, TO, out_bf16=True)[0] == 0


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_is_the_mean_of_the_visible_values(causal):
    # every probability is 1: O_i is the plain mean of the V rows query i sees
    b, Lq, Lk, d = 2, 200, 260, 128
    Q = draw((b, Lq, d), "normal", 0, 1, 996)
    K = draw((b, Lk, d), "normal", 0, 1, 997)
    V = draw((b, Lk, d), "int", -4, 4, 998)
    for items in (256, 128):
        got, _ = _run(Q, K, V, 0.0, out="f32", causal=causal, items=items)
        v = V.double().numpy()
        off = Lk - Lq
        for i in (0, 1, Lq // 2, Lq - 1):
            n = i + off + 1 if causal else Lk
            assert np.allclose(got[:, i], v[:, :n].mean(axis=1), rtol=0, atol=1e-6), (items, i)


def test_one_key_value_head_shared_by_all_slices():
    # multi-query attention: K and V with batch stride 0 serve every slice
    b, Lq, Lk, d = 6, 256, 320, 128
    Q = draw((b, Lq, d), "normal", 0, 1, 999)
    K1 = draw((1, Lk, d), "normal", 0, 1, 1000)
    V1 = draw((1, Lk, d), "normal", 0, 1, 1001)
    Qd, Kd, Vd = Q.to(DEV), K1.to(DEV), V1.to(DEV)
    for items in (256, 128):
        Ob = torch.full((b, Lq, d), float("nan"), dtype=torch.float32, device=DEV)
        asl.attn_fwd_run(Qd.data_ptr(), Kd.data_ptr(), Vd.data_ptr(), Ob.data_ptr(), b, Lq, Lk, d, d,
                         (d, 1, Lq * d), (d, 1, 0), (d, 1, 0), (d, 1, Lq * d), 0.1, asl.AS_BF16, asl.AS_F32,
                         flags=ITEMS[items], stream=torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        got = Ob.double().cpu().numpy()
        ref, TO = oracle.attention(bits(Q), bits(K1), bits(V1), b, Lq, Lk, d, d, (d, 1, Lq * d), (d, 1, 0),
                                   (d, 1, 0), 0.1)
        assert oracle.check_attention(got, ref, TO)[0] == 0


GQA = [  # (batch, kv_group, Lq, Lk, d)
    (8, 4, 300, 300, 128),
    (16, 8, 256, 384, 64),
    (6, 3, 129, 200, 128),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("items", [256, 128])
@pytest.mark.parametrize("b,g,Lq,Lk,d", GQA)
def test_grouped_key_value_heads(b, g, Lq, Lk, d, items, causal):
    # the grouped launch equals the ungrouped one on materialised repeats bit
    # for bit (each item's arithmetic is the same), and the exact pin holds
    _say("attn gqa b=%d g=%d Lq=%d Lk=%d d=%d items=%d causal=%d" % (b, g, Lq, Lk, d, items, causal))
    Q = _sparse_q(b, Lq, d, 1010 + Lq)
    K = draw((b // g, Lk, d), "int", -1, 1, 1011 + Lk)
    V = draw((b // g, Lk, d), "int", -4, 4, 1012 + d)
    Qd, Kd, Vd = Q.to(DEV), K.to(DEV), V.to(DEV)
    Ob = torch.full((b, Lq, d), float("nan"), dtype=torch.float32, device=DEV)
    flags = (asl.AS_ATTN_CAUSAL if causal else 0) | ITEMS[items]
    asl.attn_fwd_run_gqa(Qd.data_ptr(), Kd.data_ptr(), Vd.data_ptr(), Ob.data_ptr(), b, g, Lq, Lk, d, d,
                         (d, 1, Lq * d), (d, 1, Lk * d), (d, 1, Lk * d), (d, 1, Lq * d), math.log(2.0),
                         asl.AS_BF16, asl.AS_F32, flags=flags, stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = Ob.double().cpu().numpy()
    rep, _ = _run(Q, K.repeat_interleave(g, dim=0).contiguous(), V.repeat_interleave(g, dim=0).contiguous(),
                  math.log(2.0), out="f32", causal=causal, items=items)
    assert np.array_equal(got, rep)
    ref, TO = oracle.attention(bits(Q), bits(K), bits(V), b, Lq, Lk, d, d, (d, 1, Lq * d), (d, 1, Lk * d),
                               (d, 1, Lk * d), math.log(2.0), causal=causal, kv_group=g)
    assert np.all(np.abs(got - ref) <= 2.0 ** -18 * TO)


def test_attention_helper_with_grouped_heads():
    b, g, L, d = 8, 4, 256, 128
    Q = draw((b, L, d), "normal", 0, 1, 1020).to(DEV)
    K = draw((b // g, L, d), "normal", 0, 1, 1021).to(DEV)
    V = draw((b // g, L, d), "normal", 0, 1, 1022).to(DEV)
    O = asl.attention(Q, K, V, causal=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, TO = oracle.attention(bits(Q.cpu()), bits(K.cpu()), bits(V.cpu()), b, L, L, d, d, (d, 1, L * d),
                               (d, 1, L * d), (d, 1, L * d), d ** -0.5, causal=True, kv_group=g)
    assert oracle.check_attention(O.double().cpu().numpy(), ref, TO)[0] == 0
