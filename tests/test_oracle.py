"""Pins of the CPU oracle to things other than itself (CPU only).

Each pin is chosen so that a plausible slip in the oracle -- a dropped term, a
wrong sign, an exchanged index or stride, a transposed operand, a wrong
rounding rule -- fails at least one of them; ``test_pins_catch_planted_mistakes``
plants such slips on the CPU and shows they are caught.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import bits, draw

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f64(bits_arr):
    return oracle.bf16_bits_to_f64_array(bits_arr)


def _bf16_bits_of(values):
    """Exact bf16 bits of values that are representable in bf16 (checked)."""
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    b = bits(t)
    assert np.array_equal(_f64(b), np.asarray(values, dtype=np.float64)), "value not exact in bf16"
    return b


def _rowmajor_gemm(A_bits, B_bits, M, N, K, want_T=True):
    C, T = oracle.gemm(A_bits, B_bits, 1, M, N, K, (K, 1, 0), (N, 1, 0), want_T=want_T)
    return C[0], (T[0] if want_T else None)


# ------------------------------------------------------------------ bf16 --

def _read_pairs(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, b = line.split()
                rows.append((a, b))
    return rows


def test_bf16_decode_golden():
    for hexbits, expr in _read_pairs("bf16_decode.txt"):
        want = float(eval(expr, {"__builtins__": {}}))
        got = oracle.bf16_to_f64(int(hexbits, 16))
        assert got == want and np.signbit(got) == np.signbit(want), (hexbits, got, want)


def test_bf16_rne_golden():
    for expr, hexbits in _read_pairs("bf16_rne.txt"):
        x = float(eval(expr, {"__builtins__": {}}))
        assert oracle.f64_to_bf16_rne(x) == int(hexbits, 16), (expr, hex(oracle.f64_to_bf16_rne(x)))


def test_bf16_rne_matches_torch_conversion():
    # torch's float32 -> bfloat16 cast is an independent round-to-nearest-even.
    g = torch.Generator().manual_seed(7)
    x = torch.randn(20000, generator=g) * torch.exp2(torch.randint(-20, 20, (20000,), generator=g).float())
    # plant exact ties: bf16 value plus half an ulp
    ties = (torch.randn(2000, generator=g).to(torch.bfloat16).float())
    ties = ties + ties.abs() * 2.0 ** -8
    x = torch.cat([x, ties])
    want = bits(x.to(torch.bfloat16))
    got = np.array([oracle.f64_to_bf16_rne(float(v)) for v in x.tolist()], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_bf16_decode_vector_matches_scalar():
    b = np.arange(0, 65536, 97, dtype=np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]  # finite only
    vec = _f64(b)
    sca = np.array([oracle.bf16_to_f64(int(v)) for v in b])
    assert np.array_equal(vec, sca)


# ------------------------------------------------------- hand-worked GEMM --

def _read_gemm_cases():
    cases = []
    with open(os.path.join(GOLDEN, "gemm_hand.txt")) as f:
        lines = [l.strip() for l in f if l.strip() and not l.startswith("#")]
    i = 0
    while i < len(lines):
        _, name, M, N, K = lines[i].split()
        M, N, K = int(M), int(N), int(K)
        i += 1
        def take(r):
            nonlocal i
            m = np.array([[float(x) for x in lines[i + t].split()] for t in range(r)])
            i += r
            return m
        A, B, C, T = take(M), take(K), take(M), take(M)
        cases.append((name, A, B, C, T))
    return cases


@pytest.mark.parametrize("case", _read_gemm_cases(), ids=lambda c: c[0])
def test_gemm_hand_worked(case):
    name, A, B, C, T = case
    M, K = A.shape
    N = B.shape[1]
    Cg, Tg = _rowmajor_gemm(_bf16_bits_of(A), _bf16_bits_of(B), M, N, K)
    assert np.array_equal(Cg, C) and np.array_equal(Tg, T)


def test_sscore_hand_worked():
    with open(os.path.join(GOLDEN, "sscore_hand.txt")) as f:
        lines = [l.strip() for l in f if l.strip() and not l.startswith("#")]
    blocks, cur = {}, None
    for l in lines:
        if l in ("Q", "K", "S", "T"):
            cur = l
            blocks[cur] = []
        else:
            blocks[cur].append([float(x) for x in l.split()])
    Q, Kt, S, T = (np.array(blocks[k]) for k in "QKST")
    Lq, d = Q.shape
    Lk = Kt.shape[0]
    Sg, Tg = oracle.sscore(_bf16_bits_of(Q), _bf16_bits_of(Kt), 1, Lq, Lk, d, (d, 1, Lq * d), (d, 1, Lk * d))
    assert np.array_equal(Sg[0], S) and np.array_equal(Tg[0], T)


# --------------------------------------------------------------- closed forms --

@pytest.mark.parametrize("M,N", [(16, 7), (64, 64), (33, 100)])
def test_identity_A_gives_B(M, N):
    K = M
    eye = _bf16_bits_of(np.eye(M))
    B = bits(draw((K, N), "normal", 0, 1, 11))
    C, T = _rowmajor_gemm(eye, B, M, N, K)
    assert np.array_equal(C, _f64(B))
    assert np.array_equal(T, np.abs(_f64(B)))


@pytest.mark.parametrize("M,K", [(9, 16), (64, 64), (100, 33)])
def test_identity_B_gives_A(M, K):
    N = K
    A = bits(draw((M, K), "uniform", -1, 1, 12))
    C, _ = _rowmajor_gemm(A, _bf16_bits_of(np.eye(K)), M, N, K)
    assert np.array_equal(C, _f64(A))


@pytest.mark.parametrize("K", [1, 128, 512, 2048])
def test_all_ones_gives_K(K):
    M, N = 5, 6
    C, T = _rowmajor_gemm(_bf16_bits_of(np.ones((M, K))), _bf16_bits_of(np.ones((K, N))), M, N, K)
    assert np.all(C == K) and np.all(T == K)


def test_rank1_closed_form():
    M, N, K = 12, 10, 64
    alpha = 2.0 ** np.arange(-3, M - 3)
    beta = -(2.0 ** np.arange(-2, N - 2))
    A = np.repeat(alpha[:, None], K, axis=1)
    B = np.repeat(beta[None, :], K, axis=0)
    C, T = _rowmajor_gemm(_bf16_bits_of(A), _bf16_bits_of(B), M, N, K)
    assert np.array_equal(C, K * np.outer(alpha, beta))
    assert np.array_equal(T, K * np.abs(np.outer(alpha, beta)))


def test_integer_data_is_exact_against_integer_matmul():
    # integer entries in [-4, 4]: every partial sum is an exact integer, so the
    # oracle must equal numpy's int64 matmul (an independent exact routine).
    M, N, K = 37, 29, 300
    Ai = draw((M, K), "int", -4, 4, 21)
    Bi = draw((K, N), "int", -4, 4, 22)
    C, T = _rowmajor_gemm(bits(Ai), bits(Bi), M, N, K)
    a = Ai.float().numpy().astype(np.int64)
    b = Bi.float().numpy().astype(np.int64)
    assert np.array_equal(C, (a @ b).astype(np.float64))
    assert np.array_equal(T, (np.abs(a) @ np.abs(b)).astype(np.float64))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 7, 16, 33])
@pytest.mark.parametrize("N", [1, 3, 16, 33])
@pytest.mark.parametrize("K", [1, 2, 7, 33])
def test_brute_force_tiny_vs_numpy(M, N, K):
    A = bits(draw((M, K), "normal", 0, 1, 1000 + M * 100 + K))
    B = bits(draw((K, N), "uniform", -1, 1, 2000 + N * 100 + K))
    C, T = _rowmajor_gemm(A, B, M, N, K)
    a, b = _f64(A).reshape(M, K), _f64(B).reshape(K, N)
    ref = a @ b                     # numpy float64 matmul: independent library routine
    refT = np.abs(a) @ np.abs(b)
    assert np.all(np.abs(C - ref) <= 1e-12 * refT + 1e-300)
    assert np.all(np.abs(T - refT) <= 1e-12 * refT + 1e-300)


def test_bilinearity():
    M, N, K = 20, 24, 96
    A1 = draw((M, K), "int", -3, 3, 31)
    A2 = draw((M, K), "int", -3, 3, 32)
    B = bits(draw((K, N), "normal", 0, 1, 33))
    Asum = (A1.float() + A2.float()).to(torch.bfloat16)  # exact: small integers
    C1, _ = _rowmajor_gemm(bits(A1), B, M, N, K)
    C2, _ = _rowmajor_gemm(bits(A2), B, M, N, K)
    Cs, Ts = _rowmajor_gemm(bits(Asum), B, M, N, K)
    assert np.all(np.abs(Cs - (C1 + C2)) <= 1e-13 * (Ts + 1))


def test_magnitude_sum_bounds_result():
    M, N, K = 31, 17, 257
    A = bits(draw((M, K), "normal", 0, 1, 41))
    B = bits(draw((K, N), "normal", 0, 1, 42))
    C, T = _rowmajor_gemm(A, B, M, N, K)
    assert np.all(np.abs(C) <= T)
    assert np.all(T > 0)


# ------------------------------------------------------------------- layouts --

def test_column_major_A_equals_materialized():
    M, N, K = 48, 40, 72
    At = draw((K, M), "uniform", -0.5, 0.5, 51)       # storage of a column-major A
    B = bits(draw((K, N), "uniform", -0.5, 0.5, 52))
    C_col, T_col = oracle.gemm(bits(At), B, 1, M, N, K, (1, M, 0), (N, 1, 0))
    A_mat = bits(At.t().contiguous())
    C_row, T_row = oracle.gemm(A_mat, B, 1, M, N, K, (K, 1, 0), (N, 1, 0))
    assert np.array_equal(C_col, C_row) and np.array_equal(T_col, T_row)


def test_k_major_B_equals_materialized():
    M, N, K = 30, 50, 64
    A = bits(draw((M, K), "normal", 0, 1, 61))
    Bt = draw((N, K), "normal", 0, 1, 62)             # B[k, j] stored at j*K + k
    C_t, _ = oracle.gemm(A, bits(Bt), 1, M, N, K, (K, 1, 0), (1, K, 0))
    C_r, _ = oracle.gemm(A, bits(Bt.t().contiguous()), 1, M, N, K, (K, 1, 0), (N, 1, 0))
    assert np.array_equal(C_t, C_r)


def test_sscore_equals_gemm_with_materialized_transpose():
    b, Lq, Lk, d = 3, 20, 24, 32
    Q = draw((b, Lq, d), "normal", 0, 1, 71)
    Kt = draw((b, Lk, d), "normal", 0, 1, 72)
    S, T = oracle.sscore(bits(Q), bits(Kt), b, Lq, Lk, d, (d, 1, Lq * d), (d, 1, Lk * d))
    KT = Kt.transpose(1, 2).contiguous()               # [b, d, Lk]
    C, Tc = oracle.gemm(bits(Q), bits(KT), b, Lq, Lk, d, (d, 1, Lq * d), (Lk, 1, d * Lk))
    assert np.array_equal(S, C) and np.array_equal(T, Tc)


def test_sscore_symmetric_when_Q_equals_K():
    b, L, d = 2, 33, 64
    Q = bits(draw((b, L, d), "normal", 0, 1, 81))
    S, _ = oracle.sscore(Q, Q, b, L, L, d, (d, 1, L * d), (d, 1, L * d))
    assert np.array_equal(S, np.transpose(S, (0, 2, 1)))


def test_batch_stride_zero_broadcasts():
    b, M, N, K = 3, 8, 9, 16
    A = draw((b, M, K), "normal", 0, 1, 91)
    B = bits(draw((K, N), "normal", 0, 1, 92))
    C, _ = oracle.gemm(bits(A), B, b, M, N, K, (K, 1, M * K), (N, 1, 0))
    for i in range(b):
        Ci, _ = oracle.gemm(bits(A[i].contiguous()), B, 1, M, N, K, (K, 1, 0), (N, 1, 0))
        assert np.array_equal(C[i], Ci[0])


def test_points_equal_full_product():
    b, M, N, K = 2, 40, 36, 80
    A = draw((b, M, K), "normal", 0, 1, 101)
    B = draw((b, K, N), "normal", 0, 1, 102)
    sa, sb = (K, 1, M * K), (N, 1, K * N)
    C, T = oracle.gemm(bits(A), bits(B), b, M, N, K, sa, sb)
    rng = np.random.default_rng(0)
    pts = np.stack([rng.integers(0, b, 200), rng.integers(0, M, 200), rng.integers(0, N, 200)], 1)
    Cp, Tp = oracle.gemm_points(bits(A), bits(B), pts, K, sa, sb, dims=(b, M, N))
    assert np.array_equal(Cp, C[pts[:, 0], pts[:, 1], pts[:, 2]])
    assert np.array_equal(Tp, T[pts[:, 0], pts[:, 1], pts[:, 2]])
    Q = draw((b, M, K), "normal", 0, 1, 103)
    Kt = draw((b, N, K), "normal", 0, 1, 104)
    S, _ = oracle.sscore(bits(Q), bits(Kt), b, M, N, K, (K, 1, M * K), (K, 1, N * K))
    Sp, _ = oracle.sscore_points(bits(Q), bits(Kt), pts, K, (K, 1, M * K), (K, 1, N * K))
    assert np.array_equal(Sp, S[pts[:, 0], pts[:, 1], pts[:, 2]])


def test_threads_do_not_change_result():
    M, N, K = 50, 30, 100
    A = bits(draw((M, K), "normal", 0, 1, 111))
    B = bits(draw((K, N), "normal", 0, 1, 112))
    C1, T1 = oracle.gemm(A, B, 1, M, N, K, (K, 1, 0), (N, 1, 0), nthreads=1)
    C7, T7 = oracle.gemm(A, B, 1, M, N, K, (K, 1, 0), (N, 1, 0), nthreads=7)
    assert np.array_equal(C1, C7) and np.array_equal(T1, T7)


def test_view_outside_buffer_rejected():
    A = np.zeros(10, dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm(A, A, 1, 4, 4, 4, (4, 1, 0), (4, 1, 0))


# ---------------------------------------------------------------- tolerance --

def test_check_accepts_and_rejects():
    ref = np.array([1.0, -2.0, 0.0, 5.0])
    T = np.array([10.0, 2.0, 0.0, 5.0])
    bound = 1e-3 * T + 1e-5
    ok = ref + 0.99 * bound
    assert oracle.check(ok, ref, T)[0] == 0
    bad = ref.copy()
    bad[1] += 1.01 * bound[1]
    assert oracle.check(bad, ref, T)[0] == 1
    nan = ref.copy()
    nan[2] = np.nan
    assert oracle.check(nan, ref, T)[0] == 1
    inf = ref.copy()
    inf[3] = np.inf
    assert oracle.check(inf, ref, T)[0] == 1


def test_rne_array_equals_the_pinned_scalar():
    # The vector rounding used by every bf16 bit-exact comparison is the
    # scalar rule pinned above (hand-worked fixtures and torch's cast),
    # element by element: the golden values, torch's tie set, specials.
    golden = [float(eval(e, {"__builtins__": {}})) for e, _ in _read_pairs("bf16_rne.txt")]
    want_golden = [int(h, 16) for _, h in _read_pairs("bf16_rne.txt")]
    g = torch.Generator().manual_seed(11)
    ties = torch.randn(3000, generator=g).to(torch.bfloat16).double()
    ties = torch.cat([ties + ties.abs() * 2.0 ** -8, ties - ties.abs() * 2.0 ** -9,
                      torch.randn(3000, generator=g, dtype=torch.float64) * 1e3])
    x = np.concatenate([np.array(golden), ties.numpy(), [0.0, -0.0, np.inf, -np.inf, np.nan, 1e300, -1e-300]])
    arr = oracle.f64_to_bf16_rne_array(x)
    sca = np.array([oracle.f64_to_bf16_rne(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(arr, sca)
    assert list(arr[:len(golden)]) == want_golden
    # shape is kept and torch agrees on the float32-representable part
    x2 = ties.numpy()[:3000].reshape(30, 100)
    a2 = oracle.f64_to_bf16_rne_array(x2)
    assert a2.shape == (30, 100)
    assert np.array_equal(a2, bits(torch.from_numpy(x2).float().to(torch.bfloat16)))


def test_check_attention_accepts_rounded_probabilities_and_rejects_beyond():
    # What the attention tolerance is for: a result whose probabilities were
    # rounded to bf16 before the P.V product (simulated here with torch's
    # independent bf16 cast, normalised by the unrounded sum) must pass, with
    # room to spare; results moved past the bound must fail; NaN and Inf fail;
    # a bf16 output gets its own rounding (2^-8 |O|) on top.
    rng = np.random.default_rng(5)
    n, Lk, dv = 64, 300, 16
    t = rng.normal(0, 3, (n, Lk))
    p = np.exp(t - t.max(axis=1, keepdims=True))
    V = rng.normal(0, 1, (Lk, dv))
    O_ref = p @ V / p.sum(axis=1, keepdims=True)
    TO = p @ np.abs(V) / p.sum(axis=1, keepdims=True)
    p_bf = torch.from_numpy(p).to(torch.bfloat16).double().numpy()
    O_fused = p_bf @ V / p.sum(axis=1, keepdims=True)
    nfail, util = oracle.check_attention(O_fused, O_ref, TO)
    assert nfail == 0 and util <= 0.5                     # rounding p costs at most 2^-8 TO: half the bound
    bound = 2.0 ** -7 * TO + 1e-6
    assert oracle.check_attention(O_ref + 0.99 * bound, O_ref, TO)[0] == 0
    assert oracle.check_attention(O_ref - 1.01 * bound, O_ref, TO)[0] == O_ref.size
    moved = O_ref.copy()
    moved[3, 5] += 1.01 * bound[3, 5]
    assert oracle.check_attention(moved, O_ref, TO)[0] == 1
    for special in (np.nan, np.inf, -np.inf):
        bad = O_fused.copy()
        bad[7, 2] = special
        assert oracle.check_attention(bad, O_ref, TO)[0] == 1
    # bf16 output: the stored value is RNE(O), which may sit 2^-9 |O| away
    O_out = torch.from_numpy(O_fused).to(torch.bfloat16).double().numpy()
    assert oracle.check_attention(O_out, O_ref, TO, out_bf16=True)[0] == 0
    extra = 2.0 ** -8 * np.abs(O_ref)
    edge = O_ref + bound + 0.5 * extra
    assert oracle.check_attention(edge, O_ref, TO, out_bf16=True)[0] == 0
    assert oracle.check_attention(edge, O_ref, TO, out_bf16=False)[0] == np.count_nonzero(extra > 0)


# ----------------------------------------------------- tile fan-out bench --

def test_tilecast_accounting_matches_printed_run():
    with open(os.path.join(GOLDEN, "tilecast_accounting.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for consumers, iters, tile_bytes, group, expected in rows:
        consumers, iters, tile_bytes, group = int(consumers), int(iters), int(tile_bytes), int(group)
        # one fetch per group of `group` consumers when the fan-out is ideal
        got = oracle.tilecast_bytes(consumers, iters, tile_bytes) / group
        assert got == float(expected)
    # the printed reduction for a cluster of 2 is 50.00 %
    assert 1.0 - 1.0 / 2 == 0.5


@pytest.mark.parametrize("group", [1, 2, 4, 8, 16, 32])
@pytest.mark.parametrize("grouped", [True, False])
def test_tilecast_group_membership(group, grouped):
    n = 256
    groups = [oracle.tilecast_group(w, n, group, grouped) for w in range(n)]
    assert sorted(set(groups)) == list(range(n // group))
    for g in range(n // group):
        members = [w for w in range(n) if groups[w] == g]
        assert len(members) == group
        if grouped:
            assert len({w % 8 for w in members}) == 1          # one XCD
        else:
            assert members == list(range(members[0], members[0] + group))


def test_tilecast_group_rejects_bad_sizes():
    assert oracle.tilecast_group(0, 256, 3, True) == -1
    assert oracle.tilecast_group(0, 256, 64, True) == -1       # 32 workgroups per XCD
    assert oracle.tilecast_group(256, 256, 2, False) == -1


def test_tilecast_checksum_brute_force():
    rows, cols, tm, tn = 32, 48, 8, 16
    buf = np.arange(rows * cols, dtype=np.uint64) * 2654435761 % 65536
    buf = buf.astype(np.uint16)
    consumers, group, iters, stride = 16, 2, 7, 8
    for grouped in (False, True):
        for w in range(consumers):
            g = oracle.tilecast_group(w, consumers, group, grouped)
            tot, last = 0, 0
            for it in range(iters):
                t = it * stride + g
                c0 = (t % (cols // tn)) * tn
                r0 = ((t // (cols // tn)) % (rows // tm)) * tm
                tile = buf.reshape(rows, cols)[r0:r0 + tm, c0:c0 + tn].astype(np.uint64)
                s = int((tile[:, 0::2] + (tile[:, 1::2] << 16)).sum()) % 2 ** 32
                tot = (tot + s) % 2 ** 32
                last = s
            assert oracle.tilecast_checksum(buf, rows, cols, tm, tn, w, consumers, group, grouped,
                                            iters, stride) == (tot, last)


# --------------------------------------------- planted mistakes are caught --

def test_pins_catch_planted_mistakes():
    """Slips planted on the CPU (wrong strides / lengths / sign fed to the
    oracle) are each caught by one of the pins above."""
    M, N, K = 16, 16, 64
    Ai = draw((M, K), "int", -4, 4, 121)
    Bi = draw((K, N), "int", -4, 4, 122)
    a = Ai.float().numpy().astype(np.int64)
    b = Bi.float().numpy().astype(np.int64)
    exact = (a @ b).astype(np.float64)
    # transposed B operand (row/col strides exchanged)
    C, _ = oracle.gemm(bits(Ai), bits(Bi), 1, M, N, K, (K, 1, 0), (1, N, 0))
    assert not np.array_equal(C[0], exact)
    # dropped last term of the k sum
    C, _ = oracle.gemm(bits(Ai), bits(Bi), 1, M, N, K - 1, (K, 1, 0), (N, 1, 0))
    assert not np.array_equal(C[0], exact)
    # transposed A operand
    C, _ = oracle.gemm(bits(Ai), bits(Bi), 1, M, N, K, (1, M, 0), (N, 1, 0))
    assert not np.array_equal(C[0], exact)
    # sign slip: -A
    Cn, _ = oracle.gemm(bits((-Ai.float()).to(torch.bfloat16)), bits(Bi), 1, M, N, K, (K, 1, 0), (N, 1, 0))
    assert not np.array_equal(Cn[0], exact)


# ------------------------------------------------------ attention forward --

def _attn_ref_library(q, k, v, scale):
    """softmax(scale q k^T) v with scipy's softmax and numpy's matmul."""
    import scipy.special
    return scipy.special.softmax(scale * (q @ k.T), axis=1) @ v


def _attn_inputs(b, Lq, Lk, d, dv, seed, dist="normal"):
    Q = draw((b, Lq, d), dist, -1, 1, seed)
    K = draw((b, Lk, d), dist, -1, 1, seed + 1)
    V = draw((b, Lk, dv), dist, -1, 1, seed + 2)
    return Q, K, V


def _attn(Q, K, V, scale, rows=None):
    b, Lq, d = Q.shape
    Lk, dv = V.shape[1], V.shape[2]
    return oracle.attention(bits(Q), bits(K), bits(V), b, Lq, Lk, d, dv, (d, 1, Lq * d), (d, 1, Lk * d),
                            (dv, 1, Lk * dv), scale, rows=rows)


@pytest.mark.parametrize("b,Lq,Lk,d,dv", [(1, 1, 1, 1, 1), (2, 3, 5, 4, 2), (1, 7, 33, 16, 8), (3, 4, 17, 8, 5)])
def test_attention_matches_library_softmax_on_tiny_shapes(b, Lq, Lk, d, dv):
    Q, K, V = _attn_inputs(b, Lq, Lk, d, dv, 700 + Lk)
    O, TO = _attn(Q, K, V, 0.3)
    for x in range(b):
        ref = _attn_ref_library(Q[x].double().numpy(), K[x].double().numpy(), V[x].double().numpy(), 0.3)
        assert np.allclose(O[x], ref, rtol=0, atol=1e-12 * (1 + np.abs(ref).max()))
    assert np.all(TO >= np.abs(O) - 1e-12)


def test_attention_is_the_mean_of_v_when_keys_are_zero():
    # every score is 0, so the softmax is uniform: O_i = mean_j V_j
    Q, _, V = _attn_inputs(2, 5, 24, 8, 6, 710)
    K = torch.zeros((2, 24, 8), dtype=torch.bfloat16)
    O, _ = _attn(Q, K, V, 0.7)
    mean = V.double().numpy().mean(axis=1)
    for i in range(5):
        assert np.allclose(O[:, i, :], mean, rtol=0, atol=1e-14)


def test_attention_dominant_diagonal_closed_form():
    # Q = K = a*I (n x n): S = a^2 I, so row i weighs key i by e^x (x = scale a^2)
    # and every other key by 1: O_i = (e^x V_i + sum_{j != i} V_j) / (e^x + n - 1)
    n, a, scale = 12, 2.0, 0.8
    QK = torch.zeros((1, n, n), dtype=torch.bfloat16)
    for i in range(n):
        QK[0, i, i] = a
    V = draw((1, n, 5), "normal", 0, 1, 720)
    O, _ = _attn(QK, QK, V, scale)
    v = V[0].double().numpy()
    ex = np.exp(scale * a * a)
    for i in range(n):
        want = (ex * v[i] + (v.sum(axis=0) - v[i])) / (ex + n - 1)
        assert np.allclose(O[0, i], want, rtol=1e-14, atol=1e-14)


def test_attention_exact_powers_of_two():
    # integer scores and scale = ln 2: every weight is a power of two, so the
    # result is a ratio of integers known exactly (Fractions)
    from fractions import Fraction
    Q = draw((1, 3, 6), "int", -1, 1, 730)
    K = draw((1, 9, 6), "int", -1, 1, 731)
    V = draw((1, 9, 4), "int", -4, 4, 732)
    O, _ = _attn(Q, K, V, math.log(2.0))
    q, k, v = (t[0].float().numpy().astype(np.int64) for t in (Q, K, V))
    s = q @ k.T
    for i in range(3):
        m = s[i].max()
        w = [Fraction(2) ** int(s[i, j] - m) for j in range(9)]
        for c in range(4):
            want = sum(w[j] * int(v[j, c]) for j in range(9)) / sum(w)
            assert abs(O[0, i, c] - float(want)) <= 1e-14 * (1 + abs(float(want)))


def test_attention_shift_and_key_permutation_invariance():
    Q, K, V = _attn_inputs(1, 6, 20, 8, 4, 740)
    O, _ = _attn(Q, K, V, 0.5)
    # a constant added to every score of a row (an extra dimension: q -> [q, 1], k -> [k, c])
    Qx = torch.cat([Q, torch.ones((1, 6, 1), dtype=torch.bfloat16)], dim=2)
    Kx = torch.cat([K, torch.full((1, 20, 1), 3.0, dtype=torch.bfloat16)], dim=2)
    Ox, _ = _attn(Qx, Kx, V, 0.5)
    assert np.allclose(Ox, O, rtol=0, atol=1e-13)
    # keys reordered together with their values
    perm = torch.randperm(20, generator=torch.Generator().manual_seed(741))
    Op, _ = _attn(Q, K[:, perm], V[:, perm], 0.5)
    assert np.allclose(Op, O, rtol=0, atol=1e-13)


def test_attention_rows_are_convex_combinations_of_v():
    Q, K, V = _attn_inputs(2, 8, 30, 16, 6, 750)
    O, TO = _attn(Q, K, V, 0.9)
    v = V.double().numpy()
    assert np.all(O >= v.min(axis=1)[:, None, :] - 1e-13)
    assert np.all(O <= v.max(axis=1)[:, None, :] + 1e-13)
    ones = torch.ones_like(V)
    O1, _ = _attn(Q, K, ones, 0.9)
    assert np.allclose(O1, 1.0, rtol=0, atol=1e-14)


def test_attention_strides_broadcast_and_row_subset():
    b, Lq, Lk, d, dv = 2, 5, 11, 8, 3
    Q, K, V = _attn_inputs(b, Lq, Lk, d, dv, 760)
    O, TO = _attn(Q, K, V, 0.4)
    # K and V stored transposed ([b, d, Lk] / [b, dv, Lk]) give identical bits
    Kt = K.transpose(1, 2).contiguous()
    Vt = V.transpose(1, 2).contiguous()
    O2, TO2 = oracle.attention(bits(Q), bits(Kt), bits(Vt), b, Lq, Lk, d, dv, (d, 1, Lq * d),
                               (1, Lk, Lk * d), (1, Lk, Lk * dv), 0.4)
    assert np.array_equal(O2, O) and np.array_equal(TO2, TO)
    # batch stride 0 broadcasts K and V
    Ob, _ = oracle.attention(bits(Q), bits(K[:1]), bits(V[:1]), b, Lq, Lk, d, dv, (d, 1, Lq * d),
                             (d, 1, 0), (dv, 1, 0), 0.4)
    O0, _ = _attn(Q, K[:1].expand(b, -1, -1).contiguous(), V[:1].expand(b, -1, -1).contiguous(), 0.4)
    assert np.array_equal(Ob, O0)
    # selected rows equal the full result's rows
    rows = np.array([[1, 4], [0, 0], [1, 2]])
    Or, TOr = _attn(Q, K, V, 0.4, rows=rows)
    for n, (x, i) in enumerate(rows):
        assert np.array_equal(Or[n], O[x, i]) and np.array_equal(TOr[n], TO[x, i])


def test_attention_pins_catch_planted_mistakes():
    """Slips planted on the CPU (wrong scale, transposed V, a dropped key,
    the softmax taken over queries) are each caught by the library pin."""
    Lq = Lk = 9
    d = dv = 9
    Q, K, V = _attn_inputs(1, Lq, Lk, d, dv, 770)
    q, k, v = Q[0].double().numpy(), K[0].double().numpy(), V[0].double().numpy()
    ref = _attn_ref_library(q, k, v, 0.6)
    ok = lambda O: np.allclose(O[0], ref, rtol=0, atol=1e-12)
    assert ok(_attn(Q, K, V, 0.6)[0])
    assert not ok(_attn(Q, K, V, 1.0)[0])                                   # scale dropped
    Ovt, _ = oracle.attention(bits(Q), bits(K), bits(V), 1, Lq, Lk, d, dv, (d, 1, 0), (d, 1, 0), (1, dv, 0), 0.6)
    assert not ok(Ovt)                                                      # V transposed
    Od, _ = oracle.attention(bits(Q), bits(K), bits(V), 1, Lq, Lk - 1, d, dv, (d, 1, 0), (d, 1, 0), (dv, 1, 0), 0.6)
    assert not np.allclose(Od[0], ref, rtol=0, atol=1e-12)                  # last key dropped
    Oq, _ = _attn(K, Q, V, 0.6)
    assert not ok(Oq)                                                       # softmax over queries


def _attn_c(Q, K, V, scale, rows=None):
    b, Lq, d = Q.shape
    Lk, dv = V.shape[1], V.shape[2]
    return oracle.attention(bits(Q), bits(K), bits(V), b, Lq, Lk, d, dv, (d, 1, Lq * d), (d, 1, Lk * d),
                            (dv, 1, Lk * dv), scale, rows=rows, causal=True)


def _attn_ref_causal(q, k, v, scale):
    """Masked softmax with scipy: query i sees keys j <= i + (Lk - Lq)."""
    import scipy.special
    Lq, Lk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    mask = np.arange(Lk)[None, :] > (np.arange(Lq)[:, None] + (Lk - Lq))
    s[mask] = -np.inf
    return scipy.special.softmax(s, axis=1) @ v


@pytest.mark.parametrize("b,Lq,Lk,d,dv", [(1, 1, 1, 4, 2), (2, 5, 5, 4, 3), (1, 7, 33, 16, 8), (3, 9, 9, 8, 5)])
def test_causal_attention_matches_masked_library_softmax(b, Lq, Lk, d, dv):
    Q, K, V = _attn_inputs(b, Lq, Lk, d, dv, 780 + Lk)
    O, TO = _attn_c(Q, K, V, 0.4)
    for x in range(b):
        ref = _attn_ref_causal(Q[x].double().numpy(), K[x].double().numpy(), V[x].double().numpy(), 0.4)
        assert np.allclose(O[x], ref, rtol=0, atol=1e-12 * (1 + np.abs(ref).max()))


def test_causal_attention_first_and_last_rows():
    # Lq == Lk: query 0 sees key 0 only (O_0 = V_0 exactly); the last query
    # sees every key (equal to the unmasked row)
    Q, K, V = _attn_inputs(2, 12, 12, 8, 6, 790)
    O, _ = _attn_c(Q, K, V, 0.7)
    Of, _ = _attn(Q, K, V, 0.7)
    assert np.array_equal(O[:, 0, :], V[:, 0, :].double().numpy())
    assert np.allclose(O[:, -1, :], Of[:, -1, :], rtol=0, atol=1e-14)
    # Lk > Lq: the mask aligns to the last key, so query i sees i + Lk - Lq + 1 keys
    Q2, K2, V2 = _attn_inputs(1, 4, 10, 8, 3, 791)
    O2, _ = _attn_c(Q2, K2, V2, 0.5)
    for i in range(4):
        n = i + 10 - 4 + 1
        Oi, _ = _attn(Q2[:, i:i + 1], K2[:, :n], V2[:, :n], 0.5)
        assert np.allclose(O2[0, i], Oi[0, 0], rtol=0, atol=1e-14)


def test_causal_attention_ignores_masked_keys_and_catches_off_by_one():
    # changing keys/values that the mask hides changes nothing; a mask one key
    # too wide or too narrow (emulated by shifting Lk against Lq) does
    Q, K, V = _attn_inputs(1, 8, 8, 8, 4, 800)
    O, _ = _attn_c(Q, K, V, 0.6)
    K2, V2 = K.clone(), V.clone()
    K2[:, 5:], V2[:, 5:] = 3.0, -2.0
    O2, _ = _attn_c(Q, K2, V2, 0.6)
    assert np.array_equal(O[:, :5], O2[:, :5])
    assert not np.allclose(O[:, 5:], O2[:, 5:])
    q, k, v = Q[0].double().numpy(), K[0].double().numpy(), V[0].double().numpy()
    ref = _attn_ref_causal(q, k, v, 0.6)
    assert np.allclose(O[0], ref, rtol=0, atol=1e-12)
    # one key too many: the first 7 queries against the same 8 keys see
    # j <= i + 1 under the bottom-right alignment
    Ow, _ = _attn_c(Q[:, :7], K, V, 0.6)
    assert not np.allclose(Ow[0], ref[:7], rtol=0, atol=1e-12)
    # one key too few: all 8 queries against the first 7 keys are refused (Lk < Lq)
    with pytest.raises(RuntimeError):
        _attn_c(Q, K[:, :7], V[:, :7], 0.6)


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_key_value_heads_equal_materialised_repeats(causal):
    # kv_group g: query slice b reads K/V slice b // g.  The same result comes
    # from the ungrouped oracle fed K and V with each slice repeated g times
    # (an independent layout: every slice then has its own copy), bit for bit.
    b, g, Lq, Lk, d, dv = 6, 3, 7, 9, 8, 5
    Q, _, _ = _attn_inputs(b, Lq, Lk, d, dv, 810)
    _, K, V = _attn_inputs(b // g, Lq, Lk, d, dv, 811)
    Kr = K.repeat_interleave(g, dim=0).contiguous()
    Vr = V.repeat_interleave(g, dim=0).contiguous()
    O, TO = oracle.attention(bits(Q), bits(K), bits(V), b, Lq, Lk, d, dv, (d, 1, Lq * d), (d, 1, Lk * d),
                             (dv, 1, Lk * dv), 0.3, causal=causal, kv_group=g)
    Or, TOr = oracle.attention(bits(Q), bits(Kr), bits(Vr), b, Lq, Lk, d, dv, (d, 1, Lq * d), (d, 1, Lk * d),
                               (dv, 1, Lk * dv), 0.3, causal=causal)
    assert np.array_equal(O, Or) and np.array_equal(TO, TOr)
    # a grouping that sends the last group to the first K/V slice is caught
    Kw = torch.cat([Kr[:-g], Kr[:g]]).contiguous()
    Ow, _ = oracle.attention(bits(Q), bits(Kw), bits(Vr), b, Lq, Lk, d, dv, (d, 1, Lq * d), (d, 1, Lk * d),
                             (dv, 1, Lk * dv), 0.3, causal=causal)
    assert not np.allclose(O, Ow)
    with pytest.raises(ValueError):
        oracle.attention(bits(Q), bits(K), bits(V), b, Lq, Lk, d, dv, (d, 1, Lq * d), (d, 1, Lk * d),
                         (dv, 1, Lk * dv), 0.3, kv_group=4)
