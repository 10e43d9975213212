"""Parity of every HIP tile op with the fp64 oracle (GPU).

Inputs are seeded (synth.rand_*); sizes span several kernel tiles and a
ragged tail; every call goes through the C ABI. Float tolerances follow the
fp32 arithmetic: a length-k dot product in fp32 is within ~k*2^-24 of the
fp64 value relative to the sum of |terms| (worst case), the memory-bound
ops within a few units of 2^-24 of their inputs' scale.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth  # noqa: E402
import tile_task_transformer_amd as tt  # noqa: E402
from oracle import gpt2 as og  # noqa: E402
from oracle import tiled as otl  # noqa: E402
from tests.gpu_util import EPS32, assert_close_bound, assert_rel, dev, empty, host  # noqa: E402

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ GEMM

def _op(a, t):
    return a.T if t else a


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("m,n,k", [(257, 130, 70), (128, 128, 16), (300, 513, 337), (1, 1, 1), (64, 200, 1),
                                   (1100, 700, 256), (4000, 2304, 37),
                                   # >= 512 blocks of 128x128 whose last round is poorly filled -> 64x64
                                   # (short and long K), and full rounds that keep 128x128
                                   (4096, 2304, 768), (4100, 2304, 1030), (4096, 2048, 768)])
def test_gemm_parity(ta, tb, m, n, k):
    seed = m * 7 + n * 3 + k + 10 * ta + 20 * tb
    a = synth.rand_normal((k, m) if ta else (m, k), seed)
    b = synth.rand_normal((n, k) if tb else (k, n), seed + 1)
    c0 = synth.rand_normal((m, n), seed + 2)
    ref = 0.75 * _op(a.astype(np.float64), ta) @ _op(b.astype(np.float64), tb) + 0.5 * c0
    C = dev(c0)
    tt.tile_gemm(None, ta, tb, m, n, k, 0.75, dev(a), a.shape[1], dev(b), b.shape[1], 0.5, C, n)
    bound = 0.75 * (np.abs(_op(a, ta)).astype(np.float64) @ np.abs(_op(b, tb)).astype(np.float64)) * (k + 2) * EPS32
    assert_close_bound(host(C), ref, bound + 4 * EPS32 * np.abs(ref) + 1e-30, f"gemm {ta}{tb} {m}x{n}x{k}")


@pytest.mark.parametrize("ta,tb,m,n,k", [(1, 0, 768, 768, 4096), (1, 0, 700, 300, 5000), (0, 1, 1536, 768, 4096),
                                         (0, 0, 1000, 200, 2049), (1, 1, 3072, 768, 4096),
                                         (1, 0, 512, 512, 1024), (0, 1, 1024, 512, 1024), (0, 0, 1000, 300, 1100),
                                         (0, 1, 1024, 512, 512)])
def test_gemm_split_k_workspace(ta, tb, m, n, k):
    """Tall-K shapes take the split-K path when given a workspace: same result
    within the fp32 bound, bitwise equal across runs, epilogue applied once."""
    seed = m + n + k
    a = synth.rand_normal((k, m) if ta else (m, k), seed)
    b = synth.rand_normal((n, k) if tb else (k, n), seed + 1)
    c0 = synth.rand_normal((m, n), seed + 2)
    bias = synth.rand_normal((n,), seed + 3)
    need = tt.tile_gemm_workspace(m, n, k)
    assert need > 0, "shape expected to split"
    ws = torch.empty(need // 4, device="cuda")
    outs = []
    for _ in range(2):
        C = dev(c0)
        tt.tile_gemm_ws(None, ta, tb, m, n, k, 1.0, dev(a), a.shape[1], dev(b), b.shape[1], 1.0, C, n,
                        tt.TT_EPI_BIAS, dev(bias), None, 0, None, 0, ws, need)
        outs.append(C)
    ref = _op(a.astype(np.float64), ta) @ _op(b.astype(np.float64), tb) + c0 + bias
    bound = (np.abs(_op(a, ta)).astype(np.float64) @ np.abs(_op(b, tb)).astype(np.float64)) * (k + 2) * EPS32
    assert_close_bound(host(outs[0]), ref, bound + 4 * EPS32 * np.abs(ref), "split-K gemm")
    assert torch.equal(outs[0], outs[1])


def _ksum_ws(m, n, use):
    """a NaN-filled workspace of the size that allows the widest K split (a
    slice the kernels failed to write would show), or none"""
    if not use:
        return None, 0
    wsb = tt.tile_gemm_ksum_workspace(m, n)
    return torch.full((max(wsb, 4) // 4,), float("nan"), device="cuda"), wsb


@pytest.mark.parametrize("ws", [False, True])
@pytest.mark.parametrize("tb", [0, 1])
@pytest.mark.parametrize("m,n,ks,beta", [
    (4096, 768, [768] * 5 + [337], 0.0),          # the LM head's dnf: full vocab tiles + the ragged last one
    (256, 192, [64, 96, 32, 0, 128], 0.5),        # a skipped empty pair, C kept with beta
    (128, 128, [32] * 100, 1.0),                  # more pairs than one launch takes
    (2048, 4096, [48, 64], 0.0),                  # the 128x128 plan (>= 512 blocks)
    (100, 72, [40, 33], 0.25),                    # m, n off the block grid: every pair falls back
    (4096, 768, [768] * 3, 0.0),                  # the q/k/v input gradient (B transposed)
    (1024, 512, [1024] * 6, 0.5),                 # a narrow output: 32 blocks, K split into 12 slices
    (512, 384, [512, 160, 512, 96], 1.0),         # slices that start and end inside pairs of unequal K
])
def test_gemm_ksum(m, n, ks, beta, tb, ws):
    """C = alpha sum_t A_t op(B_t) + beta C against the fp64 sum (fp32 bound
    over the total K), bitwise equal across runs; B as [k][n] or [n][k];
    without and with a workspace (split K for outputs of few blocks)."""
    seed = m + n + len(ks) + 5 * tb
    As = [synth.rand_normal((m, k), seed + 2 * i) for i, k in enumerate(ks)]
    Bs = [synth.rand_normal((n, k) if tb else (k, n), seed + 2 * i + 1) for i, k in enumerate(ks)]
    c0 = synth.rand_normal((m, n), seed + 999)
    dA, dB = [dev(a) for a in As], [dev(b) for b in Bs]
    W, wsb = _ksum_ws(m, n, ws)
    outs = []
    for _ in range(2):
        C = dev(c0)
        tt.tile_gemm_ksum_ex(None, m, n, ks, 0.75, dA, ks, dB, [b.shape[1] for b in Bs], beta, C, n, transB=tb,
                             workspace=W, workspace_bytes=wsb)
        outs.append(C)
    ref = beta * c0.astype(np.float64)
    bound = np.zeros((m, n))
    for a, b in zip(As, Bs):
        b = b.T if tb else b
        ref = ref + 0.75 * (a.astype(np.float64) @ b.astype(np.float64))
        bound += 0.75 * (np.abs(a).astype(np.float64) @ np.abs(b).astype(np.float64))
    bound *= (sum(ks) + len(ks) + 2) * EPS32
    assert_close_bound(host(outs[0]), ref, bound + 4 * EPS32 * np.abs(ref) + 1e-30, f"ksum {m}x{n} {len(ks)} pairs")
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("m,n,k,count,tb,epi,ws", [
    (4096, 2048, 512, 4, 0, "bias_res", False),   # 512 blocks of 128x128 (BK 16): the attention projection's shape
    (1024, 1024, 256, 3, 0, "gelu", False),       # 64 blocks of 64x64: the MLP input layer with its activation
    (4096, 4096, 256, 2, 1, "gelu_bwd", False),   # 1024 blocks (BK 32), B stored [n][k]: the MLP output's dX
    (1024, 512, 1024, 3, 0, "bias_res", True),    # split K (6 slices), then bias + residual on the slice sum
    (1024, 1024, 512, 4, 0, "gelu", True),        # split K (4 slices), GELU on the slice sum
    (1024, 512, 512, 4, 1, "gelu_bwd", True),     # split K (4 slices), B stored [n][k], GELU'
])
def test_gemm_ksum_epilogues(m, n, k, count, tb, epi, ws):
    """K-sum with tile_gemm's epilogues on the whole sum: bias + residual,
    GELU (pre-activation kept in aux) and GELU' against the fp64 sum, also
    with K split into slices over a workspace."""
    seed = m + n + count
    As = [synth.rand_normal((m, k), seed + i, std=0.2) for i in range(count)]
    Bs = [synth.rand_normal((n, k) if tb else (k, n), seed + 50 + i, std=0.2) for i in range(count)]
    bias, res = synth.rand_normal((n,), seed + 100), synth.rand_normal((m, n), seed + 101)
    aux0 = synth.rand_normal((m, n), seed + 102)
    ref = np.zeros((m, n))
    bound = np.zeros((m, n))
    for a, b in zip(As, Bs):
        b = (b.T if tb else b).astype(np.float64)
        ref += a.astype(np.float64) @ b
        bound += np.abs(a).astype(np.float64) @ np.abs(b)
    bound *= (count * k + count + 4) * EPS32
    C, aux = empty((m, n)), dev(aux0)
    flag = {"bias_res": tt.TT_EPI_BIAS | tt.TT_EPI_RES, "gelu": tt.TT_EPI_GELU | tt.TT_EPI_BIAS,
            "gelu_bwd": tt.TT_EPI_GELU_BWD}[epi]
    W, wsb = _ksum_ws(m, n, ws)
    tt.tile_gemm_ksum_ex(None, m, n, [k] * count, 1.0, [dev(a) for a in As], [k] * count, [dev(b) for b in Bs],
                         [b.shape[1] for b in Bs], 0.0, C, n, transB=tb, epilogue=flag, bias=dev(bias), res=dev(res),
                         ldr=n, aux=aux, ldaux=n, workspace=W, workspace_bytes=wsb)
    if epi == "bias_res":
        want = ref + bias + res
        assert_close_bound(host(C), want, bound + 4 * EPS32 * np.abs(want) + 1e-6, "ksum bias+res")
    elif epi == "gelu":
        pre = ref + bias
        assert_close_bound(host(aux), pre, bound + 4 * EPS32 * np.abs(pre) + 1e-6, "ksum gelu pre-activation")
        assert_close_bound(host(C), og.gelu(pre), 1.2 * bound + 4e-6, "ksum gelu")
    else:
        want = ref * og.gelu_grad(aux0.astype(np.float64))
        assert_close_bound(host(C), want, 1.2 * bound + 4e-6 * np.abs(ref) + 1e-6, "ksum gelu'")


def test_gemm_ksum_epilogue_needs_one_launch():
    a = empty((96, 64))
    with pytest.raises(tt.TTError) as e:   # 96 rows: edge blocks, the long-K launch cannot take the pair
        tt.tile_gemm_ksum_ex(None, 96, 64, [64, 64], 1.0, [a, a], [64, 64], [a, a], [64, 64], 0.0, a, 64,
                             epilogue=tt.TT_EPI_BIAS, bias=a)
    assert e.value.code == tt._lib.TT_ERR_UNSUPPORTED


def test_gemm_ksum_empty_and_errors():
    c0 = synth.rand_normal((64, 64), 5)
    C = dev(c0)
    tt.tile_gemm_ksum(None, 64, 64, [], 1.0, [], [], [], [], 0.5, C, 64)
    assert np.array_equal(host(C), (0.5 * c0.astype(np.float32)).astype(np.float64))
    with pytest.raises(tt.TTError):
        tt.tile_gemm_ksum(None, 64, 64, [32], 1.0, [None], [32], [C], [64], 0.0, C, 64)


@pytest.mark.parametrize("ta,tb,m,n,k,count,beta,ld_pad", [
    (1, 0, 768, 768, 256, 15, 1.0, 0),     # the head's dwte_v = dz_v^T nf shape, 128x128 blocks (>= 512 in all)
    (0, 1, 512, 768, 768, 4, 0.0, 0),      # the head's z_v = nf wte_v^T shape, 64x64 blocks
    (0, 0, 300, 130, 70, 3, 0.5, 0),       # ragged m, n, k: edge blocks
    (1, 1, 200, 96, 40, 2, 0.25, 0),
    (0, 1, 96, 72, 40, 3, 1.0, 1),         # leading dimensions not multiples of 4: scalar loads
    (0, 0, 64, 64, 32, 100, 0.0, 0),       # more products than one launch takes
    (1, 0, 128, 64, 0, 2, 0.5, 0),         # k = 0: C = beta C
])
def test_gemm_batch(ta, tb, m, n, k, count, beta, ld_pad):
    """C_t = alpha op(A_t) op(B_t) + beta C_t for every product against the
    fp64 products (fp32 bound), bitwise equal across runs."""
    seed = m + 3 * n + 5 * k + count
    As = [synth.rand_normal(((k, m + ld_pad) if ta else (m, k + ld_pad)), seed + 3 * i) for i in range(count)]
    Bs = [synth.rand_normal(((n, k + ld_pad) if tb else (k, n + ld_pad)), seed + 3 * i + 1) for i in range(count)]
    Cs0 = [synth.rand_normal((m, n), seed + 3 * i + 2) for i in range(count)]
    dA, dB = [dev(a) for a in As], [dev(b) for b in Bs]
    lda, ldb = As[0].shape[1], Bs[0].shape[1]
    outs = []
    for _ in range(2):
        Cs = [dev(c) for c in Cs0]
        tt.tile_gemm_batch(None, ta, tb, m, n, k, 0.75, dA, lda, dB, ldb, beta, Cs, n)
        outs.append(Cs)
    for t in range(count):
        a = As[t][:, :m] if ta else As[t][:, :k]
        b = Bs[t][:, :k] if tb else Bs[t][:, :n]
        ref = 0.75 * (_op(a.astype(np.float64), ta) @ _op(b.astype(np.float64), tb)) + beta * Cs0[t]
        bound = 0.75 * (np.abs(_op(a, ta)).astype(np.float64) @ np.abs(_op(b, tb)).astype(np.float64)) * (k + 2) * EPS32
        assert_close_bound(host(outs[0][t]), ref, bound + 4 * EPS32 * np.abs(ref) + 1e-30,
                           f"batch {ta}{tb} {m}x{n}x{k} product {t} of {count}")
        assert torch.equal(outs[0][t], outs[1][t])


@pytest.mark.parametrize("ta,tb,ms,ns,k", [
    (1, 0, [768] * 6 + [337], [768] * 7, 256),    # dwte_v = dz_v^T nf: ragged last vocab tile (lda 337: scalar loads)
    (0, 1, [512] * 4, [768] * 3 + [337], 768),    # z_v = nf wte_v^T: ragged last tile (ldc 337)
    (0, 0, [100, 0, 64, 300], [72, 50, 0, 130], 70),  # empty products are skipped
    (1, 1, [64] * 80, [32] * 80, 48),             # more products than one launch takes
])
def test_gemm_batch_ragged_products(ta, tb, ms, ns, k):
    """Products of different sizes and leading dimensions in one call against
    the fp64 products; a vector-load product and a scalar one side by side."""
    cnt = len(ms)
    seed = 7 * cnt + k
    As = [synth.rand_normal(((k, m) if ta else (m, k)), seed + 3 * i) for i, m in enumerate(ms)]
    Bs = [synth.rand_normal(((n, k) if tb else (k, n)), seed + 3 * i + 1) for i, n in enumerate(ns)]
    Cs0 = [synth.rand_normal((m, n), seed + 3 * i + 2) for i, (m, n) in enumerate(zip(ms, ns))]
    Cs = [dev(c) for c in Cs0]
    tt.tile_gemm_batch(None, ta, tb, ms, ns, k, 1.25, [dev(a) for a in As], [a.shape[1] for a in As],
                       [dev(b) for b in Bs], [b.shape[1] for b in Bs], 0.5, Cs, list(ns))
    for t in range(cnt):
        a, b = As[t], Bs[t]
        ref = 1.25 * (_op(a.astype(np.float64), ta) @ _op(b.astype(np.float64), tb)) + 0.5 * Cs0[t]
        bound = 1.25 * (np.abs(_op(a, ta)).astype(np.float64) @ np.abs(_op(b, tb)).astype(np.float64)) * (k + 2) * EPS32
        assert_close_bound(host(Cs[t]), ref, bound + 4 * EPS32 * np.abs(ref) + 1e-30, f"batch product {t}")


@pytest.mark.parametrize("ta,tb,ms,ns,k,beta", [
    (1, 0, [768] * 3, [768] * 3, 4096, 1.0),        # the q, k, v weight gradients of one layer
    (1, 0, [700, 100], [300, 72], 5000, 0.0),       # ragged products, K not a multiple of the slice
    (0, 1, [256, 128, 384], [128, 256, 96], 2304, 0.5),
])
def test_gemm_batch_split_k(ta, tb, ms, ns, k, beta):
    """Batched split-K (few blocks, long K, with a workspace) against the
    fp64 products; bitwise equal across runs; a workspace too small to split
    gives a result within the same bound."""
    cnt = len(ms)
    need = tt.tile_gemm_batch_workspace(ms, ns, k)
    assert need > 0
    seed = 11 * cnt + k
    As = [synth.rand_normal(((k, m) if ta else (m, k)), seed + 3 * i) for i, m in enumerate(ms)]
    Bs = [synth.rand_normal(((n, k) if tb else (k, n)), seed + 3 * i + 1) for i, n in enumerate(ns)]
    Cs0 = [synth.rand_normal((m, n), seed + 3 * i + 2) for i, (m, n) in enumerate(zip(ms, ns))]
    dA, dB = [dev(a) for a in As], [dev(b) for b in Bs]
    outs = []
    for wsb in (need, need, 1024):
        ws = torch.empty(max(wsb // 4, 1), device="cuda")
        Cs = [dev(c) for c in Cs0]
        tt.tile_gemm_batch_ws(None, ta, tb, ms, ns, k, 0.75, dA, [a.shape[1] for a in As], dB, [b.shape[1] for b in Bs],
                              beta, Cs, list(ns), ws, wsb)
        outs.append(Cs)
    for t in range(cnt):
        a, b = As[t], Bs[t]
        ref = 0.75 * (_op(a.astype(np.float64), ta) @ _op(b.astype(np.float64), tb)) + beta * Cs0[t]
        bound = 0.75 * (np.abs(_op(a, ta)).astype(np.float64) @ np.abs(_op(b, tb)).astype(np.float64)) * (k + 2) * EPS32
        for run in (0, 2):
            assert_close_bound(host(outs[run][t]), ref, bound + 4 * EPS32 * np.abs(ref) + 1e-30,
                               f"split batch product {t} run {run}")
        assert torch.equal(outs[0][t], outs[1][t])


def test_gemm_batch_empty_and_errors():
    c0 = synth.rand_normal((64, 64), 6)
    C = dev(c0)
    tt.tile_gemm_batch(None, 0, 0, 64, 64, 32, 1.0, [], 32, [], 64, 0.5, [], 64)
    assert np.array_equal(host(C), c0.astype(np.float32).astype(np.float64))
    with pytest.raises(tt.TTError):
        tt.tile_gemm_batch(None, 0, 0, 64, 64, 32, 1.0, [None], 32, [C], 64, 0.0, [C], 64)
    with pytest.raises(tt.TTError):
        tt.tile_gemm_batch(None, 0, 0, 64, 64, 32, 1.0, [C], 16, [C], 64, 0.0, [C], 64)


def test_gemm_gelu_epilogue_over_the_whole_range():
    """GELU and GELU' epilogues on pre-activations from -20 to 20 (tanh
    saturated at both ends), around 0 and at tiny values, against the fp64
    oracle: the products are exact (k = 1, B = 1), so only the epilogue's
    arithmetic is measured."""
    u = np.concatenate([np.linspace(-20, 20, 4001), np.linspace(-1e-3, 1e-3, 201), [0.0, 1e-30, -1e-30, 3e-8]])
    u = u.astype(np.float32)
    m = u.size
    A, B = dev(u.reshape(m, 1)), dev(np.ones((1, 1), np.float32))
    C, aux = empty((m, 1)), empty((m, 1))
    tt.tile_gemm(None, 0, 0, m, 1, 1, 1.0, A, 1, B, 1, 0.0, C, 1, tt.TT_EPI_GELU, None, None, 0, aux, 1)
    u64 = u.astype(np.float64)
    assert np.array_equal(host(aux)[:, 0], u64)
    assert_rel(host(C)[:, 0], og.gelu(u64), 2e-6, 2e-6, "gelu over the range")
    G = dev(u.reshape(m, 1))
    tt.tile_gemm(None, 0, 0, m, 1, 1, 1.0, dev(np.ones((m, 1), np.float32)), 1, B, 1, 0.0, C, 1, tt.TT_EPI_GELU_BWD,
                 None, None, 0, G, 1)
    assert_rel(host(C)[:, 0], og.gelu_grad(u64), 2e-6, 2e-6, "gelu' over the range")


@pytest.mark.parametrize("ld_pad", [0, 1, 4])
def test_gemm_leading_dims_and_views(ld_pad):
    m, n, k = 96, 72, 40
    a = synth.rand_normal((m, k + ld_pad), 1)
    b = synth.rand_normal((k, n + ld_pad), 2)
    C = empty((m, n + ld_pad))
    tt.tile_gemm(None, 0, 0, m, n, k, 1.0, dev(a), k + ld_pad, dev(b), n + ld_pad, 0.0, C, n + ld_pad)
    ref = a[:, :k].astype(np.float64) @ b[:, :n].astype(np.float64)
    got = host(C)
    assert_rel(got[:, :n], ref, 1e-5, 1e-5, "gemm ld")
    if ld_pad:
        assert np.isnan(got[:, n:]).all(), "wrote outside the m x n block"


def test_gemm_epilogues():
    m, n, k = 200, 150, 64
    x = synth.rand_normal((m, k), 3)
    w = synth.rand_normal((k, n), 4, std=0.2)
    bias = synth.rand_normal((n,), 5)
    res = synth.rand_normal((m, n), 6)
    acc0 = synth.rand_normal((m, n), 7)
    base = x.astype(np.float64) @ w.astype(np.float64)
    # BIAS | RES, beta 0
    C = empty((m, n))
    tt.tile_gemm(None, 0, 0, m, n, k, 1.0, dev(x), k, dev(w), n, 0.0, C, n, tt.TT_EPI_BIAS | tt.TT_EPI_RES,
                 dev(bias), dev(res), n)
    assert_rel(host(C), base + bias + res, 2e-5, 2e-5, "bias+res")
    # GELU with beta 1: pre = AB + aux + bias; aux <- pre; C <- gelu(pre)
    aux = dev(acc0)
    C = empty((m, n))
    tt.tile_gemm(None, 0, 0, m, n, k, 1.0, dev(x), k, dev(w), n, 1.0, C, n, tt.TT_EPI_GELU | tt.TT_EPI_BIAS,
                 dev(bias), None, 0, aux, n)
    pre = base + acc0 + bias
    assert_rel(host(aux), pre, 2e-5, 2e-5, "gelu pre-activation")
    assert_rel(host(C), og.gelu(pre), 2e-5, 2e-5, "gelu")
    # GELU_BWD: C <- (AB + beta C) * gelu'(aux)
    u = synth.rand_normal((m, n), 8, std=2.0)
    C = dev(acc0)
    tt.tile_gemm(None, 0, 0, m, n, k, 1.0, dev(x), k, dev(w), n, 1.0, C, n, tt.TT_EPI_GELU_BWD, None, None, 0,
                 dev(u), n)
    assert_rel(host(C), (base + acc0) * og.gelu_grad(u.astype(np.float64)), 2e-5, 2e-5, "gelu_bwd")


# ------------------------------------------------------------- LayerNorm

@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 768), (300, 2048), (64, 33), (130, 512)])
def test_layernorm_fwd_fused(rows, cols):
    x = synth.rand_normal((rows, cols), rows + cols, std=3.0) + 1.5
    g = synth.rand_normal((cols,), 1) + 1
    b = synth.rand_normal((cols,), 2)
    y, stats = empty((rows, cols)), empty((rows, 2))
    tt.tile_layernorm_fwd(None, tt.TT_LN_FUSED, rows, cols, dev(x), cols, dev(g), dev(b), None, 0, 0, stats, y,
                          cols, 1e-5)
    ry, (mu, rs) = og.layernorm_fwd(x.astype(np.float64), g.astype(np.float64), b.astype(np.float64))
    assert_rel(host(y), ry, 1e-5, 1e-5, "ln y")
    assert_rel(host(stats)[:, 0], mu, 1e-5, 1e-6, "ln mean")
    assert_rel(host(stats)[:, 1], rs, 1e-5, 0, "ln rstd")


@pytest.mark.parametrize("rows,cols,et", [(40, 64, 32), (129, 2000, 512), (16, 100, 24)])
def test_layernorm_three_phase_and_bwd(rows, cols, et):
    x = synth.rand_normal((rows, cols), 11, std=2.0) - 0.7
    g = synth.rand_normal((cols,), 12) + 1
    b = synth.rand_normal((cols,), 13)
    dy = synth.rand_normal((rows, cols), 14)
    X, G, Bb, DY = dev(x), dev(g), dev(b), dev(dy)
    tiles = otl.tiles(cols, et)
    ne = len(tiles)
    parts = empty((ne, rows, 3))
    stats = empty((rows, 2))
    y = empty((rows, cols))
    for i, (c0, c1) in enumerate(tiles):
        xt = X[:, c0:c1].contiguous()
        tt.tile_layernorm_fwd(None, tt.TT_LN_PARTIAL, rows, c1 - c0, xt, c1 - c0, None, None, parts[i], 0, 0, None,
                              None, 0, 1e-5)
    tt.tile_layernorm_fwd(None, tt.TT_LN_MERGE, rows, 0, None, 0, None, None, parts, ne, rows * 3, stats, None, 0,
                          1e-5)
    for c0, c1 in tiles:
        yt = empty((rows, c1 - c0))
        tt.tile_layernorm_fwd(None, tt.TT_LN_APPLY, rows, c1 - c0, X[:, c0:c1].contiguous(), c1 - c0,
                              G[c0:c1].contiguous(), Bb[c0:c1].contiguous(), None, 0, 0, stats, yt, c1 - c0, 1e-5)
        y[:, c0:c1] = yt
    x64, g64 = x.astype(np.float64), g.astype(np.float64)
    ry, (mu, rs) = og.layernorm_fwd(x64, g64, b.astype(np.float64))
    assert_rel(host(y), ry, 2e-5, 2e-5, "ln 3-phase y")
    # backward: PARTIAL per tile, APPLY per tile (dx accumulates onto an existing gradient)
    rdx, rdg, rdb = og.layernorm_bwd(dy.astype(np.float64), x64, g64, mu, rs)
    dx0 = synth.rand_normal((rows, cols), 15)
    dx = dev(dx0)
    dgam, dbet = dev(np.full(cols, 0.25, np.float32)), dev(np.zeros(cols, np.float32))
    bparts = empty((ne, rows, 2))
    for i, (c0, c1) in enumerate(tiles):
        w = c1 - c0
        tt.tile_layernorm_bwd(None, tt.TT_LN_PARTIAL, rows, w, cols, DY[:, c0:c1].contiguous(), w,
                              X[:, c0:c1].contiguous(), w, G[c0:c1].contiguous(), stats, bparts[i], 0, 0, None, 0, 0,
                              None, None, None)
    for i, (c0, c1) in enumerate(tiles):
        w = c1 - c0
        ws = torch.empty(tt.tile_layernorm_bwd_workspace(rows, w) // 4 + 1, device="cuda")
        dxt = dx[:, c0:c1].contiguous()
        dgt, dbt = dgam[c0:c1].contiguous(), dbet[c0:c1].contiguous()
        tt.tile_layernorm_bwd(None, tt.TT_LN_APPLY, rows, w, cols, DY[:, c0:c1].contiguous(), w,
                              X[:, c0:c1].contiguous(), w, G[c0:c1].contiguous(), stats, bparts, ne, rows * 2, dxt,
                              w, 1, dgt, dbt, ws)
        dx[:, c0:c1] = dxt
        dgam[c0:c1] = dgt
        dbet[c0:c1] = dbt
    assert_rel(host(dx), dx0 + rdx, 1e-4, 1e-5, "ln dx")
    assert_rel(host(dgam), 0.25 + rdg, 1e-4, 1e-4, "ln dgamma")
    assert_rel(host(dbet), rdb, 1e-4, 1e-4, "ln dbeta")


@pytest.mark.parametrize("rows,cols", [(5, 64), (1000, 768), (64, 33)])
def test_layernorm_bwd_fused(rows, cols):
    x = synth.rand_normal((rows, cols), 21, std=2.0)
    g = synth.rand_normal((cols,), 22) + 1
    dy = synth.rand_normal((rows, cols), 23)
    ry, (mu, rs) = og.layernorm_fwd(x.astype(np.float64), g.astype(np.float64), np.zeros(cols))
    stats = dev(np.stack([mu, rs], 1).astype(np.float32))
    dx = empty((rows, cols))
    dgam, dbet = dev(np.zeros(cols, np.float32)), dev(np.zeros(cols, np.float32))
    ws = torch.empty(tt.tile_layernorm_bwd_workspace(rows, cols) // 4 + 1, device="cuda")
    tt.tile_layernorm_bwd(None, tt.TT_LN_FUSED, rows, cols, cols, dev(dy), cols, dev(x), cols, dev(g), stats, None,
                          0, 0, dx, cols, 0, dgam, dbet, ws)
    rdx, rdg, rdb = og.layernorm_bwd(dy.astype(np.float64), x.astype(np.float64), g.astype(np.float64), mu, rs)
    assert_rel(host(dx), rdx, 1e-4, 1e-5, "ln dx")
    assert_rel(host(dgam), rdg, 1e-4, 1e-4, "dgamma")
    assert_rel(host(dbet), rdb, 1e-4, 1e-4, "dbeta")


@pytest.mark.parametrize("rows,cols", [
    (96, [64, 64, 32]),            # 160 features: 256-thread rows, narrower last tile, ragged row blocks
    (33, [512, 512, 512, 512]),    # 2048 features: 512-thread rows
    (64, [2048, 2048, 2048, 1024]),  # 7168: 1024 threads, 2 float4 each
    (20, [4096, 4096, 4096, 4096]),  # 16384: 4 float4 each (the widest model's row)
])
@pytest.mark.parametrize("dx_acc", [0, 1])
def test_layernorm_multi_tile_one_pass(rows, cols, dx_acc):
    """LayerNorm over several feature tiles in one pass (forward and
    backward) against the oracle on the whole row; bitwise reproducible."""
    total = sum(cols)
    x = synth.rand_normal((rows, total), 41, std=2.0) + 0.3
    g = synth.rand_normal((total,), 42) + 1
    b = synth.rand_normal((total,), 43)
    dy = synth.rand_normal((rows, total), 44)
    edges = np.cumsum([0] + cols)
    sl = [slice(edges[i], edges[i + 1]) for i in range(len(cols))]
    xs = [dev(x[:, q]) for q in sl]
    gs, bs = [dev(g[q]) for q in sl], [dev(b[q]) for q in sl]
    ys = [empty((rows, c)) for c in cols]
    stats = empty((rows, 2))
    tt.tile_layernorm_fwd_multi(None, rows, cols, xs, gs, bs, stats, ys, 1e-5)
    x64, g64 = x.astype(np.float64), g.astype(np.float64)
    ry, (mu, rs) = og.layernorm_fwd(x64, g64, b.astype(np.float64))
    got = np.concatenate([host(y) for y in ys], 1)
    assert_rel(got, ry, 2e-5, 2e-5, "ln multi y")
    assert_rel(host(stats)[:, 0], mu, 1e-5, 1e-6, "ln multi mean")
    assert_rel(host(stats)[:, 1], rs, 1e-5, 0, "ln multi rstd")
    # backward, twice (bitwise equal), dx accumulating onto an existing gradient when dx_acc
    rdx, rdg, rdb = og.layernorm_bwd(dy.astype(np.float64), x64, g64, mu, rs)
    dx0 = synth.rand_normal((rows, total), 45)
    nws = tt.tile_layernorm_bwd_multi_workspace(rows, total)
    outs = []
    for _ in range(2):
        dxs = [dev(dx0[:, q]) if dx_acc else empty((rows, c)) for q, c in zip(sl, cols)]
        dgs = [dev(np.full(c, 0.25, np.float32)) for c in cols]
        dbs = [dev(np.zeros(c, np.float32)) for c in cols]
        ws = torch.empty(nws // 4 + 1, device="cuda")
        tt.tile_layernorm_bwd_multi(None, rows, cols, [dev(dy[:, q]) for q in sl], xs, gs, stats, dxs, dx_acc, dgs,
                                    dbs, ws, nws)
        outs.append([np.concatenate([host(a) for a in lst], -1) for lst in (dxs, dgs, dbs)])
    (dxg, dgg, dbg), again = outs
    for a, b_ in zip(outs[0], again):
        assert np.array_equal(a, b_)
    assert_rel(dxg, rdx + (dx0 if dx_acc else 0), 1e-4, 1e-5, "ln multi dx")
    assert_rel(dgg, rdg + 0.25, 1e-4, 1e-4, "ln multi dgamma")
    assert_rel(dbg, rdb, 1e-4, 1e-4, "ln multi dbeta")


def test_layernorm_multi_tile_rejects_bad_shapes():
    a = empty((8, 64))
    with pytest.raises(tt.TTError) as e:
        tt.tile_layernorm_fwd_multi(None, 8, [64], [a], [a], [a], a, [a])       # one tile: the fused phase's job
    assert e.value.code == tt._lib.TT_ERR_ARG
    for cols in ([64, 66], [32, 64], [8192, 8192, 4]):                          # width, order, total
        with pytest.raises(tt.TTError) as e:
            tt.tile_layernorm_fwd_multi(None, 8, cols, [a] * len(cols), [a] * len(cols), [a] * len(cols), a,
                                        [a] * len(cols))
        assert e.value.code == tt._lib.TT_ERR_SHAPE, cols


# ------------------------------------------------------- softmax / CE

@pytest.mark.parametrize("rows,cols,vt", [(64, 256, 32), (300, 5000, 768), (7, 2049, 2048), (33, 100, 100)])
def test_cross_entropy_tiles(rows, cols, vt):
    z = synth.rand_normal((rows, cols), 31, std=3.0)
    y = np.random.default_rng(32).integers(0, cols, rows).astype(np.int32)
    Z, Y = dev(z), dev(y)
    tiles = otl.tiles(cols, vt)
    parts = empty((len(tiles), rows, 3))
    for i, (c0, c1) in enumerate(tiles):
        tt.tile_softmax(None, tt.TT_SM_STATS, rows, c1 - c0, 0, c0, 1.0, 0, Z[:, c0:c1].contiguous(), c1 - c0, Y,
                        parts[i], 0, 0, None, None, None, 0, 1.0)
    lse, rl = empty((rows,)), empty((rows,))
    tt.tile_softmax(None, tt.TT_SM_MERGE, rows, 0, 0, 0, 1.0, 0, None, 0, None, parts, len(tiles), rows * 3, lse, rl,
                    None, 0, 1.0)
    loss = empty((1,))
    half = rows // 2
    tt.tile_xentropy(None, tt.TT_XE_LOSS, half, 0, 0, None, None, 0, None, rl, loss, 0, 1.0 / rows)
    tt.tile_xentropy(None, tt.TT_XE_LOSS, rows - half, 0, 0, None, None, 0, None, rl[half:], loss, 1, 1.0 / rows)
    rloss, rdz, rlse = og.cross_entropy(z.astype(np.float64), y)
    assert_rel(host(lse), rlse, 1e-6, 1e-6, "lse")
    assert abs(host(loss)[0] - rloss) <= 1e-5 * abs(rloss)
    dz = Z.clone()
    for c0, c1 in tiles:
        blk = dz[:, c0:c1].contiguous()
        tt.tile_xentropy(None, tt.TT_XE_GRAD, rows, c1 - c0, c0, Y, blk, c1 - c0, lse, None, None, 0, 1.0 / rows)
        dz[:, c0:c1] = blk
    assert_rel(host(dz), rdz, 1e-5, 1e-7 / rows, "dz")


@pytest.mark.parametrize("rows,cols,vt", [(300, 5000, 768), (64, 256, 32), (33, 1873, 768), (20, 6600, 100)])
def test_cross_entropy_multi_tile(rows, cols, vt):
    """tile_xentropy_multi (all vocab tiles of a token tile per launch; more
    than 64 tiles make two launches; a ragged 337-wide tile takes the scalar
    path) equals the per-tile calls bitwise, and the loss, lse and dz the
    fp64 oracle's."""
    z = synth.rand_normal((rows, cols), 41, std=3.0)
    y = np.random.default_rng(42).integers(0, cols, rows).astype(np.int32)
    Y = dev(y)
    tiles = otl.tiles(cols, vt)
    blocks = [dev(z[:, c0:c1]) for c0, c1 in tiles]          # one allocation per tile, as in the step
    lens, offs = [c1 - c0 for c0, c1 in tiles], [c0 for c0, _ in tiles]
    parts = empty((len(tiles), rows, 3))
    tt.tile_xentropy_multi(None, tt.TT_XE_STATS, rows, lens, offs, Y, blocks, lens, parts=parts, part_stride=rows * 3)
    ref_parts = empty((len(tiles), rows, 3))
    for i, (c0, c1) in enumerate(tiles):
        tt.tile_softmax(None, tt.TT_SM_STATS, rows, c1 - c0, 0, c0, 1.0, 0, blocks[i], c1 - c0, Y, ref_parts[i], 0, 0,
                        None, None, None, 0, 1.0)
    assert torch.equal(parts, ref_parts)
    lse, rl = empty((rows,)), empty((rows,))
    tt.tile_softmax(None, tt.TT_SM_MERGE, rows, 0, 0, 0, 1.0, 0, None, 0, None, parts, len(tiles), rows * 3, lse, rl,
                    None, 0, 1.0)
    rloss, rdz, rlse = og.cross_entropy(z.astype(np.float64), y)
    assert_rel(host(lse), rlse, 1e-6, 1e-6, "lse")
    assert abs(host(rl).mean() - rloss) <= 1e-5 * abs(rloss)
    singles = [b.clone() for b in blocks]
    tt.tile_xentropy_multi(None, tt.TT_XE_GRAD, rows, lens, offs, Y, blocks, lens, lse=lse, inv_n=1.0 / rows)
    for i, (c0, c1) in enumerate(tiles):
        tt.tile_xentropy(None, tt.TT_XE_GRAD, rows, c1 - c0, c0, Y, singles[i], c1 - c0, lse, None, None, 0, 1.0 / rows)
        assert torch.equal(blocks[i], singles[i])
        assert_rel(host(blocks[i]), rdz[:, c0:c1], 1e-5, 1e-7 / rows, f"dz tile {i}")


@pytest.mark.parametrize("rows,vocab,vt,k,beta", [
    (300, 1000, 256, 96, 0.0),     # ragged rows, 4 vocab tiles (the last 232 wide)
    (130, 2500, 1105, 64, 1.0),    # the wide model's ragged vocab tile width, C accumulated (beta 1)
    (64, 5000, 768, 128, 0.0),     # 7 tiles, the last 392 wide
    (96, 200, 64, 32, 0.5),        # one 64-column group per tile, rows below one block
])
def test_head_xstats_epilogue_and_group_merge(rows, vocab, vt, k, beta):
    """The head's batched products with the cross-entropy statistics in the
    epilogue, merged by 64-column groups: the logits against the fp64
    products, lse and the per-row loss against the oracle's cross-entropy of
    the fp64 logits and against the separate statistics pass over the GPU's
    own logits; the partials start as NaN, so a group the epilogue failed to
    write would show; bitwise equal across runs."""
    x = synth.rand_normal((rows, k), 81 + k, std=0.5)
    w = synth.rand_normal((vocab, k), 82 + k, std=0.5)
    c0 = synth.rand_normal((rows, vocab), 83, std=2.0)
    y = np.random.default_rng(84).integers(0, vocab, rows).astype(np.int32)
    tiles = otl.tiles(vocab, vt)
    lens = [c1 - c0_ for c0_, c1 in tiles]
    X, Y = dev(x), dev(y)
    Ws = [dev(w[a:b]) for a, b in tiles]
    groups = -(-vt // 64)
    stride = groups * rows * 3
    outs = []
    for _ in range(2):
        Zs = [dev(c0[:, a:b]) for a, b in tiles]
        parts = torch.full((len(tiles), stride), float("nan"), device="cuda")
        tt.tile_gemm_batch_xstats(None, 1, rows, lens, k, 1.0, [X] * len(tiles), [k] * len(tiles), Ws,
                                  [k] * len(tiles), beta, Zs, lens, Y, 0, vt, parts, stride)
        lse, rl = empty((rows,)), empty((rows,))
        tt.tile_xentropy_merge_groups(None, rows, lens, 64, parts, stride, lse, rl)
        outs.append((torch.cat(Zs, dim=1), lse, rl))
    assert all(torch.equal(a, b) for a, b in zip(outs[0], outs[1]))
    z_gpu, lse, rl = outs[0]
    ref = beta * c0.astype(np.float64) + x.astype(np.float64) @ w.astype(np.float64).T
    bound = (np.abs(x).astype(np.float64) @ np.abs(w).astype(np.float64).T) * (k + 2) * EPS32
    assert_close_bound(host(z_gpu), ref, bound + 4 * EPS32 * np.abs(ref) + 1e-30, "head logits")
    rloss, _, rlse = og.cross_entropy(ref, y)
    assert_rel(host(lse), rlse, 1e-5, 1e-5, "lse (fused statistics)")
    assert abs(host(rl).mean() - rloss) <= 1e-5 * abs(rloss)
    # against the separate statistics pass over the same fp32 logits
    blocks = [z_gpu[:, a:b].contiguous() for a, b in tiles]
    p1 = empty((len(tiles), rows, 3))
    tt.tile_xentropy_multi(None, tt.TT_XE_STATS, rows, lens, [a for a, _ in tiles], Y, blocks, lens, parts=p1,
                           part_stride=rows * 3)
    lse1, rl1 = empty((rows,)), empty((rows,))
    tt.tile_softmax(None, tt.TT_SM_MERGE, rows, 0, 0, 0, 1.0, 0, None, 0, None, p1, len(tiles), rows * 3, lse1, rl1,
                    None, 0, 1.0)
    assert_rel(host(lse), host(lse1), 2e-6, 2e-6, "lse fused vs separate pass")
    # the picked target logit is the GPU's own logit (a sum of one value and zeros)
    picked = host(lse) - host(rl)
    zl = host(z_gpu)[np.arange(rows), y]
    assert np.abs(picked - zl).max() <= 4 * EPS32 * (np.abs(host(lse)).max() + np.abs(zl).max())


def test_head_xstats_errors():
    a = empty((64, 64))
    lab = torch.zeros(64, dtype=torch.int32, device="cuda")
    p = empty((64 * 3,))
    with pytest.raises(tt.TTError):   # n above the vocab tile
        tt.tile_gemm_batch_xstats(None, 1, 64, [64], 64, 1.0, [a], [64], [a], [64], 0.0, [a], [64], lab, 0, 32, p,
                                  64 * 3)
    with pytest.raises(tt.TTError):   # partials too small for the groups
        tt.tile_gemm_batch_xstats(None, 1, 64, [64], 64, 1.0, [a], [64], [a], [64], 0.0, [a], [64], lab, 0, 128, p,
                                  64 * 2)
    with pytest.raises(tt.TTError):
        tt.tile_xentropy_merge_groups(None, 64, [64], 0, p, 64 * 3, p)


def test_cross_entropy_multi_errors():
    z = dev(np.zeros((4, 8), np.float32))
    y = dev(np.zeros(4, np.int32))
    tt.tile_xentropy_multi(None, tt.TT_XE_STATS, 4, [], [], y, [], [], parts=z, part_stride=12)  # count 0: no-op
    with pytest.raises(tt.TTError):
        tt.tile_xentropy_multi(None, tt.TT_XE_STATS, 4, [8], [0], y, [z], [8], parts=None, part_stride=12)
    with pytest.raises(tt.TTError):
        tt.tile_xentropy_multi(None, tt.TT_XE_GRAD, 4, [8], [0], y, [z], [8], lse=None)
    with pytest.raises(tt.TTError):
        tt.tile_xentropy_multi(None, tt.TT_XE_GRAD, 4, [4096], [0], y, [z], [4096], lse=z)
    with pytest.raises(tt.TTError):
        tt.tile_xentropy_multi(None, 7, 4, [8], [0], y, [z], [8], lse=z)


def test_softmax_causal_apply():
    rows, cols, roff, coff, scale = 40, 96, 50, 30, 0.7
    x = synth.rand_normal((rows, cols), 41)
    X = dev(x)
    parts, lse, Y = empty((1, rows, 3)), empty((rows,)), empty((rows, cols))
    tt.tile_softmax(None, tt.TT_SM_STATS, rows, cols, roff, coff, scale, 1, X, cols, None, parts, 0, 0, None, None,
                    None, 0, 1.0)
    tt.tile_softmax(None, tt.TT_SM_MERGE, rows, 0, 0, 0, 1.0, 0, None, 0, None, parts, 1, rows * 3, lse, None, None,
                    0, 1.0)
    tt.tile_softmax(None, tt.TT_SM_APPLY, rows, cols, roff, coff, scale, 1, X, cols, None, None, 0, 0, lse, None, Y,
                    cols, 1.0)
    s = x.astype(np.float64) * scale
    mask = (coff + np.arange(cols))[None, :] > (roff + np.arange(rows))[:, None]
    s[mask] = -np.inf
    assert_rel(host(Y), og.softmax(s), 1e-5, 1e-7, "causal softmax")


# ------------------------------------------------------------ attention

def _attn_inputs(b, t, h, hd, seed):
    q = synth.rand_normal((b, t, h, hd), seed)
    k = synth.rand_normal((b, t, h, hd), seed + 1)
    v = synth.rand_normal((b, t, h, hd), seed + 2)
    return q, k, v


def _attn_ref(q, k, v):
    f = lambda a: a.astype(np.float64).transpose(0, 2, 1, 3)  # noqa: E731
    o, p = og.causal_attention_fwd(f(q), f(k), f(v))
    hd = q.shape[-1]
    s = f(q) @ np.swapaxes(f(k), -1, -2) / math.sqrt(hd)
    t = q.shape[1]
    s = np.where(np.triu(np.ones((t, t), bool), 1), -np.inf, s)
    return o, p, og.logsumexp(s)


@pytest.mark.parametrize("b,t,h,hd", [(2, 32, 4, 16), (1, 200, 3, 64), (2, 256, 2, 128), (1, 130, 1, 32)])
def test_attention_fwd_single_tile(b, t, h, hd):
    q, k, v = _attn_inputs(b, t, h, hd, 51 + hd)
    O, lse = empty((b, t, h, hd)), empty((b, h, t))
    tt.tile_attention_fwd(None, b, h, t, t, hd, 0, 0, dev(q), dev(k), dev(v), O, None, lse, 1, 1, 1 / math.sqrt(hd))
    ro, _, rlse = _attn_ref(q, k, v)
    assert_rel(host(O).transpose(0, 2, 1, 3), ro, 1e-4, 2e-5, "attn O")
    assert_rel(host(lse), rlse, 1e-5, 1e-5, "attn lse")


@pytest.mark.parametrize("stored_ds", [False, True])
@pytest.mark.parametrize("hd,st", [(64, 64), (128, 96), (16, 8), (32, 40)])
def test_attention_fwd_bwd_tile_pairs(hd, st, stored_ds):
    """Both backward forms: recomputing dS in the dQ kernel, and dS handed
    from the dK/dV kernel through a workspace (the workspace is filled with
    NaN first: a block the dQ kernel reads but the other kernel did not
    write would show)."""
    b, h, t = 2, 2, 3 * st
    q, k, v = _attn_inputs(b, t, h, hd, 61)
    do = synth.rand_normal((b, t, h, hd), 64)
    scale = 1 / math.sqrt(hd)
    seq = lambda a, i: dev(np.ascontiguousarray(a[:, i * st:(i + 1) * st]))  # noqa: E731
    n = t // st
    Q = [seq(q, i) for i in range(n)]
    K = [seq(k, i) for i in range(n)]
    V = [seq(v, i) for i in range(n)]
    dO = [seq(do, i) for i in range(n)]
    O = [empty((b, st, h, hd)) for _ in range(n)]
    lse = [empty((b, h, st)) for _ in range(n)]
    ml = empty((b, h, st, 2))
    for qi in range(n):
        for ki in range(qi + 1):
            tt.tile_attention_fwd(None, b, h, st, st, hd, qi * st, ki * st, Q[qi], K[ki], V[ki], O[qi], ml, lse[qi],
                                  int(ki == 0), int(ki == qi), scale)
    ro, rp, rlse = _attn_ref(q, k, v)
    got_o = np.concatenate([host(x) for x in O], axis=1).transpose(0, 2, 1, 3)
    assert_rel(got_o, ro, 1e-4, 2e-5, "tiled attn O")
    assert_rel(np.concatenate([host(x) for x in lse], axis=2), rlse, 1e-5, 1e-5, "tiled lse")
    # backward by tile pairs
    Dv = [empty((b, h, st)) for _ in range(n)]
    dQ = [empty((b, st, h, hd)) for _ in range(n)]
    dK = [empty((b, st, h, hd)) for _ in range(n)]
    dV = [empty((b, st, h, hd)) for _ in range(n)]
    for qi in range(n):
        tt.tile_attention_bwd(None, tt.TT_ATT_PREP, b, h, st, st, hd, 0, 0, None, None, None, O[qi], dO[qi], None,
                              Dv[qi], None, None, None, 0, 0, scale)
    wsb = tt.tile_attention_bwd_workspace(b, h, st, st)
    assert wsb == b * h * (-(-st // 32)) ** 2 * 1024 * 4
    ws = torch.full((wsb // 4,), float("nan"), device="cuda")
    for qi in range(n):
        for ki in range(qi + 1):
            args = (None, tt.TT_ATT_GRAD, b, h, st, st, hd, qi * st, ki * st, Q[qi], K[ki], V[ki], None,
                    dO[qi], lse[qi], Dv[qi], dQ[qi], dK[ki], dV[ki], int(ki > 0), int(qi > ki), scale)
            if stored_ds:
                tt.tile_attention_bwd_ws(*args, ws, wsb)
            else:
                tt.tile_attention_bwd(*args)
    f = lambda a: a.astype(np.float64).transpose(0, 2, 1, 3)  # noqa: E731
    rdq, rdk, rdv = og.causal_attention_bwd(f(do), f(q), f(k), f(v), rp)
    cat = lambda xs: np.concatenate([host(x) for x in xs], axis=1).transpose(0, 2, 1, 3)  # noqa: E731
    for got, ref, name in ((cat(dQ), rdq, "dQ"), (cat(dK), rdk, "dK"), (cat(dV), rdv, "dV")):
        assert_rel(got, ref, 2e-4, 2e-4 * np.abs(ref).max(), name)


# ---------------------------------------------------------------- AdamW

@pytest.mark.parametrize("n", [1, 1000, 4096 + 3, 1 << 20])
def test_fused_adamw(n):
    p = synth.rand_normal((n,), 71)
    g = synth.rand_normal((n,), 72) * np.logspace(-6, 0, n).astype(np.float32)
    P, G = dev(p), dev(g)
    M, V = dev(np.zeros(n, np.float32)), dev(np.zeros(n, np.float32))
    step = torch.zeros(1, dtype=torch.int32, device="cuda")
    bc = empty((2,))
    # the kernel receives its hyperparameters as fp32: feed the oracle the same values
    b1, b2, lr, eps, wd = (float(np.float32(x)) for x in (0.9, 0.999, 3e-4, 1e-8, 0.1))
    rp, rm, rv = p.astype(np.float64), np.zeros(n), np.zeros(n)
    for t in (1, 2, 3):
        tt.tile_adamw_advance(None, step, bc, b1, b2)
        tt.tile_fused_adamw(None, n, P, G, M, V, lr, b1, b2, eps, wd, bc)
        rp, rm, rv = og.adamw(rp, g.astype(np.float64), rm, rv, t, lr, b1, b2, eps, wd)
    assert int(step.item()) == 3
    assert_rel(host(bc), np.array([1 - b1 ** 3, 1 - b2 ** 3]), 1e-6)
    assert_rel(host(M), rm, 1e-5, 1e-12, "m")
    assert_rel(host(V), rv, 1e-5, 1e-20, "v")
    # parameter: abs floor well below one lr step
    assert_close_bound(host(P), rp, 1e-6 * np.abs(rp) + 1e-3 * 3e-4, "p")


def test_fused_adamw_multi_equals_per_tile_launches():
    """Several tiles in one launch (mixed sizes, a ragged one, an unaligned
    one) give bitwise the per-tile results, which the test above pins to the
    oracle; more tiles than the limit, or a negative size, are errors."""
    sizes = [768, 3, 4096 + 2, 1 << 18, 1, 5000]
    base = torch.from_numpy(synth.rand_normal((sum(sizes) + 64,), 73)).cuda()
    grads = torch.from_numpy(synth.rand_normal((sum(sizes) + 64,), 74)).cuda()
    step = torch.zeros(1, dtype=torch.int32, device="cuda")
    bc = empty((2,))
    tt.tile_adamw_advance(None, step, bc, 0.9, 0.999)

    def views(t, off=1):  # offset 1 float: the second tile set is not 16-byte aligned
        out, o = [], off
        for n in sizes:
            out.append(t[o:o + n])
            o += n
        return out
    results = []
    for multi in (False, True):
        P = [x.clone() for x in views(base)]
        G = views(grads)
        M = [torch.full_like(x, 0.01) for x in P]
        V = [torch.full_like(x, 0.02) for x in P]
        if multi:
            tt.tile_fused_adamw_multi(None, P, G, M, V, 3e-4, 0.9, 0.999, 1e-8, 0.1, bc)
        else:
            for p_, g_, m_, v_ in zip(P, G, M, V):
                tt.tile_fused_adamw(None, p_.numel(), p_, g_, m_, v_, 3e-4, 0.9, 0.999, 1e-8, 0.1, bc)
        torch.cuda.synchronize()
        results.append([host(x) for x in P + M + V])
    for a, b in zip(*results):
        assert np.array_equal(a, b)
    with pytest.raises(tt.TTError):
        tt.tile_fused_adamw_multi(None, [base] * 17, [grads] * 17, [base] * 17, [base] * 17, 3e-4, 0.9, 0.999, 1e-8,
                                  0.1, bc)


def test_fill_multi():
    sizes = [1, 5, 768, 4097, 1 << 17]
    buf = torch.full((sum(sizes) + 8,), 7.0, device="cuda")
    tiles, o = [], 3
    for n in sizes:
        tiles.append(buf[o:o + n])
        o += n
    tt.tile_fill_multi(None, tiles, -2.5)
    got = host(buf)
    assert (got[:3] == 7.0).all() and (got[3:o] == -2.5).all() and (got[o:] == 7.0).all()
    with pytest.raises(tt.TTError):
        tt.tile_fill_multi(None, [buf] * 17, 0.0)


def test_sgd_multi_and_single():
    sizes = [1, 5, 768, 4097, 1 << 17]
    lr = 0.05
    ps = [synth.rand_normal((n,), 300 + i) for i, n in enumerate(sizes)]
    gs = [synth.rand_normal((n,), 400 + i) for i, n in enumerate(sizes)]
    P, Gr = [dev(x) for x in ps], [dev(x) for x in gs]
    # an unaligned tile (offset by one float) takes the scalar path
    pu = torch.from_numpy(np.concatenate([[0.0], ps[3]]).astype(np.float32)).cuda()[1:]
    gu = torch.from_numpy(np.concatenate([[0.0], gs[3]]).astype(np.float32)).cuda()[1:]
    tt.tile_sgd_multi(None, P + [pu], Gr + [gu], lr)
    for x, g, got in zip(ps + [ps[3]], gs + [gs[3]], P + [pu]):
        ref = og.sgd(x.astype(np.float32).astype(np.float64), g.astype(np.float32).astype(np.float64), lr)
        bound = 2.0 ** -23 * (np.abs(x) + lr * np.abs(g)) * 2
        assert (np.abs(host(got) - ref) <= bound + 1e-30).all()
    one = dev(ps[2])
    tt.tile_sgd(None, sizes[2], one, Gr[2], lr)
    assert np.array_equal(host(one), host(P[2]))  # same arithmetic as the multi form
    with pytest.raises(tt.TTError):
        tt.tile_sgd_multi(None, [P[0]] * 17, [Gr[0]] * 17, lr)


# ----------------------------------------------------- embedding / misc

def test_embedding_fwd_bwd():
    vocab, d, bt, st = 300, 96, 3, 40
    rows = bt * st
    wte = synth.rand_normal((vocab, d), 81)
    wpe = synth.rand_normal((st, d), 82)
    rng = np.random.default_rng(83)
    ids = rng.integers(0, vocab, rows).astype(np.int32)
    ids[:10] = 7  # repeated ids
    out = empty((rows, d))
    IDS = dev(ids)
    tt.tile_embedding_fwd(None, rows, d, IDS, vocab, 0, vocab, dev(wte), d, dev(wpe), d, st, 0, out, d)
    ref = wte[ids] + wpe[np.arange(rows) % st]
    assert np.array_equal(host(out), ref.astype(np.float32).astype(np.float64))
    srt = torch.empty(rows, dtype=torch.int32, device="cuda")
    perm = torch.empty(rows, dtype=torch.int32, device="cuda")
    tt.tile_embedding_index(None, rows, IDS, srt, perm)
    order = np.argsort(ids, kind="stable")
    assert np.array_equal(perm.cpu().numpy(), order) and np.array_equal(srt.cpu().numpy(), ids[order])
    dh = synth.rand_normal((rows, d), 84)
    dw0 = synth.rand_normal((vocab, d), 85)
    DW = dev(dw0)
    vt = 128
    for v0, v1 in otl.tiles(vocab, vt):
        blk = DW[v0:v1].contiguous()
        tt.tile_embedding_bwd(None, tt.TT_EMB_TOKEN, rows, d, srt, perm, v0, v1 - v0, st, dev(dh), d, blk, d)
        DW[v0:v1] = blk
    rdw = dw0 + otl.embedding_bwd_tiled(dh.astype(np.float64), ids, vocab, vt, d, rows)
    assert_rel(host(DW), rdw, 1e-6, 1e-6, "dwte")
    dp = dev(np.zeros((st, d), np.float32))
    tt.tile_embedding_bwd(None, tt.TT_EMB_POS, rows, d, None, None, 0, 0, st, dev(dh), d, dp, d)
    assert_rel(host(dp), dh.astype(np.float64).reshape(bt, st, d).sum(0), 1e-6, 1e-6, "dwpe")


@pytest.mark.parametrize("rows,vocab", [(1, 5), (17, 3), (4096, 50257), (5000, 40), (65536, 50257)])
def test_embedding_index_is_a_stable_sort(rows, vocab):
    """The per-token-tile index (sorted ids, permutation) equals numpy's
    stable argsort: one row, ragged workgroups, many duplicates, several LDS
    chunks, the largest tile allowed."""
    ids = np.random.default_rng(rows).integers(0, vocab, rows).astype(np.int32)
    srt = torch.empty(rows, dtype=torch.int32, device="cuda")
    perm = torch.empty(rows, dtype=torch.int32, device="cuda")
    tt.tile_embedding_index(None, rows, dev(ids), srt, perm)
    order = np.argsort(ids, kind="stable")
    assert np.array_equal(perm.cpu().numpy(), order) and np.array_equal(srt.cpu().numpy(), ids[order])


def test_embedding_out_of_range_id_gives_nan_row():
    ids = np.array([0, 5, 99, -1], np.int32)
    wte = synth.rand_normal((5, 8), 1)
    wpe = synth.rand_normal((4, 8), 2)
    out = empty((4, 8), fill=0.0)
    tt.tile_embedding_fwd(None, 4, 8, dev(ids), 5, 0, 5, dev(wte), 8, dev(wpe), 8, 4, 0, out, 8)
    got = host(out)
    assert np.isfinite(got[0]).all() and np.isnan(got[1]).all() and np.isnan(got[2]).all() and np.isnan(got[3]).all()


@pytest.mark.parametrize("rows,cols", [(1, 5), (4096, 768), (300, 3072), (1000, 33)])
def test_reduce_rows(rows, cols):
    x = synth.rand_normal((rows, cols), 91)
    out = dev(np.full(cols, 2.0, np.float32))
    ws = torch.empty(tt.tile_reduce_rows_workspace(rows, cols) // 4 + 1, device="cuda")
    tt.tile_reduce_rows(None, rows, cols, dev(x), cols, out, 1, ws)
    ref = 2.0 + x.astype(np.float64).sum(0)
    bound = (np.abs(x).astype(np.float64).sum(0) + 2) * rows * EPS32
    assert_close_bound(host(out), ref, bound, "reduce_rows")
    # deterministic: same bits on a second run
    out2 = dev(np.full(cols, 2.0, np.float32))
    tt.tile_reduce_rows(None, rows, cols, dev(x), cols, out2, 1, ws)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("rows,cols,beta", [(4096, [768, 768, 768], 1), (1000, [100, 3, 768, 257], 0),
                                             (65, [64] * 16, 1)])
def test_reduce_rows_multi(rows, cols, beta):
    """Column sums of several tiles in one pair of launches: bitwise equal to
    the per-tile calls and within the fp32 bound of the fp64 sums; ragged rows
    and columns, 16 tiles; a too-small workspace is an error."""
    xs = [synth.rand_normal((rows, c), 93 + i) for i, c in enumerate(cols)]
    need = sum(tt.tile_reduce_rows_workspace(rows, c) for c in cols)
    ws = torch.empty(need // 4 + 1, device="cuda")
    dx = [dev(x) for x in xs]
    outs = [dev(np.full(c, 2.0, np.float32)) for c in cols]
    tt.tile_reduce_rows_multi(None, rows, cols, dx, cols, outs, beta, ws, need)
    for x, c, o in zip(dx, cols, outs):
        single = dev(np.full(c, 2.0, np.float32))
        w1 = torch.empty(tt.tile_reduce_rows_workspace(rows, c) // 4 + 1, device="cuda")
        tt.tile_reduce_rows(None, rows, c, x, c, single, beta, w1)
        assert torch.equal(o, single)
    for x, o in zip(xs, outs):
        ref = 2.0 * beta + x.astype(np.float64).sum(0)
        bound = (np.abs(x).astype(np.float64).sum(0) + 2) * rows * EPS32
        assert_close_bound(host(o), ref, bound, "reduce_rows_multi")
    with pytest.raises(tt.TTError):
        tt.tile_reduce_rows_multi(None, rows, cols, dx, cols, outs, beta, ws, need - 4)


def test_fill_and_split_tokens():
    f = empty((1000,))
    tt.tile_fill(None, 1000, f, 3.5)
    assert (host(f) == 3.5).all()
    tok = np.random.default_rng(1).integers(0, 50257, (3, 9)).astype(np.int32)
    ids = torch.empty(24, dtype=torch.int32, device="cuda")
    lab = torch.empty(24, dtype=torch.int32, device="cuda")
    tt.tile_split_tokens(None, 3, 8, dev(tok), ids, lab)
    assert np.array_equal(ids.cpu().numpy().reshape(3, 8), tok[:, :8])
    assert np.array_equal(lab.cpu().numpy().reshape(3, 8), tok[:, 1:])
