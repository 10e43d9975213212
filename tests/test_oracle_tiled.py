"""The fp64 tile decompositions reproduce the untiled oracle layers across
tile shapes: untiled, 32, 16, 8, ragged 24/40/7, and single rows/heads."""
import math

import numpy as np
import pytest

from oracle import gpt2 as og
from oracle import tiled as ot

SIZES = [1000, 32, 16, 8, 24, 40, 7]


def rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


@pytest.mark.parametrize("kt", SIZES)
def test_matmul_ksplit(kt):
    rng = np.random.default_rng(0)
    a, b = rng.standard_normal((19, 70)), rng.standard_normal((70, 13))
    assert rel(ot.matmul_ksplit(a, b, kt), a @ b) <= 1e-12


@pytest.mark.parametrize("et", SIZES)
def test_layernorm_tiled(et):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5, 70)) * 2 + 1.5
    g, b = rng.standard_normal(70), rng.standard_normal(70)
    y, (mu, rs) = og.layernorm_fwd(x, g, b)
    yt, (mut, rst) = ot.ln_fwd_tiled(x, g, b, et)
    assert rel(yt, y) <= 1e-12 and rel(mut, mu) <= 1e-12 and rel(rst, rs) <= 1e-12
    dy = rng.standard_normal(x.shape)
    dx, dg, db = og.layernorm_bwd(dy, x, g, mu, rs)
    for rt in (15, 4, 1):
        dxt, dgt, dbt = ot.ln_bwd_tiled(dy, x, g, mu, rs, et, rt)
        assert rel(dxt, dx) <= 1e-12 and rel(dgt, dg) <= 1e-12 and rel(dbt, db) <= 1e-12


@pytest.mark.parametrize("vt", SIZES)
def test_cross_entropy_tiled(vt):
    rng = np.random.default_rng(2)
    z = rng.standard_normal((21, 90)) * 5
    y = rng.integers(0, 90, 21)
    loss, dz, lse = og.cross_entropy(z, y)
    for rt in (21, 8, 1):
        lt, dzt, lset = ot.cross_entropy_tiled(z, y, vt, rt)
        assert abs(lt - loss) <= 1e-12 * abs(loss)
        assert rel(dzt, dz) <= 1e-12 and rel(lset, lse) <= 1e-12


@pytest.mark.parametrize("qt,kt", [(1000, 1000), (32, 32), (16, 16), (8, 8), (8, 16), (16, 8),
                                   (24, 40), (7, 7), (1, 3)])
def test_attention_tiled(qt, kt):
    rng = np.random.default_rng(3)
    t, hd = 45, 8
    q, k, v = (rng.standard_normal((t, hd)) for _ in range(3))
    o, p = og.causal_attention_fwd(q, k, v)
    lse = og.logsumexp(np.where(np.triu(np.ones((t, t), bool), 1), -np.inf,
                                q @ k.T / math.sqrt(hd)))
    ot_, lset = ot.attention_fwd_tiled(q, k, v, qt, kt)
    assert rel(ot_, o) <= 1e-12 and rel(lset, lse) <= 1e-12
    do = rng.standard_normal(o.shape)
    dq, dk, dv = og.causal_attention_bwd(do, q, k, v, p)
    dqt, dkt, dvt = ot.attention_bwd_tiled(do, q, k, v, o, lse, qt, kt)
    assert rel(dqt, dq) <= 1e-12 and rel(dkt, dk) <= 1e-12 and rel(dvt, dv) <= 1e-12


@pytest.mark.parametrize("vt,et,rt", [(1000, 1000, 1000), (32, 16, 8), (7, 40, 24), (1, 3, 1)])
def test_embedding_bwd_tiled(vt, et, rt):
    rng = np.random.default_rng(4)
    n, d, vocab = 37, 20, 50
    dh = rng.standard_normal((n, d))
    ids = rng.integers(0, vocab, n)
    ref = np.zeros((vocab, d))
    np.add.at(ref, ids, dh)
    assert rel(ot.embedding_bwd_tiled(dh, ids, vocab, vt, et, rt), ref) <= 1e-12
