"""tile_layernorm_bwd_noalloc (column-sum partials in the library's own
device array, no allocation) against tile_layernorm_bwd with a caller
workspace: bitwise the same results, and within the oracle's bar, on two
calls in a row on one device, the second smaller than the first; sizes
beyond the array are refused before anything is launched."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth  # noqa: E402
import tile_task_transformer_amd as tt  # noqa: E402
from oracle import gpt2 as og  # noqa: E402
from tile_task_transformer_amd import _lib as L  # noqa: E402
from tests.gpu_util import assert_rel, dev, empty, host  # noqa: E402

pytestmark = pytest.mark.gpu

_fn = L.lib.tile_layernorm_bwd_noalloc
_max = L.lib.tile_layernorm_bwd_noalloc_max_bytes


def _case(rows, cols, seed):
    x = synth.rand_normal((rows, cols), seed, std=2.0) + 0.5
    g = synth.rand_normal((cols,), seed + 1) + 1
    dy = synth.rand_normal((rows, cols), seed + 2)
    dx0 = synth.rand_normal((rows, cols), seed + 3)
    _, (mu, rs) = og.layernorm_fwd(x.astype(np.float64), g.astype(np.float64), np.zeros(cols))
    stats = dev(np.stack([mu, rs], 1).astype(np.float32))
    return x, g, dy, dx0, mu, rs, stats


def _run(noalloc, rows, cols, x, g, dy, dx0, stats):
    X, G, DY = dev(x), dev(g), dev(dy)
    dx = dev(dx0)
    dgam, dbet = dev(np.full(cols, 0.5, np.float32)), dev(np.zeros(cols, np.float32))
    if noalloc:
        rc = _fn(None, L.TT_LN_FUSED, rows, cols, cols, DY.data_ptr(), cols, X.data_ptr(), cols, G.data_ptr(),
                 stats.data_ptr(), None, 0, 0, dx.data_ptr(), cols, 1, dgam.data_ptr(), dbet.data_ptr())
        L.check(rc)
    else:
        ws = torch.empty(tt.tile_layernorm_bwd_workspace(rows, cols) // 4 + 1, device="cuda")
        tt.tile_layernorm_bwd(None, tt.TT_LN_FUSED, rows, cols, cols, DY, cols, X, cols, G, stats, None, 0, 0, dx,
                              cols, 1, dgam, dbet, ws)
    return host(dx), host(dgam), host(dbet)


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    assert _max() == 16 << 20
    for rows, cols, seed in ((4096, 2048, 1), (100, 768, 7)):   # the second call smaller than the first
        x, g, dy, dx0, mu, rs, stats = _case(rows, cols, seed)
        got = _run(True, rows, cols, x, g, dy, dx0, stats)
        ref = _run(False, rows, cols, x, g, dy, dx0, stats)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), (rows, cols)
        rdx, rdg, rdb = og.layernorm_bwd(dy.astype(np.float64), x.astype(np.float64), g.astype(np.float64), mu, rs)
        assert_rel(got[0], rdx + dx0, 1e-4, 1e-5, "noalloc dx")
        assert_rel(got[1], rdg + 0.5, 1e-4, 1e-4, "noalloc dgamma")
        assert_rel(got[2], rdb, 1e-4, 1e-4, "noalloc dbeta")


def test_noalloc_refuses_sizes_beyond_its_array():
    rows, cols = 8200, 2048      # column partials of 1025 row blocks: just over 16 MiB
    assert tt.tile_layernorm_bwd_workspace(rows, cols) > _max()
    a = empty((1,))
    rc = _fn(None, L.TT_LN_FUSED, rows, cols, cols, a.data_ptr(), cols, a.data_ptr(), cols, a.data_ptr(),
             a.data_ptr(), None, 0, 0, a.data_ptr(), cols, 0, a.data_ptr(), a.data_ptr())
    assert rc == L.TT_ERR_ARG
    assert "scratch" in L.last_error()
