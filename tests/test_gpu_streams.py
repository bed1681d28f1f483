"""Calls on a caller's stream (the C ABI's stream argument): every call is
ordered on the stream it is given, the current torch stream by default, so
work queued behind it on that stream sees its output, and two handles on two
streams give the results each would give alone."""
import numpy as np
import pytest

import oracle as orc
from gpu_helpers import build, up
from synth import rmat_csr, rng_for, sparse_x, uniform_csr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dbs():
    import spmspv_graph_traversal_amd as d

    return d


def test_calls_follow_the_given_stream(dbs):
    import torch

    rp, ci, v = uniform_csr(3000, 5000, 11, rng_for("test", 960))
    A = build(dbs, 3000, 5000, rp, ci, v, dbs.DBS_F32)
    side = torch.cuda.Stream()  # default priority
    xs = [sparse_x(5000, d, rng_for("test", 961, k)) for k, d in enumerate((0.002, 0.05, 0.4))]
    refs = [orc.spmspv_pull(3000, 5000, rp, ci, v, orc.F32, xi, xv, orc.F32) for xi, xv in xs]
    with torch.cuda.stream(side):
        ys = []
        for xi, xv in xs:
            y = torch.full((3000,), float("nan"), dtype=torch.float32, device="cuda")
            # explicit stream argument, then the current stream (side) by default
            dbs.dbs_spmspv(A, up(xi), up(xv), dbs.DBS_PLUS_TIMES, y, stream=side)
            ys.append(y * 1.0)  # queued on side after the call: sees its output
    side.synchronize()
    for (yr, s), y in zip(refs, ys):
        ok, err = orc.within_tolerance(y.cpu().numpy(), yr, s)
        assert ok.all(), f"max err {err.max():.3g}"
    # the current stream of a torch.cuda.stream context is taken by default
    xi, xv = xs[1]
    with torch.cuda.stream(side):
        y = torch.full((3000,), float("nan"), dtype=torch.float32, device="cuda")
        dbs.dbs_spmspv(A, up(xi), up(xv), dbs.DBS_PLUS_TIMES, y)
        y2 = y * 1.0
    side.synchronize()
    ok, _ = orc.within_tolerance(y2.cpu().numpy(), *refs[1])
    assert ok.all()


def test_two_handles_on_two_streams(dbs):
    """Each handle owns its call scratch, so calls of two handles on two
    streams may overlap; BFS on one and OR-AND SpMSpV on the other."""
    import torch

    n = 1 << 14
    rp, ci = rmat_csr(14, 8, rng_for("test", 970))
    G1 = build(dbs, n, n, rp, ci, None, dbs.DBS_PATTERN)
    G2 = build(dbs, n, n, rp, ci, None, dbs.DBS_PATTERN)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    xi, _ = sparse_x(n, 0.02, rng_for("test", 971), with_values=False)
    lv = torch.empty(n, dtype=torch.int32, device="cuda")
    yb = torch.empty(n, dtype=torch.uint8, device="cuda")
    xi_d = up(xi)
    torch.cuda.synchronize()
    for _ in range(3):
        dbs.dbs_spmspv(G2, xi_d, None, dbs.DBS_OR_AND, yb, stream=s2)
        dbs.dbs_bfs(G1, 5, lv, stream=s1)
    s1.synchronize()
    s2.synchronize()
    np.testing.assert_array_equal(lv.cpu().numpy(), orc.bfs(n, rp, ci, 5))
    np.testing.assert_array_equal(yb.cpu().numpy(), orc.or_and_pull(n, n, rp, ci, xi))


@pytest.mark.parametrize("off", [0, 1, 2, 3, 5])
def test_outputs_at_any_offset(dbs, off):
    """y as a view that starts 4*off (f32) or off (u8) bytes into a buffer: the
    metadata kernel clears y in a head, a 16-byte body and a tail, and the
    bytes around the view stay as they were."""
    import torch

    m, n = 1234, 2000
    rp, ci, v = uniform_csr(m, n, 7, rng_for("test", 980))
    A = build(dbs, m, n, rp, ci, v, dbs.DBS_F32)
    xi, xv = sparse_x(n, 0.03, rng_for("test", 981, off))
    buf = torch.full((m + 16,), 7.0, dtype=torch.float32, device="cuda")
    y = buf[off:off + m]
    for path in (0, 1, 2):
        dbs.dbs_set_option(A, dbs.DBS_OPT_PATH, path)
        dbs.dbs_spmspv(A, up(xi), up(xv), dbs.DBS_PLUS_TIMES, y)
        yr, s = orc.spmspv_pull(m, n, rp, ci, v, orc.F32, xi, xv, orc.F32)
        ok, err = orc.within_tolerance(y.cpu().numpy(), yr, s)
        assert ok.all(), f"path {path}: max err {err.max():.3g}"
        rest = torch.cat([buf[:off], buf[off + m:]]).cpu().numpy()
        assert np.all(rest == 7.0)
    bb = torch.full((m + 32,), 9, dtype=torch.uint8, device="cuda")
    yb = bb[off:off + m]
    dbs.dbs_spmspv(A, up(xi), None, dbs.DBS_OR_AND, yb)
    np.testing.assert_array_equal(yb.cpu().numpy(), orc.or_and_pull(m, n, rp, ci, xi))
    rest = torch.cat([bb[:off], bb[off + m:]]).cpu().numpy()
    assert np.all(rest == 9)
