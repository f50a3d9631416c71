"""The decode step that allocates nothing (ttsbb_decode_step_noalloc, for callers that
cannot allocate device memory): through the C ABI, against ttsbb_decode_step on the same
inputs, two calls in a row (the second smaller), bit for bit -- the two run the same
kernels with the same launch choices; only the scratch memory differs."""
import numpy as np
import pytest

from workload import configs as CFG
from workload import device as DEV
from workload import gen
from workload.gen import stream_id

from gpu_setup import Model, torch

pytestmark = pytest.mark.gpu


def t_i32(a):
    return torch().from_numpy(np.ascontiguousarray(a, np.int32)).to("cuda")


def run_both(m, lengths, G, V, seed):
    T = m.T
    B = len(lengths)
    pt, n_pages = CFG.page_table(seed, [n + 1 for n in lengths], extra_pages=2)
    pool_a = DEV.kv_pool(seed, m.shape, m.n_layers, lengths, pt, n_pages, True)
    pool_b = pool_a.clone()
    head = DEV.host_to_device(CFG.table(seed, gen.KIND_HEAD, 0, G * V, m.shape.hidden, True))
    x_in = gen.fast_normal(seed, stream_id(gen.KIND_X_IN, 0), (B, m.shape.hidden), 1.0)
    out = []
    for fn, pool in ((T.ttsbb_decode_step, pool_a), (T.ttsbb_decode_step_noalloc, pool_b)):
        x = torch().from_numpy(x_in.copy()).to("cuda")
        pos = t_i32(lengths)
        am = torch().full((B, G), -7, dtype=torch().int32, device="cuda")
        lg = torch().empty((B, G * V), dtype=torch().float32, device="cuda")
        fn(m.ctx, B, x, pos, t_i32(pt), pt.shape[1], pool, n_pages, head, G, V, am, lg)
        # the head's logits are optional: without them the step keeps them in its scratch
        am2 = torch().full((B, G), -7, dtype=torch().int32, device="cuda")
        x2, pos2 = torch().from_numpy(x_in.copy()).to("cuda"), t_i32(lengths)
        fn(m.ctx, B, x2, pos2, t_i32(pt), pt.shape[1], pool.clone(), n_pages, head, G, V, am2, None)
        assert T.ttsbb_sync(m.ctx) == T.OK
        out.append([a.cpu().numpy() for a in (x, pos, am, lg, x2, am2)] + [pool.cpu().numpy()])
    for a, b in zip(*out):
        assert np.array_equal(a, b)
    assert np.array_equal(out[0][2], out[0][5])
    return out


def test_noalloc_decode_step_matches_the_workspace_step():
    """The paged workload's shape: 64 streams (caches up to 4000 positions, 16-token
    pages), 2 layers, 8 x 1025 heads; then 9 streams with ragged caches and a 3 x 37
    head through the same array (the first call's contents left behind)."""
    m = Model(CFG.Shape(n_layers=2), 2, True, seed=7, gains="random")
    T = m.T
    try:
        lengths = [int(v) for v in CFG.c5_lengths(CFG.c5())]
        run_both(m, lengths, 8, 1025, 7)
        run_both(m, [0, 1, 15, 16, 17, 33, 64, 100, 3000], 3, 37, 8)
        # beyond the stated limits: a clear error, nothing launched
        x = torch().zeros((65, 1024), dtype=torch().float32, device="cuda")
        st = T.ttsbb_decode_step_noalloc(m.ctx, 65, x, t_i32([1] * 65), t_i32(np.zeros((65, 1))), 1, x, 1,
                                         check=False)
        assert st == T.UNSUPPORTED
        st = T.ttsbb_decode_step_noalloc(m.ctx, 2, x, t_i32([1, 1]), t_i32(np.zeros((2, 1))), 1, x, 1, x, 9, 1000,
                                         t_i32([0] * 18), check=False)
        assert st == T.UNSUPPORTED
        assert T.ttsbb_sync(m.ctx) == T.OK
    finally:
        m.close()
