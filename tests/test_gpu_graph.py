"""HIP graph capture of the decode loop (the step orchestration row: fixed shapes per loop,
so one capture serves every step).

The batch-1 28-layer decode step (codebook embedding of 16 codes + 28 layers + final norm +
3072-way head + argmax) is captured once into a graph with torch's stream capture on the
context's own stream, then replayed step after step while the same calls run eagerly on an
identical copy of the state (KV pool, cache length).  Every replay must equal the eager
step bit for bit: the graph holds the same kernels with the same arguments, the cache length
is read and incremented on the device, and nothing in the step is a memset.  Eager work and
host synchronisations sit between the replays.
"""
import numpy as np
import pytest

from workload import configs as CFG
from workload import device as DEV
from workload import gen
from workload.gen import stream_id

from gpu_setup import Model, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_layers", [2, 28])
def test_decode_step_graph_replays_match_eager(n_layers):
    th = torch()
    w = CFG.c2()
    e = w.extra
    L0, K, V, HV = e["prefill"][0], e["n_cb"], e["cb_vocab"], e["head_vocab"]
    n_steps = 10
    side = th.cuda.Stream()
    m = Model(w.shape, n_layers, True, seed=w.seed, max_pos=2048, max_head_cols=4096, stream=side.cuda_stream)
    T = m.T
    try:
        pt, n_pages = CFG.page_table(w.seed, [L0 + n_steps + 1])
        pool_e = DEV.kv_pool(w.seed, w.shape, n_layers, [L0], pt, n_pages, True)
        pool_g = DEV.kv_pool(w.seed, w.shape, n_layers, [L0], pt, n_pages, True)
        assert th.equal(pool_e, pool_g)
        tables = DEV.host_to_device(CFG.table(w.seed, gen.KIND_CB_TABLE, 0, K * V, 1024, True))
        head = DEV.host_to_device(CFG.table(w.seed, gen.KIND_HEAD, 0, HV, 1024, True))
        codes = np.stack([gen.uniform_int(w.seed, stream_id(gen.KIND_CODES, s), (1, K), V) for s in range(n_steps)])
        codes_d = th.from_numpy(codes.astype(np.int32)).cuda()
        pt_d = th.from_numpy(pt).cuda()
        pos_e = th.tensor([L0], dtype=th.int32, device="cuda")
        pos_g = th.tensor([L0], dtype=th.int32, device="cuda")
        cur = th.empty((1, K), dtype=th.int32, device="cuda")
        x_e = th.empty((1, 1024), dtype=th.float32, device="cuda")
        x_g = th.empty_like(x_e)
        am_e = th.empty((1, 1), dtype=th.int32, device="cuda")
        am_g = th.empty_like(am_e)
        lg_e = th.empty((1, HV), dtype=th.float32, device="cuda")
        lg_g = th.empty_like(lg_e)
        th.cuda.synchronize()

        def step(codes_row, x, pos, pool, am, lg):
            T.ttsbb_codebook_embed(m.ctx, 1, K, codes_row, tables, V, None, None, None, 0, x)
            T.ttsbb_decode_step(m.ctx, 1, x, pos, pt_d, pt.shape[1], pool, n_pages, head, 1, HV, am, lg)

        g = th.cuda.CUDAGraph()
        with th.cuda.stream(side):
            with th.cuda.graph(g, stream=side):
                step(cur, x_g, pos_g, pool_g, am_g, lg_g)
        # capture records and does not run: the graph's state is untouched
        th.cuda.synchronize()
        assert pos_g.item() == L0

        with th.cuda.stream(side):
            for s in range(n_steps):
                print(f"graph replay step {s} (layers {n_layers})", flush=True)
                step(codes_d[s], x_e, pos_e, pool_e, am_e, lg_e)       # eager, same stream
                cur.copy_(codes_d[s])
                g.replay()
                if s % 3 == 2:
                    th.cuda.synchronize()
                assert th.equal(x_g, x_e), s
                assert th.equal(lg_g, lg_e), s
                assert th.equal(am_g, am_e), s
                assert pos_g.item() == pos_e.item() == L0 + s + 1
        th.cuda.synchronize()
        assert th.equal(pool_g, pool_e)
        assert T.ttsbb_sync(m.ctx) == T.OK
    finally:
        th.cuda.synchronize()
        m.close()
