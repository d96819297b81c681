"""The oracle's collective stand-ins against torch.distributed's own
collectives, with real processes on the CPU (gloo), the technique of the
check script in "Tensor and sequence parallelism" ("The implementation"):
every rank generates the same full tensors, computes its own shard, and the
ranks' results are combined by all_reduce / reduce_scatter / all_gather.

Pinned here (the library's collectives are an independent implementation of
the same sums and concatenations):
* reduce_partials (the g-forward / f-backward all-reduce) = all_reduce of the
  ranks' shard outputs;
* reduce_scatter and all_gather (the sequence-parallel boundary) =
  reduce_scatter_tensor and all_gather_into_tensor;
* sum_shared_grads (the LayerNorm weight's extra all-reduce) = all_reduce of
  the ranks' dgamma;
* the whole TP + SP block of that script in float64 over world sizes 2 and 4.
CPU only, 127.0.0.1 rendezvous.
"""
from __future__ import annotations

import os
import socket

import numpy as np
import pytest

torch = pytest.importorskip("torch")
dist = pytest.importorskip("torch.distributed")
mp = pytest.importorskip("torch.multiprocessing")


def _free_port() -> int:
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _worker(rank: int, world: int, port: int, errs):
    try:
        os.environ["MASTER_ADDR"] = "127.0.0.1"
        os.environ["MASTER_PORT"] = str(port)
        dist.init_process_group("gloo", rank=rank, world_size=world)
        import oracle
        from oracle import ln

        t = world
        rng = np.random.default_rng(123)       # every rank draws the same full tensors
        N, h, F = 4 * t, 16, 8 * t
        x = rng.standard_normal((N, h))
        gamma = rng.standard_normal(h)
        W1 = rng.standard_normal((h, F)) / 4
        W2 = rng.standard_normal((F, h)) / 6
        b2 = rng.standard_normal(h)
        dout = rng.standard_normal((N, h))
        c = oracle.column_block(rank, t, F)
        blk = oracle.sequence_block(rank, t, N)

        # --- TP: the g operator's all-reduce of the partial sums
        X = ln.layer_norm_forward(x, gamma)[0]
        parts = [oracle.shard_forward("gelu", X, W1[:, oracle.column_block(r, t, F)],
                                      W2[oracle.column_block(r, t, F), :])["Y"] for r in range(t)]
        Yr = torch.from_numpy(parts[rank].copy())
        dist.all_reduce(Yr)
        want = oracle.reduce_partials(parts)
        np.testing.assert_allclose(Yr.numpy(), want, rtol=1e-12, atol=1e-12)
        # the bias goes in once, after the sum
        np.testing.assert_allclose(Yr.numpy() + b2, oracle.reduce_partials(parts, b2), rtol=1e-12, atol=1e-12)

        # --- SP: reduce-scatter and all-gather along the token rows
        out = torch.empty(N // t, h, dtype=torch.float64)
        dist.reduce_scatter_tensor(out, torch.from_numpy(parts[rank].copy()))
        np.testing.assert_allclose(out.numpy(), oracle.reduce_scatter(parts, rank), rtol=1e-12, atol=1e-12)
        full = torch.empty(N, h, dtype=torch.float64)
        mine = ln.layer_norm_forward(x[blk], gamma)[0]
        dist.all_gather_into_tensor(full, torch.from_numpy(mine.copy()))
        blocks = [ln.layer_norm_forward(x[oracle.sequence_block(r, t, N)], gamma)[0] for r in range(t)]
        np.testing.assert_array_equal(full.numpy(), oracle.all_gather(blocks))

        # --- the whole TP + SP block, and the LayerNorm weight's all-reduce
        outs, _ = ln.sp_block_forward("gelu", x, gamma, W1, W2, t)
        bw = ln.sp_block_backward("gelu", x, gamma, W1, W2, [dout[oracle.sequence_block(r, t, N)] for r in range(t)], t)
        # this rank's pieces by the shard functions and the collectives alone
        Xg = full.numpy()
        Y_i = oracle.shard_forward("gelu", Xg, W1[:, c], W2[c, :])["Y"]
        o = torch.empty(N // t, h, dtype=torch.float64)
        dist.reduce_scatter_tensor(o, torch.from_numpy(Y_i.copy()))
        np.testing.assert_allclose(o.numpy(), outs[rank], rtol=1e-11, atol=1e-12)
        dY = torch.empty(N, h, dtype=torch.float64)
        dist.all_gather_into_tensor(dY, torch.from_numpy(dout[blk].copy()))
        dX_i = oracle.shard_backward("gelu", Xg, W1[:, c], W2[c, :], dY.numpy())["dX"]
        dln = torch.empty(N // t, h, dtype=torch.float64)
        dist.reduce_scatter_tensor(dln, torch.from_numpy(dX_i.copy()))
        dx, dg, _ = ln.layer_norm_backward(dln.numpy(), x[blk], gamma)
        np.testing.assert_allclose(dx, bw["dx"][rank], rtol=1e-10, atol=1e-11)
        dgt = torch.from_numpy(dg.copy())
        dist.all_reduce(dgt)
        np.testing.assert_allclose(dgt.numpy(), bw["dgamma"], rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(dgt.numpy(), ln.sum_shared_grads(bw["dgamma_r"]), rtol=1e-10, atol=1e-11)
        dist.destroy_process_group()
    except Exception as e:  # reported to the parent
        errs.put(f"rank {rank}: {type(e).__name__}: {e}")
        raise


@pytest.mark.parametrize("world", [2, 4])
def test_oracle_collectives_match_torch_distributed(world):
    ctx = mp.get_context("spawn")
    errs = ctx.Queue()
    port = _free_port()
    procs = [ctx.Process(target=_worker, args=(r, world, port, errs)) for r in range(world)]
    for p in procs:
        p.start()
    for p in procs:
        p.join(timeout=240)
    alive = [p for p in procs if p.is_alive()]
    for p in alive:
        p.kill()
    msgs = []
    while not errs.empty():
        msgs.append(errs.get())
    assert not alive, "a rank did not finish"
    assert not msgs and all(p.exitcode == 0 for p in procs), msgs or [p.exitcode for p in procs]
