"""corrector_run captured into a graph.  Every call of the library enqueues
kernels only (no allocation, no synchronisation, no memset), so a pass can be
captured once and replayed with new inputs copied into the same buffers.
Each replay is compared bit for bit with an eager call on the same inputs;
replays alternate with eager work and synchronisations, and inputs change
between replays."""

import numpy as np
import pytest
import torch

import parity as P
from draft_correction_amd import device

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _outputs(n, B, K):
    mk = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")  # noqa: E731
    return dict(tokens=mk((n, B), torch.int32), choice=mk((n, B), torch.int32), ids=mk((n, B, K), torch.int32),
                vals=mk((n, B, K), torch.float32), scores=mk((n, max(B - 1, 0), K, K), torch.float32))


def _run(corr, cfg, n, logits, hidden, ws, out, stream=None):
    st = device.strides(cfg)
    corr.run(n, logits, st["l_req"], st["l_slot"], hidden, st["h_req"], st["h_slot"], out["tokens"], ws,
             choice=out["choice"], ids=out["ids"], vals=out["vals"], scores=out["scores"], l_offset=st["l_off"],
             h_offset=st["h_off"], stream=stream)


@pytest.mark.parametrize("name,n,fold", [("b32", 32, False), ("b32", 1, False), ("b32", 32, True),
                                         ("cosine", 32, False)])
def test_graph_replay_matches_eager(name, n, fold):
    _log("graph %s n=%d fold=%s" % (name, n, fold))
    x = P.inputs(name, head="stress") if name == "b32" else P.inputs(name, sigma=8.0)
    cfg = x["cfg"]
    dev = P.dev_inputs(x)
    B, K = cfg["B"], cfg["K"]
    corr = device.make_corrector(cfg, dev, max_requests=cfg["n"])
    if fold:
        table = torch.empty(corr.table_bytes() // 4, dtype=torch.float32, device="cuda")
        corr.fold_table(table)
        corr.use_table(table)
    # input sets of n requests: consecutive requests of the batch, rotated
    full_l, full_h = dev["logits"], dev["hidden"]
    sets = [(full_l.roll(-k, 0)[:n].contiguous(), full_h.roll(-k, 0)[:n].contiguous()) for k in (0, 5, 17, 0)]
    static_l, static_h = sets[0][0].clone(), sets[0][1].clone()
    ws = corr.new_workspace(n)
    out = _outputs(n, B, K)
    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(corr, cfg, n, static_l, static_h, ws, out, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run(corr, cfg, n, static_l, static_h, ws, out)
    torch.cuda.synchronize()
    ws_e = corr.new_workspace(n)
    ref = _outputs(n, B, K)
    for k, (lg, hd) in enumerate(sets):
        static_l.copy_(lg)
        static_h.copy_(hd)
        for o in out.values():
            o.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _run(corr, cfg, n, lg, hd, ws_e, ref)
        torch.cuda.synchronize()
        for key in out:
            np.testing.assert_array_equal(out[key].cpu().numpy(), ref[key].cpu().numpy(),
                                          err_msg="replay %d: %s" % (k, key))
    corr.close()
