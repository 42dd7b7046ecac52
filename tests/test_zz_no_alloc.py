"""corrector_run_static, the entry point that allocates nothing (its
workspace is the library's static per-GPU array), against corrector_run with
a caller-allocated workspace: identical outputs, bit for bit, on calls in a
row whose request counts shrink (so a call after a larger one finds stale
data in the shared array), for both variants.  A request count whose
workspace exceeds the array is refused on the host."""

import numpy as np
import pytest
import torch

import parity as P
from draft_correction_amd import corrector as cr
from draft_correction_amd import device

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _static(corr, x, n, first):
    cfg = x["cfg"]
    dev = P.dev_inputs(x)
    st = device.strides(cfg)
    B, K = cfg["B"], cfg["K"]
    out = dict(tokens=torch.full((n, B), -7, dtype=torch.int32, device="cuda"),
               choice=torch.full((n, B), -7, dtype=torch.int32, device="cuda"),
               ids=torch.full((n, B, K), -7, dtype=torch.int32, device="cuda"),
               vals=torch.full((n, B, K), -7.0, dtype=torch.float32, device="cuda"),
               scores=torch.full((n, max(B - 1, 0), K, K), -7.0, dtype=torch.float32, device="cuda"))
    corr.run_static(n, dev["logits"], st["l_req"], st["l_slot"], dev["hidden"], st["h_req"], st["h_slot"],
                    out["tokens"], choice=out["choice"], ids=out["ids"], vals=out["vals"], scores=out["scores"],
                    l_offset=st["l_off"] + first * st["l_req"], h_offset=st["h_off"] + first * st["h_req"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("name,head", [("b32", "stress"), ("cosine", "normal")])
def test_run_static_matches_run(name, head):
    x = P.inputs(name, head=head) if name == "b32" else P.inputs(name, sigma=8.0)
    cfg = x["cfg"]
    corr = device.make_corrector(cfg, P.dev_inputs(x), max_requests=cfg["n"])
    for n, first in ((cfg["n"], 0), (5, 3), (1, 30)):
        _log("run_static %s n=%d first=%d" % (name, n, first))
        got = _static(corr, x, n, first)
        want = P.gpu_run(x, n=n, first=first)
        for k in got:
            np.testing.assert_array_equal(got[k], want[k], err_msg="%s n=%d: %s" % (name, n, k))
    corr.close()


def test_run_static_refuses_oversized_batches():
    _log("run_static oversized")
    x = P.inputs("tiny")
    cfg = dict(x["cfg"], n=4096, B=15, K=64, V=151936, d=4096, de=4096, r=128, h=256)
    corr = device.make_corrector(cfg, P.dev_inputs(x), max_requests=4096)
    assert corr.workspace_bytes(4096) > (64 << 20)
    t = torch.empty((4096, 15), dtype=torch.int32, device="cuda")
    with pytest.raises(cr.CorrectorError) as e:
        corr.run_static(4096, t, 0, 0, t, 0, 0, t)
    assert e.value.code == 5   # CORR_E_WORKSPACE, nothing launched
    corr.close()
