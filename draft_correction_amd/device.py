"""Move generated inputs to the device in the layout the library reads.

Marshalling only: bfloat16 tensors travel as their 16-bit patterns in int16
tensors, float32 tensors as float32; shapes and contents are unchanged.
"""

from __future__ import annotations

import numpy as np
import torch

from .corrector import Corrector

MATRICES = ("w_cand", "w_ctx", "w_fuse", "w_pair", "w1", "w_out", "w_in")
VECTORS = ("ln_gamma", "ln_beta", "b1", "w2", "b2")


def tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def weights_to_device(weights: dict, embed: np.ndarray, device="cuda") -> dict:
    out = {k: tensor(weights[k], device) for k in MATRICES if k in weights}
    out.update({k: tensor(weights[k].astype(np.float32), device) for k in VECTORS if k in weights})
    out["embed"] = tensor(embed, device)
    return out


def inputs_to_device(inputs: dict, device="cuda") -> dict:
    """logits [n][B+1][V], hidden [n][B+1][d] and all weights as device tensors."""
    return dict(logits=tensor(inputs["logits"], device), hidden=tensor(inputs["hidden"], device),
                weights=weights_to_device(inputs["weights"], inputs["embed"], device))


def make_corrector(cfg: dict, dev: dict, max_requests: int | None = None) -> Corrector:
    w = dict(dev["weights"])
    if cfg["variant"] == "mlp":
        w.pop("w_out", None)
        w.pop("w_in", None)
    return Corrector(cfg, w, max_requests or cfg["n"])


def strides(cfg: dict):
    """Element strides and offsets for the [n][B+1][*] block layout (anchor first)."""
    B1 = cfg["B"] + 1
    return dict(l_req=B1 * cfg["V"], l_slot=cfg["V"], l_off=cfg["V"],
                h_req=B1 * cfg["d"], h_slot=cfg["d"], h_off=cfg["d"])
