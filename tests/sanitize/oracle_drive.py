"""Drives every oracle entry point on small seeded inputs; run in a child
process with the oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (DRAFT_ORACLE_LIB names that build).  It checks
nothing numerically (the pins do that): a memory or undefined-behaviour error
aborts the process with the sanitizer's report."""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workload import config, gen_inputs, gen_targets  # noqa: E402


def main():
    assert os.environ.get("DRAFT_ORACLE_LIB"), "run through tests/test_sanitizers.py"
    oracle.set_threads(2)
    for name, kw, heads in (("tiny", {}, ("normal", "zero", "stress")),
                            ("tiny", dict(variant="cosine", sigma=8.0), ("normal",)),
                            ("tiny", dict(n=3, B=7, K=5, V=257, succ_top_m=2), ("stress",)),
                            ("tiny", dict(n=2, B=1), ("normal",)),
                            ("tiny", dict(n=2, B=5, K=7, logits_dtype="bf16", logits="zipf", V=997), ("stress",))):
        cfg = config(name, **kw)
        for head in heads:
            for ties in (False, True):
                x = gen_inputs(cfg, head=head, ties=ties and cfg["logits"] == "planted")
                r = oracle.run(cfg, x)
                desc = oracle.OracleDesc.from_config(cfg)
                n, B, V = cfg["n"], cfg["B"], cfg["V"]
                oracle.viterbi(desc, r["scores"], r["ids"], n)
                oracle.viterbi(desc, r["scores"], r["ids"], n, lam=0.75)
                for w in (1, 2, 4):
                    oracle.beam(desc, r["scores"].astype(np.float32), r["ids"], n, w)
                logz = oracle.log_normaliser(desc, x["logits"], n, (B + 1) * V, V, offset=V)
                oracle.confidence(r["vals"], logz)
                codes = gen_targets(cfg)
                targets = np.where(codes >= 0, np.take_along_axis(
                    r["ids"], np.maximum(codes, 0)[..., None], 2)[..., 0], -1)
                oracle.accepted_lengths(r["tokens"], targets)
    row = np.array([3.0, -0.0, 0.0, -np.inf, 3.0, 1.0], np.float32)
    for K in range(1, row.size + 1):
        oracle.topk_row(row, K)
    oracle.log_normaliser_row(row)
    oracle.layernorm(np.arange(16.0), 1e-5)
    oracle.layernorm(np.arange(16.0), 1e-5, np.ones(16, np.float32), np.zeros(16, np.float32))
    for t in (-9.0, -1.0, 0.0, 0.5, 12.0):
        oracle.gelu(t)
    oracle.accepted_lengths(np.zeros((0, 4), np.int32), np.zeros((0, 4), np.int32))
    oracle.accepted_lengths(np.zeros((2, 0), np.int32), np.zeros((2, 0), np.int32))
    print("oracle driven under sanitizers", flush=True)


if __name__ == "__main__":
    main()
