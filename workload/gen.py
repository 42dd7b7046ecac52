"""Seeded synthetic inputs and weights.

Everything is drawn with NumPy from ``SeedSequence(entropy=1000 + config
index, spawn_key=(tag, ...))`` so any slice can be regenerated independently,
and is rounded once to bfloat16 (round to nearest, ties to even) where the
tensor is stored in bfloat16.  bfloat16 tensors are returned as ``uint16``
arrays holding the raw bit patterns.

Input recipe (stand-ins for the drafter outputs the pages' workloads feed the
corrector; no dataset record or trained weight is used):

* logits, "zipf": per (request, slot) a random permutation gives each token a
  rank 1..V; logit = -s * ln(rank) + Gumbel(0, 1), with the Zipf exponent s
  chosen by the request's entropy tier (request i of n gets tier
  floor(T * i / n) of T tiers).
* logits, "planted": N(0, 2) noise with three distinct planted peaks per slot
  at 8, 7, 6 (or 8, 7, 7 with ``ties=True``).
* hidden states ~ N(0, hidden_std), embedding table ~ N(0, embed_std).
* projection and MLP matrices ~ N(0, weight_std) (bfloat16); gamma = 1 +
  N(0, weight_std); beta, b1, w2, b2 ~ N(0, weight_std) (float32).
  ``head="zero"`` sets w2 = b2 = 0 (the zero-initialised output layer);
  ``head="stress"`` draws w2 ~ N(0, 1) so the walk leaves rank 0 often.
* the anchor position (row 0 of every block) holds a large constant so that
  any read of it shows up in the results.
"""

from __future__ import annotations

import numpy as np

from .configs import config as _config

TAG_LOGITS = 1
TAG_HIDDEN = 2
TAG_EMBED = 3
TAG_WEIGHTS = 4
TAG_TARGETS = 5
TAG_PLANT = 6

ANCHOR_VALUE = 64.0
EMBED_BLOCK = 4096


def _rng(cfg: dict, *key: int) -> np.random.Generator:
    base = int(cfg.get("seed_index", cfg["index"]))
    ss = np.random.SeedSequence(entropy=1000 + base + 100 * int(cfg.get("seed", 0)),
                                spawn_key=tuple(int(k) for k in key))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _resolve(cfg) -> dict:
    if isinstance(cfg, str):
        return _config(cfg)
    return cfg


def tier_of(cfg: dict, request: int) -> float:
    tiers = cfg["tiers"]
    return float(tiers[(len(tiers) * request) // cfg["n"]])


def gen_logits(cfg, ties: bool = False, threads: int = 8) -> np.ndarray:
    """Logits laid out [n][B+1][V]; row 0 of each block is the anchor."""
    cfg = _resolve(cfg)
    n, B, V = cfg["n"], cfg["B"], cfg["V"]
    if cfg["logits"] == "planted":
        out = np.empty((n, B + 1, V), dtype=np.float32)
        out[:, 0, :] = ANCHOR_VALUE
        for i in range(n):
            g = _rng(cfg, TAG_LOGITS, i)
            p = _rng(cfg, TAG_PLANT, i)
            for s in range(1, B + 1):
                row = g.normal(0.0, 2.0, size=V).astype(np.float32)
                peaks = p.choice(V, size=3, replace=False)
                row[peaks] = (8.0, 7.0, 7.0) if ties else (8.0, 7.0, 6.0)
                out[i, s] = row
        if cfg["logits_dtype"] == "bf16":
            return f32_to_bf16_bits(out).reshape(out.shape)
        return out
    assert cfg["logits"] == "zipf"
    from concurrent.futures import ThreadPoolExecutor

    out = np.empty((n, B + 1, V), dtype=np.uint16)
    out[:, 0, :] = f32_to_bf16_bits(np.array([ANCHOR_VALUE], np.float32))[0]
    lnrank = np.log(np.arange(1, V + 1, dtype=np.float64))

    def one_request(i: int) -> None:
        s_exp = tier_of(cfg, i)
        g = _rng(cfg, TAG_LOGITS, i)
        for s in range(1, B + 1):
            perm = g.permutation(V)          # token v gets rank perm[v] + 1
            gum = g.gumbel(size=V)
            row = (-s_exp * lnrank[perm] + gum).astype(np.float32)
            out[i, s] = f32_to_bf16_bits(row)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one_request, range(n)))
    if cfg["logits_dtype"] == "f32":
        return bf16_bits_to_f32(out).reshape(out.shape)
    return out


def gen_hidden(cfg) -> np.ndarray:
    """Drafter hidden states [n][B+1][d] as bfloat16 bits; row 0 is the anchor."""
    cfg = _resolve(cfg)
    n, B, d = cfg["n"], cfg["B"], cfg["d"]
    out = np.empty((n, B + 1, d), dtype=np.uint16)
    out[:, 0, :] = f32_to_bf16_bits(np.array([ANCHOR_VALUE], np.float32))[0]
    for i in range(n):
        g = _rng(cfg, TAG_HIDDEN, i)
        x = g.standard_normal(size=(B, d), dtype=np.float32) * np.float32(cfg["hidden_std"])
        out[i, 1:] = f32_to_bf16_bits(x).reshape(B, d)
    return out


def _embed_block(cfg: dict, blk: int, out: np.ndarray) -> None:
    g = _rng(cfg, TAG_EMBED, blk)
    x = g.standard_normal(size=out.shape, dtype=np.float32)
    x *= np.float32(cfg["embed_std"])
    out[...] = f32_to_bf16_bits(x).reshape(out.shape)


def gen_embed_rows(cfg, first: int, count: int) -> np.ndarray:
    """Rows [first, first+count) of the embedding table as bfloat16 bits."""
    cfg = _resolve(cfg)
    de, V = cfg["de"], cfg["V"]
    out = np.empty((count, de), dtype=np.uint16)
    pos = first
    while pos < first + count:
        blk = pos // EMBED_BLOCK
        b0 = blk * EMBED_BLOCK
        b1 = min(b0 + EMBED_BLOCK, V)
        tmp = np.empty((b1 - b0, de), dtype=np.uint16)
        _embed_block(cfg, blk, tmp)
        lo, hi = pos, min(first + count, b1)
        out[lo - first:hi - first] = tmp[lo - b0:hi - b0]
        pos = hi
    return out


def gen_embed(cfg, threads: int = 8) -> np.ndarray:
    """The frozen token-embedding table [V][de] as bfloat16 bits.

    Blocks of rows are independent streams, so they are filled in parallel
    threads (NumPy releases the GIL while generating).
    """
    from concurrent.futures import ThreadPoolExecutor

    cfg = _resolve(cfg)
    V, de = cfg["V"], cfg["de"]
    out = np.empty((V, de), dtype=np.uint16)
    nblk = (V + EMBED_BLOCK - 1) // EMBED_BLOCK
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda b: _embed_block(cfg, b, out[b * EMBED_BLOCK:min((b + 1) * EMBED_BLOCK, V)]),
                    range(nblk)))
    return out


def gen_weights(cfg, head: str = "normal") -> dict:
    """Corrector weights.  Matrices are bfloat16 bits in [out][in] layout."""
    cfg = _resolve(cfg)
    d, de, r, h, dv = cfg["d"], cfg["de"], cfg["r"], cfg["h"], cfg["dvec"]
    sw = np.float32(cfg["weight_std"])
    shapes = [
        ("w_cand", (r, de)), ("w_ctx", (r, d)), ("w_fuse", (r, 2 * r)),
        ("w_pair", (r, 2 * d)), ("w1", (h, 3 * r + 2)),
        ("w_out", (dv, r)), ("w_in", (dv, r)),
    ]
    w = {}
    for t, (name, shp) in enumerate(shapes):
        g = _rng(cfg, TAG_WEIGHTS, t)
        w[name] = f32_to_bf16_bits(g.standard_normal(size=shp, dtype=np.float32) * sw).reshape(shp)
    vecs = [("ln_gamma", r), ("ln_beta", r), ("b1", h), ("w2", h), ("b2", 1)]
    for t, (name, m) in enumerate(vecs):
        g = _rng(cfg, TAG_WEIGHTS, 100 + t)
        w[name] = (g.standard_normal(size=m, dtype=np.float32) * sw).astype(np.float32)
    w["ln_gamma"] = (w["ln_gamma"] + np.float32(1.0)).astype(np.float32)
    if head == "zero":
        w["w2"] = np.zeros(h, np.float32)
        w["b2"] = np.zeros(1, np.float32)
    elif head == "stress":
        g = _rng(cfg, TAG_WEIGHTS, 200)
        w["w2"] = g.standard_normal(size=h, dtype=np.float32)
    else:
        assert head == "normal", head
    return w


def gen_targets(cfg, p_top: float = 0.6, p_other: float = 0.3) -> np.ndarray:
    """Synthetic greedy-verifier targets as candidate ranks, [n][B] int32.

    Per slot: rank 0 with probability p_top, another candidate rank (uniform
    over 1..K-1) with probability p_other, and -1 (a token outside the
    candidate pool) otherwise.
    """
    cfg = _resolve(cfg)
    n, B, K = cfg["n"], cfg["B"], cfg["K"]
    g = _rng(cfg, TAG_TARGETS, 0)
    u = g.random(size=(n, B))
    other = g.integers(1, max(K, 2), size=(n, B))
    codes = np.where(u < p_top, 0, np.where(u < p_top + p_other, other, -1))
    if K == 1:
        codes = np.where(codes > 0, -1, codes)
    return codes.astype(np.int32)


def gen_inputs(cfg, head: str = "normal", ties: bool = False, embed: bool = True) -> dict:
    """All inputs of one pass: logits, hidden, embedding table and weights."""
    cfg = _resolve(cfg)
    out = dict(cfg=cfg, logits=gen_logits(cfg, ties=ties), hidden=gen_hidden(cfg),
               weights=gen_weights(cfg, head=head))
    if embed:
        out["embed"] = gen_embed(cfg)
    return out
