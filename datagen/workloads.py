"""The synthetic workloads: LLaMA-3.1-8B-shaped attention layers at 1K-128K.

They stand in for the LLaMA-3.1-8B / PG-19 / NIAH / RULER evaluation of the
page "Runtime-Certified Bounded-Error Quantized Attention" (Results), which
needs a trained model and datasets.  Every tensor is drawn from the
counter-based generator in dg.c with a seed that depends only on
(config id, layer), so any layer can be produced on its own.

Planting: "+k sigma" raises the group-mean score of every token of a block
by k standard deviations of that kv-head group's bulk scores.  The shift is
added along u = mean of the group's query vectors (normalised); with the
analytic score variance sigma_h^2 = sm^2 q_h' Cov(k) q_h pooled over the
group, the amplitude is a = k * sigma / (sm * |mean q|).
"""
import math
from dataclasses import dataclass, field

import numpy as np

from . import keys, normal, to_f16, uniform, values

# The five workloads.  Sizes and distributions follow the config list of the
# build's target; readings of unstated magnitudes are noted per entry.
CONFIGS = {
    # 1: tiny single layer; "one planted block with keys = 0.5 q-direction"
    #    read as one block at +4 sigma along the group query direction.
    "tiny_1k": dict(cid=1, L=1, B=1, Hq=8, Hkv=2, d=64, T=1024, n_out=4, out_scale=8.0,
                    q_std=1.0, sm=0.125, random=(1, 4.0)),
    # 2: 8K, 3 planted blocks per kv head (magnitude unstated: +4 sigma).
    "llama_8k": dict(cid=2, L=32, B=1, Hq=32, Hkv=8, d=128, T=8192, n_out=6, out_scale=10.0,
                     q_std=1 / math.sqrt(128), sm=1.0, random=(3, 4.0)),
    # 3: 32K x 4, plus a sink block 0 at +4 sigma and the last 2 blocks at +2 sigma.
    "llama_32k": dict(cid=3, L=32, B=4, Hq=32, Hkv=8, d=128, T=32768, n_out=6, out_scale=10.0,
                      q_std=1 / math.sqrt(128), sm=1.0, random=(3, 4.0), sink=4.0,
                      recent=(2, 2.0)),
    # 4: 64K / 128K needle: rank-16 keys (U ~ N(0,1), W ~ N(0,1)/4) + N(0, 0.3^2)
    #    noise + 5% outlier channels x10; one needle block at +6 sigma.
    "needle_64k": dict(cid=4, L=32, B=1, Hq=32, Hkv=8, d=128, T=65536, n_out=6, out_scale=10.0,
                       q_std=1 / math.sqrt(128), sm=1.0, rank=16, w_std=0.25, noise_std=0.3,
                       random=(1, 6.0)),
    "needle_128k": dict(cid=6, L=32, B=1, Hq=32, Hkv=8, d=128, T=131072, n_out=6,
                        out_scale=10.0, q_std=1 / math.sqrt(128), sm=1.0, rank=16, w_std=0.25,
                        noise_std=0.3, random=(1, 6.0)),
    # 5: fallback stress, 4 layers: near-flat attention (q x 0.05), blocks in
    #    near-tie pairs (odd block = even block + U(-1,1) * 0.004 * channel
    #    scale, below a quarter of a typical INT8 step), Student-t(3) values.
    #    Layers 0-2 are documented variants so that every rung occurs
    #    ("copies": every block of the kv group is block 0 + such a
    #    perturbation, so block masses are all near ties):
    #    0: q not flattened, one +6 sigma needle pair, V ~ 3 N(0,1)   -> rung 1
    #    1: kv groups 0-4 (20 of 32 q heads) flat copies, rest as 0   -> rung 3 -> 4
    #    2: kv group 0 (4 q heads) flat copies, rest as 0             -> rung 3
    #    3: as specified: adjacent blocks flip (D ~ 300 of 130K pairs)  -> rung 2
    "stress_32k": dict(cid=5, L=4, B=1, Hq=32, Hkv=8, d=128, T=32768, n_out=6, out_scale=10.0,
                       q_std=1 / math.sqrt(128), sm=1.0, tie_eps=0.004, v_nu=3,
                       flat_heads="all",
                       layer_variants={
                           0: dict(random=(1, 6.0), flat_heads=(), v_nu=0, v_scale=3.0),
                           1: dict(random=(1, 6.0), flat_heads=tuple(range(0, 20)),
                                   copies=(0, 1, 2, 3, 4), v_nu=0, v_scale=3.0),
                           2: dict(random=(1, 6.0), flat_heads=(0, 1, 2, 3), copies=(0,),
                                   v_nu=0, v_scale=3.0),
                           3: dict(),
                       }),
}


def seed_for(cid, layer, salt=0):
    x = (cid * 1000003 + layer * 7919 + salt * 104729 + 0x5EED) & ((1 << 64) - 1)
    x = (x * 0x9E3779B97F4A7C15) & ((1 << 64) - 1)
    return x ^ (x >> 29)


def h2f(a):
    return np.asarray(a, np.uint16).view(np.float16).astype(np.float64)


@dataclass
class Layer:
    name: str
    layer: int
    q: np.ndarray  # uint16 [B][Hq][d]
    k: np.ndarray  # uint16 [B][T][Hkv][d]
    v: np.ndarray  # uint16 [B][T][Hkv][d]
    sm: float
    info: dict = field(default_factory=dict)


def _distinct_blocks(seed, tag, count, nblocks, reserved):
    """`count` distinct block indices, uniform over [0, nblocks) minus `reserved`."""
    chosen = []
    i = 0
    while len(chosen) < count and i < 1000 * (count + 1):
        b = int(uniform(seed, tag, 1, start=i)[0] * nblocks)
        i += 1
        if b in reserved or b in chosen:
            continue
        chosen.append(b)
    return chosen


def make_layer(name, layer, B=None, T=None, Hq=None, Hkv=None):
    """Generate one layer of workload `name` (optionally with a smaller
    batch / context / head count for quick tests, same recipe otherwise)."""
    cfg = dict(CONFIGS[name])
    cfg.update(cfg.pop("layer_variants", {}).get(layer, {}))
    B = B or cfg["B"]
    T = T or cfg["T"]
    Hq = Hq or cfg["Hq"]
    Hkv = Hkv or cfg["Hkv"]
    d = cfg["d"]
    G = Hq // Hkv
    NB = (T + 63) // 64
    cid = cfg["cid"]
    seed = seed_for(cid, layer)
    sm = cfg["sm"]

    # queries
    qf = normal(seed, 30, B * Hq * d).reshape(B, Hq, d) * cfg["q_std"]
    flat = cfg.get("flat_heads", ())
    if flat == "all":
        flat = tuple(range(Hq))
    for h in flat:
        if h < Hq:
            qf[:, h, :] *= 0.05
    q = to_f16(qf)
    qd = h2f(q)

    # outlier channels per kv head, fixed per layer
    chan = np.ones((Hkv, d))
    for g in range(Hkv):
        u = uniform(seed, 31, d, start=g * d)
        chan[g, np.argsort(u, kind="stable")[: cfg["n_out"]]] = cfg["out_scale"]

    rank = cfg.get("rank", 0)
    W = None
    if rank:
        W = normal(seed, 32, Hkv * rank * d).reshape(Hkv, rank, d) * cfg["w_std"]
    noise = cfg.get("noise_std", 1.0)

    # analytic bulk score variance per head, pooled per group
    amp = np.zeros((B, Hkv, NB))
    direc = np.zeros((B, Hkv, d))
    plants = {}
    for n in range(B):
        for g in range(Hkv):
            qs = qd[n, g * G:(g + 1) * G, :]
            oq = qs * chan[g][None, :]
            var = noise ** 2 * np.sum(oq ** 2, axis=1)
            if rank:
                var = var + np.sum((oq @ W[g].T) ** 2, axis=1)
            sigma = sm * math.sqrt(float(np.mean(var)))
            qbar = qs.mean(axis=0)
            nq = float(np.linalg.norm(qbar))
            if nq == 0.0:
                continue
            direc[n, g] = qbar / nq
            unit = sigma / (sm * nq)
            reserved = set()
            if "sink" in cfg:
                amp[n, g, 0] = cfg["sink"] * unit
                reserved.add(0)
            if "recent" in cfg:
                cnt, ks = cfg["recent"]
                for b in range(max(0, NB - cnt), NB):
                    amp[n, g, b] = ks * unit
                    reserved.add(b)
            rb = []
            if "random" in cfg:
                cnt, ks = cfg["random"]
                rb = _distinct_blocks(seed, 40 + n * Hkv + g, cnt, NB, reserved)
                for b in rb:
                    amp[n, g, b] = ks * unit
            if cfg.get("tie_eps"):
                # planted blocks keep their near-tie partner at the same level
                for b in list(rb):
                    partner = b ^ 1
                    if partner < NB:
                        amp[n, g, partner] = amp[n, g, b]
            plants[(n, g)] = dict(sigma=sigma, random=rb)

    tie_mode = np.ones(Hkv, np.int32)
    for g in cfg.get("copies", ()):
        if g < Hkv:
            tie_mode[g] = 2
            amp[:, g, :] = 0.0
    k = keys(seed, B, T, Hkv, d, chan, amp, direc, rank=rank, W=W, noise_std=noise,
             tie_eps=cfg.get("tie_eps", 0.0), tie_mode=tie_mode)
    v = values(seed, B, T, Hkv, d, nu=cfg.get("v_nu", 0), scale=cfg.get("v_scale", 1.0))
    return Layer(name, layer, q, k, v, sm, dict(plants=plants, chan=chan, flat=flat))
