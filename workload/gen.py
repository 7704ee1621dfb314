"""Seeded input generator.

Everything is drawn from one torch.Generator per call on the target device,
so a given (config, seed, device) always yields the same tensors. All keys
and queries are drawn directly in the post-RoPE frame (an isotropic normal is
rotation invariant, so this is the same distribution as rotating pre-RoPE
draws); planted structure is written in that frame too.

Layouts (T = sum of sequence lengths, tokens of all sequences concatenated):
  K, V       [Ly][H][T][d]              cached keys / values
  Qp         [S][Ly][H*G][P][d]         probe queries (question / tail probes)
  Qctx       [Ly][H*G][T][d]            prefill queries of every cached token
  hidden     [T][hidden_dim]            sampled hidden states (DP slots only);
             [n_depth][T][hidden_dim]   with several sampled depths
  surprisal  [T] fp32                   per-token surprisal (optional)
  Qd         [T_dec][S][Ly][H*G][d]     decode queries
  Kd, Vd     [Ly][H][S][T_dec][d]       decode-time appended keys / values
  W          [vocab][H*G*d]             seeded vocab projection
"""
from __future__ import annotations

import math
from typing import Dict, List

import numpy as np
import torch

from .configs import Config

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def _align(k: torch.Tensor, target: torch.Tensor, cosine: float = 0.8) -> torch.Tensor:
    """Return vectors with the norm of ``k`` at the given cosine to ``target``.

    k: [..., n, d]; target: [..., d] (broadcast over n). The orthogonal part of
    ``k`` supplies the remaining direction.
    """
    u = _unit(target).unsqueeze(-2)
    kn = k.norm(dim=-1, keepdim=True)
    perp = k - (k * u).sum(-1, keepdim=True) * u
    perp = _unit(perp)
    s = math.sqrt(max(0.0, 1.0 - cosine * cosine))
    return kn * (cosine * u + s * perp)


def _spans(gen: torch.Generator, L: int, n: int, lo: int, hi: int) -> List[tuple]:
    """n non-overlapping spans with lengths U{lo..hi} at random positions in [0, L)."""
    lens = torch.randint(lo, hi + 1, (n,), generator=gen).tolist()
    while sum(lens) > L and n > 0:
        n -= 1
        lens = lens[:n]
    free = L - sum(lens)
    gaps = torch.sort(torch.randint(0, free + 1, (n,), generator=gen)).values.tolist()
    out, used = [], 0
    for k in range(n):
        start = gaps[k] + used
        out.append((start, lens[k]))
        used += lens[k]
    return out


def make_inputs(cfg: Config, device: str = "cpu", seed: int | None = None,
                with_qctx: bool = True) -> Dict[str, object]:
    seed = cfg.seed if seed is None else seed
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    hgen = torch.Generator()  # small host-side draws (positions, choices)
    hgen.manual_seed(seed + 7919)

    S, Ly, H, G, d, P = cfg.S, cfg.Ly, cfg.H, cfg.G, cfg.d, cfg.P
    T = cfg.T
    dt = _DT[cfg.dtype]
    cu = [0]
    for L in cfg.lens:
        cu.append(cu[-1] + int(L))
    cu_t = torch.tensor(cu, dtype=torch.int64)

    # Draw in fp32, plant, then store in the workload dtype.
    K = torch.randn((Ly, H, T, d), generator=gen, device=dev, dtype=torch.float32)
    V = torch.randn((Ly, H, T, d), generator=gen, device=dev, dtype=torch.float32)
    Qp = torch.randn((S, Ly, H * G, P, d), generator=gen, device=dev, dtype=torch.float32)
    scales = np.ones(Ly, dtype=np.float64)
    if cfg.layer_scale:
        u = torch.rand((Ly,), generator=hgen, dtype=torch.float64).numpy()
        scales = 2.0 ** (2.0 * u - 1.0)

    Qctx = None
    if with_qctx:
        Qctx = torch.randn((Ly, H * G, T, d), generator=gen, device=dev, dtype=torch.float32)

    planted: List[List[List[int]]] = [[[] for _ in range(Ly * H)] for _ in range(S)]

    for s in range(S):
        L = cfg.lens[s]
        base = cu[s]
        if cfg.plant == "evidence":
            # single tokens at distinct positions; token e follows probe row
            # (g = e mod G, p = e mod P) in every (layer, head)
            pos = torch.randperm(L, generator=hgen)[: cfg.n_plant].tolist()
            for e, i in enumerate(pos):
                g, p = e % G, e % P
                tgt = Qp[s, :, torch.arange(H) * G + g, p, :]          # [Ly, H, d]
                K[:, :, base + i: base + i + 1, :] = _align(K[:, :, base + i: base + i + 1, :], tgt)
                for uh in range(Ly * H):
                    planted[s][uh].append(i)
        elif cfg.plant == "spans":
            for (st, n) in _spans(hgen, L, cfg.n_plant, cfg.span_len[0], cfg.span_len[1]):
                g = torch.randint(0, G, (Ly, H), generator=hgen)
                p = torch.randint(0, P, (Ly, H), generator=hgen)
                mask = torch.rand((Ly, H), generator=hgen) < 0.5
                rows = (torch.arange(H).view(1, H) * G + g)                 # [Ly, H]
                tgt = Qp[s, torch.arange(Ly).view(Ly, 1), rows.to(dev), p.to(dev), :]  # [Ly,H,d]
                blk = K[:, :, base + st: base + st + n, :]
                new = _align(blk, tgt)
                m = mask.to(dev).view(Ly, H, 1, 1)
                K[:, :, base + st: base + st + n, :] = torch.where(m, new, blk)
                for l in range(Ly):
                    for h in range(H):
                        if bool(mask[l, h]):
                            planted[s][l * H + h].extend(range(st, st + n))
        elif cfg.plant == "chains":
            # question probe -> bridge span -> answer span; the answer precedes
            # its bridge so that causal prefill attention can carry relevance
            # from the bridge back to the answer.
            for _ in range(cfg.n_plant):
                lo, hi = cfg.span_len
                nb = int(torch.randint(lo, hi + 1, (1,), generator=hgen))
                na = int(torch.randint(lo, hi + 1, (1,), generator=hgen))
                a0 = int(torch.randint(0, max(1, L // 2 - na), (1,), generator=hgen))
                b0 = int(torch.randint(a0 + na, max(a0 + na + 1, L - nb), (1,), generator=hgen))
                g = torch.randint(0, G, (Ly, H), generator=hgen)
                p = torch.randint(0, P, (Ly, H), generator=hgen)
                rows = (torch.arange(H).view(1, H) * G + g)
                tgt = Qp[s, torch.arange(Ly).view(Ly, 1), rows.to(dev), p.to(dev), :]
                K[:, :, base + b0: base + b0 + nb, :] = _align(K[:, :, base + b0: base + b0 + nb, :], tgt)
                ans = torch.randn((Ly, H, d), generator=gen, device=dev)
                K[:, :, base + a0: base + a0 + na, :] = _align(K[:, :, base + a0: base + a0 + na, :], ans)
                if Qctx is not None:
                    qa = ans.repeat_interleave(G, dim=1)                      # [Ly, H*G, d]
                    Qctx[:, :, base + b0: base + b0 + nb, :] = _align(
                        Qctx[:, :, base + b0: base + b0 + nb, :], qa)
                for uh in range(Ly * H):
                    planted[s][uh].extend(list(range(a0, a0 + na)) + list(range(b0, b0 + nb)))
        else:
            raise ValueError(cfg.plant)

    if cfg.layer_scale:
        sc = torch.tensor(scales, dtype=torch.float32, device=dev).view(Ly, 1, 1, 1)
        K = K * sc
        V = V * sc

    hidden = None
    turns = []          # (global start, length) of every trajectory segment
    if cfg.hidden_dim > 0:
        Dh = cfg.hidden_dim
        hidden = torch.empty((T, Dh), dtype=torch.float32, device=dev)
        for s in range(S):
            L = cfg.lens[s]
            i = 0
            while i < L:
                n = int(torch.randint(16, 113, (1,), generator=hgen))
                n = min(n, L - i)
                turns.append((cu[s] + i, n))
                c = _unit(torch.randn((Dh,), generator=gen, device=dev))
                u = _unit(torch.randn((Dh,), generator=gen, device=dev))
                t = torch.arange(n, device=dev, dtype=torch.float32).view(n, 1) / max(n, 1)
                noise = torch.randn((n, Dh), generator=gen, device=dev) * (0.002 / math.sqrt(Dh))
                hidden[cu[s] + i: cu[s] + i + n] = c.view(1, Dh) + 0.5 * t * u.view(1, Dh) + noise
                i += n
        hidden = hidden.to(dt)

    Td = cfg.T_dec
    Qd = torch.randn((Td, S, Ly, H * G, d), generator=gen, device=dev, dtype=torch.float32)
    # Half of the decode queries aim (cosine 0.8) at a planted key of their head.
    aim = torch.rand((Td, S, Ly, H * G), generator=hgen) < 0.5
    for s in range(S):
        for l in range(Ly):
            for h in range(H):
                pl = planted[s][l * H + h]
                if not pl:
                    continue
                for g in range(G):
                    ts = [t for t in range(Td) if bool(aim[t, s, l, h * G + g])]
                    if not ts:
                        continue
                    pick = torch.randint(0, len(pl), (len(ts),), generator=hgen).tolist()
                    idx = torch.tensor([cu[s] + pl[k] for k in pick], device=dev)
                    tgt = K[l, h, idx, :]                                   # [n, d]
                    tt = torch.tensor(ts, device=dev)
                    q = Qd[tt, s, l, h * G + g, :].unsqueeze(-2)           # [n,1,d]
                    Qd[tt, s, l, h * G + g, :] = _align(q, tgt).squeeze(-2)
    Kd = torch.randn((Ly, H, S, Td, d), generator=gen, device=dev, dtype=torch.float32)
    Vd = torch.randn((Ly, H, S, Td, d), generator=gen, device=dev, dtype=torch.float32)
    if cfg.layer_scale:
        sc = torch.tensor(scales, dtype=torch.float32, device=dev).view(Ly, 1, 1, 1, 1)
        Kd = Kd * sc
        Vd = Vd * sc

    Dm = cfg.d_model
    W = torch.randn((cfg.vocab, Dm), generator=gen, device=dev, dtype=torch.float32)
    W = (W * (cfg.logit_tau / math.sqrt(Dm))).to(_DT[cfg.w_dtype])

    # Extra sampled depths and the surprisal come from generators of their
    # own, after every other draw, so the single-depth inputs do not change.
    # Every depth turns at the same positions with its own directions.
    if hidden is not None and cfg.n_depth > 1:
        g2 = torch.Generator(device=dev)
        g2.manual_seed(seed + 7919)
        Dh = cfg.hidden_dim
        layers = [hidden]
        for _ in range(cfg.n_depth - 1):
            hd = torch.empty((T, Dh), dtype=torch.float32, device=dev)
            for (a0, n) in turns:
                c = _unit(torch.randn((Dh,), generator=g2, device=dev))
                u = _unit(torch.randn((Dh,), generator=g2, device=dev))
                t = torch.arange(n, device=dev, dtype=torch.float32).view(n, 1) / max(n, 1)
                noise = torch.randn((n, Dh), generator=g2, device=dev) * (0.002 / math.sqrt(Dh))
                hd[a0:a0 + n] = c.view(1, Dh) + 0.5 * t * u.view(1, Dh) + noise
            layers.append(hd.to(dt))
        hidden = torch.stack(layers, 0)
    surprisal = None
    if cfg.surprisal:
        g3 = torch.Generator()
        g3.manual_seed(seed + 104729)
        sur = -torch.log(torch.rand((T,), generator=g3, dtype=torch.float64).clamp_min(1e-12))
        for (a0, n) in turns:
            sur[a0] += 2.0
        surprisal = sur.float().to(dev)

    out = {
        "cu_seqlens": cu_t,
        "K": K.to(dt).contiguous(),
        "V": V.to(dt).contiguous(),
        "Qp": Qp.to(dt).contiguous(),
        "Qctx": None if Qctx is None else Qctx.to(dt).contiguous(),
        "hidden": hidden,
        "surprisal": surprisal,
        "Qd": Qd.to(dt).contiguous(),
        "Kd": Kd.to(dt).contiguous(),
        "Vd": Vd.to(dt).contiguous(),
        "W": W.contiguous(),
        "layer_scale": scales,
        "planted": planted,
    }
    return out


def make_policy(seed: int = 7, hidden: int = 128, device: str = "cpu") -> Dict[str, torch.Tensor]:
    """Seeded weights of the scoring MLP of step-wise eviction (5 features ->
    hidden -> hidden -> 1, a LayerNorm scale and shift after each hidden
    layer). No trained policy exists here: the weights are random draws with
    fan-in scaling, fp32."""
    g = torch.Generator().manual_seed(seed)

    def rnd(*shape, scale=1.0):
        return (torch.randn(shape, generator=g, dtype=torch.float64) * scale).float()

    p = {
        "w1": rnd(hidden, 5, scale=1.0 / math.sqrt(5)), "b1": rnd(hidden, scale=0.1),
        "g1": 1.0 + rnd(hidden, scale=0.1), "be1": rnd(hidden, scale=0.1),
        "w2": rnd(hidden, hidden, scale=1.0 / math.sqrt(hidden)), "b2": rnd(hidden, scale=0.1),
        "g2": 1.0 + rnd(hidden, scale=0.1), "be2": rnd(hidden, scale=0.1),
        "w3": rnd(hidden, scale=1.0 / math.sqrt(hidden)), "b3": rnd(1, scale=0.1),
    }
    return {k: v.contiguous().to(device) for k, v in p.items()}
