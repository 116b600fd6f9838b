"""Seeded synthetic top-K router output with a chosen imbalance (maxvio).

The pages benchmark on artificially skewed routing swept from maxvio 0.2 to 20
("Moonshot AI Open-Sources MoonEP", paragraph 4; "MoonshotAI/MoonEP deep dive",
section 8, exercise B, which names a routing generator but does not print it).  This
module stands in for that generator:

* per-expert popularity z_e ~ N(0, 1), per-(token, expert) noise g ~ Gumbel(0, 1);
* logit[t, e] = alpha * z_e + g[t, e]; a token's K experts are its K largest logits,
  largest first (Gumbel-top-K, i.e. sampling without replacement from p_e ~ exp(alpha z_e));
* weights = softmax over the K selected logits (the full softmax renormalised to top-K), fp32;
* alpha is bisected until the realised imbalance maxvio = max_e load_e / mean_e load_e - 1
  (mean = T*K/E) is within 1 % of the target (or the closest value found).

It draws random numbers and picks top-K; it holds none of the balanced-EP arithmetic
(no plan, no slot map, no dispatch or combine).  Everything runs in torch on the
requested device so large workloads are generated on the GPU in milliseconds.
"""

import torch


def realised_maxvio(ids: torch.Tensor, E: int) -> float:
    load = torch.bincount(ids.reshape(-1).long(), minlength=E).double()
    mean = ids.numel() / E
    return float(load.max().item() / mean - 1.0)


def _topk(logits: torch.Tensor, K: int):
    vals, idx = torch.topk(logits, K, dim=1, largest=True, sorted=True)
    return vals, idx


def make_routing(R: int, E: int, K: int, S: int, maxvio: float, seed: int,
                 device="cpu", iters: int = 60):
    """Return (ids int32 [T,K], w fp32 [T,K], alpha, achieved maxvio)."""
    if K > E:
        raise ValueError("K must not exceed E")
    T = R * S
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    z = torch.randn(E, generator=gen, device=device, dtype=torch.float32)
    u = torch.rand(T, E, generator=gen, device=device, dtype=torch.float32)
    u.clamp_(min=1e-12, max=1.0 - 1e-7)
    g = -torch.log(-torch.log(u))
    del u

    def at(alpha):
        logits = g + alpha * z
        vals, idx = _topk(logits, K)
        return vals, idx, realised_maxvio(idx, E)

    lo, hi = 0.0, 64.0
    best = None
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        vals, idx, mv = at(mid)
        if best is None or abs(mv - maxvio) < abs(best[2] - maxvio):
            best = (vals, idx, mv, mid)
        if abs(mv - maxvio) <= 0.01 * maxvio:
            break
        if mv < maxvio:
            lo = mid
        else:
            hi = mid
    vals, idx, mv, alpha = best
    w = torch.softmax(vals.float(), dim=1).contiguous()
    return idx.to(torch.int32).contiguous(), w, alpha, mv


def make_balanced_routing(R: int, E: int, K: int, S: int):
    """Perfectly balanced routing: assignment i goes to expert i mod E (needs T*K % E == 0
    for an exactly flat load).  Weights are uniform 1/K."""
    T = R * S
    i = torch.arange(T * K, dtype=torch.int64)
    ids = (i % E).to(torch.int32).reshape(T, K)
    w = torch.full((T, K), 1.0 / K, dtype=torch.float32)
    return ids, w
