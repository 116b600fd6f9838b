"""Seeded bulk inputs: hidden rows, expert scales and gradient slabs.

* hidden rows x ~ N(0, 1), stored as bf16 [T, H];
* the toy expert of the tiny workload: a per-expert fp32 scale s_e ~ U(0.5, 1.5);
* gradients ~ N(0, sigma=1e-3) fp32: home slabs [E, G_el] and replica slabs
  [R, slots, G_el].

Only random draws and dtype plumbing live here (bf16 tensors are handed to numpy as their
raw uint16 bit patterns); none of the balanced-EP arithmetic does.
"""

import numpy as np
import torch


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_hidden(T: int, H: int, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return torch.randn(T, H, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_scales(E: int, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return (0.5 + torch.rand(E, generator=g, device=device, dtype=torch.float32)).contiguous()


def make_grads(E: int, R: int, slots: int, G_el: int, seed: int, device="cpu", sigma=1e-3):
    g = _gen(seed, device)
    home = torch.randn(E, G_el, generator=g, device=device, dtype=torch.float32).mul_(sigma)
    rep = torch.randn(R, slots, G_el, generator=g, device=device,
                      dtype=torch.float32).mul_(sigma)
    return home, rep


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a bf16 tensor as a host uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_bf16(a: np.ndarray, device="cpu") -> torch.Tensor:
    """Host uint16 bit patterns -> bf16 tensor (bit copy)."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
