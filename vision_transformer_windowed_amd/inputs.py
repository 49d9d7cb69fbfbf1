"""Seeded synthetic inputs for window attention (shared by tests, bench and the smoke check).

This module holds only random-number generation and the workload table; it
contains none of the attention arithmetic.  Recipe: a CPU torch.Generator
seeded with `seed` draws Q, K, V (then dO when asked for) ~ N(0, 1) in
float32; a second generator seeded with `seed + 1000000` draws the row, then
the column RoPE frequency noise ~ N(0, 0.01^2), so theta does not depend on
whether dO is drawn.  bf16 workloads
round Q, K, V, dO to bf16 (round-to-nearest-even).  The RoPE frequencies start
from the geometric schedule 10000^(-2i/(d/2)), i < d/4, used as the
initialisation in the FlashSwin paper card's Figure S4, plus that noise.
`make_device_inputs` draws Q, K, V, dO the same way from a generator on the GPU
itself, for tensors too large to draw on the host (theta as above).
`lowrank_factors` draws the two factors of a rank-r additive bias, U then W
[heads, M*M, r] ~ N(0, 0.5^2) in float32, from a CPU generator seeded with `seed`.
"""

import torch

# name -> (B, Hg, Wg, heads, d, M, shifts, dtype, pass)
WORKLOADS = {
    "tiny_f32_m8": dict(B=1, Hg=16, Wg=16, heads=2, d=32, M=8, shifts=(0,), dtype="f32", kind="fwd", seed=1000),
    "swin_t_s1_p4_m8": dict(B=128, Hg=64, Wg=64, heads=3, d=32, M=8, shifts=(0,), dtype="bf16", kind="fwd", seed=1001),
    "flashswin_t_s1_p2_m32": dict(B=128, Hg=128, Wg=128, heads=3, d=32, M=32, shifts=(0,), dtype="bf16", kind="fwd", seed=1002),
    "flashswin_t_s2_shift16_m32": dict(B=128, Hg=64, Wg=64, heads=6, d=32, M=32, shifts=(16,), dtype="bf16", kind="fwd", seed=1003),
    "flashswin_t_s1_p2_m32_bwd": dict(B=32, Hg=128, Wg=128, heads=3, d=32, M=32, shifts=(0, 16), dtype="bf16", kind="bwd", seed=1004),
    # the M = 16 windows of the pages' comparison tables, on the stage-1 grid of the M = 32 workload
    "flashswin_t_s1_p2_m16": dict(B=128, Hg=128, Wg=128, heads=3, d=32, M=16, shifts=(0, 8), dtype="bf16", kind="fwd", seed=1005),
    # 64-wide heads (C = 192 in 3 heads) at M = 16 on the same stage-1 grid: the q/k/v bytes of the M = 32 workload
    "wide_heads_s1_p2_m16_d64": dict(B=64, Hg=128, Wg=128, heads=3, d=64, M=16, shifts=(0, 8), dtype="bf16", kind="fwd", seed=1006),
}


def geometric_theta(heads, d):
    """theta[h, i] = 10000^(-2i/(d/2)) for i < d/4, identical for every head (float64 list)."""
    return [[10000.0 ** (-2.0 * i / (d / 2)) for i in range(d // 4)] for _ in range(heads)]


def make_inputs(B, Hg, Wg, heads, d, dtype="bf16", seed=0, with_dout=False, theta_noise=0.01):
    """Return a dict of CPU tensors: q, k, v (and dout) in `dtype`, theta_row / theta_col float32 [heads, d/4]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (B, Hg, Wg, heads, d)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for name in ("q", "k", "v"):
        out[name] = torch.randn(shape, generator=g, dtype=torch.float32).to(tdt)
    if with_dout:
        out["dout"] = torch.randn(shape, generator=g, dtype=torch.float32).to(tdt)
    gt = torch.Generator(device="cpu")
    gt.manual_seed(int(seed) + 1000000)
    base = torch.tensor(geometric_theta(heads, d), dtype=torch.float64)
    for name in ("theta_row", "theta_col"):
        noise = torch.randn((heads, d // 4), generator=gt, dtype=torch.float32).double() * theta_noise
        out[name] = (base + noise).float()
    return out


def make_device_inputs(B, Hg, Wg, heads, d, dtype="bf16", seed=0, device="cuda", with_dout=False,
                       theta_noise=0.01):
    """make_inputs with Q, K, V (and dO) drawn on `device` by a generator there (a different stream of
    numbers than the CPU draw); theta is drawn on the host exactly as in make_inputs."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    shape = (B, Hg, Wg, heads, d)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for name in ("q", "k", "v") + (("dout",) if with_dout else ()):
        out[name] = torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(tdt)
    th = make_inputs(1, 1, 1, heads, d, dtype, seed, theta_noise=theta_noise)
    for name in ("theta_row", "theta_col"):
        out[name] = th[name].to(device)
    return out


def workload_inputs(name, with_dout=None, batch=None):
    """Inputs for a named workload; `batch` overrides B (a different B is a different draw)."""
    w = WORKLOADS[name]
    B = w["B"] if batch is None else batch
    wd = (w["kind"] == "bwd") if with_dout is None else with_dout
    return make_inputs(B, w["Hg"], w["Wg"], w["heads"], w["d"], w["dtype"], w["seed"], with_dout=wd)


def lowrank_factors(heads, M, rank, seed):
    """Factors U, W [heads, M*M, rank] of a rank-r additive bias, N(0, 0.5^2) float32 CPU tensors."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return (torch.randn((heads, M * M, rank), generator=g) * 0.5, torch.randn((heads, M * M, rank), generator=g) * 0.5)
