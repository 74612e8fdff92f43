"""Seeded synthetic inputs for the linear, MoE and NVFP4-style workloads.

This module only draws random numbers and stores them as bf16; it holds none
of the quantization or GEMM arithmetic, so both the GPU path and the CPU
checker can take their inputs from it.

Workloads (shapes of the layers the pages name: Meta-Llama-3-8B in the usage
examples of the fine-grained FP8 guide, DeepSeek-V3/R1 as the scheme's
origin, the Mistral-Medium-3.5-128B-NVFP4 MLP/attention split):

* ``llama``    acts N(0, 1) with 0.1% of the input channels (round(0.001 K),
               chosen by a seeded permutation) multiplied by 50 for every
               token; weights N(0, 0.02).
* ``deepseek`` acts drawn elementwise from N(0, 1) with probability 0.9 and
               from Student-t(3) with probability 0.1; weights N(0, 0.01).
* ``moe``      Zipf(1.1) expert popularity over a seeded permutation of the
               expert ids; every token picks ``top_k`` distinct experts by
               Gumbel-top-k; rows are grouped in expert order.
* ``nvfp4``    acts N(0, 1), weights N(0, 0.015).

Every draw comes from ``numpy.random.Generator(PCG64(SeedSequence(key)))``
with ``key = [seed, workload, tensor, index]``, so each tensor is
reproducible on its own.  Large device tensors can instead be drawn with
torch's device generator (``device_normal_bf16``), seeded the same way.
"""

import numpy as np

WORKLOAD_IDS = {"single": 1, "llama": 2, "deepseek": 3, "moe": 4, "nvfp4": 5}
TENSOR_IDS = {"x": 0, "w": 1, "bias": 2, "route": 3, "h": 4, "w2": 5, "misc": 9}


def rng(workload, tensor, index=0, seed=0):
    key = [int(seed), WORKLOAD_IDS[workload], TENSOR_IDS[tensor], int(index)]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def f32_to_bf16_bits(a):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even
    (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def normal_bf16(shape, sigma, workload, tensor, index=0, seed=0):
    g = rng(workload, tensor, index, seed)
    return f32_to_bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(sigma))


def llama_acts(M, K, seed=0, index=0, outlier_frac=0.001, outlier_mult=50.0):
    g = rng("llama", "x", index, seed)
    x = g.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    if n_out:
        ch = g.permutation(K)[:n_out]
        x[:, ch] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


def deepseek_acts(M, K, seed=0, index=0, heavy_frac=0.1, dof=3.0):
    g = rng("deepseek", "x", index, seed)
    x = g.standard_normal((M, K), dtype=np.float32)
    t = g.standard_t(dof, size=(M, K)).astype(np.float32)
    pick = g.random((M, K)) < heavy_frac
    return f32_to_bf16_bits(np.where(pick, t, x))


def moe_routing(tokens, experts, top_k, alpha=1.1, seed=0):
    """Returns (token_of_row int64 (tokens*top_k,), seg_offsets int32 (E+1,)).

    Rows are sorted by expert (stable in token order), so the rows of
    expert e are token_of_row[seg_offsets[e]:seg_offsets[e+1]].
    """
    g = rng("moe", "route", 0, seed)
    perm = g.permutation(experts)
    pop = np.empty(experts)
    pop[perm] = np.arange(1, experts + 1, dtype=np.float64) ** (-alpha)
    pop /= pop.sum()
    gumbel = -np.log(-np.log(g.random((tokens, experts))))
    keys = np.log(pop)[None, :] + gumbel
    choice = np.argpartition(-keys, top_k - 1, axis=1)[:, :top_k]     # distinct
    flat_e = choice.reshape(-1)
    flat_t = np.repeat(np.arange(tokens), top_k)
    order = np.lexsort((flat_t, flat_e))
    counts = np.bincount(flat_e, minlength=experts)
    off = np.zeros(experts + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return flat_t[order].astype(np.int64), off


def device_normal_bf16(shape, sigma, workload, tensor, index=0, seed=0, device="cuda"):
    """Draw N(0, sigma) on the device with torch's generator (for tensors too
    large to draw on the host); returns a torch bfloat16 tensor."""
    import torch
    key = ((int(seed) * 131 + WORKLOAD_IDS[workload]) * 131 + TENSOR_IDS[tensor]) * 1_000_003 + int(index)
    gen = torch.Generator(device=device)
    gen.manual_seed(key)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    step = 1 << 26
    for i in range(0, flat.numel(), step):
        n = min(step, flat.numel() - i)
        flat[i:i + n] = (torch.randn(n, generator=gen, device=device) * sigma).to(torch.bfloat16)
    return out


def device_llama_acts(M, K, seed=0, index=0, outlier_frac=0.001, outlier_mult=50.0,
                      device="cuda"):
    """The ``llama`` activation recipe drawn on the device: N(0, 1), with the
    outlier channels picked by the same seeded permutation as llama_acts."""
    import torch
    x = device_normal_bf16((M, K), 1.0, "llama", "x", index, seed, device).float()
    n_out = int(round(outlier_frac * K))
    if n_out:
        ch = rng("llama", "misc", index, seed).permutation(K)[:n_out]
        x[:, torch.from_numpy(ch).to(device)] *= outlier_mult
    return x.to(torch.bfloat16)


def device_deepseek_acts(M, K, seed=0, index=0, heavy_frac=0.1, dof=3.0, device="cuda"):
    """The ``deepseek`` activation recipe drawn on the device (normal with a
    Student-t(3) share), from torch's device generator."""
    import torch
    key = ((int(seed) * 131 + WORKLOAD_IDS["deepseek"]) * 131 + TENSOR_IDS["x"]) * 1_000_003 + index
    gen = torch.Generator(device=device)
    gen.manual_seed(key)
    z = torch.randn((M, K), generator=gen, device=device)
    # Student-t(dof) = N / sqrt(chi2_dof / dof); chi2_dof from dof normals
    n = torch.randn((M, K), generator=gen, device=device)
    chi = sum(torch.randn((M, K), generator=gen, device=device) ** 2 for _ in range(int(dof)))
    t = n / torch.sqrt(chi / dof)
    pick = torch.rand((M, K), generator=gen, device=device) < heavy_frac
    return torch.where(pick, t, z).to(torch.bfloat16)
