"""Seeded synthetic inputs shaped like the layers the pages describe.

This module only draws random numbers and rounds them to bf16 storage; it
holds none of the NVFP4 arithmetic (no scale computation, no encoding, no
products), so both the CPU oracle and the HIP path can take their inputs
from it.  ``random_nvfp4`` draws code and scale bytes directly, which needs
none of that arithmetic either.

Shapes and distributions:
  * "vroomfondel/glm-5.2-reap-504B-v2-W4A4" model card, "What this variant
    changes": o_proj is 6144 x 16384 and q_b_proj 16384 x 2048 (out x in).
  * "GLM-5.2-NVFP4" model card, intro: 256 routed experts, 8 per token,
    hidden size 6144.
The value distributions (weights ~ N(0, 0.02), activations ~ N(0, 1),
heavy-tailed quantize input, expert intermediate 2048, router logits
~ N(0, 1) with top-8 softmax gates) are synthetic stand-ins: the pages ship
no tensors.

bf16 tensors are returned as numpy.uint16 bit patterns (round-to-nearest-even
from float32 by torch's CPU conversion).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

O_PROJ = (6144, 16384)     # (N out, K in)
Q_B_PROJ = (16384, 2048)
MOE_T, MOE_E, MOE_TOPK, MOE_H, MOE_I = 4096, 256, 8, 6144, 2048
GEMM_M_SWEEP = (1, 8, 32, 64, 128, 256, 1024, 4096)
GEMV_M = (1, 2, 4, 8)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), RNE via torch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


# ------------------------------------------------------------------ configs --

def tiny_end_to_end(seed: int = 0):
    """W [256 x 512] ~ N(0, 0.02) then X [4 x 512] ~ N(0, 1) from one generator."""
    rng = np.random.default_rng(seed)
    w = normal_bf16(rng, (256, 512), 0.02)
    x = normal_bf16(rng, (4, 512), 1.0)
    return w, x


def heavy_tailed(rows: int, cols: int, seed: int = 1, chunk_rows: int = 4096) -> np.ndarray:
    """Student-t (df = 3) * 0.02 with 0.01 % outliers scaled by 50, drawn in
    row chunks of ``chunk_rows`` (t-draw then outlier mask per chunk)."""
    rng = np.random.default_rng(seed)
    out = np.empty((rows, cols), np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        v = rng.standard_t(3, size=(r1 - r0, cols)).astype(np.float32) * np.float32(0.02)
        mask = rng.random((r1 - r0, cols)) < 1e-4
        v[mask] *= np.float32(50.0)
        out[r0:r1] = to_bf16_bits(v)
    return out


def layer_weight(shape, seed: int = 3, std: float = 0.02) -> np.ndarray:
    return normal_bf16(np.random.default_rng(seed), shape, std)


def activations(m: int, k: int, seed: int) -> np.ndarray:
    return normal_bf16(np.random.default_rng(seed), (m, k), 1.0)


def gemv_inputs(shape_name: str):
    """(W bf16 [N, K], x bf16 [8, K]) for o_proj / q_b_proj: W seed 3, x seed 33.
    The first M rows of x are the batch-M activation."""
    shape = {"o_proj": O_PROJ, "q_b_proj": Q_B_PROJ}[shape_name]
    return layer_weight(shape, seed=3), activations(8, shape[1], seed=33)


def moe_routing(T: int = MOE_T, E: int = MOE_E, k: int = MOE_TOPK, seed: int = 5):
    """Router logits ~ N(0, 1) [T, E]; ids = the k largest per token (ties to
    the lower expert id), weights = softmax over those k logits (fp32,
    max-subtracted).  Returns (ids int32 [T, k], weights f32 [T, k])."""
    logits = np.random.default_rng(seed).standard_normal((T, E), dtype=np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, order, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return order.astype(np.int32), w


def moe_tokens(T: int = MOE_T, H: int = MOE_H, seed: int = 55) -> np.ndarray:
    return activations(T, H, seed)


def moe_expert_weight(e: int, E: int = MOE_E, H: int = MOE_H, I: int = MOE_I, seed: int = 50):
    """Expert e's (W13 bf16 [2I, H] with gate rows first, W2 bf16 [H, I]),
    both ~ N(0, 0.02), from SeedSequence(seed).spawn(E)[e]."""
    ss = np.random.SeedSequence(seed).spawn(E)[e]
    rng = np.random.default_rng(ss)
    w13 = normal_bf16(rng, (2 * I, H), 0.02)
    w2 = normal_bf16(rng, (H, I), 0.02)
    return w13, w2


def moe_expert_weights_iter(E: int = MOE_E, H: int = MOE_H, I: int = MOE_I, seed: int = 50,
                            threads: int = 8):
    """Yield (e, W13, W2) for e = 0..E-1, drawn on a small thread pool with at
    most ``2 * threads`` experts in flight."""
    window = 2 * threads
    with ThreadPoolExecutor(max_workers=threads) as pool:
        futs = {}
        for e in range(E):
            futs[e] = pool.submit(moe_expert_weight, e, E, H, I, seed)
            if e >= window - 1:
                done = e - (window - 1)
                w13, w2 = futs.pop(done).result()
                yield done, w13, w2
        for done in sorted(futs):
            w13, w2 = futs.pop(done).result()
            yield done, w13, w2


MOE_LORA_RANK = 64


def moe_lora(E: int = MOE_E, H: int = MOE_H, I: int = MOE_I, rank: int = MOE_LORA_RANK, seed: int = 56,
             std: float = 0.02):
    """bf16 LoRA adapter for the routed experts ("Getting GLM-5.2 NVFP4
    Post-Training off the ground", "Going deeper": rank 64 on the MLP, one
    LoRA-A shared by the experts, one LoRA-B per expert).  Every tensor is
    ~ N(0, std) (a trained adapter, not the all-zero B of initialisation):
    a13 [r, H], b13 [E, 2I, r] (gate rows first), a2 [r, I], b2 [E, H, r]."""
    rng = np.random.default_rng(seed)
    return {
        "a13": normal_bf16(rng, (rank, H), std),
        "b13": normal_bf16(rng, (E, 2 * I, rank), std),
        "a2": normal_bf16(rng, (rank, I), std),
        "b2": normal_bf16(rng, (E, H, rank), std),
    }


def random_nvfp4(lead, rows: int, cols: int, seed: int, device, rms: float = 0.02):
    """Random NVFP4 tensors [*lead, rows, cols] drawn as bytes on ``device``
    with a seeded torch generator: codes uniform over all 256 byte values
    (two E2M1 codes each), E4M3 scale bytes uniform in [0x30, 0x40)
    (block scales in [0.5, 2)), and one fp32 global scale per leading index
    set so that the element rms is about ``rms`` (uniform E2M1 codes have rms
    2.93, the scales about 1.2).  Used where a full-size expert stack is
    needed quickly: quantizing 256 drawn experts takes minutes on a host.
    Returns (codes uint8 [*lead, rows, cols/2], scales uint8
    [*lead, rows, cols/16], global f32 [*lead])."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    lead = tuple(lead)
    codes = torch.randint(0, 256, lead + (rows, cols // 2), generator=g, device=device, dtype=torch.uint8)
    scales = torch.randint(0x30, 0x40, lead + (rows, cols // 16), generator=g, device=device, dtype=torch.uint8)
    glob = torch.full(lead, rms / (2.93 * 1.2), dtype=torch.float32, device=device)
    return codes, scales, glob
