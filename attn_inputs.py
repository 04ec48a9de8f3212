"""Seeded synthetic inputs for the attention workloads.

This module is the only code the GPU path's tests and the oracle share.  It
holds no attention arithmetic: it draws iid N(0, 1) fp32 values from a seeded
CPU ``torch.Generator``, rounds them to bf16 (round-to-nearest-even), draws
packed sequence lengths, and picks seeded samples of (head, row) pairs.  The
same bf16 bits feed both the GPU library and the oracle (bf16 widens to fp64
exactly), so any difference between the two comes from the arithmetic alone.

Workloads (the pages measure on no dataset; these stand in for "attention at
sequence length N" with Llama-7B-like head shapes):

=========  ===============================================================
tiny       B1 H1 N128 D64, non-causal, scale 1/8; stability variant Q*8
causal     B4 H32 N4096 D128, causal, scale 1/sqrt(128)
varlen     16 sequences, lengths ~ U[128, 8192], H32 D128, causal, packed
long       B1 H32 N65536 D128, causal
backward   B2 H32 N4096 D128, causal, Q/K/V/dO
=========  ===============================================================
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


def generator(seed: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(int(seed))


def randn_bf16(shape, seed: int | torch.Generator, chunk_rows: int = 0):
    """iid N(0,1) fp32 from a seeded CPU generator, rounded to bf16.

    With ``chunk_rows`` > 0 the leading dimensions are filled in slices of
    that many rows of the last two dimensions (keeps the fp32 temporary small
    for the 65536-token workload); the stream is then defined by that slicing.
    """
    g = generator(seed) if isinstance(seed, int) else seed
    shape = tuple(int(s) for s in shape)
    if chunk_rows <= 0:
        return torch.randn(shape, generator=g, dtype=torch.float32).to(
            torch.bfloat16)
    out = torch.empty(shape, dtype=torch.bfloat16)
    flat = out.view(-1, shape[-1])
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, shape[-1]), generator=g,
                                  dtype=torch.float32).to(torch.bfloat16)
    return out


def randn_f16(shape, seed: int | torch.Generator):
    """iid N(0,1) fp32 from a seeded CPU generator, rounded to IEEE fp16."""
    g = generator(seed) if isinstance(seed, int) else seed
    return torch.randn(tuple(int(s) for s in shape), generator=g,
                       dtype=torch.float32).to(torch.float16)


def qkv(B: int, H: int, N: int, D: int, seed: int, chunk_rows: int = 0):
    """Q, K, V as bf16 [B, H, N, D], drawn in that order from one generator."""
    g = generator(seed)
    return tuple(randn_bf16((B, H, N, D), g, chunk_rows) for _ in range(3))


def default_scale(D: int) -> float:
    """fp32(1/sqrt(D)), the scale every workload uses."""
    return float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))


def varlen_lengths(seed: int, nseq: int = 16, lo: int = 128,
                   hi: int = 8192) -> list[int]:
    """nseq lengths drawn uniformly from [lo, hi] (inclusive)."""
    return [int(x) for x in torch.randint(lo, hi + 1, (nseq,),
                                          generator=generator(seed))]


def cu_seqlens(lengths) -> torch.Tensor:
    """int32 offsets [nseq + 1]: 0, l0, l0+l1, ..."""
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def sample_rows(seed: int, n_heads: int, n_rows: int, count: int = 256,
                extra=()):
    """``count`` seeded (head, row) pairs, uniform, plus fixed extras.

    Returns two int64 tensors (heads, rows).  Duplicates are kept: they are
    harmless for element-wise comparisons.
    """
    g = generator(seed)
    heads = torch.randint(0, n_heads, (count,), generator=g)
    rows = torch.randint(0, n_rows, (count,), generator=g)
    if extra:
        eh = torch.tensor([e[0] for e in extra], dtype=torch.int64)
        er = torch.tensor([e[1] for e in extra], dtype=torch.int64)
        heads, rows = torch.cat([heads, eh]), torch.cat([rows, er])
    return heads.to(torch.int64), rows.to(torch.int64)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return default_scale(self.D)


TINY = Workload("tiny B1 H1 N128 D64 non-causal", 1, 1, 128, 64, False, 0)
CAUSAL = Workload("causal fwd B4 H32 N4096 D128", 4, 32, 4096, 128, True, 1)
LONG = Workload("long causal fwd B1 H32 N65536 D128", 1, 32, 65536, 128, True,
                4)
BACKWARD = Workload("causal bwd B2 H32 N4096 D128", 2, 32, 4096, 128, True, 5)
VARLEN_NAME = "varlen causal fwd 16 seqs U[128,8192] H32 D128"
VARLEN_LENGTH_SEED = 2
VARLEN_DATA_SEED = 3
VARLEN_H = 32
VARLEN_D = 128
LONG_SAMPLE_SEED = 40


def tiny_inputs():
    """Tiny workload plus its stability variant (Q*8 is exact in bf16)."""
    q, k, v = qkv(TINY.B, TINY.H, TINY.N, TINY.D, TINY.seed)
    return q, k, v, q * 8


def varlen_inputs(nseq: int = 16, lo: int = 128, hi: int = 8192,
                  H: int = VARLEN_H, D: int = VARLEN_D,
                  length_seed: int = VARLEN_LENGTH_SEED,
                  data_seed: int = VARLEN_DATA_SEED):
    """Packed q, k, v [H, total, D] bf16 and cu_seqlens int32 [nseq+1]."""
    lengths = varlen_lengths(length_seed, nseq, lo, hi)
    cu = cu_seqlens(lengths)
    total = int(cu[-1])
    g = generator(data_seed)
    q, k, v = (randn_bf16((H, total, D), g) for _ in range(3))
    return q, k, v, cu, lengths


def backward_inputs(B=BACKWARD.B, H=BACKWARD.H, N=BACKWARD.N, D=BACKWARD.D,
                    seed=BACKWARD.seed):
    """q, k, v, dO bf16 [B, H, N, D] from one generator."""
    g = generator(seed)
    return tuple(randn_bf16((B, H, N, D), g) for _ in range(4))


def randn_bf16_device(shape, seed: int):
    """iid N(0,1) fp32 drawn on the GPU from a seeded CUDA generator, rounded
    to bf16: for inputs of several GiB, which the CPU generator would take
    minutes to fill.  A test copies the slices it checks back to the host, so
    the oracle still sees exactly the bits the GPU library read."""
    g = torch.Generator(device="cuda")
    g.manual_seed(int(seed))
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
