"""Seeded synthetic inputs for the embedding weight-gradient accumulation.

This module only draws inputs. It holds none of the method's arithmetic, and
both sides (the CPU oracle and the HIP library) are fed from it.

Five workloads, named for what they are:

  uniform3073_v512_h128      3073 int32 ids uniform in [0, 512); grad [3073,128]
                             bf16 ~ N(0, 0.01); main_grad [512,128] fp32 ~ N(0, 1e-3)
  zipf1.1_4096_v32000_h4096  4096 ids Zipf(s=1.1) over 32000; grad bf16 ~ N(0, 0.01);
                             main_grad [32000,4096] fp32 ~ N(0, 1e-3)
  zipf1.1_8192_v129280_h7168 8192 ids Zipf(s=1.1) over 129280; grad [8192,7168]
                             bf16 ~ N(0, 0.01); main_grad [129280,7168] fp32 ~ N(0, 1e-3)
                             (the vocabulary and hidden size the Megatron-Core page
                             quotes for the dense path)
  longrun_8192_v129280_h7168 id 7 at 4096 random positions, 64 other distinct ids at 32
                             positions each, the remaining 2048 uniform over 129280;
                             grad fp32 ~ N(0, 1); main_grad fp32 ~ N(0, 1e-3)
  zipf1.3_4x2048_v129280_h7168_bf16mg
                             ids [4,2048] Zipf(s=1.3) over 129280; grad [4,2048,7168]
                             bf16 ~ N(0, 0.01); main_grad bf16 ~ N(0, 1e-3)

Four more with more tokens than one LDS sort holds (MANY_WORKLOADS, for the
many-token entry point):

  zipf1.1_32768_v129280_h7168    ids [4,8192] Zipf(s=1.1) over 129280, as the
                                 headline otherwise
  zipf1.1_131072_v129280_h7168   ids [16,8192], the largest token count
  longrun_16384_v129280_h7168    the long-run law at 16384 positions (id 7 on
                                 8192 of them), fp32 grad
  zipf1.3_24576_v32000_h4096_bf16mg
                                 24576 ids Zipf(s=1.3) over 32000, bf16 main_grad

Recipe: numpy's PCG64 (`default_rng(seed)`) draws ids and grad; sigma is the
standard deviation; bf16 grad is torch's round-to-nearest-even of the fp32
draw. Zipf(s) over V means P(id = k) proportional to (k + 1)^-s for k in
[0, V), drawn exactly with `rng.choice`. main_grad is drawn by torch.randn from
a seeded torch.Generator on the device that holds it (it is large, and only
its touched rows are ever compared, after copying them back).
"""
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    ids_shape: Tuple[int, ...]
    vocab: int
    hidden: int
    ids_kind: str          # "uniform", "zipf", "longrun"
    zipf_s: float
    grad_dtype: str        # "bf16" or "fp32"
    grad_sigma: float
    main_grad_dtype: str   # "bf16" or "fp32"
    main_grad_sigma: float
    seed: int

    @property
    def num_tokens(self) -> int:
        return int(np.prod(self.ids_shape))


WORKLOADS = {
    w.name: w
    for w in [
        Workload("uniform3073_v512_h128", (3073,), 512, 128, "uniform", 0.0,
                 "bf16", 0.01, "fp32", 1e-3, 1),
        Workload("zipf1.1_4096_v32000_h4096", (4096,), 32000, 4096, "zipf", 1.1,
                 "bf16", 0.01, "fp32", 1e-3, 2),
        Workload("zipf1.1_8192_v129280_h7168", (8192,), 129280, 7168, "zipf", 1.1,
                 "bf16", 0.01, "fp32", 1e-3, 3),
        Workload("longrun_8192_v129280_h7168", (8192,), 129280, 7168, "longrun", 0.0,
                 "fp32", 1.0, "fp32", 1e-3, 4),
        Workload("zipf1.3_4x2048_v129280_h7168_bf16mg", (4, 2048), 129280, 7168, "zipf", 1.3,
                 "bf16", 0.01, "bf16", 1e-3, 5),
    ]
}

# the headline workload: 8192 tokens into a 129280 x 7168 main_grad
HEADLINE = "zipf1.1_8192_v129280_h7168"

# more tokens than one LDS sort holds (the many-token entry point): the
# headline's table and id law with 4x and 16x the tokens (micro-batches of
# 4 and 16 sequences of 8192), a long-run stress with one id on half of
# 16384 positions, and a bf16 main_grad with a steeper Zipf law
MANY_WORKLOADS = {
    w.name: w
    for w in [
        Workload("zipf1.1_32768_v129280_h7168", (4, 8192), 129280, 7168, "zipf", 1.1,
                 "bf16", 0.01, "fp32", 1e-3, 6),
        Workload("zipf1.1_131072_v129280_h7168", (16, 8192), 129280, 7168, "zipf", 1.1,
                 "bf16", 0.01, "fp32", 1e-3, 7),
        Workload("longrun_16384_v129280_h7168", (16384,), 129280, 7168, "longrun", 0.0,
                 "fp32", 1.0, "fp32", 1e-3, 8),
        Workload("zipf1.3_24576_v32000_h4096_bf16mg", (24576,), 32000, 4096, "zipf", 1.3,
                 "bf16", 0.01, "bf16", 1e-3, 9),
    ]
}
MANY_HEADLINE = "zipf1.1_32768_v129280_h7168"

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}


def zipf_ids(rng: np.random.Generator, n: int, vocab: int, s: float) -> np.ndarray:
    """n draws with P(k) proportional to (k + 1)^-s over [0, vocab)."""
    w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    return rng.choice(vocab, size=n, p=w / w.sum()).astype(np.int32)


def longrun_ids(rng: np.random.Generator, n: int, vocab: int) -> np.ndarray:
    """Half the positions hold id 7, 64 other distinct ids hold n/256 positions each,
    the last quarter is uniform over the vocabulary (collisions allowed)."""
    assert n % 256 == 0 and vocab > 65
    perm = rng.permutation(n)
    ids = np.empty(n, dtype=np.int32)
    ids[perm[: n // 2]] = 7
    others = rng.choice(vocab - 1, size=64, replace=False)
    others = others + (others >= 7)          # skip id 7
    per = n // 256
    for i, v in enumerate(others):
        ids[perm[n // 2 + i * per: n // 2 + (i + 1) * per]] = v
    ids[perm[3 * n // 4:]] = rng.integers(0, vocab, size=n - 3 * n // 4)
    return ids


def make_ids(w: Workload) -> np.ndarray:
    rng = np.random.default_rng(w.seed)
    n = w.num_tokens
    if w.ids_kind == "uniform":
        ids = rng.integers(0, w.vocab, size=n, dtype=np.int32)
    elif w.ids_kind == "zipf":
        ids = zipf_ids(rng, n, w.vocab, w.zipf_s)
    elif w.ids_kind == "longrun":
        ids = longrun_ids(rng, n, w.vocab)
    else:
        raise ValueError(w.ids_kind)
    return ids.reshape(w.ids_shape)


def normal_tensor(rng: np.random.Generator, shape, sigma: float, dtype: str) -> torch.Tensor:
    """CPU tensor of N(0, sigma) draws, fp32 or bf16 (round-to-nearest-even of the draw)."""
    x = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma))
    return x.to(TORCH_DTYPE[dtype])


def make_grad(w: Workload) -> torch.Tensor:
    """CPU tensor of shape [*ids_shape, hidden]."""
    rng = np.random.default_rng(w.seed + 1000)
    return normal_tensor(rng, (*w.ids_shape, w.hidden), w.grad_sigma, w.grad_dtype)


def make_main_grad(w: Workload, device="cpu", rows: Optional[int] = None) -> torch.Tensor:
    """[vocab, hidden] main_grad drawn on `device` from a seeded torch generator."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed + 2000)
    x = torch.randn((rows or w.vocab, w.hidden), generator=gen, device=device,
                    dtype=torch.float32)
    x.mul_(w.main_grad_sigma)
    return x.to(TORCH_DTYPE[w.main_grad_dtype])


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> numpy; bf16 as raw uint16 bits, fp32 as float32."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def from_numpy_bits(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Inverse of to_numpy_bits."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def algorithmic_bytes(num_tokens: int, hidden: int, distinct_ids: int, grad_dtype: str,
                      main_grad_dtype: str, ids_itemsize: int = 4) -> int:
    """N*H*sizeof(grad) + 2*U*H*sizeof(main_grad) + N*sizeof(id): grad read once,
    the touched main_grad rows read and written once, the ids read once."""
    size = {"bf16": 2, "fp32": 4}
    return (num_tokens * hidden * size[grad_dtype]
            + 2 * distinct_ids * hidden * size[main_grad_dtype]
            + num_tokens * ids_itemsize)
