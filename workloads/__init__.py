"""Seeded synthetic workloads for the ZeRO-DP partitioned optimizer step.

This module only describes and draws inputs: shapes, sizes, dtypes, seeds and
random values. It holds none of the method's arithmetic (no partitioning, no
averaging, no optimizer math), so the GPU library and the CPU oracle can both
be fed from it without sharing any code with each other.

Every buffer draws from its own stream, seeded by (seed, workload, buffer kind,
replica, step). Values follow the pages' mixed-precision setting
(fp16/bf16 params and grads, fp32 master/momentum/variance):

* gradient replicas: N(0, 1e-3) times the current loss scale, rounded to the
  16-bit dtype (round to nearest even);
* fp32 master: N(0, 0.02);
* momentum and variance: 0;
* the flat 16-bit parameter vector: the master rounded to 16 bits inside the
  rank's segment, N(0, 0.02) rounded elsewhere.
"""
import hashlib
from dataclasses import dataclass, field

import numpy as np

GRAD_SIGMA = 1e-3
MASTER_SIGMA = 0.02


@dataclass(frozen=True)
class GroupSpec:
    shapes: tuple          # tensor shapes laid end to end in the flat vector
    weight_decay: float = 0.0

    @property
    def numels(self):
        return tuple(int(np.prod(s, dtype=np.int64)) for s in self.shapes)


@dataclass(frozen=True)
class Workload:
    key: str
    title: str
    groups: tuple              # GroupSpec per parameter group
    n_d: int                   # data-parallel degree (gradient copies per segment)
    rank: int                  # the rank whose shard is stepped
    grad_dt: str               # "f16" | "bf16"
    param_dt: str              # "f16" | "bf16"
    steps: int
    loss_scale: float = 1.0
    dynamic_loss_scale: bool = False   # skip on overflow + halve the scale
    inf_at: tuple = None       # (call index from 1, replica, "mid") -> +inf injected
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    notes: str = ""
    extra: dict = field(default_factory=dict, compare=False, hash=False)


def _gpt2_xl_shapes(n_layer=48, d=1600, vocab=50257, n_pos=1024):
    """GPT-2 1.5B: token + position embeddings, 48 blocks with biased linears and
    LayerNorms, final LayerNorm, LM head tied to the token embedding."""
    shapes = [(vocab, d), (n_pos, d)]
    for _ in range(n_layer):
        shapes += [(d,), (d,),                  # ln_1 weight, bias
                   (d, 3 * d), (3 * d,),        # attention qkv
                   (d, d), (d,),                # attention output
                   (d,), (d,),                  # ln_2 weight, bias
                   (d, 4 * d), (4 * d,),        # MLP up
                   (4 * d, d), (d,)]            # MLP down
    shapes += [(d,), (d,)]                      # ln_f
    return tuple(shapes)


def _llama3_8b_groups(n_layer=32, d=4096, n_kv=8, head_dim=128, mlp=14336, vocab=128256):
    """LLaMA-3 8B: matrices (weight decay 0.1) and RMSNorm weights (no decay)."""
    kv = n_kv * head_dim
    mats = [(vocab, d)]
    norms = []
    for _ in range(n_layer):
        mats += [(d, d), (kv, d), (kv, d), (d, d),      # q, k, v, o
                 (mlp, d), (mlp, d), (d, mlp)]          # gate, up, down
        norms += [(d,), (d,)]                           # attention / MLP RMSNorm
    norms += [(d,)]                                     # final norm
    mats += [(vocab, d)]                                # untied LM head
    return (GroupSpec(tuple(mats), 0.1), GroupSpec(tuple(norms), 0.0))


WORKLOADS = {
    "tiny": Workload(
        key="tiny",
        title="tiny flat group [512x768],[768],[768x513],[3], N_d=4, rank 1",
        groups=(GroupSpec(((512, 768), (768,), (768, 513), (3,))),),
        n_d=4, rank=1, grad_dt="f16", param_dt="f16", steps=3,
        notes="Psi = 787,971 (odd); the rank-1 segment straddles tensor boundaries"),
    "tiny_literal": Workload(
        key="tiny_literal",
        title="tiny flat group [512x768],[768],[768x511],[3], N_d=4, rank 1",
        groups=(GroupSpec(((512, 768), (768,), (768, 511), (3,))),),
        n_d=4, rank=1, grad_dt="f16", param_dt="f16", steps=3,
        notes="the literal shape list; Psi = 786,435"),
    "gpt2_1.5b": Workload(
        key="gpt2_1.5b",
        title="GPT-2 1.5B flat vector, N_d=1, bf16, static loss scale 2^16",
        groups=(GroupSpec(_gpt2_xl_shapes()),),
        n_d=1, rank=0, grad_dt="bf16", param_dt="bf16", steps=10, loss_scale=65536.0),
    "7.5b_nd64": Workload(
        key="7.5b_nd64",
        title="7.5B flat vector, N_d=64, rank 63 (~117M-element shard), fp16",
        groups=(GroupSpec(((7_500_000_000,),)),),
        n_d=64, rank=63, grad_dt="f16", param_dt="f16", steps=10),
    "13b_nd8": Workload(
        key="13b_nd8",
        title="13B flat vector, N_d=8, rank 7 (1.625B-element shard), fp16, dynamic loss scale",
        groups=(GroupSpec(((13_000_000_000,),)),),
        n_d=8, rank=7, grad_dt="f16", param_dt="f16", steps=10, loss_scale=65536.0,
        dynamic_loss_scale=True, inf_at=(4, 5, "mid"),
        notes="+inf in replica 5 at the shard's middle element before call 4"),
    "llama3_8b": Workload(
        key="llama3_8b",
        title="LLaMA-3 8B, N_d=1, AdamW, two groups (matrices wd 0.1, norms wd 0), bf16",
        groups=_llama3_8b_groups(),
        n_d=1, rank=0, grad_dt="bf16", param_dt="bf16", steps=5),
}


# --------------------------------------------------------------------------
# Seeds and draws
# --------------------------------------------------------------------------

def derive_seed(*keys):
    """A 63-bit seed from a tuple of keys (stable across processes)."""
    h = hashlib.sha256(repr(tuple(keys)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def normal_f32_np(n, sigma, seed):
    """float32 N(0, sigma^2) on the host. ``seed`` is an int or a key tuple."""
    if not isinstance(seed, (int, np.integer)):
        seed = derive_seed(seed)
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    return (rng.standard_normal(int(n), dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def to16_bits_np(x, dt):
    """float32 -> uint16 bit patterns of fp16/bf16, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dt == "f16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16).view(np.uint16)
    import torch
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def grads16_np(n, dt, loss_scale, seed, sigma=GRAD_SIGMA):
    """One gradient replica as uint16 bits: RNE16(N(0, sigma) * loss_scale)."""
    g = normal_f32_np(n, sigma, seed) * np.float32(loss_scale)
    return to16_bits_np(g, dt)


def torch_dtype(dt):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dt]


def fill_normal_(out, sigma, seed, scale=1.0, chunk=1 << 27):
    """Fill a torch tensor (any device, any float dtype) with N(0, sigma)*scale,
    drawn in fp32 chunk by chunk from one seeded generator, then rounded to
    ``out``'s dtype. Bounded temporary memory for multi-GB buffers."""
    import torch
    flat = out.view(-1)
    if not isinstance(seed, (int, np.integer)):
        seed = derive_seed(seed)
    gen = torch.Generator(device=flat.device)
    gen.manual_seed(int(seed))
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        tmp = torch.randn(e - s, generator=gen, device=flat.device, dtype=torch.float32)
        tmp.mul_(float(sigma) * float(scale))
        flat[s:e].copy_(tmp)
    return out
