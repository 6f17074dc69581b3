"""Seeded synthetic inputs for the triangle multiplicative update.

Shared by the tests, the benchmark and the oracle checks, and by nothing that
computes the method: this module only draws random numbers, rounds them to the
storage dtype and builds 0/1 masks and index samples.

Shapes follow the fold-cp-ops README ("Use" section): the pair representation
x is (B, N, N, D) row-major, the pair mask is (B, N, N) in the same dtype, and
the layer holds LayerNorm(D) x2, Linear(D, 2D) x2 and Linear(D, D) x2 without
bias (here generalised to a hidden width C: p_in, g_in are [2C, D], p_out is
[D, C]).

Distribution conventions: "N(0, v)" means mean 0 and variance v.  Linear
weights are N(0, 1/D), drawn from one generator in the order a, b, gate_a,
gate_b, gate_out, out.  z is N(0, 1) (or another variance) from its own seed.
In bf16 workloads the GEMM weights, z and the mask are rounded to bf16 (round
to nearest even) and these rounded values are what every consumer sees; the
LayerNorm affine parameters stay fp32.
"""
from dataclasses import dataclass, field, replace
import math

import numpy as np
import torch

Z_SEED, W_SEED, MASK_SEED, SAMPLE_SEED, LN_SEED = 0, 1, 2, 3, 4

TORCH_DTYPES = {"bf16": torch.bfloat16, "fp32": torch.float32}


@dataclass
class TriMulWeights:
    """Host fp32 parameters of one layer (Linear weights stored [out][in])."""
    ln_in_w: np.ndarray    # [D]
    ln_in_b: np.ndarray    # [D]
    p_in: np.ndarray       # [2C, D]: rows [0, C) project a, rows [C, 2C) project b
    g_in: np.ndarray       # [2C, D]: rows [0, C) gate a,    rows [C, 2C) gate b
    ln_out_w: np.ndarray   # [C]
    ln_out_b: np.ndarray   # [C]
    p_out: np.ndarray      # [D, C]
    g_out: np.ndarray      # [D, D]
    eps: float = 1e-5

    @property
    def D(self):
        return int(self.ln_in_w.shape[0])

    @property
    def C(self):
        return int(self.ln_out_w.shape[0])

    def replace(self, **kw):
        return replace(self, **kw)


def round_to(arr, dtype):
    """Round float32 values to the storage dtype and return them as float32."""
    t = torch.as_tensor(np.asarray(arr, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16).to(torch.float32)
    return np.ascontiguousarray(t.numpy())


def make_weights(D, C, dtype="bf16", seed=W_SEED, random_ln=False, ln_seed=LN_SEED):
    """Linear weights N(0, 1/D) in the order a, b, gate_a, gate_b, gate_out, out.

    LayerNorm gamma = 1 and beta = 0 unless ``random_ln`` (then gamma ~ 1 +
    0.1 N(0,1), beta ~ 0.1 N(0,1) from ``ln_seed``, to exercise the affine part).
    """
    g = torch.Generator("cpu").manual_seed(seed)
    std = 1.0 / math.sqrt(D)
    wa = torch.randn((C, D), generator=g) * std
    wb = torch.randn((C, D), generator=g) * std
    wga = torch.randn((C, D), generator=g) * std
    wgb = torch.randn((C, D), generator=g) * std
    wgo = torch.randn((D, D), generator=g) * std
    wo = torch.randn((D, C), generator=g) * std
    p_in = round_to(torch.cat([wa, wb]).numpy(), dtype)
    g_in = round_to(torch.cat([wga, wgb]).numpy(), dtype)
    p_out = round_to(wo.numpy(), dtype)
    g_out = round_to(wgo.numpy(), dtype)
    if random_ln:
        gl = torch.Generator("cpu").manual_seed(ln_seed)
        ln_in_w = (1.0 + 0.1 * torch.randn(D, generator=gl)).numpy()
        ln_in_b = (0.1 * torch.randn(D, generator=gl)).numpy()
        ln_out_w = (1.0 + 0.1 * torch.randn(C, generator=gl)).numpy()
        ln_out_b = (0.1 * torch.randn(C, generator=gl)).numpy()
    else:
        ln_in_w, ln_in_b = np.ones(D, np.float32), np.zeros(D, np.float32)
        ln_out_w, ln_out_b = np.ones(C, np.float32), np.zeros(C, np.float32)
    f = lambda a: np.ascontiguousarray(np.asarray(a, np.float32))
    return TriMulWeights(f(ln_in_w), f(ln_in_b), p_in, g_in, f(ln_out_w), f(ln_out_b),
                         p_out, g_out, 1e-5)


def make_z(B, N, D, dtype="bf16", seed=Z_SEED, var=1.0, device="cpu"):
    """z ~ N(0, var) of shape [B, N, N, D] in the storage dtype, on ``device``.

    On a GPU the draw is made there in row blocks (to bound the fp32 temporary);
    on the CPU in one call.  The two generators give different values for the
    same seed; every consumer reads the one tensor that was drawn.
    """
    tdt = TORCH_DTYPES[dtype]
    std = math.sqrt(var)
    dev = torch.device(device)
    if dev.type == "cpu":
        g = torch.Generator("cpu").manual_seed(seed)
        return (torch.randn((B, N, N, D), generator=g) * std).to(tdt)
    g = torch.Generator(device=dev).manual_seed(seed)
    z = torch.empty((B, N, N, D), dtype=tdt, device=dev)
    rows = max(1, (1 << 27) // max(1, N * D))
    for b in range(B):
        for r0 in range(0, N, rows):
            r1 = min(N, r0 + rows)
            blk = torch.randn((r1 - r0, N, D), generator=g, device=dev, dtype=torch.float32)
            z[b, r0:r1].copy_((blk * std).to(tdt))
            del blk
    return z


def token_mask_tail(N, frac=0.1):
    """Token mask whose last floor(frac*N) tokens are 0 (the rest 1)."""
    n_pad = int(math.floor(frac * N))
    m = np.ones(N, np.float32)
    if n_pad:
        m[N - n_pad:] = 0.0
    return m


def chain_lengths(n_valid, n_chains=4, seed=MASK_SEED):
    """Random lengths of ``n_chains`` chains that sum to ``n_valid`` (cut points from seed)."""
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, n_valid), size=n_chains - 1, replace=False))
    edges = np.concatenate([[0], cuts, [n_valid]])
    return np.diff(edges).astype(np.int64)


def token_mask_chains(N, n_valid, n_chains=4, seed=MASK_SEED):
    """Chains fill tokens [0, n_valid) back to back; tokens [n_valid, N) are padding."""
    lens = chain_lengths(n_valid, n_chains, seed)
    assert int(lens.sum()) == n_valid <= N
    m = np.zeros(N, np.float32)
    m[:n_valid] = 1.0
    return m


def pair_mask(token_mask, B, dtype="bf16", device="cpu"):
    """Pair mask [B, N, N] = outer product of a 0/1 token mask, in the storage dtype."""
    t = torch.as_tensor(np.asarray(token_mask, np.float32))
    pm = (t[:, None] * t[None, :]).to(TORCH_DTYPES[dtype])
    return pm.unsqueeze(0).expand(B, -1, -1).contiguous().to(device)


def sample_grid(N, n=64, seed=SAMPLE_SEED, extra=()):
    """Two sorted index sets (rows I, columns J) of ``min(n, N)`` distinct tokens each.

    Both contain 0, N-1 and ``extra``; the rest are drawn from one generator
    seeded with ``seed`` (I first, then J).
    """
    n = min(n, N)
    must = sorted({0, N - 1, *[int(e) for e in extra if 0 <= int(e) < N]})
    rng = np.random.default_rng(seed)
    pool = np.setdiff1d(np.arange(N), np.array(must))
    out = []
    for _ in range(2):
        k = max(0, n - len(must))
        fill = rng.choice(pool, size=k, replace=False) if k else np.zeros(0, np.int64)
        out.append(np.sort(np.concatenate([np.array(must, np.int64), fill.astype(np.int64)])))
    return out[0], out[1]


@dataclass
class Workload:
    """One synthetic TriMul workload (sizes, dtype, directions, input recipe)."""
    name: str
    dtype: str
    directions: tuple
    B: int
    N: int
    D: int
    C: int
    z_var: float = 1.0
    mask: str = "none"          # "none" | "tail10" | "chains"
    n_valid: int = 0
    check: str = "full"         # "full" | "grid"
    tol: float = 2e-2
    extra_idx: tuple = field(default_factory=tuple)

    def token_mask(self):
        if self.mask == "none":
            return None
        if self.mask == "tail10":
            return token_mask_tail(self.N, 0.1)
        if self.mask == "chains":
            return token_mask_chains(self.N, self.n_valid, 4, MASK_SEED)
        raise ValueError(self.mask)

    def sample_extra(self):
        tm = self.token_mask()
        if tm is None:
            return ()
        nz = np.nonzero(tm)[0]
        last_valid = int(nz[-1]) if len(nz) else 0
        return (last_valid, min(self.N - 1, last_valid + 1))

    def flops(self):
        """Counted FLOPs: contraction 2BCN^3 + input projections 2BN^2 D(4C+D) + p_out 2BN^2 CD."""
        B, N, D, C = self.B, self.N, self.D, self.C
        return 2 * B * C * N ** 3 + 2 * B * N * N * D * (4 * C + D) + 2 * B * N * N * C * D


WORKLOADS = {
    "out_fp32_b1_n64_d32": Workload("out_fp32_b1_n64_d32", "fp32", ("outgoing",), 1, 64, 32, 32,
                                    tol=1e-4),
    "outin_bf16_b1_n384_d128_tailmask": Workload("outin_bf16_b1_n384_d128_tailmask", "bf16",
                                                 ("outgoing", "incoming"), 1, 384, 128, 128,
                                                 mask="tail10"),
    "outin_bf16_b2_n1024_d128": Workload("outin_bf16_b2_n1024_d128", "bf16",
                                         ("outgoing", "incoming"), 2, 1024, 128, 128),
    "out_bf16_b1_n4096_d256": Workload("out_bf16_b1_n4096_d256", "bf16", ("outgoing",),
                                       1, 4096, 256, 256, check="grid"),
    "in_bf16_b1_n8192_d128_chains": Workload("in_bf16_b1_n8192_d128_chains", "bf16",
                                             ("incoming",), 1, 8192, 128, 128, z_var=0.5,
                                             mask="chains", n_valid=7800, check="grid"),
}

HEADLINE = "out_bf16_b1_n4096_d256"
