"""Seeded synthetic workloads for MoE dispatch/combine.

This module only draws random inputs.  It holds none of the dispatch or
combine arithmetic, so the CPU reference and the HIP library can both be fed
from it without sharing any code.  Random numbers come from NumPy's PCG64;
float32 -> bfloat16 rounding of the drawn activations uses torch's CPU cast.

The workloads mirror the shapes of the pages' low-latency and fused-MoE
cases ("Low-Latency Mode API": hidden <= 7168, top-k <= 16, at most 512
experts; "[feat] A5 deep fused moe", Benchmarking: hidden 7168, uniform top-k;
"DeepEP topk_idx_t Custom Dtype Requirements": 8192 tokens, top-8 of 256
experts, int32 or int64 ids):

========  =====  ====  ===  ==  =====  ==========  ======================  ========================
name      T      H     E    k   ids    quant       routing                 combine input
========  =====  ====  ===  ==  =====  ==========  ======================  ========================
small     128    1024  8    2   int64  none        uniform, no -1          1.5 x dispatched rows
decode8   192    7168  8    8   int64  int8_token  permutations, 1% x50    dispatched buffer
a5fused   24     7168  8    8   int64  int8_token  permutations            dispatched buffer
decode    128    7168  256  8   int64  fp8_b128    uniform, 10% -1         bf16 N(0,1) rows
prefill   4096   7168  256  8   int32  mxfp8       Zipf(1.2) hot experts   dispatched buffer
large     16384  7168  256  8   int64  mxfp4       uniform, 5% -1          bf16 N(0,1) rows
========  =====  ====  ===  ==  =====  ==========  ======================  ========================

Recipe: x = standard normal float32 rounded to bf16; uniform routing is the
first k entries of a random permutation of the experts per token (a uniform
k-subset in random order; with k > E, k independent uniform draws); ``neg_frac`` of all pairs, exactly
round(neg_frac * T * k) of them chosen without replacement, are set to -1;
outlier rows (exactly round(0.01 * T)) are multiplied by 50 in float32 before
the bf16 rounding; Zipf routing gives rank r probability proportional to
r**-1.2, maps ranks to experts through a random permutation and draws k
distinct experts per token by Gumbel-top-k; topk_weights is a float32 softmax
over k of standard normal logits.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    idx_dtype: str          # "int64" | "int32"
    mode: str               # none | int8_token | fp8_b128 | mxfp8 | mxfp4
    routing: str            # "uniform" | "zipf"
    neg_frac: float = 0.0
    outlier_frac: float = 0.0
    combine_input: str = "normal"   # "scaled_dispatch" | "identity" | "normal"
    seed: int = 0
    num_max_tokens: int = 0         # 0 -> T
    row_align: int = 1              # > 1: expert blocks start at multiples of it
    expert_capacity: int = 0        # > 0: every expert block has this many rows
    interleaved: bool = False       # receive rows hold data then scales

    @property
    def t_max(self) -> int:
        return self.num_max_tokens or self.T

    @property
    def max_rows(self) -> int:
        if self.expert_capacity:
            return self.E * self.expert_capacity
        return self.t_max * self.k + self.E * (self.row_align - 1)


WORKLOADS = {
    "small": Workload("small", 128, 1024, 8, 2, "int64", "none", "uniform",
                      combine_input="scaled_dispatch", seed=1001),
    "decode8": Workload("decode8", 192, 7168, 8, 8, "int64", "int8_token", "uniform",
                        outlier_frac=0.01, combine_input="identity", seed=1002),
    "a5fused": Workload("a5fused", 24, 7168, 8, 8, "int64", "int8_token", "uniform",
                        combine_input="identity", seed=1012),
    "decode": Workload("decode", 128, 7168, 256, 8, "int64", "fp8_b128", "uniform",
                       neg_frac=0.10, combine_input="normal", seed=1003),
    "prefill": Workload("prefill", 4096, 7168, 256, 8, "int32", "mxfp8", "zipf",
                        combine_input="identity", seed=1004),
    "large": Workload("large", 16384, 7168, 256, 8, "int64", "mxfp4", "uniform",
                      neg_frac=0.05, combine_input="normal", seed=1005),
}


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16) with torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4)]


def _draw_x(rng, T: int, H: int, outlier_frac: float, chunk: int = 2048) -> np.ndarray:
    n_out = int(round(outlier_frac * T))
    out_rows = set(rng.choice(T, size=n_out, replace=False).tolist()) if n_out else set()
    x = np.empty((T, H), np.uint16)
    for r0 in range(0, T, chunk):
        r1 = min(T, r0 + chunk)
        a = rng.standard_normal((r1 - r0, H), dtype=np.float32)
        for r in out_rows:
            if r0 <= r < r1:
                a[r - r0] *= np.float32(50.0)
        x[r0:r1] = bf16_from_f32(a)
    return x


def _draw_idx(rng, w: Workload) -> np.ndarray:
    T, E, k = w.T, w.E, w.k
    if w.routing == "uniform" and k <= E:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int64)
    elif w.routing == "uniform":               # more choices than experts: repeats
        idx = rng.integers(0, E, size=(T, k)).astype(np.int64)
    elif w.routing == "zipf":
        ranks = np.arange(1, E + 1, dtype=np.float64)
        logp = -1.2 * np.log(ranks)
        perm = rng.permutation(E)
        logp_e = np.empty(E)
        logp_e[perm] = logp                 # expert perm[r-1] has rank r
        g = -np.log(-np.log(rng.random((T, E))))
        idx = np.argsort(-(logp_e[None, :] + g), axis=1)[:, :k].astype(np.int64)
    else:
        raise ValueError(w.routing)
    n_neg = int(round(w.neg_frac * T * k))
    if n_neg:
        flat = idx.reshape(-1)
        flat[rng.choice(T * k, size=n_neg, replace=False)] = -1
    return idx.astype(np.int32 if w.idx_dtype == "int32" else np.int64)


def _draw_weights(rng, T: int, k: int) -> np.ndarray:
    z = rng.standard_normal((T, k), dtype=np.float32)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def make_inputs(w: Workload) -> dict:
    """x (uint16 bf16 patterns [T, H]), topk_idx ([T, k], w.idx_dtype) and
    topk_weights (float32 [T, k])."""
    rx, ri, rw, _ = _streams(w.seed)
    return {
        "x": _draw_x(rx, w.T, w.H, w.outlier_frac),
        "topk_idx": _draw_idx(ri, w),
        "topk_weights": _draw_weights(rw, w.T, w.k),
    }


def make_expert_out(w: Workload, rows: int | None = None, chunk: int = 4096) -> np.ndarray:
    """bf16 N(0,1) expert-output rows (uint16 [rows, H]); rows defaults to
    the workload's max_rows.  Each block of ``chunk`` rows has its own PCG64
    stream (seeded from the workload seed and the block number), so the
    result does not depend on how many threads draw it."""
    from concurrent.futures import ThreadPoolExecutor
    rows = w.max_rows if rows is None else rows
    y = np.empty((rows, w.H), np.uint16)

    def block(b):
        r0, r1 = b * chunk, min(rows, (b + 1) * chunk)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 4, b])))
        y[r0:r1] = bf16_from_f32(g.standard_normal((r1 - r0, w.H), dtype=np.float32))

    nblocks = (rows + chunk - 1) // chunk
    with ThreadPoolExecutor(max_workers=min(8, max(1, nblocks))) as ex:
        list(ex.map(block, range(nblocks)))
    return y


def random_workload(seed: int, T: int, H: int, E: int, k: int, mode: str, *, idx_dtype="int64",
                    neg_frac=0.0, num_max_tokens=0, combine_input="normal") -> Workload:
    return Workload(f"rand{seed}", T, H, E, k, idx_dtype, mode, "uniform", neg_frac=neg_frac,
                    combine_input=combine_input, seed=seed, num_max_tokens=num_max_tokens)


def with_duplicates(idx: np.ndarray, seed: int, frac: float = 0.2) -> np.ndarray:
    """Copy of ``idx`` where a fraction of pairs repeat an expert already
    chosen earlier in the same token row (k >= 2)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = idx.copy()
    T, k = out.shape
    if k < 2:
        return out
    n = int(round(frac * T))
    for t in rng.choice(T, size=min(n, T), replace=False):
        j = int(rng.integers(1, k))
        out[t, j] = out[t, int(rng.integers(0, j))]
    return out


def scaled(w: Workload, **kw) -> Workload:
    return replace(w, **kw)


# ---------------------------------------------------------------------------
# expert MLP (fused MoE) workloads: one GPU's share of an expert-parallel group
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class MoeWorkload:
    """T tokens routed top-k over E_total experts, of which this GPU owns the
    first E_local; pairs routed elsewhere are -1 in the local ids.  Expert
    MLP: hidden H, intermediate I (W1 [E_local, 2I, H], W2 [E_local, H, I],
    MXFP8)."""
    name: str
    T: int
    H: int
    I: int
    E_total: int
    E_local: int
    k: int
    seed: int
    idx_dtype: str = "int64"

    @property
    def max_rows(self) -> int:
        return self.T * self.k


MOE_WORKLOADS = {
    # the 128-tokens-per-device point of the fused-MoE benchmark: 8 ranks x 128
    # tokens, 6 experts per device (48 in all), top-6, hidden 7168, inter 3072
    "moe_share": MoeWorkload("moe_share", 1024, 7168, 3072, 48, 6, 6, seed=1021),
    "moe_small": MoeWorkload("moe_small", 96, 512, 256, 12, 4, 3, seed=1022),
    # the 32 / 64 / 96-tokens-per-device points of the same benchmark
    "moe_share32": MoeWorkload("moe_share32", 256, 7168, 3072, 48, 6, 6, seed=1031),
    "moe_share64": MoeWorkload("moe_share64", 512, 7168, 3072, 48, 6, 6, seed=1032),
    "moe_share96": MoeWorkload("moe_share96", 768, 7168, 3072, 48, 6, 6, seed=1033),
}


def make_mx_weights(seed: int, E: int, N: int, K: int):
    """Synthetic MXFP8 weights drawn directly as codes and scale bytes:
    codes [E, N, K] uint8 (random sign, e4m3 exponent field 4..8 weighted
    towards 6, uniform mantissa: magnitudes 0.125 .. 3.75, never NaN) and e8m0 scale bytes
    [E, N, K/32] around 2**-round(log2(K)/2) (+-1), so a dot product over K
    stays of order one."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 77, E, N, K])))
    # one random byte per code: bit 7 the sign, bits 0-2 the mantissa; a
    # second byte picks the exponent field 4..8 with weights 26/51/90/64/25 of 256
    lut = np.repeat(np.arange(4, 9, dtype=np.uint8), [26, 51, 90, 64, 25])
    b = g.integers(0, 256, size=(E, N, K), dtype=np.uint8)
    e = lut[g.integers(0, 256, size=(E, N, K), dtype=np.uint8)]
    codes = (b & np.uint8(0x87)) | (e << np.uint8(3))
    base = 127 - int(round(np.log2(K) / 2))
    scales = (base - 1 + g.integers(0, 3, size=(E, N, K // 32))).astype(np.uint8)
    return codes, scales


def make_moe_inputs(w: MoeWorkload) -> dict:
    """x (bf16 patterns [T, H]), global ids [T, k] (uniform k-subsets of
    E_total), local ids (the global id if it is one of this GPU's experts,
    else -1), topk_weights (float32 softmax over k), and W1 / W2 codes and
    scale bytes."""
    rx, ri, rw, _ = _streams(w.seed)
    x = _draw_x(rx, w.T, w.H, 0.0)
    gid = np.argsort(ri.random((w.T, w.E_total)), axis=1)[:, :w.k].astype(np.int64)
    lid = np.where(gid < w.E_local, gid, -1)
    dt = np.int32 if w.idx_dtype == "int32" else np.int64
    w1c, w1s = make_mx_weights(w.seed, w.E_local, 2 * w.I, w.H)
    w2c, w2s = make_mx_weights(w.seed + 1, w.E_local, w.H, w.I)
    return {"x": x, "global_idx": gid.astype(dt), "topk_idx": lid.astype(dt),
            "topk_weights": _draw_weights(rw, w.T, w.k),
            "w1_codes": w1c, "w1_scales": w1s, "w2_codes": w2c, "w2_scales": w2s}
