"""Seeded synthetic workloads shaped like the attention layers the pages study.

This module only draws random inputs; it holds none of the method's arithmetic,
so both the CPU oracle and the HIP path can be fed from it.

The pages evaluate on LLaDA-8B, Dream-7B and block-diffusion models (Fast-dLLM
v2, Nemotron-Labs-Diffusion) with real datasets; no weights or datasets are
available here, so seeded Gaussian tensors with the layer shapes stand in for
them.  Outlier key channels (lognormal per-channel scales, Student-t columns)
imitate the per-channel key outliers that motivate KIVI-style per-channel key
quantization.

Every tensor is drawn from ``numpy.random.default_rng([config_id, tensor_id])``
(PCG64) in float32 and, for bf16 configurations, rounded to bf16 with round to
nearest even.  Values are returned as float32 arrays holding exactly the input
values, plus ``dtype`` telling the caller which storage type to upload.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

L_BLOCK = 32

# tensor ids of the recipe
T_Q, T_PK, T_PV, T_KB, T_VB, T_CSCALE, T_PROT, T_LENS, T_SK, T_SV, T_OUTL = range(11)
T_STEP = 11  # 11 + 3s, 12 + 3s, 13 + 3s: step-s block K, V, protected positions


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seed_id: int
    B: int
    Hq: int
    Hkv: int
    D: int
    T: int                  # prefix tokens per sequence (upper bound when ragged)
    dtype: str              # "f32" or "bf16"
    k_bits: int
    v_bits: int
    v_group: int
    prot_frac: float = 0.0
    kscale: bool = False    # lognormal(0, 1) per-(kv head, channel) K scales
    ragged: Optional[tuple] = None  # (lo, hi) inclusive prefix lengths
    suffix: int = 0         # suffix tokens (dual cache)
    t4_outliers: bool = False
    step_protect: int = 0   # protected rows in each per-step 32-token block commit
    desc: str = ""

    @property
    def r(self) -> int:
        return self.Hq // self.Hkv


CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", 1, B=1, Hq=2, Hkv=2, D=64, T=256, dtype="f32", k_bits=4, v_bits=4,
                   v_group=64, desc="batch 1, 2 heads, d 64, prefix 256, fp32, 4-bit"),
    "llada8b": Config("llada8b", 2, B=1, Hq=32, Hkv=32, D=128, T=2048, dtype="bf16", k_bits=4,
                      v_bits=4, v_group=128, prot_frac=0.05, kscale=True,
                      desc="LLaDA-8B-shaped layer: MHA 32 heads, prefix 2048, 4-bit, 5% protected"),
    "dream7b_2bit": Config("dream7b_2bit", 3, B=8, Hq=28, Hkv=4, D=128, T=8192, dtype="bf16",
                           k_bits=2, v_bits=2, v_group=64, prot_frac=0.10, kscale=True,
                           step_protect=3,
                           desc="Dream-7B-shaped layer: B 8, GQA 28/4, prefix 8192, 2-bit, 10% protected"),
    "dream7b_4bit": Config("dream7b_4bit", 3, B=8, Hq=28, Hkv=4, D=128, T=8192, dtype="bf16",
                           k_bits=4, v_bits=4, v_group=64, prot_frac=0.10, kscale=True,
                           step_protect=3,
                           desc="Dream-7B-shaped layer at 4-bit KV: B 8, GQA 28/4, prefix 8192"),
    "serve_b32": Config("serve_b32", 4, B=32, Hq=12, Hkv=2, D=128, T=4096, dtype="bf16", k_bits=4,
                        v_bits=4, v_group=128, ragged=(1024, 4096),
                        desc="batch-32 serving: GQA 12/2, ragged prefixes 1024..4096, 4-bit"),
    "dual_long": Config("dual_long", 5, B=4, Hq=28, Hkv=4, D=128, T=32768, dtype="bf16", k_bits=2,
                        v_bits=2, v_group=64, prot_frac=0.05, suffix=1024, t4_outliers=True,
                        desc="long dual cache: prefix 32768 + suffix 1024, 2-bit, 5% protected"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32.  Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are exactly bf16 (for upload)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value is not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _rng(cfg: Config, tid: int) -> np.random.Generator:
    return np.random.default_rng([cfg.seed_id, tid])


def _cast(cfg: Config, x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_to_bf16(x) if cfg.dtype == "bf16" else x


def channel_scales(cfg: Config) -> Optional[np.ndarray]:
    if not cfg.kscale:
        return None
    return _rng(cfg, T_CSCALE).lognormal(0.0, 1.0, size=(cfg.Hkv, cfg.D)).astype(np.float32)


def outlier_columns(cfg: Config) -> List[tuple]:
    """(kv head, channel) pairs drawn from Student-t(4): 1% of the K columns."""
    if not cfg.t4_outliers:
        return []
    n = int(np.floor(0.01 * cfg.Hkv * cfg.D + 0.5))
    idx = _rng(cfg, T_OUTL).choice(cfg.Hkv * cfg.D, size=n, replace=False)
    return [(int(i) // cfg.D, int(i) % cfg.D) for i in np.sort(idx)]


def _keys(cfg: Config, tid: int, B: int, n: int, std: float = 1.0) -> np.ndarray:
    g = _rng(cfg, tid)
    x = g.standard_normal(size=(B, n, cfg.Hkv, cfg.D), dtype=np.float32) * np.float32(std)
    cols = outlier_columns(cfg)
    if cols:
        t = g.standard_t(4, size=(B, n, len(cols))).astype(np.float32) * np.float32(std)
        for j, (h, d) in enumerate(cols):
            x[:, :, h, d] = t[:, :, j]
    cs = channel_scales(cfg)
    if cs is not None:
        x = x * cs[None, None, :, :]
    return _cast(cfg, x)


def _values(cfg: Config, tid: int, B: int, n: int, std: float = 1.0) -> np.ndarray:
    g = _rng(cfg, tid)
    return _cast(cfg, g.standard_normal(size=(B, n, cfg.Hkv, cfg.D), dtype=np.float32) * np.float32(std))


def prefix_lengths(cfg: Config) -> np.ndarray:
    if cfg.ragged is None:
        return np.full(cfg.B, cfg.T, dtype=np.int32)
    lo, hi = cfg.ragged
    return _rng(cfg, T_LENS).integers(lo, hi + 1, size=cfg.B).astype(np.int32)


def protected_positions(cfg: Config, lengths: np.ndarray, suffix: int = 0) -> List[np.ndarray]:
    """Sorted distinct protected positions per sequence over prefix (+suffix) tokens.

    Count = floor(frac * n + 0.5); positions >= lengths[b] fall in the suffix."""
    g = _rng(cfg, T_PROT)
    out = []
    for b in range(cfg.B):
        n = int(lengths[b]) + suffix
        k = int(np.floor(cfg.prot_frac * n + 0.5))
        out.append(np.sort(g.choice(n, size=k, replace=False)).astype(np.int32) if k else
                   np.zeros(0, dtype=np.int32))
    return out


@dataclasses.dataclass
class Workload:
    cfg: Config
    q: np.ndarray            # [B, 32, Hq, D]
    k_prefix: np.ndarray     # [B, T, Hkv, D]  (rows past lengths[b] are unused)
    v_prefix: np.ndarray
    lengths: np.ndarray      # [B] prefix tokens per sequence
    prot_prefix: List[np.ndarray]   # per b, positions within the prefix
    k_blk: np.ndarray        # [B, 32, Hkv, D]
    v_blk: np.ndarray
    k_suffix: Optional[np.ndarray] = None   # [B, S, Hkv, D]
    v_suffix: Optional[np.ndarray] = None
    prot_suffix: Optional[List[np.ndarray]] = None


def make(cfg: Config, T: Optional[int] = None, B: Optional[int] = None) -> Workload:
    """Full workload of a configuration.  T / B shrink it with the same recipe
    (a ragged configuration keeps its lo/hi ratio) for quick tests."""
    if B is not None:
        cfg = dataclasses.replace(cfg, B=B)
    if T is not None:
        ragged = None
        if cfg.ragged is not None:
            lo, hi = cfg.ragged
            ragged = (max(1, T * lo // hi), T)
        cfg = dataclasses.replace(cfg, T=T, ragged=ragged)
    lengths = prefix_lengths(cfg)
    Tmax = int(lengths.max())
    q = _cast(cfg, _rng(cfg, T_Q).standard_normal(size=(cfg.B, L_BLOCK, cfg.Hq, cfg.D), dtype=np.float32))
    kp = _keys(cfg, T_PK, cfg.B, Tmax)
    vp = _values(cfg, T_PV, cfg.B, Tmax)
    kb = _keys(cfg, T_KB, cfg.B, L_BLOCK)
    vb = _values(cfg, T_VB, cfg.B, L_BLOCK)
    prot = protected_positions(cfg, lengths, cfg.suffix)
    w = Workload(cfg, q, kp, vp, lengths, [p[p < lengths[b]] for b, p in enumerate(prot)], kb, vb)
    if cfg.suffix:
        w.k_suffix = _keys(cfg, T_SK, cfg.B, cfg.suffix, std=0.5)
        w.v_suffix = _values(cfg, T_SV, cfg.B, cfg.suffix, std=0.5)
        w.prot_suffix = [(p[p >= lengths[b]] - lengths[b]).astype(np.int32) for b, p in enumerate(prot)]
    return w


def step_block(cfg: Config, step: int, B: Optional[int] = None):
    """K/V of the 32-token block committed at decoding step `step`, and its
    protected positions (cfg.step_protect per sequence)."""
    B = cfg.B if B is None else B
    k = _keys(cfg, T_STEP + 3 * step, B, L_BLOCK)
    v = _values(cfg, T_STEP + 3 * step + 1, B, L_BLOCK)
    g = _rng(cfg, T_STEP + 3 * step + 2)
    prot = [np.sort(g.choice(L_BLOCK, size=cfg.step_protect, replace=False)).astype(np.int32)
            if cfg.step_protect else np.zeros(0, np.int32) for _ in range(B)]
    return k, v, prot


def to_csr(pos: List[np.ndarray]):
    off = np.zeros(len(pos) + 1, dtype=np.int32)
    for i, p in enumerate(pos):
        off[i + 1] = off[i] + len(p)
    idx = np.concatenate(pos).astype(np.int32) if off[-1] else np.zeros(0, np.int32)
    return off, idx


def krpbh_params(D: int, block: int, seed: int = 0):
    """Random inputs of the K-RPBH value rotation: a permutation of 0..D-1 and a
    Haar-distributed k x k orthogonal mix (k = D / block), fp32.  QR of a
    Gaussian matrix with the signs of R's diagonal moved into Q gives the Haar
    measure.  These are drawn here, as inputs; neither side of the comparison
    draws them."""
    g = np.random.default_rng([0xB07A7E, D, block, seed])
    k = D // block
    a = g.standard_normal((k, k))
    q, r = np.linalg.qr(a)
    q = q * np.sign(np.diag(r))[None, :]
    return g.permutation(D).astype(np.int32), q.astype(np.float32)
