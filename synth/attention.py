"""Workload recipes for the global attention layer (seeded, synthetic).

Shapes follow the layer the model card describes ("Agnes-3.0-Flash Preview", section 架构,
row 全局注意力): 24 query heads, 4 KV heads (GQA 6 : 1), head dim 256; rotary on the first 64
dims with base 1e7 (row 位置编码).

Distributions:
  * q, gate, k, v: N(0, PROJ_STD^2), the spread of one projection output of N(0, 1)
    activations and N(0, 0.02^2) weights over the 5120 hidden units, stored as bf16;
  * q / k norm weights: RNE_bf16(1 + 0.1 N(0, 1)), so the multiply is exercised;
  * a KV cache entry: k ~ N(0, 1) (the RMS-normalised, rotated k has unit spread), v ~
    N(0, PROJ_STD^2), both bf16.
numpy's PCG64 ``default_rng`` is the only source of randomness.
"""
import numpy as np

from .bf16 import f32_to_bf16_bits
from .configs import PROJ_STD

ATTN = dict(num_q_heads=24, num_kv_heads=4, head_dim=256, rot_dim=64, rope_base=1e7)


def _bf16(rng, shape, std):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def norm_weights(rng, d=256):
    return f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32))


def attn_prefill_inputs(rng, lens, hq=24, hkv=4, d=256):
    """Packed batch of sequences with the given lengths: q, gate [T, hq, d], k, v [T, hkv, d]
    (bf16 bits), norm weights qw, kw [d] (bf16 bits), cu_seqlens [N + 1] int32."""
    T = int(sum(lens))
    return dict(
        q=_bf16(rng, (T, hq, d), PROJ_STD),
        k=_bf16(rng, (T, hkv, d), PROJ_STD),
        v=_bf16(rng, (T, hkv, d), PROJ_STD),
        gate=_bf16(rng, (T, hq, d), PROJ_STD),
        qw=norm_weights(rng, d),
        kw=norm_weights(rng, d),
        cu=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
    )


def attn_decode_inputs(rng, lens, lmax, hq=24, hkv=4, d=256):
    """One new token for each of len(lens) sequences whose caches [B, lmax, hkv, d] hold
    lens[b] earlier tokens (entries past lens[b] are zero)."""
    lens = np.asarray(lens, dtype=np.int32)
    B = lens.size
    kc = np.zeros((B, lmax, hkv, d), dtype=np.uint16)
    vc = np.zeros((B, lmax, hkv, d), dtype=np.uint16)
    for b in range(B):
        kc[b, :lens[b]] = _bf16(rng, (int(lens[b]), hkv, d), 1.0)
        vc[b, :lens[b]] = _bf16(rng, (int(lens[b]), hkv, d), PROJ_STD)
    return dict(
        q=_bf16(rng, (B, hq, d), PROJ_STD),
        k=_bf16(rng, (B, hkv, d), PROJ_STD),
        v=_bf16(rng, (B, hkv, d), PROJ_STD),
        gate=_bf16(rng, (B, hq, d), PROJ_STD),
        qw=norm_weights(rng, d),
        kw=norm_weights(rng, d),
        k_cache=kc, v_cache=vc, lens=lens,
    )
