"""Global (softmax) attention layer, fp64 — TEST INFRASTRUCTURE.

Sources: model card "Agnes-3.0-Flash Preview", 架构 table, rows 全局注意力 (24 query heads and
4 KV heads, GQA 6 : 1, head dim 256; q and k each pass an RMS-norm; the output passes a sigmoid
gate) and 位置编码 (three-axis rotary over text / height / width, sections 11 : 11 : 10
interleaved, base 1e7, applied to the first 25 % of the head dim, 64 dims); discosf article
"Agnes 3.0 Flash 刚上线就刷屏…", section 二.1 (the same specification; only these 18 layers
keep a KV cache).

The pages give no formula.  Readings (each pinned in tests/test_oracle_attention_pins.py):
  * inputs are the projections q, gate [T, Hq, 256] and k, v [T, Hkv, 256]; query head h reads
    KV head h // (Hq / Hkv) (contiguous groups);
  * RMS-norm per head over its 256 values, x / sqrt(mean(x^2) + eps) * w, one weight [256] for
    q and one for k, eps = 1e-6; it comes before the rotary;
  * rotary on dims 0..63 of each q and k head, dim j paired with dim j + 32 (j < 32) and turned
    by the angle pos * base^(-2j/64); frequency j takes its position from axis j mod 3 of the
    token's (text, height, width) position triple, which splits the 32 frequencies 11 : 11 : 10
    in interleaved order; dims 64..255 pass unchanged.  A text token has all three positions
    equal to its index in its sequence;
  * causal softmax attention inside each sequence of cu_seqlens with scale 1/sqrt(256);
  * output = attention output * sigmoid(gate), elementwise;
  * decode: the cache holds the normalised, rotated k and the raw v of every earlier token of
    the sequence; a step writes the new token's k, v at index len and attends over len + 1 keys.
"""
import numpy as np

from .inputs import as_f64

HEAD_DIM = 256
ROT_DIM = 64
ROPE_BASE = 1e7


def rms_norm_heads(x, w, eps=1e-6):
    """x [..., 256], w [256] -> x / sqrt(mean(x^2) + eps) * w."""
    x = as_f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * as_f64(w)


def rope_inv_freq(base=ROPE_BASE, rot_dim=ROT_DIM):
    """[rot_dim / 2] angular frequencies base^(-2j / rot_dim)."""
    return base ** (-np.arange(0, rot_dim, 2, dtype=np.float64) / rot_dim)


def rope_angles(pos3, base=ROPE_BASE, rot_dim=ROT_DIM):
    """pos3 [3, T] (text, height, width positions) -> angles [T, rot_dim / 2]: frequency j
    turns with the position on axis j mod 3."""
    pos3 = np.asarray(pos3, dtype=np.float64)
    inv = rope_inv_freq(base, rot_dim)
    axis = np.arange(inv.size) % 3
    return pos3[axis].T * inv[None, :]


def apply_rotary(x, angles, rot_dim=ROT_DIM):
    """x [T, H, D], angles [T, rot_dim / 2]: (x_j, x_{j+half}) -> (x_j c - x_{j+half} s,
    x_{j+half} c + x_j s) for j < half; the other dims unchanged."""
    x = as_f64(x).copy()
    half = rot_dim // 2
    c = np.cos(angles)[:, None, :]
    s = np.sin(angles)[:, None, :]
    a = x[..., :half].copy()
    b = x[..., half:rot_dim].copy()
    x[..., :half] = a * c - b * s
    x[..., half:rot_dim] = b * c + a * s
    return x


def text_positions(cu_seqlens, total):
    """[3, T] positions of text tokens: the index in the sequence on all three axes."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    p = np.zeros(total, dtype=np.int64)
    for n in range(cu.size - 1):
        p[cu[n]:cu[n + 1]] = np.arange(cu[n + 1] - cu[n])
    return np.stack([p, p, p])


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def qk_prep(q, k, q_norm_w, k_norm_w, pos3, eps=1e-6, base=ROPE_BASE):
    """RMS-norm then rotary of q [T, Hq, D] and k [T, Hkv, D] at positions pos3 [3, T]."""
    ang = rope_angles(pos3, base)
    return (apply_rotary(rms_norm_heads(q, q_norm_w, eps), ang),
            apply_rotary(rms_norm_heads(k, k_norm_w, eps), ang))


def causal_attention(qr, kr, v, cu_seqlens, scale=None):
    """Softmax attention of prepared qr [T, Hq, D] over kr, v [T, Hkv, D], causal inside each
    sequence.  Returns [T, Hq, D]."""
    qr, kr, v = as_f64(qr), as_f64(kr), as_f64(v)
    T, hq, d = qr.shape
    grp = hq // kr.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((T, hq, d))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for n in range(cu.size - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b <= a:
            continue
        L = b - a
        mask = np.tril(np.ones((L, L), dtype=bool))
        for h in range(hq):
            s = qr[a:b, h] @ kr[a:b, h // grp].T * scale
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[a:b, h] = p @ v[a:b, h // grp]
    return out


def causal_attention_rows(qr, kr, v, cu_seqlens, rows, heads, scale=None):
    """Rows of causal_attention for the listed tokens and query heads only: [len(rows),
    len(heads), D].  For checks at sizes where the whole output is too costly."""
    qr, kr, v = as_f64(qr), as_f64(kr), as_f64(v)
    d = qr.shape[2]
    grp = qr.shape[1] // kr.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = np.zeros((len(rows), len(heads), d))
    for i, t in enumerate(rows):
        a = int(cu[np.searchsorted(cu, t, side="right") - 1])
        for j, h in enumerate(heads):
            s = kr[a:t + 1, h // grp] @ qr[t, h] * scale
            p = np.exp(s - s.max())
            out[i, j] = (p / p.sum()) @ v[a:t + 1, h // grp]
    return out


def attention_prefill(q, k, v, gate, cu_seqlens, q_norm_w, k_norm_w, pos3=None, eps=1e-6,
                      base=ROPE_BASE, scale=None):
    """The layer in prefill mode over a packed batch.  Returns (o [T, Hq, D], the normalised
    rotated k [T, Hkv, D] that the KV cache holds)."""
    T = np.asarray(q).shape[0]
    pos3 = text_positions(cu_seqlens, T) if pos3 is None else pos3
    qr, kr = qk_prep(q, k, q_norm_w, k_norm_w, pos3, eps, base)
    return causal_attention(qr, kr, v, cu_seqlens, scale) * sigmoid(as_f64(gate)), kr


def attention_decode(q, k, v, gate, k_cache, v_cache, lens, q_norm_w, k_norm_w, pos3=None,
                     eps=1e-6, base=ROPE_BASE, scale=None):
    """One token for each of B sequences.  q, gate [B, Hq, D]; k, v [B, Hkv, D]; caches
    [B, Lmax, Hkv, D] holding lens[b] tokens; pos3 [3, B] (default: lens).  Returns (o [B, Hq, D],
    new k cache, new v cache); the inputs are not modified."""
    lens = np.asarray(lens, dtype=np.int64)
    B = lens.size
    pos3 = np.stack([lens, lens, lens]) if pos3 is None else pos3
    qr, kr = qk_prep(q, k, q_norm_w, k_norm_w, pos3, eps, base)
    kc = np.array(as_f64(k_cache), copy=True)
    vc = np.array(as_f64(v_cache), copy=True)
    hq, d = qr.shape[1], qr.shape[2]
    grp = hq // kr.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((B, hq, d))
    for b in range(B):
        L = int(lens[b])
        kc[b, L] = kr[b]
        vc[b, L] = as_f64(v)[b]
        for h in range(hq):
            s = kc[b, :L + 1, h // grp] @ qr[b, h] * scale
            p = np.exp(s - s.max())
            out[b, h] = (p / p.sum()) @ vc[b, :L + 1, h // grp]
    return out * sigmoid(as_f64(gate)), kc, vc
