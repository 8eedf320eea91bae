"""fp64 CPU oracle of the gated delta-rule layer — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never calls it and shares no code with it.

What the layer computes, as the pages describe it:
  * model card "Agnes-3.0-Flash Preview", section 架构 (architecture table,
    delta-rule row): gated delta-rule recurrence with 16 key / 48 value heads of
    dimension 128, a causal convolution of kernel 4 in front, a gated RMS-norm
    behind, and an fp32 recurrent state;
  * discosf article "Agnes 3.0 Flash 刚上线就刷屏…", section 二.1 ("72 层里只有
    18 层吃 KV cache"): the state is kept in fp32 so a long recurrence does not
    drift; the model code has a chunked prefill (chunk 64) and a stepwise
    decode path for the same layer.
The pages name the method but print no formula.  The recurrence is the gated
delta rule of Yang, Kautz & Hatamizadeh, "Gated Delta Networks: Improving
Mamba2 with Delta Rule" (ICLR 2025), equation of the gated delta rule:
    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t.

The global attention layer of the same model (24 query / 4 KV heads of dimension 256, RMS-norm
on q and k, partial three-axis rotary, sigmoid output gate; same model card, rows 全局注意力 and
位置编码) is in attention.py.

Every routine works in fp64 on exactly upcast inputs.  Pins that tie each
function to something other than itself live in tests/test_oracle_pins.py;
the readings of points the pages leave open are listed at the top of each
module.  Parity unpinned: whether those readings (head mapping, conv weight
orientation, norm form, epsilons) match a trained checkpoint's conventions —
nothing on the pages can settle that.
"""
from .gdn import recurrence, recurrence_matrix_form, decode_step, key_head_of
from .conv import causal_conv, l2norm_heads, silu
from .norm import gated_rmsnorm
from .layer import prefill_layer, decode_layer_step, prefill_conv_recurrence
from .inputs import as_f64
from .attention import (
    rms_norm_heads, rope_inv_freq, rope_angles, apply_rotary, text_positions, qk_prep,
    causal_attention, causal_attention_rows, attention_prefill, attention_decode,
)

__all__ = [
    "recurrence", "recurrence_matrix_form", "decode_step", "key_head_of",
    "causal_conv", "l2norm_heads", "silu", "gated_rmsnorm", "prefill_layer", "decode_layer_step",
    "prefill_conv_recurrence",
    "as_f64",
    "rms_norm_heads", "rope_inv_freq", "rope_angles", "apply_rotary", "text_positions", "qk_prep",
    "causal_attention", "causal_attention_rows", "attention_prefill", "attention_decode",
]
