"""The layer constants the pages state (tests/golden/layer_constants.json, each cited) against the
generators, the oracle and the library's supported set.  CPU only."""
import json
import os

import numpy as np

import oracle
from synth import LAYER, ATTN

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "layer_constants.json")
G = json.load(open(GOLDEN))


def test_delta_layer_shapes_follow_the_pages():
    d = G["delta_layer"]
    assert (LAYER["num_k_heads"], LAYER["num_v_heads"], LAYER["head_dim"]) == (d["num_k_heads"], d["num_v_heads"],
                                                                             d["head_dim"])
    assert LAYER["conv_kernel"] == d["conv_kernel"]
    assert LAYER["chunk"] == G["delta_chunk"]["chunk"]
    assert LAYER["hidden"] == G["hidden"]["hidden_size"]
    assert LAYER["conv_channels"] == (2 * d["num_k_heads"] + d["num_v_heads"]) * d["head_dim"]


def test_layer_counts_add_up():
    l = G["layers"]
    assert l["delta_layers"] + l["global_layers"] == l["decoder_layers"]
    assert l["decoder_layers"] // l["global_attention_interval"] == l["global_layers"]


def test_attention_shapes_and_rotary_follow_the_pages():
    a, r = G["global_attention"], G["rotary"]
    assert (ATTN["num_q_heads"], ATTN["num_kv_heads"], ATTN["head_dim"]) == (a["num_q_heads"], a["num_kv_heads"],
                                                                           a["head_dim"])
    assert oracle.attention.HEAD_DIM == a["head_dim"]
    assert ATTN["rot_dim"] == oracle.attention.ROT_DIM == r["rot_dim"] == int(r["fraction_of_head_dim"] * a["head_dim"])
    assert ATTN["rope_base"] == oracle.attention.ROPE_BASE == r["base"]
    # the oracle's axis of each of the 32 frequencies splits them as the pages' sections
    axis = np.arange(r["rot_dim"] // 2) % 3
    assert [int((axis == k).sum()) for k in range(3)] == r["sections"]


def test_longest_context_fits_the_rotary_position_range():
    """The rotary angles of the longest context stay finite and distinct at fp64 (the library
    forms them in fp64)."""
    p = G["context_length"]["tokens"] - 1
    ang = oracle.rope_angles(np.full((3, 2), [p - 1, p]))
    assert np.isfinite(ang).all() and (ang[1] > ang[0]).all()
