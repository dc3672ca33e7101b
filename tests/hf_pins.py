"""Build transformers models that carry our synthetic weights (CPU, float64).

Used only as black-box library references for the oracle: transformers'
Qwen3 decoder pins the layer (q/k norm, rotate-half RoPE, GQA head map, SwiGLU,
tied or untied head), and Qwen2-VL's multimodal rotary function pins the
section layout of the multi-section rotation.
"""
import contextlib

import numpy as np
import torch

from oracle import bf16_bits_to_float


def _t(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = bf16_bits_to_float(a)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def qwen3_from_weights(shape, weights):
    from transformers import Qwen3Config, Qwen3ForCausalLM

    cfg = Qwen3Config(
        vocab_size=shape.vocab, hidden_size=shape.hidden, intermediate_size=shape.intermediate,
        num_hidden_layers=shape.n_layers, num_attention_heads=shape.n_q_heads,
        num_key_value_heads=shape.n_kv_heads, head_dim=shape.head_dim, rms_norm_eps=shape.rms_eps,
        rope_parameters={"rope_type": "default", "rope_theta": shape.rope_theta},
        tie_word_embeddings=shape.tied, attn_implementation="eager",
        max_position_embeddings=max(4096, shape.capacity), attention_bias=False)
    m = Qwen3ForCausalLM(cfg).to(torch.float64).eval()
    sd = {"model.embed_tokens.weight": _t(weights["embed"]),
          "model.norm.weight": _t(weights["final_norm"])}
    sd["lm_head.weight"] = _t(weights["embed"] if shape.tied else weights["lm_head"])
    names = {"in_norm": "input_layernorm", "post_norm": "post_attention_layernorm",
             "wq": "self_attn.q_proj", "wk": "self_attn.k_proj", "wv": "self_attn.v_proj",
             "wo": "self_attn.o_proj", "q_norm": "self_attn.q_norm", "k_norm": "self_attn.k_norm",
             "w_gate": "mlp.gate_proj", "w_up": "mlp.up_proj", "w_down": "mlp.down_proj"}
    for l, lw in enumerate(weights["layers"]):
        for k, v in lw.items():
            sd[f"model.layers.{l}.{names[k]}.weight"] = _t(v)
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected, unexpected
    assert all(k == "lm_head.weight" for k in missing), missing
    if shape.tied:
        assert m.lm_head.weight.data_ptr() == m.model.embed_tokens.weight.data_ptr()
    return m


def layer_outputs(model):
    """Register hooks that record each decoder layer's output; returns (list, remover)."""
    outs = []
    hs = [lyr.register_forward_hook(lambda mod, a, o: outs.append(o[0] if isinstance(o, tuple) else o))
          for lyr in model.model.layers]
    return outs, lambda: [h.remove() for h in hs]


@contextlib.contextmanager
def multimodal_rotary(model, sections):
    """Swap the Qwen3 rotation for Qwen2-VL's multi-section one.

    The model's rotary module is replaced by Qwen2-VL's (which takes three
    position streams), and the rotation applied inside attention by
    ``apply_multimodal_rotary_pos_emb`` with the given sections.
    """
    import transformers.models.qwen3.modeling_qwen3 as q3
    from transformers import Qwen2VLTextConfig
    from transformers.models.qwen2_vl import modeling_qwen2_vl as q2

    c = model.config
    vcfg = Qwen2VLTextConfig(hidden_size=c.hidden_size, num_attention_heads=c.num_attention_heads,
                             num_key_value_heads=c.num_key_value_heads,
                             rope_parameters={"rope_type": "default",
                                              "rope_theta": c.rope_parameters["rope_theta"],
                                              "mrope_section": list(sections)},
                             max_position_embeddings=c.max_position_embeddings)
    vcfg.head_dim = c.head_dim          # read by Qwen2-VL's default inverse-frequency rule
    rot = q2.Qwen2VLRotaryEmbedding(vcfg)
    assert rot.inv_freq.numel() == c.head_dim // 2
    old_rot, old_apply = model.model.rotary_emb, q3.apply_rotary_pos_emb
    model.model.rotary_emb = rot
    q3.apply_rotary_pos_emb = lambda q, k, cos, sin, unsqueeze_dim=1: q2.apply_multimodal_rotary_pos_emb(
        q, k, cos, sin, list(sections), unsqueeze_dim)
    try:
        yield
    finally:
        model.model.rotary_emb, q3.apply_rotary_pos_emb = old_rot, old_apply
