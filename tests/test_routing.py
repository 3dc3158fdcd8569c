"""Routing of layers to quantization schemes (CPU only), pinned to the rules of
"vLLM-Omni Online Quantization complete guide", sections "Per-component routing"
and "Key parameters in detail"."""
import pytest

from precision_quantized_linear_amd import routing as R


def test_input_forms():
    assert R.build_quant_config(None) is None
    assert R.build_quant_config("none") is None and R.build_quant_config("None") is None
    c = R.build_quant_config("fp8")
    assert isinstance(c, R.MethodConfig) and c.scheme_for("blocks.0.attn.to_qkv") == "fp8_row"
    c = R.build_quant_config({"method": "fp8", "ignored_layers": ["img_mlp"]})
    assert c.ignored_layers == ["img_mlp"]
    c2 = R.build_quant_config("fp8", ignored_layers=["img_mlp"])          # keyword form
    assert c2.ignored_layers == ["img_mlp"]
    assert R.build_quant_config(c) is c                                     # an existing config
    assert R.build_quant_config({"quant_method": "int8"}).scheme == "int8_row"
    with pytest.raises(ValueError):
        R.build_quant_config(42)


def test_method_aliases_and_unknown_methods():
    for name in ("auto-round", "auto_round", "AUTO-ROUND", "Auto_Round"):
        assert R.canonical_method(name) == "auto_round"
    assert R.build_quant_config("MXFP8").scheme == "mxfp8"
    with pytest.raises(ValueError) as e:
        R.build_quant_config("nvfp4")
    assert "supported" in str(e.value) and "mxfp4" in str(e.value)


def test_per_component_longest_prefix_none_and_default():
    c = R.build_quant_config({"transformer": {"method": "fp8"}, "vae": None,
                              "transformer.blocks.0": "int8", "default": "mxfp8"})
    assert isinstance(c, R.ComponentConfig)
    assert c.scheme_for("transformer.blocks.1.ff") == "fp8_row"
    assert c.scheme_for("transformer.blocks.0.ff") == "int8_row"          # longer prefix wins
    assert c.scheme_for("transformer.blocks.01.ff") == "fp8_row"          # whole components only
    assert c.scheme_for("vae.decoder.conv") is None                       # None: unquantized
    assert c.scheme_for("text_encoder.layers.0") == "mxfp8"               # default
    no_default = R.build_quant_config({"transformer": "fp8", "vae": None})
    assert no_default.scheme_for("text_encoder.layers.0") is None


def test_per_component_detection():
    # a dict with a method key is a flat config, even if other values look like components
    c = R.build_quant_config({"method": "fp8", "ignored_layers": ["to_out"]})
    assert isinstance(c, R.MethodConfig)
    with pytest.raises(ValueError):
        R.build_quant_config({"transformer": 3})       # not str / dict / None: not per-component, no method


def test_ignored_layers_all_methods():
    for m in ("fp8", "int8", "mxfp8", "mxfp4", "auto_round"):
        c = R.build_quant_config({"method": m, "ignored_layers": ["img_mlp", "to_out"]})
        assert c.scheme_for("blocks.3.img_mlp.net.0.proj") is None
        assert c.scheme_for("blocks.3.attn.to_out.0") is None
        assert c.scheme_for("blocks.3.img_mlp2") is not None
        assert c.scheme_for("blocks.3.attn.to_qkv") is not None


def test_activation_scheme_rules():
    with pytest.raises(ValueError):
        R.build_quant_config({"method": "int8", "activation_scheme": "static"})
    c = R.build_quant_config({"method": "fp8", "scheme": "fp8_tensor", "activation_scheme": "static"})
    assert c.scheme_for("blocks.0.ff") == "fp8_tensor"
    with pytest.raises(ValueError):   # no static per-row scheme
        R.build_quant_config({"method": "fp8", "activation_scheme": "static"})
    with pytest.raises(ValueError):
        R.build_quant_config({"method": "fp8", "scheme": "mxfp8"})


def test_dualscale_fallback_priority():
    c = R.build_quant_config({"method": "mxfp4-dualscale", "ignored_layers": ["blocks.7.ffn"]})
    assert c.num_bf16_fallback_layers == 5                               # the default
    assert all(c.scheme_for(f"blocks.{i}.attn.to_q") is None for i in range(5))   # rule 2
    assert c.scheme_for("blocks.7.ffn.net.0") is None                    # rule 1, anywhere
    assert c.scheme_for("blocks.5.attn.to_q") == "mxfp4_dual"           # rule 3: the dual-scale kernel
    assert c.scheme_for("condition_embedder.linear_1") == "mxfp4_dual"  # outside blocks.N: quantized
    c0 = R.build_quant_config({"method": "mxfp4_dualscale", "num_bf16_fallback_layers": 0})
    assert c0.scheme_for("blocks.0.attn.to_q") == "mxfp4_dual"
    with pytest.raises(ValueError):
        R.build_quant_config({"method": "mxfp4_dualscale", "num_bf16_fallback_layers": -1})


def test_every_routed_scheme_is_a_library_scheme():
    import precision_quantized_linear_amd as pql
    for m, choices in R.SCHEME_CHOICES.items():
        for s in choices:
            assert s in pql.SCHEMES, (m, s)
        if R.METHODS[m] is not None:
            assert R.METHODS[m] in pql.SCHEMES
