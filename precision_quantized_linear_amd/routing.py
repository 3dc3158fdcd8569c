"""Which layers of a model get which quantization scheme (host logic only).

This is the routing layer above the quantized-linear kernels: given a
quantization spec and a layer's runtime prefix (its name after weight-name
mapping, e.g. "transformer.blocks.3.attn.to_qkv"), it answers with the
library scheme that layer runs (``"fp8_row"``, ``"mxfp8"``, ...) or ``None``
for "keep the checkpoint's bf16 weights".  It follows "vLLM-Omni Online
Quantization complete guide", sections "Per-component routing" and "Key
parameters in detail":

* a spec is ``None`` / ``"none"``, a method name, a flat dict with a
  ``"method"`` key and extra parameters (``ignored_layers``,
  ``activation_scheme``, ``num_bf16_fallback_layers``), a per-component dict
  (no ``method`` / ``quant_method`` key, every value a str, dict or None), or
  an already-built config;
* method names are case-insensitive and treat ``-`` and ``_`` alike; an
  unknown method is a ``ValueError`` that lists the supported ones;
* per-component keys are runtime layer prefixes; the longest matching prefix
  wins; a ``None`` value keeps the matched component unquantized; a
  ``"default"`` key handles prefixes nothing else matches; the matched
  sub-config decides for the layer;
* ``ignored_layers`` keeps every layer whose prefix contains one of the names
  unquantized (all methods);
* int8 accepts dynamic activation scales only (a static scheme is a
  ``ValueError``); FP8 takes ``"static"`` when calibrated scales exist;
* ``num_bf16_fallback_layers`` (dual-scale MXFP4 only, default 5) keeps the
  first N transformer blocks (``blocks.<i>.`` with i < N) in bf16 after the
  explicit ``ignored_layers``.

Readings where the page is silent: an ignored-layer name matches a layer when
it equals one dot-separated component run of the prefix (``"img_mlp"``
matches ``"blocks.0.img_mlp.net.0"`` but not ``"blocks.0.img_mlp2"``); a
prefix key matches a layer when the layer equals it or continues it at a dot.
The method names map to this library's schemes as: fp8 -> fp8_row (dynamic
per-token activations, per-channel weights; fp8_tensor / fp8_block128 are
selected with ``"scheme"``), int8 -> int8_row, mxfp8 -> mxfp8, mxfp4 ->
mxfp4, mxfp4_dualscale -> mxfp4_dual (online: the calibrated multiplier is
all ones), auto_round / inc -> w4a16_asym.
"""
from __future__ import annotations

import re
from dataclasses import dataclass, field

# canonical method name -> default library scheme
METHODS = {
    "fp8": "fp8_row",
    "int8": "int8_row",
    "mxfp8": "mxfp8",
    "mxfp4": "mxfp4",
    "mxfp4_dualscale": "mxfp4_dual",
    "auto_round": "w4a16_asym",
    "inc": "w4a16_asym",
}
# schemes a spec may name explicitly for a method
SCHEME_CHOICES = {
    "fp8": ("fp8_tensor", "fp8_row", "fp8_block128"),
    "int8": ("int8_row",),
    "mxfp8": ("mxfp8",),
    "mxfp4": ("mxfp4",),
    "mxfp4_dualscale": ("mxfp4_dual",),
    "auto_round": ("w4a16_asym", "w4a16_sym"),
    "inc": ("w4a16_asym", "w4a16_sym"),
}
_BLOCK_RE = re.compile(r"^blocks\.(\d+)\.")


def canonical_method(name: str) -> str:
    """Case-insensitive, '-' and '_' equivalent; ValueError for unknown methods."""
    key = str(name).strip().lower().replace("-", "_")
    if key not in METHODS:
        raise ValueError(f"unknown quantization method {name!r}; supported: {sorted(METHODS)}")
    return key


def _names_match(name: str, prefix: str) -> bool:
    parts, want = prefix.split("."), name.split(".")
    return any(parts[i:i + len(want)] == want for i in range(len(parts) - len(want) + 1))


def _prefix_match(key: str, prefix: str) -> bool:
    return prefix == key or prefix.startswith(key + ".")


@dataclass
class MethodConfig:
    """One quantization method with its parameters."""
    method: str
    scheme: str | None = None
    ignored_layers: list = field(default_factory=list)
    activation_scheme: str = "dynamic"
    num_bf16_fallback_layers: int = 5

    def __post_init__(self):
        self.method = canonical_method(self.method)
        choices = SCHEME_CHOICES[self.method]
        if self.scheme is None:
            self.scheme = METHODS[self.method]
        elif self.scheme not in choices:
            raise ValueError(f"method {self.method!r} runs schemes {choices}, not {self.scheme!r}")
        if self.activation_scheme not in ("dynamic", "static"):
            raise ValueError(f"activation_scheme must be 'dynamic' or 'static', not {self.activation_scheme!r}")
        if self.activation_scheme == "static":
            if self.method == "int8":
                raise ValueError("int8 supports dynamic activation scales only")
            if self.method != "fp8" or self.scheme not in ("fp8_tensor", "fp8_block128"):
                raise ValueError("static activation scales exist for fp8 per-tensor and per-128-block scales only")
        if isinstance(self.ignored_layers, str):
            self.ignored_layers = [self.ignored_layers]
        self.ignored_layers = list(self.ignored_layers or [])
        if int(self.num_bf16_fallback_layers) < 0:
            raise ValueError("num_bf16_fallback_layers must be >= 0")
        self.num_bf16_fallback_layers = int(self.num_bf16_fallback_layers)

    def scheme_for(self, prefix: str) -> str | None:
        """The library scheme for the layer at ``prefix``, or None to keep it in bf16."""
        if any(_names_match(n, prefix) for n in self.ignored_layers):
            return None
        if self.method == "mxfp4_dualscale":
            m = _BLOCK_RE.match(prefix)
            if m and int(m.group(1)) < self.num_bf16_fallback_layers:
                return None
        return self.scheme


@dataclass
class ComponentConfig:
    """Per-component routing: {layer prefix: MethodConfig or None}, longest prefix first."""
    components: dict
    default: MethodConfig | None = None

    def route(self, prefix: str):
        """The sub-config that decides for ``prefix`` (None: unquantized)."""
        for key in sorted(self.components, key=len, reverse=True):
            if _prefix_match(key, prefix):
                return self.components[key]
        return self.default

    def scheme_for(self, prefix: str) -> str | None:
        sub = self.route(prefix)
        return None if sub is None else sub.scheme_for(prefix)   # the sub-config sees the same prefix


def _is_per_component(spec: dict) -> bool:
    return ("method" not in spec and "quant_method" not in spec
            and all(v is None or isinstance(v, (str, dict)) for v in spec.values()))


def build_quant_config(spec=None, **extra):
    """Resolve a spec into None, a MethodConfig or a ComponentConfig."""
    if isinstance(spec, (MethodConfig, ComponentConfig)):
        if extra:
            raise ValueError("extra parameters apply to a method name or a flat dict, not a built config")
        return spec
    if spec is None or (isinstance(spec, str) and spec.strip().lower() == "none"):
        if extra:
            raise ValueError("extra parameters given without a method")
        return None
    if isinstance(spec, str):
        return MethodConfig(spec, **extra)
    if not isinstance(spec, dict):
        raise ValueError(f"cannot build a quantization config from {type(spec).__name__}")
    if _is_per_component(spec):
        if extra:
            raise ValueError("extra parameters apply to a flat config, not a per-component dict")
        comps, default = {}, None
        for k, v in spec.items():
            sub = build_quant_config(v)
            if k == "default":
                default = sub
            else:
                comps[k] = sub
        return ComponentConfig(comps, default)
    d = dict(spec)
    method = d.pop("method", None) or d.pop("quant_method", None)
    if method is None:
        raise ValueError("a flat config needs a 'method'")
    d.update(extra)
    return MethodConfig(method, **d)
