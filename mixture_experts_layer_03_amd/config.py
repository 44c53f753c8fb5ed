"""Layer configuration with the Bailing/Ling MoE family's defaults.

Field names and defaults follow the model family's Hugging Face config as the
mlxcel #838 page describes it ("Config fields the checkpoint does not
contain"): n_group 1, score_function "softmax", no expert bias, routed scaling
factor 1.0; the shared expert is one MLP of width shared_dim *
num_shared_experts with shared_dim = moe_shared_expert_intermediate_size or
moe_intermediate_size, present when num_shared_experts > 0 and
moe_router_enable_shared_expert ("Shared experts are one wide MLP").
moe_router_enable_routed_scaling is read and ignored: upstream always scales
("moe_router_enable_routed_scaling is dead code upstream").  A config setting
norm_softmax true is rejected ("Vendor config keys upstream partly ignores").
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass, fields

from . import _lib

_DT = {"f32": _lib.DT_F32, "bf16": _lib.DT_BF16, "u8": _lib.DT_U8_AFFINE, "u4": _lib.DT_U4_AFFINE}
_SCORE = {"softmax": _lib.SCORE_SOFTMAX, "sigmoid": _lib.SCORE_SIGMOID}
_PATH = {"auto": _lib.PATH_AUTO, "decode": _lib.PATH_DECODE, "prefill": _lib.PATH_PREFILL}


@dataclass
class MoEConfig:
    hidden: int
    num_experts: int
    top_k: int
    moe_intermediate: int
    shared_intermediate: int = 0
    n_group: int = 1
    topk_group: int = 1
    score_function: str = "softmax"
    norm_topk_prob: bool = True
    use_expert_bias: bool = False
    routed_scaling_factor: float = 1.0
    act_dtype: str = "bf16"        # x, y, router, shared expert: "bf16" | "f32"
    expert_dtype: str = "bf16"     # routed experts: act_dtype, "u8" or "u4" (affine, group 64)
    quant_group: int = 64
    path: str = "auto"             # "auto" | "decode" | "prefill"

    @classmethod
    def from_hf_dict(cls, d: dict, act_dtype: str = "bf16", expert_dtype: str | None = None,
                     path: str = "auto") -> "MoEConfig":
        if d.get("norm_softmax", False):
            raise ValueError("norm_softmax=true: no released implementation defines it; "
                             "refusing the config")
        sf = d.get("score_function", "softmax")
        if sf not in _SCORE:
            raise ValueError(f"unknown score_function {sf!r} (softmax or sigmoid)")
        for key in ("hidden_size", "num_experts", "num_experts_per_tok", "moe_intermediate_size"):
            if key not in d:
                raise ValueError(f"config lacks {key}")
        moe_i = int(d["moe_intermediate_size"])
        shared_dim = d.get("moe_shared_expert_intermediate_size") or moe_i
        n_shared = int(d.get("num_shared_experts", 0) or 0)
        shared_on = bool(d.get("moe_router_enable_shared_expert", True))
        _ = d.get("moe_router_enable_routed_scaling")  # parsed, no effect (always scaled)
        rsf = d.get("routed_scaling_factor")
        return cls(
            hidden=int(d["hidden_size"]),
            num_experts=int(d["num_experts"]),
            top_k=int(d["num_experts_per_tok"]),
            moe_intermediate=moe_i,
            shared_intermediate=int(shared_dim) * n_shared if (n_shared > 0 and shared_on) else 0,
            n_group=int(d.get("n_group") or 1),
            topk_group=int(d.get("topk_group") or 1),
            score_function=sf,
            norm_topk_prob=bool(d.get("norm_topk_prob", True)),
            use_expert_bias=bool(d.get("moe_router_enable_expert_bias", False)),
            routed_scaling_factor=1.0 if rsf is None else float(rsf),
            act_dtype=act_dtype,
            expert_dtype=expert_dtype or act_dtype,
            path=path,
        )

    @classmethod
    def from_object(cls, obj, **overrides) -> "MoEConfig":
        """Config from any object carrying attributes with this class's field names."""
        kw = {f.name: getattr(obj, f.name) for f in fields(cls) if hasattr(obj, f.name)}
        kw.update(overrides)
        return cls(**kw)

    def to_c(self) -> _lib.moe_config:
        try:
            c = _lib.moe_config(
                hidden=int(self.hidden), num_experts=int(self.num_experts), top_k=int(self.top_k),
                moe_intermediate=int(self.moe_intermediate),
                shared_intermediate=int(self.shared_intermediate), n_group=int(self.n_group),
                topk_group=int(self.topk_group), score_function=_SCORE[self.score_function],
                norm_topk_prob=int(bool(self.norm_topk_prob)),
                use_expert_bias=int(bool(self.use_expert_bias)),
                routed_scaling_factor=float(self.routed_scaling_factor),
                act_dtype=_DT[self.act_dtype], router_dtype=_DT[self.act_dtype],
                expert_dtype=_DT[self.expert_dtype], shared_dtype=_DT[self.act_dtype],
                quant_group=int(self.quant_group), path=_PATH[self.path])
        except KeyError as e:
            raise ValueError(f"bad enumerated config value {e}") from None
        return c

    def validate(self) -> "MoEConfig":
        c = self.to_c()
        _lib.check(_lib.lib().moe_validate_config(C.byref(c)))
        return self

    def workspace_size(self, T: int) -> int:
        c = self.to_c()
        n = C.c_size_t(0)
        _lib.check(_lib.lib().moe_workspace_size(C.byref(c), int(T), C.byref(n)))
        return int(n.value)

    def kernel_path(self, T: int) -> str:
        """"decode" (weight-streaming kernels) or "prefill" (tiled GEMMs): the kernels a
        call with T tokens runs under this configuration."""
        c = self.to_c()
        v = C.c_int32(-1)
        _lib.check(_lib.lib().moe_select_path(C.byref(c), int(T), C.byref(v)))
        return "decode" if v.value == _lib.PATH_DECODE else "prefill"

    def as_dict(self) -> dict:
        return {f.name: getattr(self, f.name) for f in fields(self)}
