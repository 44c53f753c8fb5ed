"""The C ABI on the host (no GPU): the library loads, exports every declared
symbol, and rejects each invalid configuration with the documented status.

One rejection test per rule of the pages' defensive requirements (mlxcel #838
"Defensive requirements": magnitude ceilings, zero checks before divisibility,
routing bounds), plus the config-file mapping (defaults of "Config fields the
checkpoint does not contain", the dead routed-scaling flag, norm_softmax).
"""
import ctypes as C
import os
import re

import pytest

import mixture_experts_layer_03_amd as moe
from mixture_experts_layer_03_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    names = header_functions()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/moe.h but not exported"
    assert L.moe_abi_version() == 1


def test_struct_layout_matches_header():
    # int64 x7, int32 x3, float, int32 x4, int64, int32 (+ padding) as declared
    assert C.sizeof(_lib.moe_config) == 7 * 8 + 3 * 4 + 4 + 4 * 4 + 8 + 8
    assert C.sizeof(_lib.moe_weights) == 15 * 8


def test_config_default_values():
    c = _lib.moe_config()
    assert _lib.lib().moe_config_default(C.byref(c)) == 0
    assert (c.n_group, c.topk_group, c.score_function, c.norm_topk_prob, c.use_expert_bias) == (1, 1, 0, 1, 0)
    assert c.routed_scaling_factor == 1.0 and c.quant_group == 64 and c.path == 0
    assert c.act_dtype == c.expert_dtype == c.router_dtype == c.shared_dtype == _lib.DT_BF16


def good(**kw):
    base = dict(hidden=2048, num_experts=64, top_k=6, moe_intermediate=1408, shared_intermediate=2816)
    base.update(kw)
    return moe.MoEConfig(**base)


def status_of(cfg):
    c = cfg.to_c()
    return _lib.lib().moe_validate_config(C.byref(c)), _lib.lib().moe_last_error().decode()


def test_valid_configs_of_every_workload():
    import synth
    for spec in synth.SPECS.values():
        assert status_of(moe.MoEConfig.from_object(spec)) == (0, "")


@pytest.mark.parametrize("kw,field", [
    (dict(hidden=0), "hidden"), (dict(hidden=16384 + 64), "hidden"), (dict(hidden=-64), "hidden"),
    (dict(num_experts=0), "num_experts"), (dict(num_experts=1025), "num_experts"),
    (dict(moe_intermediate=0), "moe_intermediate"), (dict(moe_intermediate=32768 + 64), "moe_intermediate"),
    (dict(shared_intermediate=-1), "shared_intermediate"),
    (dict(shared_intermediate=32768 + 64), "shared_intermediate"),
    (dict(top_k=0), "top_k"), (dict(top_k=65, num_experts=64), "top_k"), (dict(top_k=17), "top_k"),
    (dict(n_group=0), "n_group"), (dict(n_group=65, num_experts=64), "n_group"),
    (dict(n_group=3), "divisible"),
    (dict(n_group=64), "group score needs two"),
    (dict(n_group=8, topk_group=0), "topk_group"), (dict(n_group=8, topk_group=9), "topk_group"),
    (dict(topk_group=2), "topk_group"),
    (dict(n_group=8, topk_group=1, top_k=9), "kept groups"),
    (dict(routed_scaling_factor=0.0), "routed_scaling_factor"),
    (dict(routed_scaling_factor=-1.0), "routed_scaling_factor"),
    (dict(routed_scaling_factor=float("nan")), "routed_scaling_factor"),
    (dict(routed_scaling_factor=float("inf")), "routed_scaling_factor"),
    (dict(expert_dtype="u8", quant_group=32), "quant_group"),
    (dict(act_dtype="f32", expert_dtype="u8"), "expert_dtype"),
    (dict(expert_dtype="u4", quant_group=128), "quant_group"),
    (dict(act_dtype="f32", expert_dtype="u4"), "expert_dtype"),
    (dict(act_dtype="f32", expert_dtype="bf16"), "expert_dtype"),
])
def test_invalid_config_rejected(kw, field):
    st, msg = status_of(good(**kw))
    assert st == _lib.MOE_EINVAL_CONFIG, (st, msg)
    assert field in msg, msg


def test_zero_group_count_checked_before_divisibility():
    # n_group = 0 must be reported as a range error, never reach "E % n_group"
    st, msg = status_of(good(n_group=0))
    assert st == _lib.MOE_EINVAL_CONFIG and "n_group" in msg and "divisible" not in msg


def test_raw_struct_rejections():
    L = _lib.lib()
    for field, val, word in (("score_function", 2, "score_function"), ("norm_topk_prob", 2, "norm_topk_prob"),
                             ("use_expert_bias", 7, "use_expert_bias"), ("path", 3, "path"),
                             ("router_dtype", _lib.DT_F32, "router_dtype"),
                             ("shared_dtype", _lib.DT_F32, "shared_dtype"), ("act_dtype", 9, "act_dtype")):
        c = good().to_c()
        setattr(c, field, val)
        assert L.moe_validate_config(C.byref(c)) == _lib.MOE_EINVAL_CONFIG
        assert word in L.moe_last_error().decode()
    assert L.moe_validate_config(None) == _lib.MOE_EINVAL_ARG


@pytest.mark.parametrize("kw", [dict(hidden=2048 + 32), dict(moe_intermediate=1400),
                                dict(shared_intermediate=100), dict(path="prefill", act_dtype="f32",
                                                                    expert_dtype="f32")])
def test_unsupported_but_valid(kw):
    st, _ = status_of(good(**kw))
    assert st == _lib.MOE_EUNSUPPORTED


U4 = dict(expert_dtype="u4", moe_intermediate=1024)


@pytest.mark.parametrize("kw,word", [(dict(hidden=2048 + 64), "128"), (dict(moe_intermediate=1472), "128"),
                                     (dict(path="prefill"), "streaming")])
def test_u4_limits(kw, word):
    """u4 experts: only the weight-streaming kernels exist, stepping 128 elements."""
    st, msg = status_of(good(**{**U4, **kw}))
    assert st == _lib.MOE_EUNSUPPORTED and word in msg, (st, msg)
    assert status_of(good(**U4)) == (0, "")
    assert status_of(good(**U4, path="decode")) == (0, "")


def test_u4_weight_checks_before_any_launch():
    """u4 group parameters are copied two at a time: 2-byte aligned is not enough."""
    L = _lib.lib()
    c = good(**U4).to_c()
    fake = C.c_void_p(0x1000)
    full = dict(router=0x1000, gate=0x1000, up=0x1000, down=0x1000, shared_gate=0x1000, shared_up=0x1000,
                shared_down=0x1000, gate_scale=0x1000, gate_zero=0x1000, up_scale=0x1000, up_zero=0x1000,
                down_scale=0x1000, down_zero=0x1000)
    w = _lib.moe_weights(**{**full, "down_zero": None})
    st = L.moe_experts(C.byref(c), 4, fake, C.byref(w), fake, fake, fake, fake, 1 << 30, None)
    assert st == _lib.MOE_EINVAL_ARG and "down_zero" in L.moe_last_error().decode()
    w = _lib.moe_weights(**{**full, "up_scale": 0x1002})
    st = L.moe_experts(C.byref(c), 4, fake, C.byref(w), fake, fake, fake, fake, 1 << 30, None)
    assert st == _lib.MOE_EINVAL_ARG and "up_scale" in L.moe_last_error().decode()


def test_workspace_size_and_T_bounds():
    cfg = good()
    assert cfg.workspace_size(0) >= 0
    a, b = cfg.workspace_size(64), cfg.workspace_size(4096)
    assert 0 < a < b
    with pytest.raises(moe.MoEError) as e:
        cfg.workspace_size(-1)
    assert e.value.status == _lib.MOE_EINVAL_ARG
    with pytest.raises(moe.MoEError):
        cfg.workspace_size((1 << 20) + 1)


def test_path_choice():
    """The automatic path streams up to 64 tokens or at most min(20, 40960 / H) routed
    tokens per expert on average (20 at hidden 2048, 10 at 4096); u4 experts and fp32
    layers always stream; a forced path is kept."""
    import synth
    spec2, spec4 = synth.SPECS[2], synth.SPECS[4]           # H 2048 E 64 k 6; H 4096 E 512 k 8
    c2, c4 = moe.MoEConfig.from_object(spec2), moe.MoEConfig.from_object(spec4)
    assert [c2.kernel_path(T) for T in (1, 64, 213, 214, 4096)] == \
        ["decode", "decode", "decode", "prefill", "prefill"]
    assert [c4.kernel_path(T) for T in (8, 640, 641, 8192)] == ["decode", "decode", "prefill", "prefill"]
    assert moe.MoEConfig.from_object(synth.SPECS[6]).kernel_path(8192) == "decode"   # u4
    assert moe.MoEConfig.from_object(synth.SPECS[1]).kernel_path(4096) == "decode"   # fp32
    assert moe.MoEConfig.from_object(spec2, path="prefill").kernel_path(1) == "prefill"
    assert moe.MoEConfig.from_object(spec2, path="decode").kernel_path(4096) == "decode"
    c = c2.to_c()
    v = C.c_int32(-1)
    assert _lib.lib().moe_select_path(C.byref(c), 64, None) == _lib.MOE_EINVAL_ARG
    assert _lib.lib().moe_select_path(C.byref(c), -1, C.byref(v)) == _lib.MOE_EINVAL_ARG
    assert _lib.lib().moe_select_path(None, 64, C.byref(v)) == _lib.MOE_EINVAL_ARG


def test_entry_points_reject_bad_arguments_before_any_launch():
    """Null pointers, too-small workspace: refused on the host, nothing touches a device."""
    L = _lib.lib()
    c = good().to_c()
    fake = C.c_void_p(0x1000)          # never dereferenced: checks fail first
    ws_need = good().workspace_size(4)
    st = L.moe_route(C.byref(c), 4, None, fake, None, None, fake, fake, fake, ws_need, None)
    assert st == _lib.MOE_EINVAL_ARG and "x" in L.moe_last_error().decode()
    st = L.moe_route(C.byref(c), 4, C.c_void_p(0x1001), fake, None, None, fake, fake, fake, ws_need, None)
    assert st == _lib.MOE_EINVAL_ARG and "aligned" in L.moe_last_error().decode()
    st = L.moe_route(C.byref(c), 4, fake, fake, None, None, fake, fake, fake, ws_need - 1, None)
    assert st == _lib.MOE_EWORKSPACE
    st = L.moe_route(C.byref(c), 4, fake, fake, None, None, fake, fake, C.c_void_p(0x1010), ws_need, None)
    assert st == _lib.MOE_EWORKSPACE   # not 256-byte aligned
    st = L.moe_route(C.byref(c), -3, fake, fake, None, None, fake, fake, fake, ws_need, None)
    assert st == _lib.MOE_EINVAL_ARG
    # T == 0 is a valid no-op even with null pointers
    assert L.moe_route(C.byref(c), 0, None, None, None, None, None, None, None, 0, None) == 0
    w = _lib.moe_weights()
    st = L.moe_forward(C.byref(c), 4, fake, C.byref(w), fake, None, None, None, fake, ws_need, None)
    assert st == _lib.MOE_EINVAL_ARG and "router" in L.moe_last_error().decode()
    cb = good(use_expert_bias=True).to_c()
    st = L.moe_route(C.byref(cb), 4, fake, fake, None, None, fake, fake, fake, ws_need, None)
    assert st == _lib.MOE_EINVAL_ARG and "expert_bias" in L.moe_last_error().decode()
    cu8 = good(expert_dtype="u8").to_c()
    w = _lib.moe_weights(router=0x1000, gate=0x1000, up=0x1000, down=0x1000, shared_gate=0x1000,
                         shared_up=0x1000, shared_down=0x1000)
    st = L.moe_experts(C.byref(cu8), 4, fake, C.byref(w), fake, fake, fake, fake, 1 << 30, None)
    assert st == _lib.MOE_EINVAL_ARG and "scale" in L.moe_last_error().decode()
    assert L.moe_profile_collect(1, None, None) == _lib.MOE_EINVAL_ARG
    assert L.moe_profile_enable(1, 0) == _lib.MOE_EINVAL_ARG


def test_status_strings():
    L = _lib.lib()
    for s in range(6):
        assert L.moe_status_str(s)
    assert L.moe_status_str(99) == b"unknown status"


# ------------------------------------------------------------ config mapping
LING_LITE = {  # the fields the validation checkpoint's config carries (mlxcel #838)
    "hidden_size": 2048, "intermediate_size": 1408, "moe_intermediate_size": 1408, "num_experts": 64,
    "num_experts_per_tok": 6, "num_shared_experts": 2, "norm_topk_prob": True,
}


def test_hf_config_defaults():
    cfg = moe.MoEConfig.from_hf_dict(LING_LITE)
    assert cfg.n_group == 1 and cfg.topk_group == 1 and cfg.score_function == "softmax"
    assert not cfg.use_expert_bias and cfg.routed_scaling_factor == 1.0
    assert cfg.shared_intermediate == 2816          # 1408 * 2 (one wide MLP)
    cfg.validate()


def test_hf_shared_expert_switches():
    assert moe.MoEConfig.from_hf_dict(dict(LING_LITE, num_shared_experts=0)).shared_intermediate == 0
    assert moe.MoEConfig.from_hf_dict(dict(LING_LITE, moe_router_enable_shared_expert=False)).shared_intermediate == 0
    assert moe.MoEConfig.from_hf_dict(dict(LING_LITE, moe_shared_expert_intermediate_size=512)).shared_intermediate == 1024


def test_hf_routed_scaling_flag_is_ignored():
    # upstream always scales; the flag is parsed and has no effect
    cfg = moe.MoEConfig.from_hf_dict(dict(LING_LITE, routed_scaling_factor=2.5,
                                          moe_router_enable_routed_scaling=False))
    assert cfg.routed_scaling_factor == 2.5


def test_hf_rejects_norm_softmax_and_unknown_score_function():
    with pytest.raises(ValueError, match="norm_softmax"):
        moe.MoEConfig.from_hf_dict(dict(LING_LITE, norm_softmax=True))
    moe.MoEConfig.from_hf_dict(dict(LING_LITE, norm_softmax=False))
    with pytest.raises(ValueError, match="score_function"):
        moe.MoEConfig.from_hf_dict(dict(LING_LITE, score_function="relu"))
    assert moe.MoEConfig.from_hf_dict(dict(LING_LITE, score_function="sigmoid")).score_function == "sigmoid"


def test_hf_grouped_fields():
    cfg = moe.MoEConfig.from_hf_dict(dict(LING_LITE, num_experts=256, num_experts_per_tok=8, n_group=8,
                                          topk_group=4, score_function="sigmoid",
                                          moe_router_enable_expert_bias=True))
    assert (cfg.n_group, cfg.topk_group, cfg.use_expert_bias) == (8, 4, True)
    cfg.validate()


def test_python_shape_checks_use_real_shapes():
    import torch
    from mixture_experts_layer_03_amd.layer import check_weights
    cfg = moe.MoEConfig(hidden=128, num_experts=4, top_k=2, moe_intermediate=64)
    w = moe.MoEWeights(router=torch.zeros(5, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="router has shape"):
        check_weights(cfg, w, torch.device("cpu"), need_router=True, need_experts=False)
    w = moe.MoEWeights(router=torch.zeros(4, 128, dtype=torch.float32))
    with pytest.raises(ValueError, match="dtype"):
        check_weights(cfg, w, torch.device("cpu"), need_router=True, need_experts=False)


# ------------------------------------------------------------ dense MLP entry points
def dense_status(cfg, I, T=4):
    n = C.c_size_t(0)
    c = cfg.to_c()
    return _lib.lib().moe_dense_workspace_size(C.byref(c), I, T, C.byref(n)), _lib.lib().moe_last_error().decode(), n.value


def test_dense_workspace_and_validation():
    assert dense_status(good(), 9216)[0] == 0
    assert dense_status(good(), 9216, T=0)[0] == 0
    st, msg, _ = dense_status(good(), 100)
    assert st == _lib.MOE_EUNSUPPORTED and "multiples of 64" in msg
    st, msg, _ = dense_status(good(), 0)
    assert st == _lib.MOE_EINVAL_ARG and "intermediate" in msg
    st, msg, _ = dense_status(good(), 32768 + 64)
    assert st == _lib.MOE_EINVAL_ARG
    st, msg, _ = dense_status(good(act_dtype="f32", expert_dtype="f32", path="prefill"), 256)
    assert st == _lib.MOE_EUNSUPPORTED and "BF16" in msg
    st, _, _ = dense_status(good(), 256, T=-1)
    assert st == _lib.MOE_EINVAL_ARG
    # routing fields are not read: a configuration the layer would reject is fine here
    c = good().to_c()
    c.top_k = 99
    n = C.c_size_t(0)
    assert _lib.lib().moe_dense_workspace_size(C.byref(c), 256, 4, C.byref(n)) == 0
    # the streaming path (T <= 192) keeps an fp32 output buffer, the tiled path does not
    assert dense_status(good(), 256, T=192)[2] > dense_status(good(), 256, T=193)[2]
    assert _lib.lib().moe_dense_workspace_size(None, 256, 4, C.byref(n)) == _lib.MOE_EINVAL_ARG


def test_dense_rejects_bad_arguments_before_any_launch():
    L = _lib.lib()
    c = good().to_c()
    fake = C.c_void_p(0x1000)
    need = dense_status(good(), 256)[2]
    st = L.moe_dense_mlp(C.byref(c), 256, 4, None, fake, fake, fake, fake, fake, need, None)
    assert st == _lib.MOE_EINVAL_ARG and "x" in L.moe_last_error().decode()
    st = L.moe_dense_mlp(C.byref(c), 256, 4, fake, C.c_void_p(0x1008), fake, fake, fake, fake, need, None)
    assert st == _lib.MOE_EINVAL_ARG and "gate" in L.moe_last_error().decode()
    st = L.moe_dense_mlp(C.byref(c), 256, 4, fake, fake, fake, None, fake, fake, need, None)
    assert st == _lib.MOE_EINVAL_ARG and "down" in L.moe_last_error().decode()
    st = L.moe_dense_mlp(C.byref(c), 256, 4, fake, fake, fake, fake, fake, fake, need - 1, None)
    assert st == _lib.MOE_EWORKSPACE
    st = L.moe_dense_mlp(C.byref(c), 256, 4, fake, fake, fake, fake, fake, C.c_void_p(0x1010), need, None)
    assert st == _lib.MOE_EWORKSPACE
    assert L.moe_dense_mlp(C.byref(c), 256, 0, None, None, None, None, None, None, 0, None) == 0
    # the tiled path's 32-bit operand offsets
    big = 1 << 20
    st = L.moe_dense_mlp(C.byref(good(path="prefill").to_c()), 32768, big, fake, fake, fake, fake, fake, fake,
                         1 << 62, None)
    assert st == _lib.MOE_EUNSUPPORTED


def test_noalloc_rejects_calls_beyond_its_scratch_on_the_host():
    """moe_forward_noalloc refuses a call whose workspace exceeds the fixed scratch, on
    the host, before touching the GPU, naming the bytes needed (no GPU in this test)."""
    cfg = good()
    T = 4096
    need = cfg.workspace_size(T)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    c = cfg.to_c()
    wc = _lib.moe_weights(**{n: 256 for n, _ in _lib.moe_weights._fields_})  # never dereferenced
    st = _lib.lib().moe_forward_noalloc(C.byref(c), T, 256, C.byref(wc), 256, None, None, None, None)
    msg = _lib.lib().moe_last_error().decode()
    assert st == _lib.MOE_EWORKSPACE and str(need) in msg, (st, msg)
    # argument checks come first, as in moe_forward
    st = _lib.lib().moe_forward_noalloc(C.byref(c), T, 8, C.byref(wc), 256, None, None, None, None)
    assert st == _lib.MOE_EINVAL_ARG and "x" in _lib.lib().moe_last_error().decode()
    assert _lib.lib().moe_forward_noalloc(C.byref(c), 0, None, C.byref(wc), None, None, None, None, None) == 0
