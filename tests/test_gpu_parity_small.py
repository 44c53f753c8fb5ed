"""GPU parity on reduced layers (same routing structure as the workloads,
small hidden/intermediate sizes) against the fp64 oracle, through the C ABI.

Every case spans several tiles and ragged tails; the oracle runs on every token.
"""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as om
import synth
from gpu_util import (SMALL, check_forward, check_route, device_weights, log, moe_cfg,
                      oracle_cfg, to_dev, y_to_f64)

pytestmark = pytest.mark.gpu

_CACHE = {}


def layer(cid):
    if cid not in _CACHE:
        spec = SMALL[cid]
        L = synth.make_layer(spec)
        _CACHE[cid] = (spec, L, device_weights(L))
    return _CACHE[cid]


def xs(spec, T):
    x = synth.make_x(spec, T)
    return x, to_dev(x)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5, 7])
@pytest.mark.parametrize("T", [1, 7, 64, 300])
def test_route(cid, T):
    import mixture_experts_layer_03_amd as moe
    spec, L, W = layer(cid)
    x, xd = xs(spec, T)
    log(f"route cfg{cid} {spec.name} T={T}")
    idx, w = moe.route(xd, W.router, moe_cfg(spec), W.router_bias, W.expert_bias)
    torch.cuda.synchronize()
    st = check_route(spec, idx.cpu().numpy(), w.cpu().numpy(), L, x)
    log(f"  ok: near-ties {st['near_ties']}/{st['tokens']}, masked picks {st['masked_picks']}")


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
@pytest.mark.parametrize("T", [5, 300])
def test_permute(cid, T):
    import mixture_experts_layer_03_amd as moe
    spec, L, W = layer(cid)
    x, xd = xs(spec, T)
    log(f"permute cfg{cid} T={T}")
    cfg = moe_cfg(spec)
    idx, _ = moe.route(xd, W.router, cfg, W.router_bias, W.expert_bias)
    counts, offsets, perm = moe.permute(idx, cfg)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    c_o, off_o = om.expert_counts(idx_h, spec.num_experts)
    assert np.array_equal(counts.cpu().numpy(), c_o)
    assert np.array_equal(offsets.cpu().numpy(), off_o)
    perm_h = perm.cpu().numpy()
    for e, slots in enumerate(om.expert_slots(idx_h, spec.num_experts)):
        got = np.sort(perm_h[off_o[e]:off_o[e + 1]])
        assert np.array_equal(got, slots), f"expert {e}"


@pytest.mark.parametrize("T,E,k", [(1000, 40, 8), (2049, 512, 8), (600, 7, 7)])
def test_permute_multi_block(T, E, k):
    """Slot counts above one workgroup's share (2048-slot chunks, ragged last chunk),
    with some dropped slots."""
    import mixture_experts_layer_03_amd as moe
    cfg = moe.MoEConfig(hidden=64, num_experts=E, top_k=k, moe_intermediate=64)
    rng = np.random.default_rng(T + E)
    idx_h = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx_h[rng.random((T, k)) < 0.01] = -7
    log(f"permute multi-block T={T} E={E} k={k}")
    counts, offsets, perm = moe.permute(torch.from_numpy(idx_h).cuda(), cfg)
    torch.cuda.synchronize()
    valid = (idx_h >= 0) & (idx_h < E)
    c_o = np.bincount(idx_h[valid], minlength=E)
    assert np.array_equal(counts.cpu().numpy(), c_o)
    off_o = np.concatenate([[0], np.cumsum(c_o)])
    assert np.array_equal(offsets.cpu().numpy(), off_o)
    p = perm.cpu().numpy()
    flat = np.where(valid, idx_h, -1).reshape(-1)
    for e in range(E):
        assert np.array_equal(np.sort(p[off_o[e]:off_o[e + 1]]), np.nonzero(flat == e)[0]), f"expert {e}"
    assert (p[off_o[-1]:] == -1).all()


def test_permute_drops_out_of_range_indices():
    import mixture_experts_layer_03_amd as moe
    spec = SMALL[2]
    cfg = moe_cfg(spec)
    rng = np.random.default_rng(4)
    idx_h = rng.integers(0, spec.num_experts, size=(50, spec.top_k)).astype(np.int32)
    idx_h[3, 1] = -1
    idx_h[10, 0] = spec.num_experts
    idx_h[11, 5] = 1 << 30
    log("permute with out-of-range indices")
    counts, offsets, perm = moe.permute(torch.from_numpy(idx_h).cuda(), cfg)
    torch.cuda.synchronize()
    valid = (idx_h >= 0) & (idx_h < spec.num_experts)
    c_o = np.bincount(idx_h[valid], minlength=spec.num_experts)
    assert np.array_equal(counts.cpu().numpy(), c_o)
    p = perm.cpu().numpy()
    assert (p[valid.sum():] == -1).all()
    assert set(p[:valid.sum()].tolist()) == set(np.nonzero(valid.reshape(-1))[0].tolist())


CASES = [(1, 16, "auto"), (1, 3, "auto"), (1, 100, "auto"),
         (2, 1, "auto"), (2, 13, "auto"), (2, 64, "auto"), (2, 200, "auto"), (2, 700, "auto"),
         (3, 1, "auto"), (3, 64, "auto"), (3, 300, "auto"),
         (4, 1, "auto"), (4, 40, "auto"), (4, 500, "auto"),
         (5, 1, "auto"), (5, 64, "auto"), (5, 500, "auto"),
         (2, 200, "decode"), (3, 100, "decode"), (5, 130, "decode"),
         (2, 13, "prefill"), (3, 1, "prefill"), (5, 40, "prefill"),
         (6, 1, "auto"), (6, 7, "auto"), (6, 64, "auto"), (6, 300, "auto"), (6, 90, "decode"),
         (7, 1, "auto"), (7, 13, "auto"), (7, 64, "auto"), (7, 300, "auto"),
         (2, 16, "auto"), (4, 16, "auto"),
         # the automatic choice streams these (at most 20 routed tokens per expert):
         # the same batches through the tiled kernels
         (3, 300, "prefill"), (4, 500, "prefill"), (5, 500, "prefill"), (7, 300, "prefill")]


@pytest.mark.parametrize("cid,T,path", CASES)
def test_forward(cid, T, path):
    import mixture_experts_layer_03_amd as moe
    spec, L, W = layer(cid)
    x, xd = xs(spec, T)
    log(f"forward cfg{cid} {spec.name} T={T} path={path}")
    y, (idx, w, counts) = moe.forward(xd, W, moe_cfg(spec, path), return_routing=True)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    check_route(spec, idx_h, w.cpu().numpy(), L, x)
    assert np.array_equal(counts.cpu().numpy(), np.bincount(idx_h.reshape(-1), minlength=spec.num_experts))
    st = check_forward(spec, y_to_f64(y), idx_h, L, x)
    log(f"  ok: max rel err {st['max_rel']:.3e}, near-ties {st['near_ties']}")


@pytest.mark.parametrize("cid,T,path", [(2, 64, "decode"), (2, 64, "prefill"), (4, 300, "prefill"),
                                        (4, 300, "decode"), (1, 16, "decode"), (6, 300, "auto")])
def test_experts_given_routing(cid, T, path):
    """The expert stage alone, fed the oracle's routing."""
    import mixture_experts_layer_03_amd as moe
    spec, L, W = layer(cid)
    x, xd = xs(spec, T)
    ocfg = oracle_cfg(spec)
    y_o, d = om.forward(x, L, ocfg)
    log(f"experts cfg{cid} T={T} path={path}")
    idx = torch.from_numpy(d["idx"].astype(np.int32)).cuda()
    wt = torch.from_numpy(d["w"].astype(np.float32)).cuda()
    y = moe.experts(xd, W, idx, wt, moe_cfg(spec, path))
    torch.cuda.synchronize()
    yg = y_to_f64(y)
    rel = np.abs(yg - y_o).max(axis=1) / np.abs(y_o).max(axis=1)
    assert rel.max() <= (2e-2 if spec.act_dtype == "bf16" else 1e-4), rel.max()


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_experts_skip_invalid_indices(path):
    """Slots whose expert index is outside [0, E) contribute nothing."""
    import mixture_experts_layer_03_amd as moe
    spec, L, W = layer(2)
    T = 40
    x, xd = xs(spec, T)
    ocfg = oracle_cfg(spec)
    _, d = om.forward(x, L, ocfg)
    idx = d["idx"].astype(np.int32)
    idx[::3, 2] = -1
    idx[1::5, 0] = spec.num_experts + 3
    log(f"experts with invalid slots path={path}")
    y = moe.experts(xd, W, torch.from_numpy(idx).cuda(), torch.from_numpy(d["w"].astype(np.float32)).cuda(),
                    moe_cfg(spec, path))
    torch.cuda.synchronize()
    X = om.to_f64(x)
    ref = np.zeros_like(X)
    for t in range(T):
        for j in range(spec.top_k):
            e = idx[t, j]
            if 0 <= e < spec.num_experts:
                ref[t] += d["w"][t, j] * om.swiglu_mlp(X[t:t + 1], om.to_f64(L["gate"][e]),
                                                       om.to_f64(L["up"][e]), om.to_f64(L["down"][e]))[0]
    ref += om.swiglu_mlp(X, om.to_f64(L["shared_gate"]), om.to_f64(L["shared_up"]),
                         om.to_f64(L["shared_down"]))
    rel = np.abs(y_to_f64(y) - ref).max(axis=1) / np.abs(ref).max(axis=1)
    assert rel.max() <= 2e-2


def test_no_shared_expert_and_top1():
    import mixture_experts_layer_03_amd as moe
    base = SMALL[3].variant("no-shared-top1", 150, shared_intermediate=0, top_k=1)
    L = synth.make_layer(base)
    W = device_weights(L)
    for T, path in ((9, "auto"), (200, "auto")):
        x = synth.make_x(base, T)
        log(f"forward without shared expert, top_k=1, T={T}")
        y, (idx, w, _) = moe.forward(to_dev(x), W, moe_cfg(base, path), return_routing=True)
        torch.cuda.synchronize()
        check_route(base, idx.cpu().numpy(), w.cpu().numpy(), L, x)
        check_forward(base, y_to_f64(y), idx.cpu().numpy(), L, x)


def test_odd_expert_count_and_single_group():
    """E not a multiple of 16 or 64, n_group == topk_group (mask is a no-op)."""
    import mixture_experts_layer_03_amd as moe
    spec = SMALL[3].variant("odd-E", 151, num_experts=40, n_group=4, topk_group=4, top_k=5)
    L = synth.make_layer(spec)
    W = device_weights(L)
    for T, path in ((3, "auto"), (150, "auto"), (150, "prefill")):
        x = synth.make_x(spec, T)
        log(f"forward E=40 G=g=4 T={T} path={path}")
        y, (idx, w, _) = moe.forward(to_dev(x), W, moe_cfg(spec, path), return_routing=True)
        torch.cuda.synchronize()
        check_route(spec, idx.cpu().numpy(), w.cpu().numpy(), L, x)
        check_forward(spec, y_to_f64(y), idx.cpu().numpy(), L, x)


_SPEC_CACHE = {}


def layer_of(spec):
    if spec.name not in _SPEC_CACHE:
        L = synth.make_layer(spec)
        _SPEC_CACHE[spec.name] = (L, device_weights(L))
    return _SPEC_CACHE[spec.name]


@pytest.mark.parametrize("path,T", [("decode", 1), ("decode", 40), ("prefill", 33), ("prefill", 300),
                                    ("auto", 100)])
def test_top_k_16(path, T):
    """The largest top_k the library takes: sixteen routed terms per token through the
    routing, the permutation and both combines (the decode kernel and the shared-down
    epilogue)."""
    import mixture_experts_layer_03_amd as moe
    spec = SMALL[2].variant("top16", 152, num_experts=48, top_k=16)
    L, W = layer_of(spec)
    x = synth.make_x(spec, T)
    log(f"forward top_k=16 E=48 T={T} path={path}")
    y, (idx, w, _) = moe.forward(to_dev(x), W, moe_cfg(spec, path), return_routing=True)
    torch.cuda.synchronize()
    check_route(spec, idx.cpu().numpy(), w.cpu().numpy(), L, x)
    check_forward(spec, y_to_f64(y), idx.cpu().numpy(), L, x)


@pytest.mark.parametrize("I,T,path", [(1024, 700, "prefill"), (1152, 700, "prefill"), (1024, 64, "decode")])
def test_every_token_on_one_expert(I, T, path):
    """The most skewed routing: one expert among every token's picks, so it holds all T
    tokens (six 128-row M-tiles and three 256-position chunks of one expert at 700
    tokens; the 128 x 512 gate/up tiles at I = 1024, the split kernel at I = 1152, four
    16-token chunks in the decode kernels).  The oracle's forced-routing mode gives the
    weights of those sets."""
    import mixture_experts_layer_03_amd as moe
    spec = SMALL[2].variant(f"one-expert-{I}", 153, moe_intermediate=I)
    L, W = layer_of(spec)
    x = synth.make_x(spec, T)
    ocfg = oracle_cfg(spec)
    _, d0 = om.forward(x, L, ocfg)
    hot = 5
    forced = d0["idx"].copy()
    for t in range(T):
        row = [int(e) for e in forced[t]]
        if hot in row:
            row.remove(hot)
        else:
            row.pop()
        forced[t] = [hot] + row
    y_o, d = om.forward(x, L, ocfg, forced_idx=forced)
    assert (d["idx"] == hot).any(axis=1).all()
    log(f"experts with every token on expert {hot}: I={I} T={T} path={path}")
    idx = torch.from_numpy(d["idx"].astype(np.int32)).cuda()
    wt = torch.from_numpy(d["w"].astype(np.float32)).cuda()
    y = moe.experts(to_dev(x), W, idx, wt, moe_cfg(spec, path))
    torch.cuda.synchronize()
    rel = np.abs(y_to_f64(y) - y_o).max(axis=1) / np.abs(y_o).max(axis=1)
    assert rel.max() <= 2e-2, rel.max()


@pytest.mark.parametrize("cid,path,T", [(5, "decode", 40), (5, "prefill", 300), (6, "auto", 64), (6, "auto", 7)])
def test_fractional_zero_points(cid, path, T):
    """Zero points are fp16 and need not be integers (the synthetic quantiser writes
    integers): every zero point shifted by 0.375, against the oracle, which takes
    s * (q - z) exactly."""
    import mixture_experts_layer_03_amd as moe
    spec = SMALL[cid]
    L = dict(synth.make_layer(spec))
    for n in ("gate_zero", "up_zero", "down_zero"):
        L[n] = (np.asarray(L[n], dtype=np.float32) + np.float32(0.375)).astype(np.float16)
    W = device_weights(L)
    x = synth.make_x(spec, T)
    log(f"fractional zero points cfg{cid} T={T} path={path}")
    y, (idx, w, _) = moe.forward(to_dev(x), W, moe_cfg(spec, path), return_routing=True)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    check_route(spec, idx_h, w.cpu().numpy(), L, x)
    st = check_forward(spec, y_to_f64(y), idx_h, L, x)
    log(f"  ok: max rel err {st['max_rel']:.3e}")


def test_zero_tokens_is_noop():
    import mixture_experts_layer_03_amd as moe
    spec, L, W = layer(2)
    xd = torch.empty((0, spec.hidden), dtype=torch.bfloat16, device="cuda")
    y = moe.forward(xd, W, moe_cfg(spec))
    assert y.shape == (0, spec.hidden)


def test_deterministic():
    import mixture_experts_layer_03_amd as moe
    spec, L, W = layer(4)
    for T, path in ((37, "auto"), (400, "auto"), (700, "prefill")):
        x, xd = xs(spec, T)
        log(f"determinism T={T} path={path}")
        a = moe.forward(xd, W, moe_cfg(spec, path))
        b = moe.forward(xd, W, moe_cfg(spec, path))
        torch.cuda.synchronize()
        assert torch.equal(a, b)


@pytest.mark.parametrize("cid,T,path", [(2, 13, "auto"), (2, 300, "auto"), (5, 64, "auto"), (4, 500, "auto"),
                                        (4, 700, "prefill"), (6, 64, "auto"), (3, 1, "auto"), (7, 16, "auto")])
def test_graph_replay_matches_eager(cid, T, path):
    """The forward captured in a HIP graph (prefill runs the shared expert on a second
    stream, joined inside the graph) gives the eager result on every replay, with other
    eager work and synchronisations between the replays."""
    import mixture_experts_layer_03_amd as moe
    spec, L, W = layer(cid)
    x, xd = xs(spec, T)
    cfg = moe_cfg(spec, path)
    log(f"graph replay cfg{cid} T={T} path={path}")
    ws = torch.empty(cfg.workspace_size(T), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, spec.hidden), dtype=xd.dtype, device="cuda")
    moe.forward(xd, W, cfg, ws=ws, out=y)  # eager call first (creates the library's second stream)
    torch.cuda.synchronize()
    ref = y.clone()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        moe.forward(xd, W, cfg, ws=ws, out=y)
    for rep in range(3):
        y.zero_()
        noise = torch.randn_like(ref, dtype=torch.float32)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {rep}"
        del noise


@pytest.mark.parametrize("cid,T", [(2, 1), (4, 5)])
def test_small_batches_on_two_streams(cid, T):
    """Small batches issued on two streams at once, each stream with its own workspace,
    give the single-stream result on every call."""
    import mixture_experts_layer_03_amd as moe
    spec, L, W = layer(cid)
    cfg = moe_cfg(spec)
    x, xd = xs(spec, T)
    ref = moe.forward(xd, W, cfg)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.empty(cfg.workspace_size(T), dtype=torch.uint8, device="cuda") for _ in streams]
    outs = [[torch.empty_like(ref) for _ in range(8)] for _ in streams]
    log(f"two streams cfg{cid} T={T}")
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for i in range(8):
        for j, st in enumerate(streams):
            with torch.cuda.stream(st):
                moe.forward(xd, W, cfg, ws=wss[j], out=outs[j][i])
    torch.cuda.synchronize()
    for j in range(2):
        for i in range(8):
            assert torch.equal(outs[j][i], ref), f"stream {j} call {i}"


@pytest.mark.parametrize("I", [1152, 2112])
def test_gate_up_last_tile_over_256_position_chunks(I):
    """Prefill gate/up whose last 256-column tile is at most half full but holds no more
    than an eighth of padding (1152 = 4 x 256 + 128; 2112 = 8 x 256 + 64, whose last
    tile also has rows past N): those columns are computed over chunks of 256
    positions of each expert, the others over 128-position tiles; experts with one to
    three chunks."""
    import mixture_experts_layer_03_amd as moe
    spec = SMALL[2].variant(f"split-I{I}", 152, moe_intermediate=I)
    L = synth.make_layer(spec)
    W = device_weights(L)
    for T in (700, 90):
        x = synth.make_x(spec, T)
        log(f"prefill I={I} T={T}")
        y, (idx, w, _) = moe.forward(to_dev(x), W, moe_cfg(spec, "prefill"), return_routing=True)
        torch.cuda.synchronize()
        idx_h = idx.cpu().numpy()
        check_route(spec, idx_h, w.cpu().numpy(), L, x)
        check_forward(spec, y_to_f64(y), idx_h, L, x)


@pytest.mark.parametrize("H,I", [(512, 192), (1024, 512)])
def test_u8_copy_pipeline(H, I):
    """Prefill with u8 experts whose reduction sizes are multiples of 512 (gate/up: H;
    down: I, in the second case): codes and group parameters copied to LDS (parameters
    once per 8 K-steps, both buffers in use when K spans several windows), dequantised
    per fragment; every token against the oracle."""
    import mixture_experts_layer_03_amd as moe
    spec = SMALL[5].variant(f"u8-dma-H{H}", 153, hidden=H, moe_intermediate=I)
    L = synth.make_layer(spec)
    W = device_weights(L)
    for T in (300, 70):
        x = synth.make_x(spec, T)
        log(f"u8 prefill H={H} I={I} T={T}")
        y, (idx, w, _) = moe.forward(to_dev(x), W, moe_cfg(spec, "prefill"), return_routing=True)
        torch.cuda.synchronize()
        idx_h = idx.cpu().numpy()
        check_route(spec, idx_h, w.cpu().numpy(), L, x)
        check_forward(spec, y_to_f64(y), idx_h, L, x)


# a Ling-lite-like layer whose one-token gate/up launch has more blocks (704) than the
# CUs hold at once, so the layer routes one token in its own one-wavefront launch
# rather than inside gate/up
WIDE_LITE = synth.SPECS[2].variant("ling-lite-wide", 112, hidden=256)


@pytest.mark.parametrize("cid,T", [(2, 1), (3, 1), (4, 1), (5, 1), (6, 1), (7, 1), ("wide", 1),
                                   (2, 8), (3, 8), (6, 8), ("wide", 8)])
def test_small_batch_routing_tables_match_the_general_permutation(cid, T):
    """Batches of up to 16 tokens are routed and permuted by one-token or one-workgroup
    launches (or, for one token, inside the gate/up launch); the expert stage fed the
    same routing builds its tables with the general permutation kernel.  Every token's
    arithmetic after routing is the same, so the outputs must be bit-identical."""
    import mixture_experts_layer_03_amd as moe
    if cid == "wide":
        if "wide" not in _CACHE:
            L = synth.make_layer(WIDE_LITE)
            _CACHE["wide"] = (WIDE_LITE, L, device_weights(L))
        spec, L, W = _CACHE["wide"]
    else:
        spec, L, W = layer(cid)
    x, xd = xs(spec, T)
    cfg = moe_cfg(spec, "decode")
    log(f"routing tables cfg{cid} {spec.name} T={T}: kernels {cfg.kernel_path(T)}")
    y, (idx, w, counts) = moe.forward(xd, W, cfg, return_routing=True)
    y2 = moe.experts(xd, W, idx, w, cfg)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    assert np.array_equal(counts.cpu().numpy(), np.bincount(idx_h.reshape(-1), minlength=spec.num_experts))
    assert torch.equal(y, y2), "forward and experts-given-its-routing differ"
    check_route(spec, idx_h, w.cpu().numpy(), L, x)
    st = check_forward(spec, y_to_f64(y), idx_h, L, x)
    log(f"  ok: bit-identical, max rel err {st['max_rel']:.3e}")


@pytest.mark.parametrize("cid", [2, 3, 5, 6, "wide"])
@pytest.mark.parametrize("pattern", ["one-invalid", "out-of-range", "duplicate", "none-valid"])
def test_one_token_down_with_irregular_picks(cid, pattern):
    """One token through the expert stage with picks the router never makes: a slot
    marked invalid (-1), an index past E, one expert in two slots, no valid slot at all.
    With one token the down launch also forms the weighted sum, reading the expert of
    each position through the permutation; every valid slot is one term (bf16, u8 and
    u4 experts)."""
    import mixture_experts_layer_03_amd as moe
    if cid == "wide":
        if "wide" not in _CACHE:
            L = synth.make_layer(WIDE_LITE)
            _CACHE["wide"] = (WIDE_LITE, L, device_weights(L))
        spec, L, W = _CACHE["wide"]
    else:
        spec, L, W = layer(cid)
    x, xd = xs(spec, 1)
    _, d = om.forward(x, L, oracle_cfg(spec))
    idx = d["idx"].astype(np.int32).copy()
    wt = d["w"].astype(np.float32).copy()
    if pattern == "one-invalid":
        idx[0, 1] = -1
    elif pattern == "out-of-range":
        idx[0, 0] = spec.num_experts + 2
    elif pattern == "duplicate":
        idx[0, 2] = idx[0, 4]
        wt[0, 2] = 0.375
    else:
        idx[0, :] = -1
    log(f"one-token experts cfg{cid} {spec.name} picks {pattern}: {idx[0].tolist()}")
    y = moe.experts(xd, W, torch.from_numpy(idx).cuda(), torch.from_numpy(wt).cuda(), moe_cfg(spec, "decode"))
    torch.cuda.synchronize()
    X = om.to_f64(x)
    ref = om.swiglu_mlp(X, om.to_f64(L["shared_gate"]), om.to_f64(L["shared_up"]), om.to_f64(L["shared_down"]))
    for j in range(spec.top_k):
        e = idx[0, j]
        if 0 <= e < spec.num_experts:
            ref = ref + wt[0, j] * om.swiglu_mlp(X, om.expert_matrix(L, "gate", e, 64),
                                                 om.expert_matrix(L, "up", e, 64), om.expert_matrix(L, "down", e, 64))
    rel = np.abs(y_to_f64(y) - ref).max() / np.abs(ref).max()
    log(f"  max rel err {rel:.3e}")
    assert rel <= 2e-2, rel
