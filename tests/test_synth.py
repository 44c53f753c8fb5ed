"""Seeded input generator: determinism, bf16 encoding, u8 encoder bounds (P13)."""
import numpy as np

import oracle.moe_oracle as om
import synth


def test_bf16_round_to_nearest_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0],
                 dtype=np.float32)
    bits = synth.bf16_bits(v)
    # 1+2^-8 is halfway between 1 and 1+2^-7: ties to even -> 1.0;
    # 1+3*2^-8 is halfway between 1+2^-7 and 1+2^-6: ties to even -> 1+2^-6
    assert synth.bf16_values(bits).tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0]
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    back = synth.bf16_values(synth.bf16_bits(r))
    assert np.all(np.abs(back - r) <= np.abs(r) * 2 ** -8)


def test_generator_is_deterministic_and_keyed():
    spec = synth.SPECS[1]
    a, b = synth.make_layer(spec), synth.make_layer(spec)
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k
    c = synth.make_layer(spec, copy=1)
    assert not np.array_equal(a["gate"], c["gate"])
    assert np.array_equal(synth.make_x(spec, 16), synth.make_x(spec, 16))
    assert not np.array_equal(synth.make_x(spec, 16)[:8], synth.make_x(spec, 8))


def test_u8_encoder_round_trip_within_half_step():
    rng = np.random.default_rng(1)
    w = synth.bf16_values(synth.bf16_bits(rng.standard_normal((17, 256)).astype(np.float32) * 0.02))
    w[3, :64] = np.abs(w[3, :64])          # a group with no negative value
    w[4, 64:128] = 0.0                      # an all-zero group
    q, s, z = synth.quantize_u8(w, 64)
    deq = om.dequant_u8(q, s, z, 64)
    step = np.repeat(s.astype(np.float64), 64, axis=1)
    assert np.all(np.abs(deq - w) <= step / 2 * (1 + 1e-9))
    assert np.all(z.astype(np.float64) == np.rint(z.astype(np.float64)))


def test_zipf_router_bias_is_centred_log_rank():
    spec = synth.SPECS[4].variant("zipf-small", 900, hidden=64, num_experts=32, moe_intermediate=64,
                                  shared_intermediate=64)
    L = synth.make_layer(spec)
    b = L["router_bias"].astype(np.float64)
    assert abs(b.mean()) < 1e-5
    ranks = np.argsort(np.argsort(-b)) + 1          # rank 1 = largest bias
    assert np.allclose(b, -1.1 * np.log(ranks) + 1.1 * np.log(ranks).mean(), atol=1e-5)
