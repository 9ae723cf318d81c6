"""The seeded input generator and the workload presets."""
import os

import numpy as np

import moe_synth as synth
import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_shapes.txt")


def _golden():
    out = {}
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split()
            out[k] = float(v)
    return out


def test_generator_is_counter_based_and_deterministic():
    a = synth.normal_bf16(0, 10, 0, 10000, 0.0, 0.02)
    b = synth.normal_bf16(0, 10, 0, 10000, 0.0, 0.02)
    np.testing.assert_array_equal(a, b)
    # A slice equals the same range of the whole tensor.
    c = synth.normal_bf16(0, 10, 1234, 777, 0.0, 0.02)
    np.testing.assert_array_equal(c, a[1234:1234 + 777])
    d = synth.normal_bf16(1, 10, 0, 10000, 0.0, 0.02)
    assert (a != d).mean() > 0.9


def test_generator_moments():
    z = synth.normal_f32(0, 1, 0, 1 << 20, 0.0, 1.0).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    assert abs((z ** 4).mean() - 3) < 0.05  # Gaussian kurtosis
    w = synth.bf16_to_f32(synth.normal_bf16(0, 11, 0, 1 << 20, 0.0, 0.02))
    assert abs(w.std() - 0.02) < 2e-4


def test_permutation_and_zipf_bias():
    p = synth.permutation(0, 3, 256)
    np.testing.assert_array_equal(np.sort(p), np.arange(256))
    b = synth.zipf_bias(0, 256, 1.2)
    np.testing.assert_allclose(np.sort(b)[::-1], (1.0 + np.arange(256)) ** -1.2)


def test_presets_follow_the_pages_shapes():
    g = _golden()
    W = synth.WORKLOADS
    assert g["experts_per_layer"] * g["moe_layers"] == g["experts_all_layers"]
    assert g["ep64_experts_per_gpu"] * g["moe_layers"] == g["ep64_experts_per_gpu_all_layers"]
    for name in ("c2_ep64_bf16", "c3_ep8_bf16", "c4_full_bf16"):
        assert W[name].E == g["experts_per_layer"] and W[name].k == g["experts_per_token"]
    assert W["c2_ep64_bf16"].n_local == g["experts_per_layer"] / 64 == g["ep64_experts_per_gpu"]
    assert W["c3_ep8_bf16"].n_local == g["experts_per_layer"] / 8 == g["ep8_experts_per_gpu"]
    assert 1 - g["experts_per_token"] / W["c3_ep8_bf16"].n_local == g["ep8_cold_fraction"]
    assert W["c5_mxfp8"].E == g["mixtral_ep"] and W["c5_mxfp8"].H % g["mx_block"] == 0
    # the two supplementary presets differ from their parents only where named
    c3, c3l = W["c3_ep8_bf16"], W["c3_literal_ep8_bf16"]
    assert (c3l.T, c3l.n_local) == (W["c2_ep64_bf16"].T, c3.n_local)
    assert (c3l.H, c3l.I, c3l.E, c3l.k, c3l.zipf_s) == (c3.H, c3.I, c3.E, c3.k, c3.zipf_s)
    c5, c5b = W["c5_mxfp8"], W["c5_shape_bf16"]
    assert (c5b.T, c5b.H, c5b.I, c5b.E, c5b.k) == (c5.T, c5.H, c5.I, c5.E, c5.k)
    assert c5b.dtype == "bf16" and c5b.router == c5.router and c5b.zipf_s is None


def test_ep_share_rows_per_expert_ratio():
    # Routing 4096 tokens with Gaussian + Zipf(1.1) logits: the EP64 share
    # (experts 0-3 of all 4096 tokens) sees about 8x the rows per expert of
    # the EP8 share (experts 0-31 of one 512-token instance).
    c2, c3 = synth.WORKLOADS["c2_ep64_bf16"], synth.WORKLOADS["c3_ep8_bf16"]
    inp = synth.make_inputs(c2, with_weights=False)
    idx, _ = orc.topk_softmax(inp["logits"], c2.k)
    r2 = orc.permute(idx, 0, c2.n_local)["R"]
    r3 = orc.permute(idx[:c3.T], 0, c3.n_local)["R"]
    assert 400 <= r2 <= 620, r2          # "about 512 rows"
    assert 10 <= r3 / c3.n_local <= 24   # "about 16 rows per expert"
    ratio = (r2 / c2.n_local) / (r3 / c3.n_local)
    assert 5 <= ratio <= 12, ratio
