"""The seeded generators are deterministic and produce the stated formats."""
import numpy as np

from workloads import CONFIGS, make_inputs, make_swiglu_weights
from oracle import codecs


def test_shapes_and_determinism():
    for name, cfg in CONFIGS.items():
        small = cfg.with_tokens(8)
        a, b = make_inputs(small), make_inputs(small)
        assert a["logits"].shape == (8, cfg.n_experts) and a["logits"].dtype == np.float32
        assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["logits"], b["logits"])
        want = {"f32": np.float32, "bf16": np.uint16, "f8": np.uint8}[cfg.dtype]
        assert a["x"].dtype == want and a["x"].shape == (8, cfg.hidden)
        if cfg.dtype == "f8":
            assert a["x_scales"].shape == (8, cfg.hidden // 128)
        else:
            assert a["x_scales"] is None


def test_fp8_blocks_reconstruct_input():
    cfg = CONFIGS["segment"].with_tokens(4)
    inp = make_inputs(cfg)
    q = codecs.fp8_bits_to_f64(inp["x"]).reshape(4, -1, 128)
    s = inp["x_scales"].astype(np.float64)
    # each block's largest magnitude maps to the largest finite code, 448
    assert np.allclose(np.abs(q).max(axis=2), 448.0)
    assert np.isfinite(q).all()
    # dequantised values are within e4m3's half-ulp (2^-4 relative) of a normal draw
    deq = (q * s[:, :, None]).reshape(4, -1)
    assert np.abs(deq).max() < 8


def test_prefill_logits_are_biased_toward_few_experts():
    cfg = CONFIGS["prefill"].with_tokens(256)
    inp = make_inputs(cfg)
    top = np.argmax(inp["logits"], axis=1)
    counts = np.bincount(top, minlength=cfg.n_experts)
    assert counts.max() > 8 * counts.mean()


def test_swiglu_weights_subset_is_consistent():
    from dataclasses import replace
    cfg = replace(CONFIGS["mixtral"], ffn=16, hidden=8)
    full = make_swiglu_weights(cfg)
    part = make_swiglu_weights(cfg, experts=[3])
    for k in full:
        assert np.array_equal(full[k][3], part[k][3])
        assert full[k].dtype == np.uint16
