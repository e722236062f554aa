"""The seeded generators: determinism, subset consistency, bf16 rounding (CPU only)."""
import numpy as np
import torch

from workloads import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make, variant


def test_five_workloads_have_the_stated_shapes():
    shapes = {c.name: (c.batch, c.L, c.V, c.d, c.dtype, c.walk) for c in CONFIGS}
    assert shapes == {
        "tiny": (1, 8, 32000, 1024, "f32", "greedy"),
        "single_stream": (1, 16, 151936, 5120, "bf16", "greedy"),
        "small_batch": (32, 16, 151936, 5120, "bf16", "greedy"),
        "throughput": (256, 16, 151936, 5120, "bf16", "greedy"),
        "sampled": (64, 16, 262144, 4096, "bf16", "gumbel"),
    }


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 3,
        # exact halfway cases between bf16 neighbours, both parities
        (np.arange(0x3F800000, 0x3F800000 + 0x40000, 0x8000, dtype=np.uint32) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -1e-40], np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(x), want)
    np.testing.assert_array_equal(bf16_bits_to_f32(want), torch.from_numpy(want.view(np.int16)).view(
        torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_subset_consistent():
    cfg = variant("small_batch", V=4000, d=64, batch=6)
    a = make(cfg)
    b = make(cfg)
    for f in ("logits", "hidden", "prev_token", "A", "B", "W_h"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    s = make(cfg, seqs=[4, 1])
    np.testing.assert_array_equal(s.logits, a.logits[[4, 1]])
    np.testing.assert_array_equal(s.hidden, a.hidden[[4, 1]])
    np.testing.assert_array_equal(s.prev_token, a.prev_token[[4, 1]])
    np.testing.assert_array_equal(s.seq_ids, [4, 1])
    assert a.logits.dtype == np.uint16 and a.logits.shape == (6, 16, 4000)
    assert ((a.prev_token >= 0) & (a.prev_token < 4000)).all()


def test_planted_peaks_sit_above_the_background():
    cfg = variant("single_stream", V=20000, d=64)
    x = bf16_bits_to_f32(make(cfg).logits[0])  # [L, V]
    for t in range(cfg.L):
        top = np.sort(x[t])[::-1]
        # 16 planted values above every background value (bf16 rounding may tie some)
        assert (top[:16] > top[16]).sum() >= 15
    tiny = make(variant("tiny", V=3000))
    xt = tiny.logits[0]
    hits = sum(int(np.argmax(xt[t]) == tiny.true_tokens[0, t]) for t in range(8))
    assert hits >= 6  # +4 on N(0,1) wins almost always


def test_tie_and_neg_inf_variants():
    cfg = variant("single_stream", V=3000, d=64, tie_levels=8, neg_inf_frac=0.5, peak_kind="none")
    x = bf16_bits_to_f32(make(cfg).logits[0])
    finite = x[np.isfinite(x)]
    assert len(np.unique(finite)) <= 9
    assert np.isneginf(x).mean() > 0.4
