"""The seeded input generator: storage rounding and determinism."""

import math

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, np.inf, -np.inf],
                                 dtype=np.float32)])
    # exact ties: mantissa ...1 1000 0000 0000 0000 and ...0 1000 0000 0000 0000
    ties = np.array([0x3F818000, 0x3F808000, 0xBF818000, 0x3F80FFFF], dtype=np.uint32).view(np.float32)
    x = np.concatenate([x, ties])
    ours = synth.round_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_chunk_independent():
    w = synth.WORKLOADS["small_200m"]
    a = synth.generate(w, seq_len=256)
    b = synth.generate(w, seq_len=256)
    for key in ("q", "k", "v", "beta"):
        assert np.array_equal(a[key], b[key])
    rng = np.random.default_rng(w.seed)
    q_small_chunks = synth._draw_qkv(rng, a["q"].shape, w.d, w.dtype, chunk=1000)
    assert np.array_equal(q_small_chunks, a["q"])


def test_workload_table():
    W = synth.WORKLOADS
    assert [w.n_segments for w in W.values()] == [4, 16, 8, 16, 512]
    c4 = W["llama3_8b_gqa"]
    assert c4.n_q_heads // c4.n_kv_heads == 4 and c4.d == 128
    c3 = synth.generate(W["llama300m_16k"], seq_len=2048)
    k = synth.as_f64(c3["k"], "bf16")
    # outlier rows are 4x the others: 102 = floor(0.05 * 2048) per (b, head)
    norms = np.linalg.norm(k, axis=-1)
    big = norms > 3.0 * np.median(norms)
    assert abs(big.sum(axis=-1).mean() - math.floor(0.05 * 2048)) <= 2
    assert c3["beta"].dtype == np.float32 and c3["M0"].shape == (4, 16, 64, 64)
