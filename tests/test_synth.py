"""Seeded input generator: determinism, per-piece independence and bf16 rounding."""
import numpy as np
import torch

import synth


def test_same_seed_same_bytes():
    wl = synth.WORKLOADS["tiny"]
    a = synth.q_chunk(wl, 1)
    b = synth.q_chunk(wl, 1)
    assert a.dtype == np.uint16 and a.shape == (512, 4, 64)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, synth.q_chunk(wl.with_seed(1), 1))
    assert not np.array_equal(a, synth.do_chunk(wl, 1))


def test_pages_independent_of_context():
    wl = synth.WORKLOADS["tiny"]
    k, v = synth.kv_tokens(wl, 3, 4)
    assert np.array_equal(k[wl.page:2 * wl.page], synth.k_page(wl, 4))
    assert np.array_equal(v[:wl.page], synth.v_page(wl, 3))


def test_key_offset_is_per_page_and_head():
    wl = synth.WORKLOADS["dense256k"]
    kp = synth.bf16_widen(synth.k_page(wl, 5)).astype(np.float64)
    # The per-(page, head) offset shifts the token mean of each (head, dim) away from zero.
    mean = kp.mean(axis=0)
    assert np.std(mean) > 0.3


def test_permutation():
    wl = synth.WORKLOADS["qwen32k"]
    perm = synth.page_permutation(wl)
    assert perm.dtype == np.int32 and sorted(perm.tolist()) == list(range(wl.n_pages))
    bigger = synth.page_permutation(wl, 2 * wl.n_pages)
    assert len(set(bigger.tolist())) == wl.n_pages and bigger.max() < 2 * wl.n_pages


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # Exact ties: low 16 bits equal to 0x8000 with both parities of the kept lsb.
    ties = (rng.integers(0, 64, 1000, dtype=np.uint32) << np.uint32(17)) | np.uint32(0x3F800000) | np.uint32(0x8000)
    ties2 = ties | np.uint32(0x10000)
    x = np.concatenate([x, ties.view(np.float32), ties2.view(np.float32), np.float32([0.0, -0.0, 1e-30, -1e30])])
    ours = synth.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_widen(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())
