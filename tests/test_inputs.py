"""Host-side checks of the seeded input generators and layout arrays (CPU only)."""

import numpy as np
import pytest
import torch

from csa_inputs import (bf16_round, contiguous_positions, zigzag_positions,
                        seq_ids_for_positions, cu_from_lengths, make_workload,
                        tiny_block_workload)
from csa_inputs.workloads import _thd_lengths


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0,
                                  3.0e38, 1e-40], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(bf16_round(x), ref)


@pytest.mark.parametrize("maker", [contiguous_positions, zigzag_positions])
def test_layouts_partition_the_sequence(maker):
    total, cp = 64, 4
    seen = np.concatenate([maker(total, cp, r) for r in range(cp)])
    assert sorted(seen.tolist()) == list(range(total))


def test_zigzag_owns_symmetric_chunks():
    pos = zigzag_positions(32768, 4, 1)
    assert pos[0] == 4096 and pos[4095] == 8191
    assert pos[4096] == 24576 and pos[-1] == 28671


def test_seq_ids_with_empty_sequences():
    cu = cu_from_lengths([3, 0, 2, 0])
    np.testing.assert_array_equal(seq_ids_for_positions([0, 2, 3, 4], cu), [0, 0, 2, 2])


def test_thd_lengths_cover_the_stream():
    rng = np.random.default_rng(123)
    lengths = _thd_lengths(rng, 65536, 1024, 16384)
    assert sum(lengths) == 65536
    assert all(1024 <= x <= 16384 for x in lengths[:-1])
    assert 0 < lengths[-1] <= 16384


def test_named_workload_shapes():
    w = make_workload("dense_f32")
    assert w.q.shape == (128, 2, 64) and w.k.shape == (512, 2, 64)
    assert w.q_pos[0] == 256 and w.q_pos[-1] == 383 and w.dtype == "f32"
    w = make_workload("moba_mha_8k")
    assert w.q.shape == (2048, 16, 128) and w.q_pos[0] == 6144
    assert np.array_equal(bf16_round(w.q), w.q)


def test_tiny_workload_is_deterministic():
    a = tiny_block_workload(seed=3)
    b = tiny_block_workload(seed=3)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k)
