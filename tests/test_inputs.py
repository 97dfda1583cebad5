"""The seeded input generator (no GPU)."""

import numpy as np
import torch

from mcs_inputs import (WORKLOADS, bf16_bits, hash_projections, head_base, head_rotation, head_step,
                        keep_count, position_embedding, round_bf16, text_embedding, token_embedding)


def test_position_embedding_norm_and_origin():
    for d in (64, 128):
        p = position_embedding((3, 4, 5), d)
        assert p.shape == (60, d)
        assert np.allclose((p.astype(np.float64) ** 2).sum(1), d / 2, atol=1e-5)
        # token 0 sits at the origin: every sin feature is 0 and every cos is 1
        w = (d // 4, 3 * d // 8, 3 * d // 8)
        off = 0
        for wi in w:
            assert np.all(p[0, off:off + wi // 2] == 0.0) and np.all(p[0, off + wi // 2:off + wi] == 1.0)
            off += wi


def test_rotation_orthogonal_and_deterministic():
    w = head_rotation(0, 2, 3, 64).astype(np.float64)
    assert np.allclose(w @ w.T, np.eye(64), atol=1e-5)
    assert np.array_equal(head_rotation(0, 2, 3, 64), head_rotation(0, 2, 3, 64))
    assert not np.array_equal(head_rotation(0, 2, 3, 64), head_rotation(0, 2, 4, 64))


def test_round_bf16_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(10000).astype(np.float32) * 10,
                        # exact ties between two bf16 neighbours
                        (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32) * 1.0])
    want = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = round_bf16(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    bits = bf16_bits(got)
    assert np.array_equal(torch.tensor(bits.view(np.int16)).view(torch.bfloat16).float().numpy(), want)


def test_head_inputs_structure():
    grid, d = (4, 4, 8), 64
    q, k, v = head_base(0, 1, 0, grid, d)
    assert q.shape == k.shape == v.shape == (128, d) and q.dtype == np.float32
    # Q and K share the 3 P W term: their difference is pure noise (std 0.5*sqrt(2))
    assert abs(np.std(q - k) - 0.5 * np.sqrt(2)) < 0.05
    q0, k0, v0 = head_step((q, k, v), 0, 1, 0, 0, 0.02, bf16=True)
    assert np.array_equal(q0, round_bf16(q))
    q3, k3, v3 = head_step((q, k, v), 0, 1, 0, 3, 0.02, bf16=False)
    assert abs(np.std(v3 - v) - 0.06) < 0.01
    q3b = head_step((q, k, v), 0, 1, 0, 3, 0.02, bf16=False)[0]
    assert np.array_equal(q3, q3b)


def test_keep_rule_matches_workloads():
    assert keep_count(0.10, 24960) == 2496
    assert keep_count(0.05, 75600) == 3776
    assert [keep_count(f, 32768) for f in (0.0625, 0.125, 0.25)] == [2048, 4096, 8192]
    assert [keep_count(f, 32760) for f in (0.02, 0.05, 0.10, 0.25, 1.0)] == [640, 1600, 3264, 8128, 32760]
    assert WORKLOADS[1].keeps().tolist() == [128]
    k4 = WORKLOADS[4].keeps()
    assert set(k4.tolist()) <= {2048, 4096, 8192} and len(k4) == 16
    assert np.array_equal(k4, WORKLOADS[4].keeps())


def test_workload_sizes():
    assert WORKLOADS[1].seq_len == 1024 and WORKLOADS[2].seq_len == 24960
    assert WORKLOADS[3].seq_len == 75600 and WORKLOADS[3].num_groups == 1182
    assert WORKLOADS[4].seq_len == 32768 and WORKLOADS[5].seq_len == 32760
    w6 = WORKLOADS[6]
    assert w6.seq_len == 24960 + 226 and w6.num_groups == 394 and w6.keeps()[0] == 2496
    assert hash_projections(0, 1, 64).shape == (8, 64)


def test_text_tokens_follow_the_grid():
    """Joint sequences: the grid tokens' position embeddings, then text
    embeddings of the same squared norm d/2, seeded, independent of the grid."""
    for d in (64, 128):
        e = token_embedding((2, 3, 4), d, 7, seed=3, workload_id=6)
        assert e.shape == (31, d)
        assert np.array_equal(e[:24], position_embedding((2, 3, 4), d))
        assert np.array_equal(e[24:], text_embedding(3, 6, 7, d))
        assert np.allclose((e[24:].astype(np.float64) ** 2).sum(1), d / 2, rtol=1e-6)
        assert not np.array_equal(text_embedding(3, 6, 7, d), text_embedding(4, 6, 7, d))
    assert np.array_equal(token_embedding((2, 3, 4), 64), position_embedding((2, 3, 4), 64))
