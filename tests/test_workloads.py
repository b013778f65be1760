"""The seeded input generators produce the structure the workloads claim:
index maps that are permutations grouped by expert with a Zipf skew, the
stated invalid share, NaN only where nothing may be read, and the same bits
for the same seed."""
from __future__ import annotations

import numpy as np

import workloads as wl


def test_zipf_grouped_map_is_a_permutation_grouped_by_expert():
    rng = np.random.Generator(np.random.PCG64(11))
    T, K, E = 4096, 8, 256
    idx = wl.zipf_grouped_index_map(rng, T, K, E, 1.1)
    assert idx.shape == (T, K) and idx.dtype == np.int32
    assert np.array_equal(np.sort(idx.reshape(-1)), np.arange(T * K))
    # recover each pair's expert from the same draw and check the grouping:
    # rows of one expert form one contiguous range, in token order
    rng = np.random.Generator(np.random.PCG64(11))
    logp = -1.1 * np.log(np.arange(1, E + 1, dtype=np.float64))
    experts = np.argsort(-(logp[None, :] + rng.gumbel(size=(T, E))), axis=1,
                         kind="stable")[:, :K]
    assert all(len(set(row)) == K for row in experts[:64])      # distinct per token
    row_expert = np.empty(T * K, np.int64)
    row_token = np.empty(T * K, np.int64)
    row_expert[idx.reshape(-1)] = experts.reshape(-1)
    row_token[idx.reshape(-1)] = np.repeat(np.arange(T), K)
    assert np.all(np.diff(row_expert) >= 0)                      # grouped by expert
    same = np.diff(row_expert) == 0
    assert np.all(np.diff(row_token)[same] > 0)                  # token order inside
    counts = np.bincount(row_expert, minlength=E)
    # Zipf skew: the first experts carry clearly more rows than the last ones
    assert counts[:16].mean() > 3 * counts[-64:].mean()


def test_invalid_share_and_poison():
    c = wl.decode(poison=True, nan_rows_beyond=2)
    bad = (c.idx < 0) | (c.idx >= c.num_rows)
    assert int(bad.sum()) == 41                                  # 2 % of 2048 slots
    g = c.gemm2_storage
    nan = lambda a: ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)
    assert np.all(nan(g[:, c.hidden:]))                          # padding columns
    assert np.all(nan(g[c.num_rows:]))                           # rows past num_rows
    assert not np.any(nan(g[:c.num_rows, :c.hidden]))            # readable part is clean
    b = wl.make_token_major_case(3, capacity=40, top_k=8, hidden=512, live_tokens=30,
                                 weights="uniform", routed_scale=2.5, poison_dead=True)
    assert np.all(nan(b.expert_outputs[b.live_tokens:]))
    assert not np.any(nan(b.expert_outputs[:b.live_tokens]))
    assert np.all(np.isnan(b.expert_weights[b.live_tokens:]))


def test_weights_are_normalised_routing_weights():
    c = wl.tiny()
    assert np.allclose(c.expert_weights.sum(axis=1), 1.0, atol=1e-6)
    b = wl.make_token_major_case(3, capacity=64, top_k=8, hidden=256, live_tokens=64,
                                 weights="uniform")
    assert np.allclose(b.expert_weights.sum(axis=1), 1.0, atol=1e-6)
    assert np.all(b.expert_weights > 0)


def test_same_seed_same_bits():
    a, b = wl.tiny(), wl.tiny()
    assert np.array_equal(a.gemm2_storage, b.gemm2_storage)
    assert np.array_equal(a.idx, b.idx)
    assert np.array_equal(a.expert_weights, b.expert_weights)
    c = wl.make_index_map_case(99, num_tokens=16, hidden=256)
    assert not np.array_equal(c.gemm2_storage[:16], a.gemm2_storage[:16, :256])
