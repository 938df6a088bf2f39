"""The input generators: published reference values and cross-implementation
agreement (C core, numpy, torch)."""
import numpy as np
import pytest
import torch

from synth import gen
from synth import workloads as wl


def test_splitmix64_reference_values():
    # SplitMix64 seeded with 0: the first outputs of the published generator
    assert [int(x) for x in gen.u64(0, 3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert int(gen.u64(12345, 1, start=7)[0]) == int(gen.mix64(np.uint64(12345) + np.uint64(8) * gen.GAMMA))


def test_bf16_rounding_matches_torch():
    x = gen.normal_f32(gen.stream_key(3), 100000, 3.0)
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 65504.0]   # exact ties and a large value
    ours = gen.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(gen.normal_bf16(gen.stream_key(3), 1000, 3.0), gen.to_bf16_bits(gen.normal_f32(gen.stream_key(3), 1000, 3.0)))


def test_normals_look_normal():
    z = gen.normal(gen.stream_key(9), 1_000_000)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    assert abs(np.mean(z ** 4) - 3.0) < 0.05


def test_commit_pattern_three_ways():
    sl = np.array([0, 5, 77, 123456])
    a = gen.commit_pattern_slabs(sl, 37, 24)
    b = gen.commit_pattern_bits(sl.reshape(-1, 1, 1), np.arange(37).reshape(1, -1, 1), np.arange(24).reshape(1, 1, -1))
    c = gen.commit_pattern_torch(torch.tensor(sl).view(-1, 1, 1), torch.arange(37).view(1, -1, 1),
                                 torch.arange(24).view(1, 1, -1)).numpy().view(np.uint16)
    assert np.array_equal(a, b) and np.array_equal(a, c)
    assert len(np.unique(a)) > 3000   # wide spread of bit patterns


def test_workload_generators_follow_their_rules():
    for w in wl.WORKLOADS:
        par = wl.trees(w)
        assert par.shape == (w.B, w.T) and (par[:, 0] == 0).all()
        for b in range(w.B):
            dep = np.zeros(w.T, int)
            kids = np.zeros(w.T, int)
            for i in range(1, w.T):
                assert 0 <= par[b, i] < i
                dep[i] = dep[par[b, i]] + 1
                kids[par[b, i]] += 1
            assert dep.max() <= w.depth_cap
            if w.tree == "bushy":
                assert (kids[dep <= 1] <= 4).all() and (kids[dep > 1] <= 2).all()
        lens = wl.lengths(w)
        assert lens.min() >= w.len_lo and lens.max() <= w.len_hi


def test_logits_designated_top_is_argmax():
    x, des = gen.logits_with_designated_top(gen.stream_key(11), 50, 3000)
    assert (np.argmax(x, axis=1) == des).all()
    assert np.abs(np.delete(x, des + 3000 * np.arange(50))).max() <= 6.0


@pytest.mark.parametrize("M,depth", [(8, 4), (16, 10), (32, 10), (255, 6), (5, 10), (1, 1)])
def test_layered_trees(M, depth):
    par = gen.tree_layered(gen.stream_key(123, M, depth), M, depth)
    lvl = np.zeros(M + 1, np.int64)
    for i in range(1, M + 1):
        assert par[i] < i
        lvl[i] = lvl[par[i]] + 1
    D = min(depth, M)
    assert lvl.max() == D
    counts = np.bincount(lvl[1:], minlength=D + 1)[1:]
    assert counts.max() - counts.min() <= 1 and counts.sum() == M
