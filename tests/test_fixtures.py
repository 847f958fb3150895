"""The seeded generator (fixtures/) against its published definition."""
import json
import os

import numpy as np
import torch

from fixtures import host, workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_vector():
    g = json.load(open(os.path.join(GOLD, "splitmix64.json")))
    L = host.lib()
    got = [L.fx_stream(g["seed"], n) for n in range(len(g["first_outputs"]))]
    assert got == [int(v) for v in g["first_outputs"]]


def test_normal_moments_and_support():
    x = host.normal_bf16(0, host.FX_WQKV, 3, 1, 0, 12345, 1 << 20, 0.02).float().numpy().astype(np.float64)
    assert abs(x.mean()) < 5 * 0.02 / np.sqrt(x.size)
    assert abs(x.std() / 0.02 - 1.0) < 0.01
    assert np.abs(x).max() <= 6 * 0.02 * (1 + 2 ** -8)
    # fourth moment of Irwin-Hall(12) is 3 - 1.2/12 = 2.9 (normal: 3)
    k4 = ((x / x.std()) ** 4).mean()
    assert abs(k4 - 2.9) < 0.05


def test_pure_function_of_index():
    a = host.normal_bf16(7, host.FX_GATE, 5, 9, 0, 1000, 64, 0.02)
    b = host.normal_bf16(7, host.FX_GATE, 5, 9, 0, 0, 1064, 0.02)[1000:]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    c = host.normal_bf16(8, host.FX_GATE, 5, 9, 0, 1000, 64, 0.02)
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_bf16_rounding_is_nearest_even():
    L = host.lib()
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: ties to even (1.0)
    assert L.fx_bf16_rne(1.0 + 2 ** -8) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even): goes up
    assert L.fx_bf16_rne(1.0 + 3 * 2 ** -8) == 0x3F82
    assert L.fx_bf16_rne(1.0 + 2 ** -8 + 2 ** -20) == 0x3F81
    assert L.fx_bf16_rne(-2.0) == 0xC000


def test_uniform_and_permutation():
    u = host.uniform(0, host.FX_CTX, 10000, 512, 32768)
    assert u.min() >= 512 and u.max() <= 32768
    assert abs(u.mean() - (512 + 32768) / 2) < 0.03 * 32768
    p = host.permutation(0, 1000)
    assert sorted(p.tolist()) == list(range(1000))
    assert p.tolist() != list(range(1000))
    assert np.array_equal(p, host.permutation(0, 1000))


def test_workload_resolution():
    w = workloads.resolve(workloads.workload("moe48_b32_ragged"))
    assert len(w["ctx"]) == 32 and all(512 <= c <= 32768 for c in w["ctx"])
    need = sum((c + 256 + 15) // 16 for c in w["ctx"])
    assert w["pool_pages"] >= int(need * 1.1)
    assert all(0 <= t < 151936 for t in w["tokens"])
