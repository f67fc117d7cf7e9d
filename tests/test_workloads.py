"""The seeded input generators: determinism, layout and the workload recipes."""
import math

import numpy as np
import pytest
import torch

from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_case, make_config


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1e-3, 1.0, 1e3)])
    # ties: values exactly half-way between two bf16 neighbours
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.array([0.0, -0.0, np.inf, -np.inf], np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    assert f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_deterministic_and_thread_independent():
    a = make_case([100, 37], seed=3, threads=1)
    b = make_case([100, 37], seed=3, threads=4)
    for f in ("q", "k_pool", "v_pool", "block_table", "context_lens"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = make_case([100, 37], seed=4)
    assert not np.array_equal(a.k_pool, c.k_pool)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
def test_config_layout(name):
    c = make_config(name)
    assert c.q.shape == (c.B, 16, 128) and c.k_pool.shape[1:] == (16, 8, 128)
    assert c.k_pool.dtype == np.uint16 and c.block_table.dtype == np.int32
    used = []
    for b in range(c.B):
        n = int(c.context_lens[b])
        need = (n + 15) // 16
        row = c.block_table[b]
        assert np.all(row[:need] >= 0) and np.all(row[:need] < c.num_pages)
        assert np.all(row[need:] == -1)
        used.extend(row[:need].tolist())
    assert len(used) == len(set(used)), "a page is used twice"
    assert math.isclose(c.scale, 1 / math.sqrt(128))


def test_config_recipes():
    c1 = make_config("c1")
    assert c1.B == 1 and c1.context_lens[0] == 512 and c1.num_pages == 64 and c1.out_dtype == "f32"
    c2 = make_config("c2")
    assert c2.B == 16 and c2.num_pages == 512 and c2.max_blocks == 27
    assert c2.context_lens.min() >= 200 and c2.context_lens.max() <= 420
    c3 = make_config("c3")
    assert c3.context_lens[0] == 28672 and c3.num_pages == 2048 and c3.max_blocks == 1792
    # 1% of key positions were scaled by 4: their rows have ~4x the spread
    k = bf16_bits_to_f32(c3.k_pool[c3.block_table[0]]).reshape(28672, -1)
    big = np.abs(k).mean(axis=1) > 2.0
    assert big.sum() == 286
    c5 = make_config("c5")
    assert c5.B == 32 and c5.context_lens[0] == 67500 and c5.max_blocks == 4219
    assert c5.context_lens.min() >= 256 and c5.context_lens.max() <= 67500
    assert c5.num_pages == c5.used_pages()
    assert np.array_equal(c5.q[0::2], c5.q[1::2])


def test_poison_marks_only_unused_slots():
    c = make_case([5, 16, 0], seed=1, poison=True, Hq=4, Hkv=2, D=8, page=4, pool_pages=12)
    kf = bf16_bits_to_f32(c.k_pool)
    for b, n in enumerate(c.context_lens):
        for t in range(int(n)):
            assert np.all(np.isfinite(kf[c.block_table[b, t // 4], t % 4]))
    assert np.isnan(kf).any()
    assert np.isnan(kf[c.block_table[0, 1], 1:]).all()  # tail of request 0's last page
