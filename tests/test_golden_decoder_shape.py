"""The workloads, the benchmark and the append's RoPE use the decoder shape
and prefill chunk size that the source pages print (tests/golden/decoder_shape.txt,
which cites the page and section of each value)."""
import os

import bench
import workloads
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "decoder_shape.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = float(v)
    return vals


def test_fixture_has_every_value():
    assert set(_golden()) == {"hidden", "layers", "q_heads", "kv_heads", "rope_theta", "prefill_chunk_tokens"}


def test_heads_and_layers():
    g = _golden()
    assert gen.HQ == g["q_heads"] and gen.HKV == g["kv_heads"]
    assert bench.LAYERS == g["layers"]                 # tokens/s = B / (layers x time per layer)
    c1 = workloads.make_config("c1")                   # the small named workload, built in full
    assert (c1.Hq, c1.Hkv) == (g["q_heads"], g["kv_heads"])


def test_rope_base():
    assert gen.ROPE_THETA == _golden()["rope_theta"]


def test_prefill_chunks():
    chunk = int(_golden()["prefill_chunk_tokens"])
    for name, (_seed, ctx, new) in gen.PREFILL_CONFIGS.items():
        assert all(n == chunk for n in new), name
        assert all(c % chunk == 0 for c in ctx), name   # whole chunks: p1 is the seventh of a 28,672-token prompt
