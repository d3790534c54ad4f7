"""Stack schedules of the attention sweep (host logic, no GPU).

The hybrid backbone interleaves 27 gated SWA layers with 5 global layers (hyper.ai summary
of the paper, section 方法; "ZGCM-1-7B 完全解説", section アーキテクチャ), and its per-token
KV cache is 20 KiB against 128 KiB for 32 global layers, 6.4x less (jaehun.me review,
section "KV 캐시가 6.4배 줄어드는 이유").
"""

from oracle import attn as O
from workloads import C4, STACKS, stack_kinds


def test_hybrid_schedule_matches_the_model():
    kinds = stack_kinds(STACKS["hybrid_5to1"])
    assert len(kinds) == 32
    assert kinds.count("global") == 5 and kinds.count("swa") == 27
    assert kinds == O.layer_kinds(32)
    assert [i for i, k in enumerate(kinds) if k == "global"] == [5, 11, 17, 23, 29]


def test_alternative_stacks():
    assert stack_kinds(STACKS["full"]) == ["global"] * 32
    k31 = stack_kinds(STACKS["swa_3to1"])
    assert k31.count("global") == 8 and k31.count("swa") == 24
    assert all(k31[i] == ("global" if i % 4 == 3 else "swa") for i in range(32))


def test_kv_bytes_per_token_of_the_stacks():
    per = {n: 2 * stack_kinds(p).count("global") * C4.Hkv * C4.d * 2 for n, p in STACKS.items()}
    assert per["hybrid_5to1"] == 20 * 1024 and per["full"] == 128 * 1024
    assert per["full"] / per["hybrid_5to1"] == 6.4
    assert per["hybrid_5to1"] * 262144 == 5 * 2 ** 30 and per["full"] * 262144 == 32 * 2 ** 30
    assert per["hybrid_5to1"] == O.kv_bytes_per_token(5)
