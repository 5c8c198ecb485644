"""Capture-side prefill: the prompt's own causal attention computed chunk by chunk against the
pages captured so far, writing its pages as it goes.  Its outputs are checked against the
oracle's causal attention over the whole prompt (no pages, no chunks, no shards), and the
pools it leaves against a direct capture, bit for bit."""
import numpy as np
import pytest
import torch

from _cases import assert_close, log, np32
from oracle import attention as orc
from suffix_attention_amd import api, datagen, driver

pytestmark = pytest.mark.gpu


def _inputs(P, hq, hkv, d, dtype, seed):
    s = lambda tag: 7919 * seed + tag  # noqa: E731
    q = datagen.normal((P, hq, d), s(4), dtype).cuda()
    k = datagen.normal((P, hkv, d), s(2), dtype).cuda()
    v = datagen.normal((P, hkv, d), s(3), dtype).cuda()
    n_pages = api.n_logical_pages(P)
    table = datagen.page_table(n_pages, s(1)).to(torch.int32).cuda()
    return q, k, v, table, n_pages


@pytest.mark.parametrize("dtype,d,chunk,S", [(torch.bfloat16, 256, 192, 3), (torch.bfloat16, 128, 64, 1),
                                             (torch.float32, 64, 128, 2)])
def test_prefill_matches_causal_oracle_and_direct_capture(dtype, d, chunk, S):
    P, hq, hkv = 700, 6, 2
    log(f"case: prefill P={P} chunk={chunk} S={S} d={d} {dtype}")
    q, k, v, table, n_pages = _inputs(P, hq, hkv, d, dtype, seed=80 + d)
    pre, o, lse = driver.prefill_capture(q, k, v, table, n_pages, chunk, n_shards=S)
    torch.cuda.synchronize()
    empty = np.zeros((0, hkv, d))
    O, L = orc.forward(np32(q), empty, empty, np32(k), np32(v), 0)
    assert_close("O", np32(o), O)
    assert_close("LSE", np32(lse), L)
    kd, vd = api.capture_pages(k, v, table, n_pages)
    assert torch.equal(pre.k_pages, kd) and torch.equal(pre.v_pages, vd)
    assert pre.prefix_len == P and pre.n_shards == S


def test_prefill_then_replay_sees_the_captured_prompt():
    """A response replayed over the prefilled pages equals one replayed over directly captured
    pages, bit for bit."""
    P, R, hq, hkv, d = 640, 96, 12, 4, 256
    log(f"case: prefill P={P} then replay R={R}")
    q, k, v, table, n_pages = _inputs(P, hq, hkv, d, torch.bfloat16, seed=90)
    pre, _, _ = driver.prefill_capture(q, k, v, table, n_pages, 256, n_shards=2, keep_o=False)
    kd, vd = api.capture_pages(k, v, table, n_pages)
    direct = api.Prefix(hq, hkv, d, torch.bfloat16, P, table, kd, vd, api.even_shard_bounds(n_pages, 2))
    qr = datagen.normal((R, hq, d), 91, torch.bfloat16).cuda()
    kr = datagen.normal((R, hkv, d), 92, torch.bfloat16).cuda()
    vr = datagen.normal((R, hkv, d), 93, torch.bfloat16).cuda()
    o1, l1, _ = api.replay_fwd(pre, qr, 0, kr, vr)
    o2, l2, _ = api.replay_fwd(direct, qr, 0, kr, vr)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.timeout(600)
def test_prefill_at_the_benchmark_size_on_sampled_rows():
    """The prefill workload the benchmark times (P = 524,288 in chunks of 4,096 over 8 shards,
    Hq 24 / Hkv 4, d 256, bf16): the pools equal a direct capture bit for bit, and sampled rows
    -- the first and last of a chunk, rows deep in the prompt, the last row -- against the
    oracle's causal attention over every key they see (two kv heads each)."""
    P, hq, hkv, d, chunk, S = 524288, 24, 4, 256, 4096, 8
    g = hq // hkv
    log(f"case: prefill P={P} chunk={chunk} S={S} sampled rows")
    s = lambda tag: 7919 * 95 + tag  # noqa: E731
    q = datagen.normal((P, hq, d), s(4), torch.bfloat16, device="cuda")
    k = datagen.normal((P, hkv, d), s(2), torch.bfloat16, device="cuda")
    v = datagen.normal((P, hkv, d), s(3), torch.bfloat16, device="cuda")
    n_pages = api.n_logical_pages(P)
    table = datagen.page_table(n_pages, s(1)).to(torch.int32).cuda()
    pre, o, lse = driver.prefill_capture(q, k, v, table, n_pages, chunk, n_shards=S)
    torch.cuda.synchronize()
    kd, vd = api.capture_pages(k, v, table, n_pages)
    assert torch.equal(pre.k_pages, kd) and torch.equal(pre.v_pages, vd)
    del kd, vd
    rng = np.random.default_rng(95)
    tokens = [0, chunk - 1, chunk, 7 * chunk + 100, P // 2 + 17, P - chunk, P - 1] + \
        sorted(int(t) for t in rng.integers(0, P, 2))
    empty = np.zeros((0, 1, d))
    for t in tokens:
        for kv in (0, hkv - 1):
            hs = slice(kv * g, (kv + 1) * g)
            O, L = orc.forward(np32(q[t:t + 1, hs]), empty, empty, np32(k[:t + 1, kv:kv + 1]),
                               np32(v[:t + 1, kv:kv + 1]), t)
            log(f"  token {t} kv head {kv}")
            assert_close("O", np32(o[t:t + 1, hs]), O)
            assert_close("LSE", np32(lse[t:t + 1, hs]), L)
