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
