"""Pre-step scoring: several members' whole responses scored forward-only in one batched call
(ls_score_fwd) against one captured prompt.  Each member is checked element by element against
the oracle's forward of its own rows, and, on the matrix-core path, bit for bit against the
single-member replay forward of the same rows."""
import numpy as np
import pytest
import torch

from _cases import Case, assert_close, log, np32
from oracle import attention as orc
from suffix_attention_amd import api

pytestmark = pytest.mark.gpu


def _members(M, P, R, hq, hkv, d, dtype, S, seed):
    """M members (own Q, K_r, V_r) over the prompt of the first one."""
    cs = [Case(P, R, hq, hkv, d, dtype, seed=seed + m, S=S) for m in range(M)]
    for c in cs[1:]:
        c.kp, c.vp, c.table, c.n_phys, c.bounds = cs[0].kp, cs[0].vp, cs[0].table, cs[0].n_phys, cs[0].bounds
    return cs


def _score(cs, pre):
    q = torch.stack([c.q for c in cs]).cuda()
    kr = torch.stack([c.kr for c in cs]).cuda()
    vr = torch.stack([c.vr for c in cs]).cuda()
    o, lse, _ = api.score_fwd(pre, q, kr, vr)
    torch.cuda.synchronize()
    return o, lse


def _check_oracle(cs, o, lse):
    for m, c in enumerate(cs):
        log(f"  member {m}")
        O, L = orc.forward(np32(c.q), np32(c.kp), np32(c.vp), np32(c.kr), np32(c.vr), 0)
        assert_close("O", np32(o[m]), O)
        assert_close("LSE", np32(lse[m]), L)


def test_score_bf16_three_members_ragged():
    log("case: score bf16 M=3 P=700 R=90 hq=24 hkv=4 d=256 S=3")
    cs = _members(3, 700, 90, 24, 4, 256, torch.bfloat16, S=3, seed=40)
    pre = cs[0].prefix()
    o, lse = _score(cs, pre)
    _check_oracle(cs, o, lse)


def test_score_bf16_equals_single_member_replay_bitwise():
    """Same rows, same tiles, same arithmetic: the batched forward gives the replay's bits."""
    log("case: score vs replay bitwise M=4 P=1000 R=150 hq=24 hkv=4 d=256 S=2")
    cs = _members(4, 1000, 150, 24, 4, 256, torch.bfloat16, S=2, seed=50)
    pre = cs[0].prefix()
    o, lse = _score(cs, pre)
    for m, c in enumerate(cs):
        o1, l1, _ = api.replay_fwd(pre, c.q.cuda(), 0, c.kr.cuda(), c.vr.cuda())
        torch.cuda.synchronize()
        assert torch.equal(o[m], o1) and torch.equal(lse[m], l1), f"member {m}"


@pytest.mark.parametrize("d", [64, 256])
def test_score_f32_members(d):
    log(f"case: score fp32 M=2 P=300 R=40 hq=4 hkv=2 d={d} S=2")
    cs = _members(2, 300, 40, 4, 2, d, torch.float32, S=2, seed=60)
    pre = cs[0].prefix()
    o, lse = _score(cs, pre)
    _check_oracle(cs, o, lse)


def test_score_promptless_and_single_row():
    log("case: score bf16 P=0 M=2 R=70; then R=1")
    cs = _members(2, 0, 70, 6, 2, 256, torch.bfloat16, S=1, seed=70)
    o, lse = _score(cs, cs[0].prefix())
    _check_oracle(cs, o, lse)
    cs = _members(3, 130, 1, 6, 1, 256, torch.bfloat16, S=2, seed=71)
    o, lse = _score(cs, cs[0].prefix())
    _check_oracle(cs, o, lse)


def test_score_at_2m_tokens_equals_replay_and_oracle_rows():
    """The 2M-token prompt (c2m shape, permuted pages, 8 shards), two members batched: each
    member's rows equal its own replay forward bit for bit, and sampled rows equal the oracle
    computed one row at a time over all prompt and response keys."""
    from suffix_attention_amd import configs, datagen

    cfg = configs.CONFIGS["c2m"]
    R = 256
    log(f"case: score at P={cfg.P}, 2 members x {R} rows")
    dev = "cuda"
    table = datagen.page_table(cfg.n_pages, datagen.seed(cfg.cfg_id, datagen.TAG_PERM), dev)
    kp, vp = datagen.prefix_kv(cfg, dev)
    k_pages, v_pages = api.capture_pages(kp, vp, table, cfg.n_pages)
    pre = api.Prefix(cfg.hq, cfg.hkv, cfg.d, cfg.dtype, cfg.P, table, k_pages, v_pages,
                     api.even_shard_bounds(cfg.n_pages, cfg.S))
    ms = [datagen.member_inputs(cfg, i, dev) for i in range(2)]
    q = torch.stack([m["q"][:R] for m in ms])
    kr = torch.stack([m["kr"][:R] for m in ms])
    vr = torch.stack([m["vr"][:R] for m in ms])
    o, lse, ws = api.score_fwd(pre, q, kr, vr)
    del ws
    torch.cuda.synchronize()
    for i in range(2):
        o1, l1, ws1 = api.replay_fwd(pre, q[i].contiguous(), 0, kr[i].contiguous(), vr[i].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o[i], o1) and torch.equal(lse[i], l1), f"member {i}"
        del ws1
    kp_h, vp_h = np32(kp), np32(vp)
    for i, row in ((0, 0), (0, R - 1), (1, 97)):
        O, L = orc.forward(np32(q[i, row:row + 1]), kp_h, vp_h, np32(kr[i]), np32(vr[i]), row)
        assert_close(f"O[{i},{row}]", np32(o[i, row:row + 1]), O)
        assert_close(f"LSE[{i},{row}]", np32(lse[i, row:row + 1]), L)
