"""Parity with the oracle at the workloads' own sizes.

* c128k in full: P = 131,072 prompt tokens (2,048 pages behind a seeded permuted table, 8
  shards), G = 2 members with 1,024-row responses (one block each), Hq 24 / Hkv 4, d 256, bf16.
  Both members go through the group driver with the stored-dS backward, and every output of
  every member, plus the prompt K/V gradient pages summed over the two members, are compared
  with the oracle over all keys.
* c2m subset block: a 64-row block at a seeded offset of the 2M-token workload's last response
  block, run through the stored-dS backward with first-touch gradient pages, so that the pages
  hold exactly this block's contribution.  All 2,097,152 prompt keys' dK and dV, for every kv
  head, are compared with the oracle's contribution of the same 64 rows (streamed key chunk by
  key chunk, so host memory stays bounded); its O, LSE and dQ rows must also be those of the
  full 1,024-row block (rows are independent) up to the order of float32 sums.
(Explainer, "Serial replay makes G a schedule": exact attention; digest, "Method": the exact
global output from the shards' local statistics.)
"""
import math

import numpy as np
import pytest
import torch

from _cases import ATOL, REL_L2, assert_close, log, np32
from oracle import attention as orc
from suffix_attention_amd import api, configs, datagen, driver

pytestmark = pytest.mark.gpu


def _prefix(cfg):
    table = datagen.page_table(cfg.n_pages, datagen.seed(cfg.cfg_id, datagen.TAG_PERM), "cuda")
    kp, vp = datagen.prefix_kv(cfg, "cuda")
    k_pages, v_pages = api.capture_pages(kp, vp, table, cfg.n_pages)
    pre = api.Prefix(cfg.hq, cfg.hkv, cfg.d, cfg.dtype, cfg.P, table, k_pages, v_pages,
                     api.even_shard_bounds(cfg.n_pages, cfg.S))
    return pre, kp, vp


def _logical_pages(pages: torch.Tensor, table: torch.Tensor, P: int, kv: int) -> torch.Tensor:
    """Gradient pages of kv head kv, [n_phys, hkv, 64, d] on the device -> logical order [P, d]."""
    d = pages.shape[-1]
    return pages[:, kv][table.long()].reshape(-1, d)[:P]


class Streamed:
    """Running max |x - y|, sum (x - y)^2 and sum y^2 over chunks, for tensors too large to hold
    twice on the host."""

    def __init__(self):
        self.max_abs, self.sq_diff, self.sq_ref = 0.0, 0.0, 0.0

    def add(self, got: np.ndarray, ref: np.ndarray):
        diff = np.asarray(got, np.float64) - ref
        assert np.all(np.isfinite(got))
        self.max_abs = max(self.max_abs, float(np.abs(diff).max()) if diff.size else 0.0)
        self.sq_diff += float((diff * diff).sum())
        self.sq_ref += float((ref * ref).sum())

    def check(self, name):
        rel = math.sqrt(self.sq_diff / self.sq_ref)
        log(f"    {name:10s} max_abs={self.max_abs:.3e} rel_l2={rel:.3e}")
        assert self.max_abs <= ATOL and rel <= REL_L2, name


@pytest.mark.timeout(900)
def test_c128k_group_in_full():
    cfg = configs.CONFIGS["c128k"]
    log(f"case: c128k in full: P={cfg.P} S={cfg.S} G={cfg.G} R={cfg.R} B={cfg.B}, stored dS")
    pre, kp, vp = _prefix(cfg)
    members = [datagen.member_inputs(cfg, i, "cuda") for i in range(cfg.G)]
    grp, results = driver.replay_group(pre, members, cfg.B, store_ds=True)
    torch.cuda.synchronize()
    assert grp.plan == driver.BwdPlan(cfg.hkv, cfg.S + 1)
    g = cfg.g
    prompt = {"dK_prompt": Streamed(), "dV_prompt": Streamed()}
    gpu_dk = [_logical_pages(grp.dk_pages, pre.page_table, cfg.P, kv) for kv in range(cfg.hkv)]
    gpu_dv = [_logical_pages(grp.dv_pages, pre.page_table, cfg.P, kv) for kv in range(cfg.hkv)]
    sum_dk = np.zeros((cfg.P, cfg.hkv, cfg.d))
    sum_dv = np.zeros((cfg.P, cfg.hkv, cfg.d))
    kp_np, vp_np = np32(kp), np32(vp)
    for i, (m, r) in enumerate(zip(members, results)):
        q, kr, vr, do = (np32(m[k]) for k in ("q", "kr", "vr", "do"))
        for kv in range(cfg.hkv):
            hs = slice(kv * g, (kv + 1) * g)
            O, L = orc.forward(q[:, hs], kp_np[:, kv:kv + 1], vp_np[:, kv:kv + 1], kr[:, kv:kv + 1],
                               vr[:, kv:kv + 1], 0)
            gr = orc.backward(q[:, hs], kp_np[:, kv:kv + 1], vp_np[:, kv:kv + 1], kr[:, kv:kv + 1],
                              vr[:, kv:kv + 1], do[:, hs], 0, o=orc.round_bf16(O), lse=L)
            log(f"  member {i} kv head {kv}")
            assert_close("O", np32(r.o[:, hs]), O)
            assert_close("LSE", np32(r.lse[:, hs]), L)
            assert_close("dQ", np32(r.dq[:, hs]), gr["dq"])
            assert_close("dK_resp", np32(r.dk_resp[:, kv:kv + 1]), gr["dkr"])
            assert_close("dV_resp", np32(r.dv_resp[:, kv:kv + 1]), gr["dvr"])
            sum_dk[:, kv] += gr["dkp"][:, 0]
            sum_dv[:, kv] += gr["dvp"][:, 0]
    log("  prompt gradient pages summed over both members")
    for kv in range(cfg.hkv):
        prompt["dK_prompt"].add(np32(gpu_dk[kv]), sum_dk[:, kv])
        prompt["dV_prompt"].add(np32(gpu_dv[kv]), sum_dv[:, kv])
    for name, st in prompt.items():
        st.check(name)


@pytest.mark.timeout(900)
def test_c2m_subset_block_all_prompt_gradients():
    cfg = configs.CONFIGS["c2m"]
    rng = np.random.default_rng(datagen.seed(cfg.cfg_id, 77))
    blk0 = cfg.R - cfg.B                          # the last reverse block [3072, 4096)
    off = blk0 + int(rng.integers(0, cfg.B - 64))  # seeded offset of the 64-row subset
    n = 64
    log(f"case: c2m subset block rows [{off}, {off + n}) of P={cfg.P}: every prompt key's dK, dV")
    pre, kp, vp = _prefix(cfg)
    m = datagen.member_inputs(cfg, 0, "cuda")
    g, d = cfg.g, cfg.d

    def block(q_start, rows):
        q, do = m["q"][q_start:q_start + rows].contiguous(), m["do"][q_start:q_start + rows].contiguous()
        o, lse, _ = api.replay_fwd(pre, q, q_start, m["kr"], m["vr"])
        dkr = torch.empty(m["kr"].shape, dtype=torch.float32, device="cuda")
        dvr = torch.empty_like(dkr)
        dkp = torch.empty(pre.k_pages.shape, dtype=torch.float32, device="cuda")
        dvp = torch.empty_like(dkp)
        dq = api.replay_bwd(pre, q, q_start, m["kr"], m["vr"], o, lse, do, dkr, dvr, True, dkp, dvp,
                            shard_first_touch=[True] * pre.n_shards, store_ds=True)
        torch.cuda.synchronize()
        return dict(o=o, lse=lse, dq=dq, dkr=dkr, dvr=dvr, dkp=dkp, dvp=dvp)

    # rows are independent: the subset's O, LSE and dQ are the full block's rows, up to the order
    # of float32 sums (a 64-row block splits the shards into page ranges, the full block does
    # not).  O is stored in bf16, so a reordered sum can move its last bit (rel-L2 about 3e-3 at
    # the bf16 rounding level), and delta = rowsum(dO * O) carries that into dS and dQ (about 2e-4).
    full = block(blk0, cfg.B)
    sub = block(off, n)
    r0 = off - blk0
    for k, tol in (("o", 8e-3), ("lse", 1e-6), ("dq", 1e-3)):
        a, b = sub[k].float(), full[k][r0:r0 + n].float()
        rel = float((a - b).norm() / b.norm())
        log(f"    {k} against the full block's rows: rel_l2={rel:.2e}")
        assert rel <= tol, k
    del full

    kend = off + n
    stats = {name: Streamed() for name in ("dK_prompt", "dV_prompt")}
    for kv in range(cfg.hkv):
        hs = slice(kv * g, (kv + 1) * g)
        q = np32(m["q"][off:kend, hs])
        do = np32(m["do"][off:kend, hs])
        kp1, vp1 = np32(kp[:, kv:kv + 1]), np32(vp[:, kv:kv + 1])
        kr1, vr1 = np32(m["kr"][:kend, kv:kv + 1]), np32(m["vr"][:kend, kv:kv + 1])
        gk = _logical_pages(sub["dkp"], pre.page_table, cfg.P, kv)
        gv = _logical_pages(sub["dvp"], pre.page_table, cfg.P, kv)

        def sink(_kv, a, b, dk_c, dv_c):
            stats["dK_prompt"].add(np32(gk[a:b]), dk_c)
            stats["dV_prompt"].add(np32(gv[a:b]), dv_c)

        O, L = orc.forward(q, kp1, vp1, kr1, vr1, off)
        gr = orc.backward(q, kp1, vp1, kr1, vr1, do, off, o=orc.round_bf16(O), lse=L, prefix_grad_sink=sink)
        log(f"  kv head {kv}")
        assert_close("O", np32(sub["o"][:, hs]), O)
        assert_close("LSE", np32(sub["lse"][:, hs]), L)
        assert_close("dQ", np32(sub["dq"][:, hs]), gr["dq"])
        assert_close("dK_resp", np32(sub["dkr"][:kend, kv:kv + 1]), gr["dkr"])
        assert_close("dV_resp", np32(sub["dvr"][:kend, kv:kv + 1]), gr["dvr"])
        del gk, gv, kp1, vp1
    for name, st in stats.items():
        st.check(name)
