"""Parity at the benchmark's full sizes, in the launch configuration it times.

The 2M-token workload (P = 2,097,152 in 64-token pages behind a seeded permuted table, 8
shards, Hq 24 / Hkv 4, d 256, bf16, one 1024-row block at the end of a 4096-token response)
is too large for the oracle to redo in full, so these tests check
  * sampled rows, which the oracle computes one at a time over all 2M + response keys;
  * identities of the gradient that hold at any size (sums of dK and dV over all keys);
  * a closed form at full size (all keys zero: uniform attention), for every output;
and, at a smaller prompt, that the group driver's accumulation is linear in the members,
that its peak memory is flat in G, and that the block size does not change the result.
"""
import math

import numpy as np
import pytest
import torch

from _cases import ATOL, REL_L2, assert_close, log, np32
from oracle import attention as orc
from suffix_attention_amd import api, configs, datagen, driver

pytestmark = pytest.mark.gpu

C2M = configs.CONFIGS["c2m"]


def _prefix(cfg, kp, vp, table):
    k_pages, v_pages = api.capture_pages(kp, vp, table, cfg.n_pages)
    return api.Prefix(cfg.hq, cfg.hkv, cfg.d, cfg.dtype, cfg.P, table, k_pages, v_pages,
                      api.even_shard_bounds(cfg.n_pages, cfg.S))


def _block(pre, m, q_start, n, store_ds=True, parts=None, fused=False):
    """One replayed block (forward + first-touch backward) through the C ABI; by default with
    the stored-dS backward that the benchmark runs at the 2M-token size.  parts: run the
    stored-dS backward one kv head by `parts` consecutive key parts at a time.  fused: the fused
    forward + dQ pass, then the backward without dQ (bench.py --workload fused)."""
    q, do = m["q"][q_start:q_start + n].contiguous(), m["do"][q_start:q_start + n].contiguous()
    if fused:
        o, lse, dq, _ = api.replay_fwd_dq(pre, q, q_start, m["kr"], m["vr"], do)
    else:
        o, lse, _ = api.replay_fwd(pre, q, q_start, m["kr"], m["vr"])
    dkr = torch.empty(m["kr"].shape, dtype=torch.float32, device="cuda")
    dvr = torch.empty_like(dkr)
    dkp = torch.empty(pre.k_pages.shape, dtype=torch.float32, device="cuda")
    dvp = torch.empty_like(dkp)
    ws = None
    if parts is not None:
        nbytes = api.bwd_ds_workspace_bytes(pre, n, q_start + n, heads=1, parts=parts)
        ws = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device="cuda")
    r = api.replay_bwd(pre, q, q_start, m["kr"], m["vr"], o, lse, do, dkr, dvr, True, dkp, dvp,
                       shard_first_touch=[True] * pre.n_shards, store_ds=store_ds, workspace=ws,
                       dq_pass=not fused)
    dq = dq if fused else r
    del ws
    torch.cuda.synchronize()
    return dict(o=o, lse=lse, dq=dq, dkr=dkr, dvr=dvr, dkp=dkp, dvp=dvp, q=q, do=do)


def _sampled_rows_and_gradient_sums(cfg, q_start, n, rows, store_ds, parts=None, fused=False):
    """The block [q_start, q_start + n) of member 0 at the config's full size: sampled rows of
    one kv head against the oracle over every key they see, and the gradient identities over
    all keys.  With the fused pass, dQ's reference takes delta from the exact output (it forms
    delta = sum P dP from its own unrounded products)."""
    table = datagen.page_table(cfg.n_pages, datagen.seed(cfg.cfg_id, datagen.TAG_PERM), "cuda")
    kp, vp = datagen.prefix_kv(cfg, "cuda")
    pre = _prefix(cfg, kp, vp, table)
    m = datagen.member_inputs(cfg, 0, "cuda")
    res = _block(pre, m, q_start, n, store_ds=store_ds, parts=parts, fused=fused)
    g = cfg.g
    kend = q_start + n

    # sampled rows of one kv head, each against all prompt and response keys, by the oracle
    kvh = 1
    heads = slice(kvh * g, (kvh + 1) * g)
    kp1, vp1 = np32(kp[:, kvh:kvh + 1]), np32(vp[:, kvh:kvh + 1])
    kr1, vr1 = np32(m["kr"][:kend, kvh:kvh + 1]), np32(m["vr"][:kend, kvh:kvh + 1])
    for r in rows:
        pos = q_start + r
        qr = np32(m["q"][pos:pos + 1, heads])
        dor = np32(m["do"][pos:pos + 1, heads])
        O, L = orc.forward(qr, kp1, vp1, kr1, vr1, pos)
        gr = orc.backward(qr, kp1, vp1, kr1, vr1, dor, pos, o=O if fused else orc.round_bf16(O), lse=L,
                          prefix_grad_sink=lambda *a: None)
        log(f"  row {pos}")
        assert_close("O", np32(res["o"][r:r + 1, heads]), O)
        assert_close("LSE", np32(res["lse"][r:r + 1, heads]), L)
        assert_close("dQ", np32(res["dq"][r:r + 1, heads]), gr["dq"])
    del kp1, vp1, kp, vp

    # sum over every key the block sees of dV = sum over its rows and group heads of dO;
    # sum of dK = scale * sum_rows sum_keys dS q = 0, because sum_keys dS = delta - delta
    f64 = torch.float64
    dv_sum = res["dvp"].sum(dim=(0, 2), dtype=f64) + res["dvr"][:kend].sum(dim=0, dtype=f64)      # [hkv, d]
    dk_sum = res["dkp"].sum(dim=(0, 2), dtype=f64) + res["dkr"][:kend].sum(dim=0, dtype=f64)
    do_sum = m["do"][q_start:kend].view(n, cfg.hkv, g, cfg.d).sum(dim=(0, 2), dtype=f64)
    rel_dv = float((dv_sum - do_sum).norm() / do_sum.norm())
    dk_sq = sum(float(torch.linalg.vector_norm(x, dtype=f64) ** 2) for x in (res["dkp"], res["dkr"][:kend]))
    rel_dk = float(dk_sum.norm()) / math.sqrt(dk_sq)
    log(f"    sum dV vs sum dO rel={rel_dv:.3e}; |sum dK| / ||dK||_F = {rel_dk:.3e}")
    assert rel_dv <= REL_L2
    # sum_j dK_j is exactly 0, so what remains is the sum of the per-key errors; errors that are
    # independent across keys add up to their Frobenius norm, so |sum dK| / ||dK||_F is about the
    # relative L2 error of dK itself, which the per-element parity bounds by REL_L2
    assert rel_dk <= REL_L2


def test_c2m_block_sampled_rows_and_gradient_sums():
    cfg = C2M
    q_start, n = cfg.R - cfg.B, cfg.B
    log(f"case: c2m P={cfg.P} block rows [{q_start}, {q_start + n}) sampled rows + gradient sums")
    _sampled_rows_and_gradient_sums(cfg, q_start, n, (0, 511, n - 1), store_ds=True)


def test_c2m_block_fused_pass_sampled_rows_and_gradient_sums():
    """The same block through the fused forward + dQ pass and the backward without dQ."""
    cfg = C2M
    q_start, n = cfg.R - cfg.B, cfg.B
    log(f"case: c2m P={cfg.P} block rows [{q_start}, {q_start + n}) fused pass: sampled rows + gradient sums")
    _sampled_rows_and_gradient_sums(cfg, q_start, n, (0, 511, n - 1), store_ds=False, fused=True)


def test_c1m_block_sampled_rows_and_gradient_sums():
    """The 1M-token workload's last reverse block of 512 rows (of a 2,048-token response)."""
    cfg = configs.CONFIGS["c1m"]
    q_start, n = cfg.R - cfg.B, cfg.B
    log(f"case: c1m P={cfg.P} block rows [{q_start}, {q_start + n}) sampled rows + gradient sums")
    _sampled_rows_and_gradient_sums(cfg, q_start, n, (0, 300, n - 1), store_ds=True)


@pytest.mark.parametrize("form", ["recompute", "stored dS, 1 kv head x 2 key parts"])
def test_stress_block_sampled_rows_and_gradient_sums(form):
    """The stress workload's last reverse block: 8,192 rows at the end of a 262,144-token
    response over a 4,194,304-token prompt in 16 shards, so its rows see 4,456,448 keys.  One
    block's dS over all keys would take 1.75 TB, so the backward either recomputes or stores dS
    one kv head by two key parts (two shards, or the response keys) at a time: 52 GB."""
    cfg = configs.CONFIGS["stress"]
    q_start, n = cfg.R - cfg.B, cfg.B
    log(f"case: stress P={cfg.P} S={cfg.S} block rows [{q_start}, {q_start + n}) {form}: sampled rows + gradient sums")
    if form == "recompute":
        _sampled_rows_and_gradient_sums(cfg, q_start, n, (0, 4097, n - 1), store_ds=False)
    else:
        _sampled_rows_and_gradient_sums(cfg, q_start, n, (0, 4097, n - 1), store_ds=False, parts=2)


def test_c2m_zero_keys_closed_form():
    """All keys zero: every visible key gets probability 1/n_vis, so O is the mean of the
    visible values, LSE = log(n_vis), dQ = 0 exactly, and dK / dV have closed forms."""
    cfg = C2M
    q_start, n = cfg.R - cfg.B, cfg.B
    log(f"case: c2m P={cfg.P} zero keys, rows [{q_start}, {q_start + n})")
    table = datagen.page_table(cfg.n_pages, datagen.seed(cfg.cfg_id, datagen.TAG_PERM), "cuda")
    _, vp = datagen.prefix_kv(cfg, "cuda")
    kp = torch.zeros_like(vp)
    pre = _prefix(cfg, kp, vp, table)
    m = datagen.member_inputs(cfg, 1, "cuda")
    m["kr"] = torch.zeros_like(m["kr"])
    res = _block(pre, m, q_start, n)
    g, d, hkv, P = cfg.g, cfg.d, cfg.hkv, cfg.P
    scale = 1.0 / math.sqrt(d)
    kend = q_start + n

    # closed forms in float64 from the inputs
    f64 = torch.float64
    vsum_p = vp.to(f64).sum(dim=0).cpu().numpy()                                  # [hkv, d]
    vr = np32(m["vr"]).astype(np.float64)                                         # [R, hkv, d]
    vcum = np.cumsum(vr, axis=0)                                                  # inclusive
    pos = q_start + np.arange(n)
    nvis = (P + pos + 1).astype(np.float64)                                       # [n]
    kv_of = np.arange(cfg.hq) // g
    O = (vsum_p[kv_of][None] + vcum[pos][:, kv_of]) / nvis[:, None, None]         # [n, hq, d]
    assert_close("O", np32(res["o"]), O)
    assert_close("LSE", np32(res["lse"]), np.broadcast_to(np.log(nvis)[:, None], (n, cfg.hq)))
    assert torch.count_nonzero(res["dq"]) == 0, "dQ must be exactly zero when every key is zero"

    q = np32(m["q"][q_start:kend]).astype(np.float64)
    do = np32(m["do"][q_start:kend]).astype(np.float64)
    dlt = (do * orc.round_bf16(O)).sum(-1)                                        # [n, hq]
    w = 1.0 / nvis
    rng = np.random.default_rng(5)
    sample = np.sort(rng.choice(P, 4096, replace=False))
    tab = table.cpu().numpy()
    for kv in range(hkv):
        hs = slice(kv * g, (kv + 1) * g)
        qg, dog, dlg = q[:, hs], do[:, hs], dlt[:, hs]                             # [n, g, d], [n, g]
        # prompt keys: every row sees them, so every prompt key has the same dV
        dv_exp = (w[:, None] * dog.sum(axis=1)).sum(axis=0)                       # sum_r w sum_g dO
        dvp = res["dvp"][:, kv].reshape(-1, d).to(f64)                            # all 2M keys
        dv_t = torch.as_tensor(dv_exp, device="cuda")
        err = float((dvp - dv_t).abs().max())
        rel = float((dvp - dv_t).norm() / (dv_t.norm() * math.sqrt(dvp.shape[0])))
        log(f"    dV_pr{kv}: max_abs={err:.3e} rel_l2={rel:.3e}")
        assert err <= ATOL and rel <= REL_L2
        M = (qg * w[:, None, None]).reshape(-1, d).T @ dog.reshape(-1, d)         # sum w q dO^T
        c = ((w[:, None] * dlg)[:, :, None] * qg).sum(axis=(0, 1))                # sum w delta q
        vs = np32(vp[torch.as_tensor(sample, device="cuda"), kv]).astype(np.float64)
        dk_exp = scale * (vs @ M.T - c[None])                                     # scale (M v - c) per key
        phys = torch.as_tensor(tab[sample // 64], device="cuda", dtype=torch.long)
        slot = torch.as_tensor(sample % 64, device="cuda", dtype=torch.long)
        assert_close(f"dK_pr{kv}", np32(res["dkp"][phys, kv, slot]), dk_exp)
        # response keys j < kend: rows whose position is >= j see them
        vis = (pos[:, None] >= np.arange(kend)[None, :])                          # [n, kend]
        wv = w[:, None] * vis                                                     # [n, kend]
        dvr_exp = wv.T @ dog.sum(axis=1)
        X = dog.reshape(-1, d) @ vr[:kend, kv].T - dlg.reshape(-1)[:, None]       # [n g, kend]: dO.V_j - delta
        Y = X * np.repeat(wv, g, axis=0)
        dkr_exp = scale * (Y.T @ qg.reshape(-1, d))
        assert_close(f"dV_resp{kv}", np32(res["dvr"][:kend, kv]), dvr_exp)
        assert_close(f"dK_resp{kv}", np32(res["dkr"][:kend, kv]), dkr_exp)


SMALL = configs.CONFIGS["c128k"].with_(R=1024, G=3)


def _small_prefix(cfg):
    table = datagen.page_table(cfg.n_pages, datagen.seed(cfg.cfg_id, datagen.TAG_PERM), "cuda")
    kp, vp = datagen.prefix_kv(cfg, "cuda")
    return _prefix(cfg, kp, vp, table)


def test_group_accumulation_is_linear_and_peak_memory_flat():
    """The prompt gradient pages after G serial members equal the sum of each member's pages
    replayed alone; every member's peak device memory is the same (flat in G: the gradient
    pages are allocated once, by the first member, and everything a member allocates is freed
    before the next)."""
    cfg = SMALL
    log(f"case: group of {cfg.G} members, P={cfg.P}, R={cfg.R}, B=512")
    pre = _small_prefix(cfg)
    members = [lambda i=i: datagen.member_inputs(cfg, i, "cuda") for i in range(cfg.G)]
    grp, results = driver.replay_group(pre, members, 512, keep="none", track_peak=True)
    peaks = [r.peak_bytes for r in results]
    log(f"    per-member peak device memory: {peaks}")
    assert len(set(peaks)) == 1, peaks
    total_k = torch.zeros_like(grp.dk_pages, dtype=torch.float64)
    total_v = torch.zeros_like(total_k)
    for i in range(cfg.G):
        alone, _ = driver.replay_group(pre, [members[i]], 512, keep="none")
        total_k += alone.dk_pages.to(torch.float64)
        total_v += alone.dv_pages.to(torch.float64)
        del alone
    for name, got, ref in (("dK_pages", grp.dk_pages, total_k), ("dV_pages", grp.dv_pages, total_v)):
        rel = float((got.to(torch.float64) - ref).norm() / ref.norm())
        log(f"    {name} accumulated vs summed alone: rel_l2={rel:.3e}")
        assert rel <= 1e-5


def test_group_with_kv_head_chunks_of_stored_ds():
    """With a memory budget that holds the dS of only two of the four kv heads, the driver runs
    the stored-dS backward a chunk of two kv heads at a time: every member's outputs and the
    group's gradient pages equal those of the unchunked replay bit for bit, and each member's
    peak memory is below the unchunked one (by the same amount for every member; the members'
    kept outputs raise later members' peaks equally in both runs)."""
    cfg = SMALL.with_(G=2)
    log(f"case: group of {cfg.G} members, P={cfg.P}, R={cfg.R}, B=512, stored dS in chunks of 2 kv heads")
    pre = _small_prefix(cfg)
    members = [lambda i=i: datagen.member_inputs(cfg, i, "cuda") for i in range(cfg.G)]
    full_ws = api.bwd_ds_workspace_bytes(pre, 512, cfg.R)
    two = api.bwd_ds_workspace_bytes(pre, 512, cfg.R, heads=2)
    assert two < full_ws
    g_full, r_full = driver.replay_group(pre, members, 512, ds_budget=full_ws, track_peak=True)
    g_two, r_two = driver.replay_group(pre, members, 512, ds_budget=two, track_peak=True)
    assert g_full.plan == driver.BwdPlan(cfg.hkv, cfg.S + 1) and g_two.plan == driver.BwdPlan(2, cfg.S + 1)
    for a, b in zip(r_full, r_two):
        for name in ("o", "lse", "dq", "dk_resp", "dv_resp"):
            assert torch.equal(getattr(a, name), getattr(b, name)), name
    assert torch.equal(g_full.dk_pages, g_two.dk_pages) and torch.equal(g_full.dv_pages, g_two.dv_pages)
    peaks_full, peaks_two = [r.peak_bytes for r in r_full], [r.peak_bytes for r in r_two]
    log(f"    peak bytes per member: all heads {peaks_full}, two-head chunks {peaks_two}")
    saved = [f - t for f, t in zip(peaks_full, peaks_two)]
    assert saved[0] > 0 and len(set(saved)) == 1, saved


def test_block_size_does_not_change_the_result():
    cfg = SMALL
    log(f"case: member replayed with B=1024 and B=384 (ragged), P={cfg.P}, R={cfg.R}")
    pre = _small_prefix(cfg)
    m = datagen.member_inputs(cfg, 0, "cuda")
    out = {}
    for B in (1024, 384):
        grp = driver.GroupReplay(pre)
        r = grp.replay_member(m["q"], m["kr"], m["vr"], m["do"], B)
        torch.cuda.synchronize()
        out[B] = (r, grp)
    (a, ga), (b, gb) = out[1024], out[384]
    # The blocks differ in size, so in the order of float32 sums (a 384-row block splits the
    # shards into page ranges, a 1,024-row one does not): the bf16 O may move by its last bit,
    # 2^-8 relative, and every other tensor stays within a fifth of the oracle bound.
    for name, x, y in (("O", a.o, b.o), ("LSE", a.lse, b.lse), ("dQ", a.dq, b.dq), ("dK_resp", a.dk_resp, b.dk_resp),
                       ("dV_resp", a.dv_resp, b.dv_resp), ("dK_pages", ga.dk_pages, gb.dk_pages),
                       ("dV_pages", ga.dv_pages, gb.dv_pages)):
        rel = 2.0 ** -8 if name == "O" else REL_L2 / 5
        assert_close(name, np32(y), np32(x).astype(np.float64), atol=ATOL, rel_l2=rel)


def test_prefix_reuse_cycles_are_steady():
    """Consecutive optimizer cycles over one capture (each a fresh group: gradient pages
    allocated at its first backward and released at its end) give bit-identical gradient pages
    and the same peak memory every cycle."""
    cfg = configs.CONFIGS["c128k"].with_(P=65536, R=512, B=256, G=2)
    log(f"case: prefix reuse, 3 cycles at P={cfg.P}, G={cfg.G}, R={cfg.R}, B={cfg.B}")
    table = datagen.page_table(cfg.n_pages, datagen.seed(cfg.cfg_id, datagen.TAG_PERM), "cuda")
    kp, vp = datagen.prefix_kv(cfg, "cuda")
    pre = _prefix(cfg, kp, vp, table)
    members = [datagen.member_inputs(cfg, i, "cuda") for i in range(cfg.G)]
    pages, peaks = [], []
    for _ in range(3):
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        grp, _ = driver.replay_group(pre, members, cfg.B, keep="none")
        torch.cuda.synchronize()
        peaks.append(torch.cuda.max_memory_allocated())
        pages.append((grp.dk_pages.cpu(), grp.dv_pages.cpu()))  # host copies: device memory stays the same
        del grp
    for c in (1, 2):
        assert torch.equal(pages[c][0], pages[0][0]) and torch.equal(pages[c][1], pages[0][1]), c
    log(f"    peaks {peaks}")
    assert peaks[1] == peaks[2]
