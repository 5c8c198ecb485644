"""Parity of the HIP path (through the C ABI) with the CPU oracle, element by element, at sizes
the oracle finishes in seconds: several tiles, ragged tails, GQA, every part kind."""
import numpy as np
import pytest
import torch

from _cases import Case, assert_close, check_against_oracle, log, np32
from oracle import attention as orc
from suffix_attention_amd import api, datagen

pytestmark = pytest.mark.gpu


def test_tiny_config_fp32():
    """The tiny workload in full: P=4096 (64 pages, permuted), R=256, Hq=4, Hkv=1, d=64, fp32, S=2."""
    log("case: tiny fp32 P=4096 R=256 hq=4 hkv=1 d=64 S=2")
    c = Case(4096, 256, 4, 1, 64, torch.float32, seed=1, S=2)
    check_against_oracle(c, 0, 256)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_bf16_small_all_head_dims(d):
    log(f"case: bf16 P=700 R=160 hq=6 hkv=2 d={d} S=3")
    c = Case(700, 160, 6, 2, d, torch.bfloat16, seed=2, S=3)
    check_against_oracle(c, 32, 96)


def test_bf16_gqa6_ragged_blocks():
    """The real head shape (24/4/256) with a ragged prompt tail and a mid-response block."""
    log("case: bf16 P=1000 R=300 hq=24 hkv=4 d=256 S=8 rows [100, 300)")
    c = Case(1000, 300, 24, 4, 256, torch.bfloat16, seed=3, S=8)
    check_against_oracle(c, 100, 200)


@pytest.mark.parametrize("n", [85, 86])
def test_bf16_both_sides_of_the_forward_tile_threshold(n):
    """510 and 516 group rows (GQA 6): the forward runs 128-row workgroups below 512 group rows
    and 256-row ones from there on, each with a ragged last tile (126 of 128 rows, 4 of 256)."""
    log(f"case: bf16 P=1000 R=200 hq=24 hkv=4 d=256 S=3 rows [60, {60 + n}) = {6 * n} group rows")
    c = Case(1000, 200, 24, 4, 256, torch.bfloat16, seed=11, S=3)
    check_against_oracle(c, 60, n)


def test_bf16_uneven_and_empty_shards():
    log("case: bf16 P=1280 (20 pages) bounds [0,0,3,3,11,20]")
    c = Case(1280, 64, 12, 4, 256, torch.bfloat16, seed=4, bounds=[0, 0, 3, 3, 11, 20])
    check_against_oracle(c, 0, 64)


def test_fp32_d256_and_d128():
    for d in (128, 256):
        log(f"case: fp32 P=300 R=70 hq=4 hkv=2 d={d} S=2")
        c = Case(300, 70, 4, 2, d, torch.float32, seed=5, S=2)
        check_against_oracle(c, 10, 60)


def test_promptless_block():
    log("case: bf16 P=0 R=200 rows [72, 200)")
    c = Case(0, 200, 6, 2, 256, torch.bfloat16, seed=6, S=1)
    check_against_oracle(c, 72, 128)


def test_single_row_block():
    log("case: bf16 P=130 R=5 single row at q_start=4")
    c = Case(130, 5, 6, 1, 256, torch.bfloat16, seed=7, S=2)
    check_against_oracle(c, 4, 1)


def test_page_permutation_invariance_bitwise():
    """Outputs do not depend on where pages live: identity vs permuted tables agree bit for bit."""
    log("case: permutation invariance P=2000 hq=24 hkv=4 d=256")
    a = Case(2000, 128, 24, 4, 256, torch.bfloat16, seed=8, S=4, table="perm", n_phys_extra=5)
    b = Case(2000, 128, 24, 4, 256, torch.bfloat16, seed=8, S=4, table="identity")
    ra, rb = a.gpu(0, 128), b.gpu(0, 128)
    for k in ("o", "lse", "dq", "dkr", "dvr"):
        assert torch.equal(ra[k], rb[k]), k
    assert np.array_equal(a.logical(ra["dk_pages"]), b.logical(rb["dk_pages"]))
    assert np.array_equal(a.logical(ra["dv_pages"]), b.logical(rb["dv_pages"]))


def test_determinism_bitwise():
    log("case: determinism P=1500 hq=12 hkv=2 d=256")
    c = Case(1500, 96, 12, 2, 256, torch.bfloat16, seed=9, S=3)
    pre = c.prefix()
    r1, r2 = c.gpu(0, 96, prefix=pre), c.gpu(0, 96, prefix=pre)
    for k in ("o", "lse", "dq", "dkr", "dvr", "dk_pages", "dv_pages"):
        assert torch.equal(r1[k], r2[k]), k


def test_unseen_and_padding_keys_never_read():
    """Response keys past the block and prompt rows past P (the partial last page) may hold
    NaN: results stay finite and identical."""
    log("case: NaN poisoning P=650 R=256 rows [64, 128)")
    c = Case(650, 256, 6, 2, 256, torch.bfloat16, seed=10, S=2)
    clean = c.gpu(64, 64)
    kr = c.kr.clone()
    vr = c.vr.clone()
    kr[128:] = float("nan")
    vr[128:] = float("nan")
    pre = c.prefix(pool_fill=float("nan"))  # unused pool rows (tail of the last page) are NaN
    dirty = c.gpu(64, 64, prefix=pre, kr=kr, vr=vr)
    for k in ("o", "lse", "dq"):
        assert torch.equal(clean[k], dirty[k]), k
    assert torch.equal(clean["dkr"][:128], dirty["dkr"][:128])
    assert np.array_equal(c.logical(clean["dk_pages"]), c.logical(dirty["dk_pages"]))


def test_large_magnitude_masked_keys():
    """Masked in-block response keys with huge scores must not leak into visible rows."""
    log("case: adversarial masked keys")
    c = Case(256, 128, 6, 2, 256, torch.bfloat16, seed=11, S=1)
    c.kr[40:128] = c.kr[40:128] * 60.0  # keys only later rows see
    # dQ = scale * sum dS K is linear in |K|: its max-abs bound scales with the x60 keys
    # (bf16 rounding of dS is relative); every rel-L2 bound is unchanged.
    check_against_oracle(c, 0, 128, parts=False, atol={"dQ": 60 * 2e-2})


def test_accumulation_vs_first_touch():
    """Second backward into the same pages adds: first touch writes g, then g + g."""
    log("case: accumulate")
    c = Case(600, 64, 6, 2, 256, torch.bfloat16, seed=12, S=2)
    pre = c.prefix()
    dev = "cuda"
    q, do = c.q.to(dev), c.do.to(dev)
    kr, vr = c.kr.to(dev), c.vr.to(dev)
    o, lse, _ = api.replay_fwd(pre, q, 0, kr, vr)
    dk_r = torch.empty(kr.shape, dtype=torch.float32, device=dev)
    dv_r = torch.empty_like(dk_r)
    dk_p = torch.empty(pre.k_pages.shape, dtype=torch.float32, device=dev)
    dv_p = torch.empty_like(dk_p)
    api.replay_bwd(pre, q, 0, kr, vr, o, lse, do, dk_r, dv_r, True, dk_p, dv_p, [True, True])
    g1 = (dk_p.clone(), dv_p.clone(), dk_r.clone(), dv_r.clone())
    api.replay_bwd(pre, q, 0, kr, vr, o, lse, do, dk_r, dv_r, False, dk_p, dv_p, [False, False])
    torch.cuda.synchronize()
    for a, b in zip(g1, (dk_p, dv_p, dk_r, dv_r)):
        idx = torch.isfinite(a)
        assert torch.equal((a + a)[idx], b[idx])


def test_lse_merge_matches_oracle():
    log("case: lse_merge 5 parts with empty parts")
    g = torch.Generator().manual_seed(3)
    n_parts, rows, d = 5, 333, 256
    o = torch.randn(n_parts, rows, d, generator=g)
    lse = torch.randn(n_parts, rows, generator=g) * 5
    lse[1] = float("-inf")
    o[1] = 0
    lse[3, :100] = float("-inf")
    o[3, :100] = 0
    lse[:, 7] = float("-inf")  # a row with no key at all
    o[:, 7] = 0
    Om, Lm = orc.lse_merge(o.numpy(), lse.numpy())
    go, gl = api.lse_merge(o.cuda(), lse.cuda(), torch.float32)
    gl = np32(gl)
    assert np.isneginf(gl[7]) and np.all(np32(go)[7] == 0)
    keep = np.arange(rows) != 7
    assert_close("merge O", np32(go)[keep], Om[keep], atol=1e-5, rel_l2=1e-6)
    assert_close("merge L", gl[keep], Lm[keep], atol=1e-5, rel_l2=1e-6)
    # one part: exact identity
    go1, gl1 = api.lse_merge(o[:1].cuda().contiguous(), lse[:1].cuda().contiguous(), torch.float32)
    assert torch.equal(go1.cpu(), o[0]) and torch.equal(gl1.cpu(), lse[0])
    # bf16 output is the float32 result rounded to nearest-even
    gob, _ = api.lse_merge(o.cuda(), lse.cuda(), torch.bfloat16)
    assert torch.equal(gob.cpu(), go.cpu().to(torch.bfloat16))


def test_bf16_numerator_merge_variant():
    """The pages' BF16-numerator merge (ls_lse_merge_bf16num) against its oracle on the same
    float32 parts, and the error it adds against the exact result on a real block (9 parts:
    8 prompt shards and the response)."""
    log("case: bf16-numerator merge, synthetic parts and a P=1000 S=8 block")
    g = torch.Generator().manual_seed(4)
    n_parts, rows, d = 9, 257, 256
    o = torch.randn(n_parts, rows, d, generator=g)
    lse = torch.randn(n_parts, rows, generator=g) * 4
    lse[2, :50] = float("-inf")
    o[2, :50] = 0
    Ov, Lv = orc.lse_merge_bf16_numerator(o.numpy(), lse.numpy())
    go, gl = api.lse_merge(o.cuda(), lse.cuda(), torch.float32, bf16_numerator=True)
    assert_close("bf16num O", np32(go), Ov, atol=2e-2, rel_l2=1e-3)
    assert_close("bf16num L", np32(gl), Lv, atol=1e-5, rel_l2=1e-6)
    # a single part: the part rounded to bf16, exactly
    go1, _ = api.lse_merge(o[:1].cuda().contiguous(), lse[:1].cuda().contiguous(), torch.float32, bf16_numerator=True)
    assert torch.equal(go1.cpu(), o[0].to(torch.bfloat16).to(torch.float32))
    # on a real block: the variant against the exact output, next to the float32 merge's error
    c = Case(1000, 128, 24, 4, 256, torch.bfloat16, seed=12, S=8)
    pre = c.prefix()
    q = c.q.cuda()
    o32, _, ws = api.replay_fwd(pre, q, 0, c.kr.cuda(), c.vr.cuda())
    op, lp = api.fwd_parts(pre, 128, ws)
    hd = op.shape[-1]
    ob, _ = api.lse_merge(op.reshape(op.shape[0], -1, hd).contiguous(), lp.reshape(lp.shape[0], -1).contiguous(),
                          torch.float32, bf16_numerator=True)
    torch.cuda.synchronize()
    O, _ = orc.forward(np32(c.q), np32(c.kp), np32(c.vp), np32(c.kr), np32(c.vr), 0)
    O = O.reshape(-1, hd)
    assert_close("fp32 merge vs exact", np32(o32).reshape(-1, hd), O)
    # the variant's own error (measured 4.6e-3 rel-L2 here, against 2.2e-3 for the float32 merge
    # with its bf16 output): bounded loosely, since it is what is being measured, not a claim
    assert_close("bf16 numerator vs exact", np32(ob), O, rel_l2=1e-2)


def test_capture_gather_exact():
    """Capture then gather is a bit copy for a permuted table, a partial last page and chunked
    capture; f32 -> bf16 capture rounds to nearest-even."""
    log("case: capture/gather")
    P, hkv, d = 64 * 7 + 13, 3, 128
    for dt in (torch.bfloat16, torch.float32):
        x = datagen.normal((P, hkv, d), 5, dt)
        y = datagen.normal((P, hkv, d), 6, dt)
        table = datagen.page_table(10, 9)[:8].to(torch.int32)
        kpg, vpg = torch.zeros((10, hkv, 64, d), dtype=dt, device="cuda"), torch.zeros((10, hkv, 64, d), dtype=dt,
                                                                                       device="cuda")
        # chunked: pages [0, 3) then the rest
        api.capture_pages(x[:192].cuda(), y[:192].cuda(), table.cuda(), 10, k_pages=kpg, v_pages=vpg)
        api.capture_pages(x[192:].cuda(), y[192:].cuda(), table.cuda(), 10, first_tok=192, k_pages=kpg,
                          v_pages=vpg)
        assert torch.equal(api.gather_pages(kpg, table.cuda(), P).cpu(), x)
        assert torch.equal(api.gather_pages(vpg, table.cuda(), P).cpu(), y)
        ref = orc.capture_pages(np32(x), table.numpy(), 64, 10)
        assert np.array_equal(np32(kpg), ref)
        assert torch.equal(api.gather_pages(kpg, table.cuda(), 50, first_tok=128).cpu(), x[128:178])
    x = datagen.normal((P, hkv, d), 7, torch.float32)
    table = torch.arange(8, dtype=torch.int32)
    kpg, vpg = api.capture_pages(x.cuda(), x.cuda(), table.cuda(), 8, page_dtype=torch.bfloat16)
    assert torch.equal(api.gather_pages(kpg, table.cuda(), P).cpu(), x.to(torch.bfloat16))


# ---- the stored-dS backward: the dK/dV pass writes dS, the dQ pass reads it back

STORED_DS_CASES = [
    # (P, R, hq, hkv, d, S, q_start, n_rows, seed): every head dim, GQA 6 with a ragged prompt
    # tail and a mid-response block, a row count that is not a multiple of the dQ pass's
    # 256-row block, a promptless block, a single row
    (700, 160, 6, 2, 64, 3, 32, 96, 21),
    (700, 160, 6, 2, 128, 3, 32, 96, 22),
    (700, 160, 6, 2, 256, 3, 32, 96, 23),
    (1000, 300, 24, 4, 256, 8, 100, 200, 24),
    (1500, 700, 12, 2, 256, 5, 0, 700, 25),
    (0, 200, 6, 2, 256, 1, 72, 128, 26),
    (130, 5, 6, 1, 256, 2, 4, 1, 27),
]


@pytest.mark.parametrize("case", STORED_DS_CASES, ids=lambda c: f"P{c[0]}_R{c[1]}_h{c[2]}x{c[3]}_d{c[4]}_S{c[5]}_rows{c[6]}+{c[7]}")
def test_stored_ds_matches_oracle(case):
    P, R, hq, hkv, d, S, q0, n, seed = case
    log(f"case: stored dS bf16 P={P} R={R} hq={hq} hkv={hkv} d={d} S={S} rows [{q0}, {q0 + n})")
    c = Case(P, R, hq, hkv, d, torch.bfloat16, seed=seed, S=S)
    check_against_oracle(c, q0, n, parts=False, store_ds=True)


def test_stored_ds_uneven_and_empty_shards():
    log("case: stored dS, bounds [0,0,3,3,11,20]")
    c = Case(1280, 64, 12, 4, 256, torch.bfloat16, seed=28, bounds=[0, 0, 3, 3, 11, 20])
    check_against_oracle(c, 0, 64, parts=False, store_ds=True)


def test_stored_ds_equals_recompute():
    """Both dQ passes see the same dS: the forward and dK/dV are bit-identical (the dK/dV pass
    only adds the exact zeros of the rows it now also walks), and dQ agrees to the rounding of
    the two contraction orders."""
    log("case: stored dS vs recompute P=2000 R=384 hq=24 hkv=4 d=256 S=4 rows [128, 384)")
    c = Case(2000, 384, 24, 4, 256, torch.bfloat16, seed=29, S=4)
    pre = c.prefix()
    a = c.gpu(128, 256, prefix=pre)
    b = c.gpu(128, 256, prefix=pre, store_ds=True)
    for k in ("o", "lse", "dkr", "dvr", "dk_pages", "dv_pages"):
        assert torch.equal(a[k][torch.isfinite(a[k])], b[k][torch.isfinite(a[k])]), k
    assert_close("dQ", np32(b["dq"]), np32(a["dq"]).astype(np.float64), atol=2e-3, rel_l2=1e-4)


def test_stored_ds_keys_never_read_and_deterministic():
    """NaN in unseen response keys and in the unused rows of the partial last page changes
    nothing on the stored-dS path either, and two runs agree bit for bit."""
    log("case: stored dS, NaN poisoning P=650 R=256 rows [64, 128)")
    c = Case(650, 256, 6, 2, 256, torch.bfloat16, seed=30, S=2)
    clean = c.gpu(64, 64, store_ds=True)
    again = c.gpu(64, 64, store_ds=True)
    for k in ("o", "lse", "dq", "dkr", "dvr", "dk_pages", "dv_pages"):
        fin = torch.isfinite(clean[k])
        assert torch.equal(clean[k][fin], again[k][fin]), k
    kr = c.kr.clone()
    vr = c.vr.clone()
    kr[128:] = float("nan")
    vr[128:] = float("nan")
    pre = c.prefix(pool_fill=float("nan"))
    dirty = c.gpu(64, 64, prefix=pre, kr=kr, vr=vr, store_ds=True)
    for k in ("o", "lse", "dq"):
        assert torch.equal(clean[k], dirty[k]), k
    assert torch.equal(clean["dkr"][:128], dirty["dkr"][:128])
    assert np.array_equal(c.logical(clean["dk_pages"]), c.logical(dirty["dk_pages"]))


@pytest.mark.parametrize("bounds", [[0, 8, 16, 24], [0, 5, 5, 13, 24]])
def test_stored_ds_in_chunks_is_bitwise_the_same(bounds):
    """A workspace with room for the dS of 1, 2 or 3 of the 4 kv heads runs the stored-dS
    backward a chunk of kv heads at a time, and one with room for less than one kv head's dS
    over all keys runs one kv head by k consecutive key parts at a time (a page pair cut by a
    chunk's odd page bound is walked by both chunks, each writing its own page); kv heads and key
    parts are independent, so every output is the same bit for bit as with room for all of them.
    The workspace starts as NaN, so a slot read but never written would show."""
    log(f"case: stored dS in chunks P=1500 R=256 hq=24 hkv=4 d=256 shards {bounds} rows [64, 256)")
    c = Case(1500, 256, 24, 4, 256, torch.bfloat16, seed=31, bounds=bounds)
    pre = c.prefix()
    dev = "cuda"
    q0, n = 64, 192
    q, do = c.q[q0:q0 + n].to(dev).contiguous(), c.do[q0:q0 + n].to(dev).contiguous()
    kr, vr = c.kr.to(dev), c.vr.to(dev)
    o, lse, _ = api.replay_fwd(pre, q, q0, kr, vr)

    def run(heads, parts):
        nbytes = api.bwd_ds_workspace_bytes(pre, n, q0 + n, heads=heads, parts=parts)
        ws = torch.full(((nbytes + 3) // 4,), float("nan"), dtype=torch.float32, device=dev)
        dk_r = torch.empty(kr.shape, dtype=torch.float32, device=dev)
        dv_r = torch.empty_like(dk_r)
        dk_p = torch.empty(pre.k_pages.shape, dtype=torch.float32, device=dev)
        dv_p = torch.empty_like(dk_p)
        dq = api.replay_bwd(pre, q, q0, kr, vr, o, lse, do, dk_r, dv_r, True, dk_p, dv_p,
                            shard_first_touch=[True] * pre.n_shards, workspace=ws)
        torch.cuda.synchronize()
        return dq, dk_r[:q0 + n], dv_r[:q0 + n], dk_p, dv_p

    full = run(None, None)
    ref = c.oracle(q0, n, o_used=c.stored(c.oracle(q0, n)["o"]))
    assert_close("dQ", np32(full[0]), ref["dq"])
    assert_close("dK_prompt", c.logical(full[3]), ref["dkp"])
    n_all = pre.n_shards + 1
    sizes = [api.bwd_ds_workspace_bytes(pre, n, q0 + n, heads=1, parts=k) for k in range(1, n_all + 1)]
    # (not monotonic in k with uneven shards: chunks are cut greedily from the first part)
    assert max(sizes[:-1]) < api.bwd_ds_workspace_bytes(pre, n, q0 + n)
    plans = [(h, n_all) for h in (1, 2, 3)] + [(1, k) for k in range(1, n_all)]
    for heads, parts in plans:
        got = run(heads, parts)
        for name, a, b in zip(("dq", "dk_r", "dv_r", "dk_p", "dv_p"), full, got):
            assert torch.equal(a, b), (heads, parts, name)


@pytest.mark.parametrize("store_ds", [False, True])
def test_small_block_over_a_long_prompt_splits_its_shards(store_ds):
    """A 16-row block over a 65,536-token prompt in two uneven shards (3 and 1,021 pages): the
    forward's and the stored-dS dQ pass's grids would hold only a few workgroups, so both split
    every shard into 8 page ranges (the 3-page shard into mostly empty ones) and combine them.
    Every output and each shard's partial (O, LSE) match the oracle."""
    c = Case(65536, 64, 6, 2, 256, seed=31, bounds=[0, 3, 1024])
    log(f"case: 16-row block over P=65536 in shards {c.bounds}, {'stored dS' if store_ds else 'recompute'}")
    check_against_oracle(c, 24, 16, store_ds=store_ds)
