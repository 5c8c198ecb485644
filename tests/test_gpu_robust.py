"""Debug checks and robustness of the backward on the GPU.

* One writer per gradient element.  Every member's K/V gradients accumulate into the same pages
  (LongStraw digest, "Method", step 3) with no atomics, which is correct only if each gradient
  element has one writer per call.  With the library's one-writer counters registered, a
  backward over a block must count exactly 1 for every prompt and response gradient half-page
  and every dQ part row it writes, and 0 for the pool pages no logical page maps to; the
  expected counts are built here from the slot layout the header documents.  Recompute, stored
  dS over all keys, and stored dS in chunks of one kv head by two key parts (whose chunk edges
  cut page pairs, the case the ownership rule is subtle in) are each checked, and counting must
  not change any result.
* NaN in one query row (one head of one token) stays in that row: the call returns normally,
  every other row's O, LSE and dQ are bit for bit those of a clean run, the other kv head's key
  gradients are unchanged, and the row's own outputs and the gradients of every key the row
  sees are NaN.  (Gradients of keys the row does not see are left unspecified: IEEE products
  of a zero weight with the row's NaN are NaN.)
"""
import pytest
import torch

from _cases import Case, log
from suffix_attention_amd import api

pytestmark = pytest.mark.gpu

# 2,000 prompt tokens over 3 uneven shards behind a permuted table with 3 spare pool pages; a
# block of 172 rows at q_start 128 (response keys end at 300, a partial last response page).
P, R, HQ, HKV, D = 2000, 300, 24, 4, 256
BOUNDS = [0, 5, 19, 32]
Q_START, N_ROWS = 128, 172


def _expected_counts(table, n_phys, n_rows, key_end):
    n_parts = len(BOUNDS)
    r0 = n_phys * HKV * 2
    q0 = r0 + (key_end + 63) // 64 * HKV * 2
    exp = torch.zeros(q0 + n_parts * n_rows * HQ, dtype=torch.int32)
    for phys in table.tolist():
        exp[phys * HKV * 2:(phys + 1) * HKV * 2] = 1
    exp[r0:] = 1
    return exp


PLANS = {"recompute": None, "stored dS": (HKV, len(BOUNDS)), "stored dS, 1 kv head x 2 key parts": (1, 2)}


@pytest.mark.parametrize("plan", list(PLANS))
def test_backward_has_one_writer_per_gradient_element(plan):
    log(f"case: one-writer counters, P={P} S=3 {BOUNDS} rows [{Q_START}, {Q_START + N_ROWS}) ({plan})")
    c = Case(P, R, HQ, HKV, D, seed=11, bounds=list(BOUNDS), n_phys_extra=3)
    pre = c.prefix()
    dev = "cuda"
    key_end = Q_START + N_ROWS
    q = c.q[Q_START:key_end].to(dev).contiguous()
    do = c.do[Q_START:key_end].to(dev).contiguous()
    kr, vr = c.kr.to(dev), c.vr.to(dev)
    o, lse, _ = api.replay_fwd(pre, q, Q_START, kr, vr)
    ws = None
    if PLANS[plan] is not None:
        heads, parts = PLANS[plan]
        nbytes = api.bwd_ds_workspace_bytes(pre, N_ROWS, key_end, heads=heads, parts=parts)
        ws = torch.empty(((nbytes + 3) // 4,), dtype=torch.float32, device=dev)

    def run():
        g = [torch.zeros(kr.shape, dtype=torch.float32, device=dev) for _ in range(2)]
        g += [torch.zeros(pre.k_pages.shape, dtype=torch.float32, device=dev) for _ in range(2)]
        dq = api.replay_bwd(pre, q, Q_START, kr, vr, o, lse, do, g[0], g[1], True, g[2], g[3],
                            shard_first_touch=[True] * pre.n_shards, workspace=ws)
        torch.cuda.synchronize()
        return [dq] + g

    oc = api.OwnerCounts(api.owner_slots(pre, N_ROWS, key_end), dev)
    with oc:
        counted = run()
    got = oc.check(plan)
    exp = _expected_counts(c.table, c.n_phys, N_ROWS, key_end)
    assert got.shape == exp.shape
    diff = torch.nonzero(got != exp).flatten()
    assert diff.numel() == 0, f"slot {int(diff[0])}: counted {int(got[diff[0]])}, expected {int(exp[diff[0]])}"
    log(f"    {int(got.sum())} slots written once, none twice")
    for name, a, b in zip(("dQ", "dK_resp", "dV_resp", "dK_pages", "dV_pages"), counted, run()):
        assert torch.equal(a, b), f"{name} changed by counting"


@pytest.mark.parametrize("store_ds", [False, True])
def test_one_writer_per_element_with_split_shards(store_ds):
    """A 16-row block over 65,536 prompt tokens in 2 shards: the stored-dS dQ pass splits each
    shard into page ranges, each forming its own dQ partial, so the counters hold one dQ region
    per range (the header's "dQ partial" slots, sized by ls_debug_owner_slots); each must be
    written once, and the recomputing backward writes only the first n_shards + 1 of them."""
    Pl, hq, hkv, d, bounds = 65536, 6, 2, 256, [0, 300, 1024]
    c = Case(Pl, 64, hq, hkv, d, seed=33, bounds=list(bounds))
    pre = c.prefix()
    dev = "cuda"
    q_start, n = 24, 16
    key_end = q_start + n
    log(f"case: one-writer counters, 16-row block over P={Pl} ({'stored dS' if store_ds else 'recompute'})")
    q = c.q[q_start:key_end].to(dev).contiguous()
    do = c.do[q_start:key_end].to(dev).contiguous()
    kr, vr = c.kr.to(dev), c.vr.to(dev)
    o, lse, _ = api.replay_fwd(pre, q, q_start, kr, vr)
    g = [torch.zeros(kr.shape, dtype=torch.float32, device=dev) for _ in range(2)]
    g += [torch.zeros(pre.k_pages.shape, dtype=torch.float32, device=dev) for _ in range(2)]
    slots = api.owner_slots(pre, n, key_end)
    r0 = c.n_phys * hkv * 2
    q0 = r0 + (key_end + 63) // 64 * hkv * 2
    n_dq = (slots - q0) // (n * hq)
    assert n_dq > len(bounds), "expected the dQ pass to split the shards"
    with api.OwnerCounts(slots, dev) as oc:
        api.replay_bwd(pre, q, q_start, kr, vr, o, lse, do, g[0], g[1], True, g[2], g[3],
                       shard_first_touch=[True] * pre.n_shards, store_ds=store_ds)
        torch.cuda.synchronize()
    got = oc.check()
    exp = torch.zeros(slots, dtype=torch.int32)
    for phys in c.table.tolist():
        exp[phys * hkv * 2:(phys + 1) * hkv * 2] = 1
    exp[r0:q0] = 1
    exp[q0:q0 + (n_dq if store_ds else len(bounds)) * n * hq] = 1
    diff = torch.nonzero(got != exp).flatten()
    assert diff.numel() == 0, f"slot {int(diff[0])}: counted {int(got[diff[0]])}, expected {int(exp[diff[0]])}"
    log(f"    {n_dq} dQ partial regions, {int(got.sum())} slots written once")


@pytest.mark.parametrize("store_ds", [False, True])
def test_nan_in_one_query_row_stays_in_its_row(store_ds):
    c = Case(700, 160, 6, 2, 128, seed=5, S=3)  # g = 3: heads 0-2 on kv head 0
    pre = c.prefix()
    dev = "cuda"
    q_start, n, r, head = 32, 96, 40, 1  # the NaN row is token 72, head 1 (kv head 0)
    log(f"case: NaN in q[token {q_start + r}, head {head}], P=700 rows [{q_start}, {q_start + n}), "
        f"{'stored dS' if store_ds else 'recompute'}")
    do = c.do[q_start:q_start + n].to(dev).contiguous()
    kr, vr = c.kr.to(dev), c.vr.to(dev)

    def run(q):
        o, lse, _ = api.replay_fwd(pre, q, q_start, kr, vr)
        g = [torch.zeros(kr.shape, dtype=torch.float32, device=dev) for _ in range(2)]
        g += [torch.zeros(pre.k_pages.shape, dtype=torch.float32, device=dev) for _ in range(2)]
        dq = api.replay_bwd(pre, q, q_start, kr, vr, o, lse, do, g[0], g[1], True, g[2], g[3],
                            shard_first_touch=[True] * pre.n_shards, store_ds=store_ds)
        torch.cuda.synchronize()
        return dict(o=o, lse=lse, dq=dq, dkr=g[0], dvr=g[1], dkp=g[2], dvp=g[3])

    q = c.q[q_start:q_start + n].to(dev).contiguous()
    clean = run(q)
    qn = q.clone()
    qn[r, head] = float("nan")
    bad = run(qn)
    row = torch.zeros((n, c.hq), dtype=torch.bool, device=dev)
    row[r, head] = True
    for k in ("o", "lse", "dq"):
        assert torch.isnan(bad[k][r, head]).all(), k
        assert torch.equal(bad[k][~row], clean[k][~row]), f"{k} of another row changed"
    for k in ("dkr", "dvr", "dkp", "dvp"):
        assert torch.equal(bad[k][:, 1], clean[k][:, 1]), f"{k} of the other kv head changed"
    seen = q_start + r + 1  # response keys the row sees
    for k in ("dkr", "dvr"):
        assert torch.isnan(bad[k][:seen, 0]).all(), k
    for k in ("dkp", "dvp"):
        logical = torch.from_numpy(c.logical(bad[k]))  # [P, hkv, d]: every prompt key is seen
        assert torch.isnan(logical[:, 0]).all(), k
    log("    the row's outputs and its seen keys' gradients are NaN; everything else is unchanged")
