"""Pins for the CPU oracle: each checks it against something other than itself.

* brute force: materialized masked softmax with pure-Python loops on tiny inputs;
* a library routine: float64 torch autograd of the explicit masked-softmax formula, and
  torch's causal scaled_dot_product_attention for the prompt-free special case;
* central finite differences of the oracle's own forward for every gradient;
* the merge identity (local results composed by LSE equal the unsharded result);
* the closed form at K = 0 (uniform weights);
* hand-derived worked examples under tests/golden/.

A plausible mistake (a dropped mask term, a wrong GQA head, a transposed operand, a
sign or scale error, a missing delta) fails at least one of these; test_pins_catch_planted
plants some of them in a copy of the oracle and checks that they are caught.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _case(seed, P, Rk, n, q_start, hq, hkv, d):
    rng = np.random.default_rng(seed)
    return dict(
        q=_rand(rng, n, hq, d), kp=_rand(rng, P, hkv, d), vp=_rand(rng, P, hkv, d),
        kr=_rand(rng, Rk, hkv, d), vr=_rand(rng, Rk, hkv, d), do=_rand(rng, n, hq, d),
        q_start=q_start)


# ---------------------------------------------------------------------------------------
# brute force (pure Python)
# ---------------------------------------------------------------------------------------

def _brute_forward(c, scale=None):
    q, kp, vp, kr, vr, q_start = c["q"], c["kp"], c["vp"], c["kr"], c["vr"], c["q_start"]
    n, hq, d = q.shape
    hkv = kp.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    O = np.zeros((n, hq, d))
    L = np.zeros((n, hq))
    for i in range(n):
        for h in range(hq):
            kv = h // (hq // hkv)
            keys = [kp[j, kv] for j in range(kp.shape[0])] + [kr[j, kv] for j in range(q_start + i + 1)]
            vals = [vp[j, kv] for j in range(vp.shape[0])] + [vr[j, kv] for j in range(q_start + i + 1)]
            s = [scale * sum(float(q[i, h, t]) * float(k[t]) for t in range(d)) for k in keys]
            z = sum(math.exp(x) for x in s)
            L[i, h] = math.log(z)
            for k, x in enumerate(s):
                O[i, h] += (math.exp(x) / z) * vals[k]
    return O, L


@pytest.mark.parametrize("P,Rk,n,q_start,hq,hkv,d", [
    (7, 5, 3, 2, 4, 2, 3),     # GQA 2, rows mid-response
    (0, 4, 4, 0, 2, 1, 2),     # no prompt: pure causal
    (5, 9, 2, 6, 3, 3, 4),     # MHA, response keys past the block exist but are unseen
    (65, 3, 3, 0, 2, 1, 5),    # prompt longer than one 64-token page
])
def test_forward_bruteforce(P, Rk, n, q_start, hq, hkv, d):
    c = _case(11 + P, P, Rk, n, q_start, hq, hkv, d)
    O, L = orc.forward(c["q"], c["kp"], c["vp"], c["kr"], c["vr"], q_start)
    Ob, Lb = _brute_forward(c)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)


def test_forward_custom_scale_bruteforce():
    c = _case(3, 6, 4, 2, 1, 2, 1, 3)
    O, L = orc.forward(c["q"], c["kp"], c["vp"], c["kr"], c["vr"], 1, scale=0.37)
    Ob, Lb = _brute_forward(c, scale=0.37)
    np.testing.assert_allclose(L, Lb, atol=1e-12)
    np.testing.assert_allclose(O, Ob, atol=1e-12)


# ---------------------------------------------------------------------------------------
# library routines (torch float64)
# ---------------------------------------------------------------------------------------

def _torch_reference(c):
    """Explicit formula in torch float64 over the concatenated keys with a boolean mask."""
    q = torch.tensor(c["q"], requires_grad=True)
    kp = torch.tensor(c["kp"], requires_grad=True)
    vp = torch.tensor(c["vp"], requires_grad=True)
    kr = torch.tensor(c["kr"], requires_grad=True)
    vr = torch.tensor(c["vr"], requires_grad=True)
    n, hq, d = q.shape
    hkv = kp.shape[1]
    g = hq // hkv
    P, Rk = kp.shape[0], kr.shape[0]
    kc = torch.cat([kp, kr], 0).repeat_interleave(g, dim=1)  # [P+Rk, hq, d]
    vc = torch.cat([vp, vr], 0).repeat_interleave(g, dim=1)
    s = torch.einsum("ihd,jhd->hij", q, kc) / math.sqrt(d)
    jj = torch.arange(P + Rk)[None, :]
    ii = torch.arange(n)[:, None]
    visible = (jj < P) | ((jj - P) <= (c["q_start"] + ii))
    s = s.masked_fill(~visible[None], float("-inf"))
    lse = torch.logsumexp(s, dim=-1)  # [h, i]
    o = torch.einsum("hij,jhd->ihd", torch.softmax(s, dim=-1), vc)
    loss = (o * torch.tensor(c["do"])).sum()
    loss.backward()
    return dict(o=o.detach().numpy(), lse=lse.T.detach().numpy(), dq=q.grad.numpy(),
                dkp=kp.grad.numpy(), dvp=vp.grad.numpy(), dkr=kr.grad.numpy(), dvr=vr.grad.numpy())


@pytest.mark.parametrize("P,Rk,n,q_start,hq,hkv,d", [
    (37, 20, 8, 5, 6, 2, 8),
    (130, 16, 16, 0, 4, 1, 16),
    (0, 12, 12, 0, 2, 2, 4),
])
def test_against_torch_autograd(P, Rk, n, q_start, hq, hkv, d):
    c = _case(100 + P + n, P, Rk, n, q_start, hq, hkv, d)
    ref = _torch_reference(c)
    O, L = orc.forward(c["q"], c["kp"], c["vp"], c["kr"], c["vr"], q_start)
    g = orc.backward(c["q"], c["kp"], c["vp"], c["kr"], c["vr"], c["do"], q_start)
    np.testing.assert_allclose(O, ref["o"], atol=1e-12)
    np.testing.assert_allclose(L, ref["lse"], atol=1e-12)
    for k in ("dq", "dkp", "dvp", "dkr", "dvr"):
        np.testing.assert_allclose(g[k], ref[k], atol=1e-11, err_msg=k)


def test_promptless_matches_torch_causal_sdpa():
    """With no prompt and the block at the response start the op is causal attention."""
    c = _case(5, 0, 24, 24, 0, 4, 2, 8)
    O, L = orc.forward(c["q"], c["kp"], c["vp"], c["kr"], c["vr"], 0)
    q = torch.tensor(c["q"]).transpose(0, 1)                       # [h, n, d]
    k = torch.tensor(c["kr"]).repeat_interleave(2, dim=1).transpose(0, 1)
    v = torch.tensor(c["vr"]).repeat_interleave(2, dim=1).transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    np.testing.assert_allclose(O, ref.transpose(0, 1).numpy(), atol=1e-12)


def test_single_visible_key():
    """One visible key: O is that key's value and LSE its score."""
    c = _case(9, 0, 3, 1, 0, 2, 1, 5)
    O, L = orc.forward(c["q"], c["kp"], c["vp"], c["kr"], c["vr"], 0)
    s = (c["q"][0] @ c["kr"][0, 0]) / math.sqrt(5)
    np.testing.assert_allclose(L[0], s, atol=1e-13)
    np.testing.assert_allclose(O[0], np.broadcast_to(c["vr"][0, 0], (2, 5)), atol=1e-13)


# ---------------------------------------------------------------------------------------
# finite differences
# ---------------------------------------------------------------------------------------

def test_backward_finite_differences():
    c = _case(21, 9, 7, 4, 3, 4, 2, 3)
    args = ("q", "kp", "vp", "kr", "vr")
    g = orc.backward(c["q"], c["kp"], c["vp"], c["kr"], c["vr"], c["do"], c["q_start"])
    names = dict(q="dq", kp="dkp", vp="dvp", kr="dkr", vr="dvr")
    rng = np.random.default_rng(0)
    h = 1e-6

    def loss(cc):
        O, _ = orc.forward(cc["q"], cc["kp"], cc["vp"], cc["kr"], cc["vr"], cc["q_start"])
        return float((O * cc["do"]).sum())

    for a in args:
        arr = c[a]
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            cp = dict(c)
            plus = arr.copy(); plus[idx] += h
            minus = arr.copy(); minus[idx] -= h
            cp[a] = plus
            lp = loss(cp)
            cp[a] = minus
            lm = loss(cp)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[names[a]][idx]) < 1e-7, (a, idx, fd, g[names[a]][idx])
    # response keys the block never sees get exactly zero gradient
    kend = c["q_start"] + c["q"].shape[0]
    assert np.all(g["dkr"][kend:] == 0) and np.all(g["dvr"][kend:] == 0)


# ---------------------------------------------------------------------------------------
# merge identity
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("bounds", [
    [(0, 64), (64, 192)],                 # two shards
    [(0, 0), (0, 130), (130, 192)],       # an empty shard
    [(0, 64), (64, 128), (128, 192)],     # one page each
    [(0, 192)],                           # one shard
])
def test_merge_identity(bounds):
    c = _case(31, 192, 20, 6, 10, 4, 2, 8)
    O, L = orc.forward(c["q"], c["kp"], c["vp"], c["kr"], c["vr"], c["q_start"])
    Op, Lp = orc.forward_parts(c["q"], c["kp"], c["vp"], c["kr"], c["vr"], bounds, c["q_start"])
    assert Op.shape[0] == len(bounds) + 1
    for p, (a, b) in enumerate(bounds):
        if a == b:
            assert np.all(np.isneginf(Lp[p])) and np.all(Op[p] == 0)
    Om, Lm = orc.lse_merge(Op, Lp)
    np.testing.assert_allclose(Lm, L, atol=1e-12)
    np.testing.assert_allclose(Om, O, atol=1e-12)


def test_merge_single_part_is_identity():
    rng = np.random.default_rng(2)
    Op = rng.standard_normal((1, 5, 3, 4))
    Lp = rng.standard_normal((1, 5, 3))
    Om, Lm = orc.lse_merge(Op, Lp)
    assert np.array_equal(Lm, Lp[0]) and np.array_equal(Om, Op[0])


def test_shard_token_bounds():
    assert orc.shard_token_bounds(64, 2, 64, 4096) == [(0, 2048), (2048, 4096)]
    assert orc.shard_token_bounds(5, 3, 64, 300) == [(0, 64), (64, 192), (192, 300)]
    assert orc.shard_token_bounds(2, 4, 64, 128) == [(0, 0), (0, 64), (64, 64), (64, 128)]


# ---------------------------------------------------------------------------------------
# closed form at K = 0
# ---------------------------------------------------------------------------------------

def closed_form_k0(q, vp, vr, do, q_start, scale):
    """All keys zero: every visible key has weight 1/N_i, N_i = P + q_start + i + 1."""
    n, hq, d = q.shape
    P, hkv = vp.shape[0], vp.shape[1]
    g = hq // hkv
    Rk = vr.shape[0]
    N = P + q_start + np.arange(n) + 1
    o = np.zeros((n, hq, d))
    for i in range(n):
        for h in range(hq):
            kv = h // g
            o[i, h] = (vp[:, kv].sum(0) + vr[:q_start + i + 1, kv].sum(0)) / N[i]
    lse = np.broadcast_to(np.log(N)[:, None], (n, hq)).copy()
    dlt = (o * do).sum(-1)
    dkp = np.zeros((P, hkv, d)); dvp = np.zeros((P, hkv, d))
    dkr = np.zeros((Rk, hkv, d)); dvr = np.zeros((Rk, hkv, d))
    for kv in range(hkv):
        hs = range(kv * g, (kv + 1) * g)
        # prompt keys are seen by every row
        A = sum(np.outer(q[i, h], do[i, h]) / N[i] for i in range(n) for h in hs)
        b = sum(dlt[i, h] * q[i, h] / N[i] for i in range(n) for h in hs)
        c_ = sum(do[i, h] / N[i] for i in range(n) for h in hs)
        dkp[:, kv] = scale * (vp[:, kv] @ A.T - b)
        dvp[:, kv] = c_
        for j in range(Rk):
            rows = [i for i in range(n) if q_start + i >= j]
            if not rows:
                continue
            A = sum(np.outer(q[i, h], do[i, h]) / N[i] for i in rows for h in hs)
            b = sum(dlt[i, h] * q[i, h] / N[i] for i in rows for h in hs)
            dkr[j, kv] = scale * (A @ vr[j, kv] - b)
            dvr[j, kv] = sum(do[i, h] / N[i] for i in rows for h in hs)
    return dict(o=o, lse=lse, dq=np.zeros_like(q), dkp=dkp, dvp=dvp, dkr=dkr, dvr=dvr)


def test_closed_form_zero_keys():
    c = _case(41, 70, 12, 5, 4, 6, 2, 4)
    c["kp"][:] = 0
    c["kr"][:] = 0
    cf = closed_form_k0(c["q"], c["vp"], c["vr"], c["do"], c["q_start"], 0.5)
    O, L = orc.forward(c["q"], c["kp"], c["vp"], c["kr"], c["vr"], c["q_start"])
    g = orc.backward(c["q"], c["kp"], c["vp"], c["kr"], c["vr"], c["do"], c["q_start"])
    np.testing.assert_allclose(L, cf["lse"], atol=1e-13)
    np.testing.assert_allclose(O, cf["o"], atol=1e-13)
    for k in ("dq", "dkp", "dvp", "dkr", "dvr"):
        np.testing.assert_allclose(g[k], cf[k], atol=1e-12, err_msg=k)


# ---------------------------------------------------------------------------------------
# golden fixtures (hand-derived)
# ---------------------------------------------------------------------------------------

def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = np.array([float(x) for x in v.split()])
    return vals


def test_golden_two_key_example():
    gd = _read_golden("two_key_attention.txt")
    t = lambda k: gd[k].reshape(1, 1, -1)  # noqa: E731
    O, L = orc.forward(t("q"), t("kp"), t("vp"), t("kr"), t("vr"), 0)
    np.testing.assert_allclose(O[0, 0], gd["o"], atol=1e-12)
    np.testing.assert_allclose(L[0, 0], gd["lse"][0], atol=1e-12)
    g = orc.backward(t("q"), t("kp"), t("vp"), t("kr"), t("vr"), t("do"), 0)
    for k in ("dq", "dkp", "dvp", "dkr", "dvr"):
        np.testing.assert_allclose(g[k][0, 0], gd[k], atol=1e-12, err_msg=k)


def test_golden_merge_example():
    gd = _read_golden("lse_merge_example.txt")
    Op = np.stack([gd["o_part0"], gd["o_part1"], gd["o_part2"]])[:, None, :]
    Lp = gd["lse_parts"][:, None]
    O, L = orc.lse_merge(Op, Lp)
    np.testing.assert_allclose(L[0], gd["lse"][0], atol=1e-12)
    np.testing.assert_allclose(O[0], gd["o"], atol=1e-12)


# ---------------------------------------------------------------------------------------
# pages
# ---------------------------------------------------------------------------------------

def test_capture_gather_roundtrip():
    rng = np.random.default_rng(7)
    T, H, d, ps = 200, 2, 3, 64          # 4 pages, last one partial
    x = rng.standard_normal((T, H, d)).astype(np.float32)
    table = np.array([5, 0, 3, 1], dtype=np.int32)
    pool = orc.capture_pages(x, table, ps, 6)
    assert np.array_equal(orc.gather_pages(pool, table, T), x)
    # page 3 (logical) lives at physical 1, rows 8.. are padding and stay zero
    assert np.array_equal(pool[1, :, : T - 192, :], x[192:].transpose(1, 0, 2))
    assert np.all(pool[1, :, T - 192:, :] == 0)
    # untouched physical pages stay zero
    assert np.all(pool[[2, 4]] == 0)


# ---------------------------------------------------------------------------------------
# planted mistakes are caught (mutations of a copy of the oracle, on the CPU)
# ---------------------------------------------------------------------------------------

def test_pins_catch_planted(monkeypatch):
    c = _case(5, 9, 6, 3, 2, 4, 2, 3)
    Ob, Lb = _brute_forward(c)

    def fwd():
        return orc.forward(c["q"], c["kp"], c["vp"], c["kr"], c["vr"], c["q_start"])

    # 1) causal mask off by one
    orig_mask = orc._resp_mask
    monkeypatch.setattr(orc, "_resp_mask", lambda n, g, qs, a, b: orig_mask(n, g, qs + 1, a, b))
    O, _ = fwd()
    assert not np.allclose(O, Ob, atol=1e-9)
    monkeypatch.setattr(orc, "_resp_mask", orig_mask)
    # 2) wrong GQA grouping (heads interleaved instead of contiguous)
    orig_group = orc._group_rows
    monkeypatch.setattr(orc, "_group_rows", lambda q, kv, g: orig_group(q[:, ::-1, :], kv, g))
    O, _ = fwd()
    assert not np.allclose(O, Ob, atol=1e-9)
    monkeypatch.setattr(orc, "_group_rows", orig_group)
    O, L = fwd()
    assert np.allclose(O, Ob, atol=1e-12) and np.allclose(L, Lb, atol=1e-12)


def test_round_bf16_matches_torch_rne_and_is_idempotent():
    """round_bf16 against torch's CPU float32 -> bfloat16 conversion (round to nearest even)
    on float32-representable values, including exact ties, signs, zeros and powers of two."""
    import torch
    rng = np.random.default_rng(11)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(10.0) ** rng.integers(-6, 6, 200_000)
    # exact ties: bf16 values plus half an ulp (bit 15 set, lower bits clear)
    ties = (rng.integers(0, 1 << 16, 5000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32)
    exp_field = ties & 0x7F800000
    ties = ties[(exp_field != 0x7F800000) & (exp_field != 0)].view(np.float32)  # normal numbers
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1.0, -2.0, 0.5, 3.0], np.float32)])
    got = orc.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(orc.round_bf16(got), got)


# ---------------------------------------------------------------------------------------
# The pages' BF16-numerator merge variant
# ---------------------------------------------------------------------------------------

def test_bf16_numerator_merge_single_part_rounds_once():
    """One non-empty part: weight 1, denominator 1, so the result is that part rounded to bf16."""
    rng = np.random.default_rng(5)
    Op = rng.standard_normal((3, 4, 8))
    Lp = np.full((3, 4), -np.inf)
    Lp[1] = rng.standard_normal(4)
    O, L = orc.lse_merge_bf16_numerator(Op, Lp)
    assert np.array_equal(O, orc.round_bf16(Op[1]))
    assert np.allclose(L, Lp[1], rtol=0, atol=1e-15)


def test_bf16_numerator_merge_rounds_the_running_sum():
    """Two parts of equal LSE (weights 1, denominator 2): a sum that bf16 holds exactly is
    exact, and a term below half a bf16 step of the running sum is lost -- which a float64 or
    float32 accumulation of the same bf16 terms would keep."""
    Lp = np.zeros((2, 1))
    O, _ = orc.lse_merge_bf16_numerator(np.array([[[1.5]], [[0.25]]]), Lp)
    assert O[0, 0] == 0.875
    O, _ = orc.lse_merge_bf16_numerator(np.array([[[1.0]], [[2.0 ** -9]]]), Lp)
    assert O[0, 0] == 0.5  # exact merge: (1 + 2^-9) / 2
    O, _ = orc.lse_merge(np.array([[[1.0]], [[2.0 ** -9]]]), Lp)
    assert O[0, 0] == (1 + 2.0 ** -9) / 2


def test_bf16_numerator_merge_error_is_bounded():
    """Against the exact merge the error is at most one bf16 rounding per term and per
    addition: |dO| <= sum_p (2 p + 1) 2^-9 max|partial sum| / denominator (a loose bound), and
    empty rows stay O = 0, L = -inf."""
    rng = np.random.default_rng(6)
    n_parts, rows, d = 9, 50, 16
    Op = rng.standard_normal((n_parts, rows, d))
    Lp = rng.standard_normal((n_parts, rows)) * 3
    Lp[2, :10] = -np.inf
    Lp[:, -1] = -np.inf
    O, L = orc.lse_merge_bf16_numerator(Op, Lp)
    Oe, Le = orc.lse_merge(Op, Lp)
    assert np.all(O[-1] == 0) and np.isneginf(L[-1])
    m = np.max(Lp[:, :-1], axis=0)
    w = np.exp(Lp[:, :-1] - m)
    den = w.sum(axis=0)
    scale = (np.abs(w[..., None] * Op[:, :-1]).sum(axis=0)) / den[:, None]
    bound = sum(2 * p + 1 for p in range(n_parts)) * 2.0 ** -9 * scale
    assert np.all(np.abs(O[:-1] - Oe[:-1]) <= bound)
    assert np.max(np.abs(O[:-1] - Oe[:-1])) > 0  # the variant does lose precision
    assert np.array_equal(np.isneginf(L), np.isneginf(Le))
    fin = np.isfinite(L)
    np.testing.assert_allclose(L[fin], Le[fin], rtol=0, atol=1e-12)
