"""Plain float64 CPU oracle for replay attention over a captured, paged prompt KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code with the HIP library and imports nothing from the product package.

What it computes (LongStraw, "LongStraw: Long-Context RL Beyond 2M Tokens under a Fixed
GPU Budget", paper digest, section "Method"; explainer page, section "Two incompatible
architectures, same transaction"):

* The prompt of P tokens is evaluated once without autograd and its attention keys and
  values are kept as pages (digest, "Method", step 1: the retained conditional state
  includes CP-sharded KV pages).  :func:`capture_pages` / :func:`gather_pages` state
  what a page table means: logical token t of a prompt lives in row t % page_size of
  physical page table[t // page_size].
* A response of R tokens is replayed under autograd with exact attention over the whole
  prompt plus the response itself, causally (explainer, "Serial replay makes G a
  schedule": an exact-attention response-only step).  Response row i sits at absolute
  position P + i and sees prompt keys 0..P-1 and response keys 0..i inclusive.
  :func:`forward` and :func:`backward` are that attention and its gradient, written out
  from the definition of softmax attention with no paging, sharding or online softmax.
* The prompt keys are split across context-parallel owners whose local softmax
  statistics are composed into the exact global output (digest, "Method", Qwen
  implementation: a global LSE/output merge; explainer, "Two incompatible
  architectures").  :func:`forward_parts` computes each owner's local result and
  :func:`lse_merge` is the composition, in float64 here (the pages' own merge keeps a
  BF16 numerator, explainer "The fine print"; the numerator here is exact).
* Group members are replayed one after another and their gradients accumulate
  (digest, "Method", step 3).  Accumulation across members is a plain sum done by the
  caller; nothing member-specific lives here.

Readings where the pages are silent (each also listed in the design notes):
  - GQA head mapping: query head h uses kv head h // (Hq // Hkv).
  - Score scale: s = scale * q.k with scale = 1/sqrt(d) unless given; LSE is the natural
    log of sum_j exp(s_j).
  - The response's own keys form one extra part after the prompt shards.
  - A part with no visible key has LSE = -inf and O = 0.
  - The upstream gradient dO is an input; the implied loss is sum(O * dO); LSE is not a
    differentiable output.

Arrays: q, do [n, Hq, d]; prompt keys/values kp, vp [P, Hkv, d] in logical order;
response keys/values kr, vr [Rk, Hkv, d].  Rows of q are response positions
q_start .. q_start + n - 1.  Any float dtype is accepted; all arithmetic is float64.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


def _f64(x):
    return np.asarray(x, dtype=F64)


# ---------------------------------------------------------------------------------------
# Page table (digest "Method" step 1: KV pages as the captured state)
# ---------------------------------------------------------------------------------------

def capture_pages(x, table, page_size, n_phys):
    """Scatter logical tokens x [T, H, d] into a page pool [n_phys, H, page_size, d].

    Logical token t goes to row t % page_size of physical page table[t // page_size];
    rows past T in the last page stay zero.  The result keeps x's dtype (a bit copy).
    """
    x = np.asarray(x)
    T, H, d = x.shape
    pool = np.zeros((n_phys, H, page_size, d), dtype=x.dtype)
    for t in range(T):
        pool[table[t // page_size], :, t % page_size, :] = x[t]
    return pool


def gather_pages(pool, table, n_tok):
    """Read logical tokens [0, n_tok) back out of a pool: the inverse of capture_pages."""
    pool = np.asarray(pool)
    page_size = pool.shape[2]
    out = np.empty((n_tok, pool.shape[1], pool.shape[3]), dtype=pool.dtype)
    for t in range(n_tok):
        out[t] = pool[table[t // page_size], :, t % page_size, :]
    return out


# ---------------------------------------------------------------------------------------
# Key sets and scores
# ---------------------------------------------------------------------------------------

def _key_chunks(n_keys, chunk):
    for a in range(0, n_keys, chunk):
        yield a, min(n_keys, a + chunk)


def _chunk_len(n_rows):
    # Keep one float64 score chunk near 64 MB and one float64 key chunk at most 64K rows;
    # a pure memory bound, with no effect on values beyond summation order.
    return min(1 << 16, max(256, (1 << 23) // max(1, n_rows)))


def _group_rows(q, kv, g):
    """Rows of the kv head's group: [n*g, d], row index i*g + j is (token i, head kv*g+j)."""
    n, _, d = q.shape
    return _f64(q[:, kv * g:(kv + 1) * g, :]).reshape(n * g, d)


def _resp_mask(n, g, q_start, a, b):
    """Boolean [n*g, b-a]: response key a+c is visible to the row (i, j)."""
    rows_i = np.repeat(np.arange(n), g)
    keys = np.arange(a, b)
    return keys[None, :] < (q_start + rows_i + 1)[:, None]


def _scores_prefix(Qg, kp, kv, a, b, scale):
    return scale * (Qg @ _f64(kp[a:b, kv, :]).T)


def _scores_resp(Qg, kr, kv, a, b, scale, n, g, q_start):
    s = scale * (Qg @ _f64(kr[a:b, kv, :]).T)
    s[~_resp_mask(n, g, q_start, a, b)] = -np.inf
    return s


# ---------------------------------------------------------------------------------------
# Forward (definition of softmax attention; explainer "Serial replay ...": exact attention)
# ---------------------------------------------------------------------------------------

def _lse_over(n, g, Qg, kv, scale, kp, kr, q_start, p_range, r_range):
    """Natural-log LSE of each row over prompt keys in p_range and response keys in
    r_range, two passes: exact maximum first, then the shifted sum."""
    rows = n * g
    m = np.full(rows, -np.inf)
    chunk = _chunk_len(rows)
    pa, pb = p_range
    ra, rb = r_range
    for a, b in _key_chunks(pb - pa, chunk):
        m = np.maximum(m, _scores_prefix(Qg, kp, kv, pa + a, pa + b, scale).max(axis=1))
    for a, b in _key_chunks(rb - ra, chunk):
        m = np.maximum(m, _scores_resp(Qg, kr, kv, ra + a, ra + b, scale, n, g, q_start).max(axis=1))
    ssum = np.zeros(rows)
    msafe = np.where(np.isfinite(m), m, 0.0)
    for a, b in _key_chunks(pb - pa, chunk):
        ssum += np.exp(_scores_prefix(Qg, kp, kv, pa + a, pa + b, scale) - msafe[:, None]).sum(axis=1)
    for a, b in _key_chunks(rb - ra, chunk):
        ssum += np.exp(_scores_resp(Qg, kr, kv, ra + a, ra + b, scale, n, g, q_start) - msafe[:, None]).sum(axis=1)
    with np.errstate(divide="ignore"):
        return np.where(ssum > 0, msafe + np.log(ssum), -np.inf)


def _out_over(n, g, Qg, kv, scale, kp, vp, kr, vr, q_start, lse, p_range, r_range):
    """O = sum_j exp(s_j - LSE) v_j over the given key ranges."""
    rows = n * g
    d = vp.shape[2] if vp.shape[0] else vr.shape[2]
    out = np.zeros((rows, d))
    chunk = _chunk_len(rows)
    lsafe = np.where(np.isfinite(lse), lse, 0.0)
    pa, pb = p_range
    ra, rb = r_range
    for a, b in _key_chunks(pb - pa, chunk):
        p = np.exp(_scores_prefix(Qg, kp, kv, pa + a, pa + b, scale) - lsafe[:, None])
        out += p @ _f64(vp[pa + a:pa + b, kv, :])
    for a, b in _key_chunks(rb - ra, chunk):
        p = np.exp(_scores_resp(Qg, kr, kv, ra + a, ra + b, scale, n, g, q_start) - lsafe[:, None])
        out += p @ _f64(vr[ra + a:ra + b, kv, :])
    out[~np.isfinite(lse)] = 0.0
    return out


def _dims(q, kp, kr):
    n, Hq, d = q.shape
    Hkv = kp.shape[1] if kp.ndim == 3 and kp.shape[0] else kr.shape[1]
    assert Hq % Hkv == 0
    return n, Hq, d, Hkv, Hq // Hkv


def _resp_key_end(q_start, n):
    return q_start + n


def forward(q, kp, vp, kr, vr, q_start=0, scale=None):
    """Exact attention of response rows over the whole prompt plus the causal response.

    Returns (O [n, Hq, d] float64, LSE [n, Hq] float64, natural log).
    """
    n, Hq, d, Hkv, g = _dims(q, kp, kr)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    P = kp.shape[0]
    kend = _resp_key_end(q_start, n)
    assert kr.shape[0] >= kend
    O = np.zeros((n, Hq, d))
    L = np.zeros((n, Hq))
    for kv in range(Hkv):
        Qg = _group_rows(q, kv, g)
        lse = _lse_over(n, g, Qg, kv, scale, kp, kr, q_start, (0, P), (0, kend))
        o = _out_over(n, g, Qg, kv, scale, kp, vp, kr, vr, q_start, lse, (0, P), (0, kend))
        O[:, kv * g:(kv + 1) * g, :] = o.reshape(n, g, d)
        L[:, kv * g:(kv + 1) * g] = lse.reshape(n, g)
    return O, L


def shard_token_bounds(n_pages, n_shards, page_size, prefix_len):
    """Contiguous logical page ranges [floor(s*n/S), floor((s+1)*n/S)) as token ranges."""
    out = []
    for s in range(n_shards):
        pa = (s * n_pages) // n_shards
        pb = ((s + 1) * n_pages) // n_shards
        out.append((min(prefix_len, pa * page_size), min(prefix_len, pb * page_size)))
    return out


def forward_parts(q, kp, vp, kr, vr, prefix_token_bounds, q_start=0, scale=None):
    """Each owner's local attention: one part per prompt token range, plus a last part
    over the response keys the rows see.

    Returns (O_parts [n_parts, n, Hq, d], LSE_parts [n_parts, n, Hq]); a part whose key
    set is empty for a row has LSE = -inf and O = 0 there.
    """
    n, Hq, d, Hkv, g = _dims(q, kp, kr)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    kend = _resp_key_end(q_start, n)
    ranges = [((a, b), (0, 0)) for a, b in prefix_token_bounds] + [((0, 0), (0, kend))]
    Op = np.zeros((len(ranges), n, Hq, d))
    Lp = np.zeros((len(ranges), n, Hq))
    for p, (pr, rr) in enumerate(ranges):
        for kv in range(Hkv):
            Qg = _group_rows(q, kv, g)
            lse = _lse_over(n, g, Qg, kv, scale, kp, kr, q_start, pr, rr)
            o = _out_over(n, g, Qg, kv, scale, kp, vp, kr, vr, q_start, lse, pr, rr)
            Op[p, :, kv * g:(kv + 1) * g, :] = o.reshape(n, g, d)
            Lp[p, :, kv * g:(kv + 1) * g] = lse.reshape(n, g)
    return Op, Lp


def lse_merge(o_parts, lse_parts):
    """Compose local softmax results into the global one (digest "Method", Qwen: global
    LSE/output merge).  L = log sum_p exp(L_p); O = sum_p exp(L_p - L) O_p.

    o_parts [n_parts, ..., d], lse_parts [n_parts, ...]; parts with L_p = -inf add
    nothing.  Rows where every part is empty get L = -inf and O = 0.
    """
    Lp = _f64(lse_parts)
    Op = _f64(o_parts)
    m = Lp.max(axis=0)
    msafe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(Lp - msafe[None])  # exp(-inf) = 0 for empty parts
    ssum = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        L = np.where(ssum > 0, msafe + np.log(ssum), -np.inf)
    Lsafe = np.where(np.isfinite(L), L, 0.0)
    wn = np.where(np.isfinite(Lp), np.exp(Lp - Lsafe[None]), 0.0)
    O = (wn[..., None] * Op).sum(axis=0)
    O[~np.isfinite(L)] = 0.0
    return O, L


def lse_merge_bf16_numerator(o_parts, lse_parts):
    """The pages' own merge, whose numerator is BF16 (explainer, "The fine print").  Reading
    (the pages give no more detail): each part's term exp(L_p - m) O_p is rounded to bf16 and
    the running sum over the parts, in part order, is rounded to bf16 after every addition --
    what a bf16 sum over the owners does; m, L and the denominator sum_p exp(L_p - m) are
    exact; O = numerator / denominator.  Empty parts add nothing; empty rows give O = 0 and
    L = -inf as in :func:`lse_merge`.
    """
    Lp = _f64(lse_parts)
    Op = _f64(o_parts)
    m = Lp.max(axis=0)
    msafe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(Lp - msafe[None])  # 0 for empty parts
    den = w.sum(axis=0)
    num = np.zeros(Op.shape[1:])
    for p in range(Op.shape[0]):
        num = round_bf16(num + round_bf16(w[p][..., None] * Op[p]))
    with np.errstate(divide="ignore", invalid="ignore"):
        L = np.where(den > 0, msafe + np.log(den), -np.inf)
        O = np.where((den > 0)[..., None], num / np.where(den > 0, den, 1.0)[..., None], 0.0)
    return O, L


# ---------------------------------------------------------------------------------------
# Output rounding (the replayed block's output is a tensor of the model's dtype, bf16 on the
# pages' runs: digest "Method", Qwen implementation; the backward's delta is formed from that
# stored output)
# ---------------------------------------------------------------------------------------

def round_bf16(x):
    """x rounded to the nearest bfloat16 value (8 significant bits, ties to even), returned
    as float64.  Written from the definition of the format; values below the bf16 normal
    range keep 8 significant bits (none occur in the tests' data)."""
    x = _f64(x)
    m, e = np.frexp(x)                     # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


# ---------------------------------------------------------------------------------------
# Backward (gradient of L = sum(O * dO) w.r.t. q, prompt k/v and response k/v)
# ---------------------------------------------------------------------------------------

def delta(o, do):
    """delta[i, h] = sum_d dO[i, h, :] * O[i, h, :]."""
    return (_f64(o) * _f64(do)).sum(axis=-1)


def backward(q, kp, vp, kr, vr, do, q_start=0, scale=None, o=None, lse=None,
             prefix_grad_sink=None):
    """Gradients of L = sum(O * dO) for the attention of :func:`forward`.

    With p = exp(s - LSE), dP = dO . v, delta = rowsum(dO * O), dS = p (dP - delta):
      dQ = scale sum_j dS_j k_j, dK_j = scale sum_rows dS_j q, dV_j = sum_rows p_j dO.
    o / lse default to this module's forward; a caller may pass the O it actually
    returned (the GPU path rounds O before delta is formed).

    Returns dict(dq [n,Hq,d], dkp/dvp [P,Hkv,d] or None, dkr/dvr [Rk,Hkv,d]).  If
    prefix_grad_sink is given, prompt gradients are handed to it chunk by chunk as
    sink(kv, a, b, dk_chunk, dv_chunk) instead of being stored (bounded host memory).
    """
    n, Hq, d, Hkv, g = _dims(q, kp, kr)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    P = kp.shape[0]
    Rk = kr.shape[0]
    kend = _resp_key_end(q_start, n)
    if o is None or lse is None:
        o_f, lse_f = forward(q, kp, vp, kr, vr, q_start, scale)
        o = o_f if o is None else o
        lse = lse_f if lse is None else lse
    dq = np.zeros((n, Hq, d))
    store_prefix = prefix_grad_sink is None
    dkp = np.zeros((P, Hkv, d)) if store_prefix else None
    dvp = np.zeros((P, Hkv, d)) if store_prefix else None
    dkr = np.zeros((Rk, Hkv, d))
    dvr = np.zeros((Rk, Hkv, d))
    dlt = delta(o, do)
    for kv in range(Hkv):
        Qg = _group_rows(q, kv, g)
        dOg = _group_rows(do, kv, g)
        lse_g = _f64(lse[:, kv * g:(kv + 1) * g]).reshape(n * g)
        dl_g = dlt[:, kv * g:(kv + 1) * g].reshape(n * g)
        lsafe = np.where(np.isfinite(lse_g), lse_g, 0.0)
        dQg = np.zeros((n * g, d))
        chunk = _chunk_len(n * g)

        def grads(s, kc, vc):
            p = np.exp(s - lsafe[:, None])
            dP = dOg @ vc.T
            dS = p * (dP - dl_g[:, None])
            return p, dS

        for a, b in _key_chunks(P, chunk):
            kc = _f64(kp[a:b, kv, :])
            vc = _f64(vp[a:b, kv, :])
            p, dS = grads(scale * (Qg @ kc.T), kc, vc)
            dQg += scale * (dS @ kc)
            dk_c = scale * (dS.T @ Qg)
            dv_c = p.T @ dOg
            if store_prefix:
                dkp[a:b, kv, :] = dk_c
                dvp[a:b, kv, :] = dv_c
            else:
                prefix_grad_sink(kv, a, b, dk_c, dv_c)
        for a, b in _key_chunks(kend, chunk):
            kc = _f64(kr[a:b, kv, :])
            vc = _f64(vr[a:b, kv, :])
            p, dS = grads(_scores_resp(Qg, kr, kv, a, b, scale, n, g, q_start), kc, vc)
            dQg += scale * (dS @ kc)
            dkr[a:b, kv, :] = scale * (dS.T @ Qg)
            dvr[a:b, kv, :] = p.T @ dOg
        dq[:, kv * g:(kv + 1) * g, :] = dQg.reshape(n, g, d)
    return dict(dq=dq, dkp=dkp, dvp=dvp, dkr=dkr, dvr=dvr)

