"""Shared helpers for the GPU parity tests: seeded cases, the HIP path through the C ABI, the
oracle on the same inputs, and the tolerance check."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import attention as orc
from suffix_attention_amd import api, datagen

# Tolerances for bf16 inputs with float32 accumulation: max |x - y| <= 2e-2 and
# ||x - y||_2 / ||y||_2 <= 5e-3, per tensor.
ATOL = 2e-2
REL_L2 = 5e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy()


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / nrm if nrm > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(name, got, ref, atol=ATOL, rel_l2=REL_L2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    max_abs, rel = errors(got, ref)
    log(f"    {name:10s} max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= atol and rel <= rel_l2, f"{name}: max_abs={max_abs:.3e} rel_l2={rel:.3e}"


class Case:
    """A seeded prompt + one member, generated on the CPU and copied to the GPU."""

    def __init__(self, P, R, hq, hkv, d, dtype=torch.bfloat16, seed=0, S=1, bounds=None, table="perm",
                 n_phys_extra=0):
        self.P, self.R, self.hq, self.hkv, self.d, self.dtype = P, R, hq, hkv, d, dtype
        s = lambda tag: 7919 * seed + tag  # noqa: E731
        self.kp = datagen.normal((P, hkv, d), s(2), dtype)
        self.vp = datagen.normal((P, hkv, d), s(3), dtype)
        self.q = datagen.normal((R, hq, d), s(4), dtype)
        self.kr = datagen.normal((R, hkv, d), s(5), dtype)
        self.vr = datagen.normal((R, hkv, d), s(6), dtype)
        self.do = datagen.normal((R, hq, d), s(7), dtype)
        n_pages = api.n_logical_pages(P)
        self.n_phys = n_pages + n_phys_extra
        if table == "perm":
            perm = datagen.page_table(self.n_phys, s(1))[:n_pages]
        else:
            perm = torch.arange(n_pages, dtype=torch.int32)
        self.table = perm.to(torch.int32)
        self.bounds = bounds if bounds is not None else api.even_shard_bounds(n_pages, S)

    def token_bounds(self):
        return [(min(self.P, a * 64), min(self.P, b * 64)) for a, b in zip(self.bounds[:-1], self.bounds[1:])]

    def prefix(self, pool_fill=None):
        dev = "cuda"
        kp, vp, table = self.kp.to(dev), self.vp.to(dev), self.table.to(dev)
        k_pages = torch.zeros((self.n_phys, self.hkv, 64, self.d), dtype=self.dtype, device=dev)
        v_pages = torch.zeros_like(k_pages)
        if pool_fill is not None:
            k_pages.fill_(pool_fill)
            v_pages.fill_(pool_fill)
        if self.P > 0:
            api.capture_pages(kp, vp, table, self.n_phys, k_pages=k_pages, v_pages=v_pages)
        return api.Prefix(self.hq, self.hkv, self.d, self.dtype, self.P, table, k_pages, v_pages,
                          list(self.bounds))

    def gpu(self, q_start, n_rows, prefix=None, kr=None, vr=None, first_touch=True, store_ds=False):
        """Forward + backward of rows [q_start, q_start + n_rows) through the C ABI.  store_ds
        gives the backward a workspace large enough for its stored-dS dQ pass, filled with NaN
        so that any slot the dK/dV pass did not write and the dQ pass still used would show."""
        pre = prefix or self.prefix()
        dev = "cuda"
        q = self.q[q_start:q_start + n_rows].to(dev).contiguous()
        do = self.do[q_start:q_start + n_rows].to(dev).contiguous()
        kr = (self.kr if kr is None else kr).to(dev)
        vr = (self.vr if vr is None else vr).to(dev)
        o, lse, ws = api.replay_fwd(pre, q, q_start, kr, vr)
        o_parts, lse_parts = api.fwd_parts(pre, n_rows, ws)
        o_parts, lse_parts = o_parts.clone(), lse_parts.clone()
        dk_r = torch.full(kr.shape, float("nan"), dtype=torch.float32, device=dev)
        dv_r = torch.full(kr.shape, float("nan"), dtype=torch.float32, device=dev)
        dk_p = torch.full(pre.k_pages.shape, float("nan"), dtype=torch.float32, device=dev)
        dv_p = torch.full(pre.k_pages.shape, float("nan"), dtype=torch.float32, device=dev)
        ws = None
        if store_ds:
            nbytes = api.bwd_ds_workspace_bytes(pre, n_rows, q_start + n_rows)
            assert nbytes > api.bwd_workspace_bytes(pre, n_rows)
            ws = torch.full(((nbytes + 3) // 4,), float("nan"), dtype=torch.float32, device=dev)
        dq = api.replay_bwd(pre, q, q_start, kr, vr, o, lse, do, dk_r, dv_r, True, dk_p, dv_p,
                            shard_first_touch=[first_touch] * pre.n_shards, workspace=ws)
        torch.cuda.synchronize()
        return dict(o=o, lse=lse, dq=dq, dkr=dk_r, dvr=dv_r, dk_pages=dk_p, dv_pages=dv_p,
                    o_parts=o_parts, lse_parts=lse_parts, prefix=pre)

    def logical(self, pages: torch.Tensor) -> np.ndarray:
        """Gradient pages [n_phys, hkv, 64, d] -> logical prompt order [P, hkv, d]."""
        pg = np32(pages)
        t = np.arange(self.P)
        tab = self.table.numpy()
        return pg[tab[t // 64], :, t % 64, :]

    def stored(self, o):
        """The oracle's output as the library stores it: rounded to the input dtype."""
        return orc.round_bf16(o) if self.dtype == torch.bfloat16 else np.asarray(o, np.float32).astype(np.float64)

    def oracle(self, q_start, n_rows, o_used=None):
        q = np32(self.q[q_start:q_start + n_rows])
        do = np32(self.do[q_start:q_start + n_rows])
        kp, vp, kr, vr = np32(self.kp), np32(self.vp), np32(self.kr), np32(self.vr)
        O, L = orc.forward(q, kp, vp, kr, vr, q_start)
        g = orc.backward(q, kp, vp, kr, vr, do, q_start, o=o_used if o_used is not None else O, lse=L)
        return dict(o=O, lse=L, **g)

    def oracle_parts(self, q_start, n_rows):
        q = np32(self.q[q_start:q_start + n_rows])
        return orc.forward_parts(q, np32(self.kp), np32(self.vp), np32(self.kr), np32(self.vr),
                                 self.token_bounds(), q_start)


def check_against_oracle(case: Case, q_start: int, n_rows: int, res=None, parts=True, atol=None, store_ds=False):
    """atol: optional per-tensor max-abs bounds (for inputs scaled away from N(0, 1))."""
    atol = atol or {}
    res = res or case.gpu(q_start, n_rows, store_ds=store_ds)
    # The backward's delta is formed from the stored output, which has the input dtype; the
    # oracle's reference backward takes its own output rounded the same way.
    ref_exact = case.oracle(q_start, n_rows)
    ref = case.oracle(q_start, n_rows, o_used=case.stored(ref_exact["o"]))
    assert_close("O", np32(res["o"]), ref_exact["o"])
    assert_close("LSE", np32(res["lse"]), ref_exact["lse"])
    assert_close("dQ", np32(res["dq"]), ref["dq"], atol=atol.get("dQ", ATOL))
    kend = q_start + n_rows
    assert_close("dK_resp", np32(res["dkr"])[:kend], ref["dkr"][:kend], atol=atol.get("dK_resp", ATOL))
    assert_close("dV_resp", np32(res["dvr"])[:kend], ref["dvr"][:kend])
    assert np.all(np32(res["dkr"])[kend:] == 0) and np.all(np32(res["dvr"])[kend:] == 0)
    if case.P > 0:
        assert_close("dK_prompt", case.logical(res["dk_pages"]), ref["dkp"])
        assert_close("dV_prompt", case.logical(res["dv_pages"]), ref["dvp"])
    if parts:
        Op, Lp = case.oracle_parts(q_start, n_rows)
        gop, glp = np32(res["o_parts"]), np32(res["lse_parts"])
        for p in range(Op.shape[0]):
            empty = np.isneginf(Lp[p])
            assert np.array_equal(np.isneginf(glp[p]), empty), f"part {p}: empty rows differ"
            if np.all(empty):
                assert np.all(gop[p] == 0)
                continue
            assert_close(f"O_part{p}", gop[p], Op[p])
            assert_close(f"LSE_part{p}", glp[p][~empty], Lp[p][~empty])
    return res, ref
