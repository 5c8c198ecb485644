"""Build liblongstraw.so (HIP for gfx950) in-tree with hipcc.

    python -m suffix_attention_amd.build [--jobs N] [--save-temps DIR]

Every source under csrc/ is compiled to an object in csrc/_build/, then linked into
suffix_attention_amd/liblongstraw.so next to this file.  The measurement microbenchmarks under
bench/hip/ (matrix-core and HBM ceilings, which bench.py reports against) are built the same way
into bench/libmicrobench.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(HERE, "liblongstraw.so")
SOURCES = ["abi.cpp", "profile.cpp", "capture.hip", "reduce.hip", "attn_generic.hip", "attn_mfma_fwd.hip",
           "attn_mfma_bwd.hip", "attn_mfma_dq.hip", "attn_mfma_dqs.hip", "attn_mfma_fwd_dq.hip", "noalloc.hip"]

ROOT = os.path.dirname(HERE)
BENCH_HIP = os.path.join(ROOT, "bench", "hip")
BENCH_SOURCES = ["mfma_peak.hip", "hbm_bw.hip", "lds_bw.hip"]
BENCH_LIB = os.path.join(ROOT, "bench", "libmicrobench.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU ops are kept off: the compiler never emits them and none is written by
# hand.  -ffp-contract=fast lets multiply-adds fuse; no other fast-math flag is used, so
# infinities and NaN keep their IEEE meaning (masked scores are -inf).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=fast",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


# Matrix-core accumulators go to VGPRs in the dQ pass (its S / dP tiles feed vector-ALU work
# every page, its read-only Q / dO operands sit in AGPRs), in the dK/dV pass (its S / dP
# tiles likewise; its 256 dK / dV accumulators are kept in AGPRs by explicit AGPR-form matrix
# instructions) and in the forward (the score tiles feed the softmax directly, and the output
# tile is rescaled by plain vector multiplies).
PER_SOURCE = {"attn_mfma_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "attn_mfma_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "attn_mfma_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "attn_mfma_dqs.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "attn_mfma_fwd_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src, extra, src_dir=CSRC, obj_dir=BUILD):
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *PER_SOURCE.get(src, []), *extra, "-c", os.path.join(src_dir, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = [ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    return src, obj, r.returncode, "\n".join(noise), cmd


def build(jobs: int | None = None, save_temps: str | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    extra = []
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        extra = [f"-save-temps={'obj'}"]
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, obj, rc, err, cmd in ex.map(lambda s: _compile(s, extra), SOURCES):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{err}")
            if err and verbose:
                print(f"[{src}] {err}", file=sys.stderr)
            objs.append(obj)
    _link(objs, LIB)
    build_microbench()
    return LIB


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)


def build_microbench() -> str:
    obj_dir = os.path.join(BENCH_HIP, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=len(BENCH_SOURCES)) as ex:
        for src, obj, rc, err, cmd in ex.map(lambda s_: _compile(s_, [], BENCH_HIP, obj_dir), BENCH_SOURCES):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{err}")
            objs.append(obj)
    _link(objs, BENCH_LIB)
    return BENCH_LIB


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ns = ap.parse_args()
    print(build(ns.jobs, verbose=ns.verbose))
