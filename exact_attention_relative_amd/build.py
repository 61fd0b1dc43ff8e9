"""Builds librelpos_attn.so (HIP, gfx950) in-tree with hipcc.

    python -m exact_attention_relative_amd.build
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librelpos_attn.so")
SOURCES = ["relpos_api.hip", "relpos_prep.hip", "relpos_fwd.hip", "relpos_bwd.hip", "relpos_agg.hip",
           "relpos_proj.hip", "relpos_bwd_txl_key.hip", "relpos_bwd_fat_q.hip", "relpos_bwd_trk.hip",
           "relpos_bwd_f32.hip", "relpos_noalloc.hip"]
# per-source options: the T-XL passes and the key-side passes of Shaw and DeBERTa schedule with
# the register-pressure trackers (fewer spills at the 256-register budget); the query-side
# general passes of Shaw and DeBERTa keep their MFMA accumulators in VGPRs (fewer copies between
# register files; measured)
EXTRA_FLAGS = {"relpos_bwd_txl_key.hip": ["-mllvm", "-amdgpu-use-amdgpu-trackers=1"],
               "relpos_bwd_trk.hip": ["-mllvm", "-amdgpu-use-amdgpu-trackers=1"],
               "relpos_bwd_fat_q.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
# measurement-only MFMA throughput probe, a library of its own
PROBE_LIB = os.path.join(PKG, "librelpos_probe.so")
PROBE_SOURCES = ["relpos_probe.hip"]

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         # keep the compiler from emitting packed fp32 arithmetic
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), "-I", os.path.join(PKG, "..", "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES + PROBE_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
