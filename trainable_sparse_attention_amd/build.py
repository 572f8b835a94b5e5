"""Build the HIP library lib/libqsa.so for gfx950 with hipcc (in-tree).

Usage: python -m trainable_sparse_attention_amd.build
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libqsa.so")
SOURCES = ["abi.hip", "pool_keys.hip", "index_prefill.hip", "index_exact.hip", "index_decode.hip",
           "attn.hip", "attn_bwd.hip", "distill.hip", "dense_attn.hip", "probe_gather.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function", "-Wno-unused-variable",
         # packed fp32 instructions are kept out of every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# per-file additions: the attention kernels keep MFMA accumulators in VGPRs,
# where the online-softmax rescale can scale them without AGPR round trips
EXTRA = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         # float atomics of the gradient scatter as hardware adds
         "attn_bwd.hip": ["-munsafe-fp-atomics"], "distill.hip": ["-munsafe-fp-atomics"]}


def _compile(src, obj):
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-I", os.path.join(HERE, "..", "include"), "-c",
                             os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    return r.returncode, " ".join(cmd), msgs


def build(verbose=False):
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        res = list(ex.map(_compile, SOURCES, objs))
    for rc, cmd, msgs in res:
        if msgs.strip() and (verbose or rc):
            print(msgs, file=sys.stderr)
        if rc:
            raise RuntimeError("hipcc failed: " + cmd)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
