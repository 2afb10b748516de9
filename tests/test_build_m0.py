"""The LDS-direct H copies set m0 in inline assembly, a register the compiler
reserves and does not track across such a block.  That is sound only while no
instruction the compiler generates in the stream kernels reads or writes m0
(the library never calls the copy builtin, which would set m0 itself).  This
compiles the kernel sources to gfx950 assembly and checks, in every kernel that
holds such a block, that every m0 reference sits inside an inline-assembly
block, and that each block writes m0 right before its copy.  (Kernels without a
copy block may use m0 as the compiler likes.)"""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STREAM_SOURCES = ("fs_stream_flat.hip", "fs_stream_group.hip", "fs_stream_store.hip", "fs_stream_topk.hip",
                  "fs_kernels.hip")


def _build_module():
    import importlib.util

    spec = importlib.util.spec_from_file_location("_fs_build_m0", os.path.join(ROOT, "lm_head_matmul_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_m0_only_in_copy_blocks():
    b = _build_module()
    try:
        cc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        procs = []
        for f in STREAM_SOURCES:
            out = os.path.join(tmp, f + ".s")
            cmd = [cc, *b.HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-S", "--cuda-device-only",
                   os.path.join(b.CSRC, f), "-o", out]
            procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), f, out))
        n_blocks = 0
        for proc, f, out in procs:
            _, err = proc.communicate()
            assert proc.returncode == 0, f"{f}: {err[-2000:]}"
            # split the assembly into functions; check those holding a copy block
            funcs, cur = [], None
            for line in open(out):
                if re.match(r"^\s*\.type\s+\S+,@function", line):
                    cur = [line.split()[1].rstrip(",")]
                    funcs.append(cur)
                elif cur is not None:
                    cur.append(line)
            for lines in funcs:
                name, body = lines[0], lines[1:]
                if not any("global_load_lds_dwordx4" in l and "ASM" not in l for l in body):
                    continue
                inside = False
                for line in body:
                    t = line.split(";")[0].strip() if not line.lstrip().startswith(";;#ASM") else line.strip()
                    if t.startswith(";;#ASMSTART"):
                        inside = True
                        continue
                    if t.startswith(";;#ASMEND"):
                        inside = False
                        continue
                    if re.search(r"\bm0\b", t):
                        assert inside, f"{f} {name}: compiler-generated m0 use: {t}"
                        if t.startswith("s_mov_b32 m0"):
                            n_blocks += 1
        assert n_blocks > 0, "no LDS-direct copy blocks found"
