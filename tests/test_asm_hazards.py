"""Device assembly check: no matrix-core instruction reads a VGPR that an
inline-asm VALU instruction wrote fewer than two wait states before.

A VALU write of a VGPR needs two wait states before an MFMA reads that
register.  The compiler inserts them after its own VALU instructions but does
not count an inline-asm instruction as such a write, so kernels whose MFMA
operands come out of inline asm must supply them themselves (the rotary
attention kernels once did not, which made their outputs depend on the
schedule).  Every kernel source is compiled to gfx950 assembly with the
library's flags and scanned in program order within each kernel: `s_nop k`
counts k + 1 wait states, every other instruction one.  The scan ignores
branches, which only add instructions between a write and a read on the
paths they skip.  A probe kernel with a known violation checks the scanner."""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

from kv_cache_calibration_amd import build as B

NEED = 2
WRITERS = ("v_", "ds_read", "ds_bpermute", "ds_permute", "ds_swizzle", "global_load",
           "buffer_load", "flat_load", "scratch_load")

PROBE = r"""
#include <hip/hip_runtime.h>
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__global__ void probe(const u32x4* a, const float* x, v16f* out) {
  int l = threadIdx.x;
  u32x4 b = a[l];
  unsigned w = b.w;
  asm("v_fma_mixhi_f16 %0, %1, 1.0, -%1 op_sel:[0,0,0] op_sel_hi:[0,0,0]" : "+v"(w) : "v"(x[l]));
  b.w = w;
  v16f acc = out[l];
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a[l + 64]),
                                               __builtin_bit_cast(v8h, b), acc, 0, 0, 0);
  out[l] = acc;
}
"""


def _regs(tok):
    tok = tok.strip().lstrip("-").strip("|")
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def scan(asm_text):
    """(kernel, wait states, writer, mfma) for every MFMA source register
    whose last writer is inline asm fewer than NEED wait states earlier."""
    found = []
    kernel, in_asm, recent, pos = None, False, [], 0
    for ln in asm_text.split("\n"):
        if re.match(r"^[A-Za-z_]\S*:\s*(;.*)?$", ln) and not ln.startswith("."):
            if ln.startswith("_Z") or re.match(r"^\w+:\s*;\s*@", ln):
                kernel, recent, pos = ln.split(":")[0], [], 0
            continue
        s = ln.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith(";") or s.startswith(".") or s.endswith(":"):
            continue
        op = s.split()[0]
        if op == "s_nop":
            pos += int(s.split()[1].rstrip(";")) + 1
            continue
        args = s[len(op):].split(",")
        if op.startswith("v_mfma"):
            srcs = set()
            for a in args[1:4]:
                if a.strip():
                    srcs |= _regs(a.split()[0])
            for regs, p, is_asm, txt in reversed(recent):
                hit = regs & srcs
                if hit:
                    if is_asm and pos - p - 1 < NEED:
                        found.append((kernel, pos - p - 1, txt, s))
                    srcs -= hit
                    if not srcs:
                        break
        if op.startswith(WRITERS) and args and args[0].strip():
            d = _regs(args[0].split()[0])
            if d:
                recent.append((d, pos, in_asm, s))
                recent = recent[-256:]
        pos += 1
    return found


def _asm(src_path, out_dir):
    out = os.path.join(out_dir, os.path.basename(src_path) + ".s")
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    r = subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", src_path, "-o", out],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read()


def _have_hipcc():
    return shutil.which(B.HIPCC) or os.path.exists(B.HIPCC)


@pytest.mark.slow
def test_scanner_finds_a_planted_violation():
    if not _have_hipcc():
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "probe.hip")
        open(src, "w").write(PROBE)
        found = scan(_asm(src, d))
    assert found and all(w < NEED for _, w, _, _ in found), found


@pytest.mark.slow
@pytest.mark.parametrize("src", ["attention.hip", "quantize_mfma.hip", "quantize.hip", "codebook.hip"])
def test_no_inline_asm_mfma_operand_hazard(src):
    if not _have_hipcc():
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        found = scan(_asm(os.path.join(B.CSRC, src), d))
    assert not found, "\n".join(f"{k[:80]}: {w} wait states: {a} -> {m}" for k, w, a, m in found[:10])
