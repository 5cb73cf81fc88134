"""Properties of the generated gfx950 code that the compiler does not check
for inline assembly, on the CPU (hipcc cross-compiles; no device needed).

The prefill kernel reads raw MFMA results with an inline-asm v_max3_f32 and
issues LDS reads in asm blocks without their wait. The matrix cores do not
interlock their results, and the compiler inserts no wait states for an asm
operand, nor does it know that an asm block's LDS results are still in
flight. Two checks over every prefill instantiation's code:
  * at least MIN_WAIT wait states (s_nop N counts N + 1, every other
    instruction 1) between the MFMA that writes a register and a v_max3_f32
    that reads it;
  * no instruction reads or writes the destination of an LDS read before an
    s_waitcnt lgkmcnt covers it.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_split_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# MFMA result to VALU read on gfx950, with margin: the 16x16x32 bf16 product
# needs fewer; 19 is what the kernel's own wait block provides
MIN_WAIT = 19


def _asm(tmp_path, source):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path / "k.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           "-o", str(out), os.path.join(CSRC, source)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _functions(asm, pattern):
    for name in re.findall(r"^(" + pattern + r"\w*):", asm, re.M):
        i = asm.index(name + ":")
        j = asm.index(".Lfunc_end", i)
        lines = [l.strip() for l in asm[i:j].splitlines()
                 if l.startswith("\t") and not l.strip().startswith((".", ";"))]
        yield name, lines


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _split(line):
    op = line.split()[0]
    return op, [a.strip() for a in line[len(op):].split(",")]


@pytest.fixture(scope="module")
def prefill_asm(tmp_path_factory):
    return _asm(tmp_path_factory.mktemp("isa"), "prefill.hip")


def test_mfma_results_reach_inline_asm_after_enough_wait_states(prefill_asm):
    seen = 0
    for name, lines in _functions(prefill_asm, r"_ZN6pdattn12_GLOBAL__N_114prefill_kernel"):
        ws = [0]
        for l in lines:
            m = re.match(r"s_nop\s+(\d+)", l)
            ws.append(ws[-1] + (int(m.group(1)) + 1 if m else 1))
        last = {}
        for k, l in enumerate(lines):
            op, args = _split(l)
            if op == "v_max3_f32":
                for a in args[1:]:
                    for r in _regs(a):
                        if r in last:
                            seen += 1
                            gap = ws[k] - ws[last[r] + 1]
                            assert gap >= MIN_WAIT, (name, l, gap)
            dst = _regs(args[0]) if args else set()
            if op.startswith("v_mfma"):
                for r in dst:
                    last[r] = k
            elif op.startswith(("v_", "ds_read")):
                for r in dst:
                    last.pop(r, None)
    assert seen > 0  # the bf16 instantiations do read MFMA results this way


def test_lds_read_destinations_untouched_until_their_wait(prefill_asm):
    checked = 0
    for name, lines in _functions(prefill_asm, r"_ZN6pdattn12_GLOBAL__N_114prefill_kernel"):
        pending = set()
        for l in lines:
            op, args = _split(l)
            if op == "s_waitcnt" and "lgkmcnt" in l:
                pending = set()
                continue
            stores = op.startswith(("ds_write", "global_store", "buffer_store"))
            srcs = set()
            for a in (args if stores else args[1:]):
                for t in a.split():
                    srcs |= _regs(t)
            dst = set() if stores or op.startswith("s_") or not args else _regs(args[0])
            if not op.startswith("ds_read"):
                assert not (pending & (srcs | dst)), (name, l)
            else:
                pending |= dst
                checked += 1
    assert checked > 0


def test_checks_catch_a_planted_hazard(tmp_path):
    """The wait-state check is not vacuous: an MFMA followed at once by an
    asm v_max3 of its result fails it."""
    src = tmp_path / "planted.hip"
    src.write_text(r'''
#include <hip/hip_runtime.h>
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
__global__ void prefill_kernel_planted(const bf16x8* a, float* o) {
  f32x4 s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[threadIdx.x], a[threadIdx.x + 64], f32x4{0, 0, 0, 0}, 0, 0, 0);
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(s[0]), "v"(s[1]), "v"(s[2]));
  o[threadIdx.x] = r;
}
''')
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path / "planted.s"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "--cuda-device-only", "-S", "-o", str(out), str(src)],
                   check=True, capture_output=True)
    asm = out.read_text()
    gaps = []
    for name, lines in _functions(asm, r"_Z22prefill_kernel_planted"):
        ws = [0]
        for l in lines:
            m = re.match(r"s_nop\s+(\d+)", l)
            ws.append(ws[-1] + (int(m.group(1)) + 1 if m else 1))
        last = {}
        for k, l in enumerate(lines):
            op, args = _split(l)
            if op == "v_max3_f32":
                gaps += [ws[k] - ws[last[r] + 1] for a in args[1:] for r in _regs(a) if r in last]
            if op.startswith("v_mfma"):
                for r in _regs(args[0]):
                    last[r] = k
    assert gaps and min(gaps) < MIN_WAIT
