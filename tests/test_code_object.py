"""Checks on the built gfx950 code object (CPU only: it is disassembled, not run).

The bf16 work-group kernels (every mask kind), the unmasked fp32 kernels
and the short-key streaming kernel issue their direct global->LDS loads from
inline assembly that sets M0 and leaves it set.  That is only sound while no
instruction in those kernels relies on M0 keeping a value across other code.
They are checked for that here: M0 is only ever written, and each
instruction that reads it (the direct loads) follows its own M0 write, with
at most one wait state in between.  (The masked fp32 kernels use the
compiler's own direct-load builtin, whose M0 the compiler tracks; they are
not checked.)
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "flashattention_forward_04_amd", "libfa_mi355x.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tool(name):
    path = os.path.join(LLVM, name)
    return path if os.path.exists(path) else shutil.which(name)


def _disassemble(tmp_path):
    """Disassembly of every gfx950 code object in the library, as one text."""
    objcopy, bundler, objdump = _tool("llvm-objcopy"), _tool("clang-offload-bundler"), _tool("llvm-objdump")
    if not os.path.exists(LIB):
        pytest.skip("library not built")
    if not (objcopy and bundler and objdump):
        pytest.skip("ROCm LLVM tools not found")
    fat = tmp_path / "fatbin.bin"
    subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fat}", LIB], check=True, capture_output=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert starts, "no offload bundle in .hip_fatbin"
    text = []
    for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
        chunk = tmp_path / f"bundle{n}.bin"
        chunk.write_bytes(data[a:b])
        listed = subprocess.run([bundler, "--list", "--type=o", f"--input={chunk}"], capture_output=True, text=True)
        if TARGET not in listed.stdout.split():
            continue
        co = tmp_path / f"bundle{n}.co"
        subprocess.run([bundler, "--unbundle", "--type=o", f"--targets={TARGET}", f"--input={chunk}",
                        f"--output={co}"], check=True, capture_output=True)
        dis = subprocess.run([objdump, "-d", "--no-show-raw-insn", str(co)], check=True, capture_output=True,
                             text=True)
        text.append(dis.stdout)
    assert text, "no gfx950 code object in the library"
    return "\n".join(text)


def _kernels(text):
    """{symbol: [instruction lines]} for every function in the disassembly."""
    out, cur = {}, None
    for line in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m:
            cur = out.setdefault(m.group(1), [])
            continue
        if cur is None:
            continue
        ins = line.split("//")[0].strip()
        if ins and not ins.endswith(":"):
            cur.append(ins)
    return out


def _operands(ins):
    parts = ins.split(None, 1)
    return parts[0], [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


# kernels whose direct loads are hand-written: every bf16 work-group kernel,
# mask kind 0 (none) of the fp32 kernels, the streaming kernel and the
# backward dQ kernel
HAND = re.compile(r"fwd_bf16_kernelILi\d+ELi\d+E|fwd_f32_kernelILi\d+ELi0E|fwd_bf16_stream_kernel|bwd_dq_kernel")


def test_m0_is_set_right_before_each_reader(tmp_path):
    kernels = {k: v for k, v in _kernels(_disassemble(tmp_path)).items() if HAND.search(k)}
    assert any("fwd_bf16_kernel" in k for k in kernels) and any("fwd_f32_kernel" in k for k in kernels)
    assert any("stream" in k for k in kernels)
    problems = []
    n_loads = 0
    for name, body in kernels.items():
        for i, ins in enumerate(body):
            op, args = _operands(ins)
            uses_m0 = "m0" in args
            if op.startswith(("global_load_lds", "buffer_load")) and (op.startswith("global_load_lds") or "lds" in args):
                n_loads += 1
                prev = [body[j] for j in range(max(0, i - 2), i)]
                writes = [k for k, p in enumerate(prev) if _operands(p)[1][:1] == ["m0"]]
                ok = bool(writes) and all(p.startswith("s_nop") for p in prev[writes[-1] + 1:])
                if not ok:
                    problems.append(f"{name}: direct load without its own M0 write: {prev} / {ins}")
                continue
            if uses_m0 and args[0] != "m0":
                problems.append(f"{name}: M0 read by {ins}")
    assert n_loads > 0, "no direct loads found: the scan is not seeing the kernels"
    assert not problems, "\n".join(problems[:20])


def test_no_flat_memory_instructions(tmp_path):
    """Every load and store in the library addresses global memory or LDS
    explicitly.  A flat one (a pointer whose address space the compiler lost,
    e.g. one rebuilt from integers) also counts against the LDS-read wait
    counter, so an LDS wait placed for an operand read would wait for it too."""
    kernels = _kernels(_disassemble(tmp_path))
    assert kernels
    problems = [f"{name}: {ins}" for name, body in kernels.items() for ins in body if ins.startswith("flat_")]
    assert not problems, "\n".join(problems[:20])
