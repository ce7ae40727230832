"""Register budgets the launch shapes depend on, checked on the compiled
gfx950 code (host-only: hipcc cross-compiles without a GPU).

A 1024-thread GEMV workgroup is sixteen waves, four per SIMD; two of them share
a CU only while every wave holds at most 64 VGPRs (eight waves per SIMD out of
512 registers).  The one-row 4-bit, MXFP4 and NVFP4 GEMV instances and the g = 128
quantize kernel are compiled to that bound; crossing it halves their
workgroups per CU without any other symptom, so the bound and the absence of
register spills are checked here."""
import os
import re
import subprocess
import tempfile

import pytest

from w4a16_bit_matmul_amd import _build


def _kernel_metadata(src_name):
    src = os.path.join(_build.CSRC, src_name)
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [_build.HIPCC, *_build.COMMON, *_build.PER_FILE[src_name], "-Wno-unused-value",
               "--cuda-device-only", "-S", src, "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            pytest.fail(res.stdout + res.stderr)
        text = open(out).read()
    meta = {}
    # the metadata block lists, per kernel, .name, .private_segment_fixed_size and .vgpr_count
    for block in text.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        vgpr = int(re.search(r"\.vgpr_count:\s+(\d+)", block).group(1))
        scratch = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1))
        meta[name] = (vgpr, scratch)
    return meta


def _find(meta, fragment):
    hits = [(n, v) for n, v in meta.items() if fragment in n]
    assert hits, f"no kernel matching {fragment}"
    return hits


@pytest.mark.skipif(not os.path.exists(_build.HIPCC), reason="hipcc is not installed")
def test_one_row_gemv_fits_two_workgroups_per_cu():
    meta = _kernel_metadata("wq_gemv.hip")
    # 4-bit codes: gemv_mfma_half_kernel<W=16, KQ=4, G> (the one-row launch) and
    # gemv_mfma_kernel<MT=1, W=16, KQ=4, G, RB=1, FMT> at g = 128 and 32, and for
    # MXFP4 (G = 32) and NVFP4 (G = 16)
    for frag in ("gemv_mfma_half_kernelILi16ELi4ELi128E", "gemv_mfma_half_kernelILi16ELi4ELi32E",
                 "gemv_mfma_kernelILi1ELi16ELi4ELi128E", "gemv_mfma_kernelILi1ELi16ELi4ELi32E",
                 "gemv_mfma_kernelILi1ELi16ELi4ELi16E"):
        for name, (vgpr, scratch) in _find(meta, frag):
            assert vgpr <= 64 and scratch == 0, (name, vgpr, scratch)


@pytest.mark.skipif(not os.path.exists(_build.HIPCC), reason="hipcc is not installed")
def test_multi_row_gemv_register_budgets():
    # the 4-bit GEMV with eight rows of x over one or two row blocks runs two
    # eight-wave workgroups per CU (at most 128 VGPRs: 16 waves on 4 SIMDs);
    # with sixteen rows over four blocks two four-wave workgroups (at most 256);
    # crossing either bound halves the workgroups per CU (a 20 % slower product)
    meta = _kernel_metadata("wq_gemv.hip")
    # (the MXFP4 instances have G = 32 too; NVFP4's G = 16)
    for g in (128, 32, 16):
        for rb in (1, 2):
            for name, (vgpr, scratch) in _find(meta, f"gemv_mfma_kernelILi8ELi8ELi4ELi{g}ELi{rb}E"):
                assert vgpr <= 128 and scratch == 0, (name, vgpr, scratch)
        for name, (vgpr, scratch) in _find(meta, f"gemv_mfma_kernelILi16ELi4ELi4ELi{g}ELi4E"):
            assert vgpr <= 256 and scratch == 0, (name, vgpr, scratch)
        # eight rows over two blocks, or over one block of a narrow output, in
        # sixteen-wave workgroups: four waves per SIMD
        for rb in (1, 2):
            for name, (vgpr, scratch) in _find(meta, f"gemv_mfma_kernelILi8ELi16ELi4ELi{g}ELi{rb}E"):
                assert vgpr <= 128 and scratch == 0, (name, vgpr, scratch)


@pytest.mark.skipif(not os.path.exists(_build.HIPCC), reason="hipcc is not installed")
def test_no_gemv_instance_spills():
    # every compiled GEMV instance (all code formats, tile heights and row
    # blocks the plans can launch) keeps its values in registers
    meta = _kernel_metadata("wq_gemv.hip")
    gemv = [(n, v) for n, v in meta.items() if "gemv_mfma" in n]
    assert len(gemv) >= 30, len(gemv)
    for name, (vgpr, scratch) in gemv:
        assert scratch == 0 and vgpr <= 256, (name, vgpr, scratch)


@pytest.mark.skipif(not os.path.exists(_build.HIPCC), reason="hipcc is not installed")
def test_g128_quantize_fits_eight_workgroups_per_cu():
    meta = _kernel_metadata("wq_quant.hip")
    # quantize_kernel<DT, G=128, SYM, SCALED=false> for every input dtype
    for dt in range(3):
        for sym in "01":
            for name, (vgpr, scratch) in _find(meta, f"quantize_kernelILi{dt}ELi128ELb{sym}ELb0E"):
                assert vgpr <= 64 and scratch == 0, (name, vgpr, scratch)


def _kernel_asm(src_name):
    src = os.path.join(_build.CSRC, src_name)
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [_build.HIPCC, *_build.COMMON, *_build.PER_FILE[src_name], "-Wno-unused-value",
               "--cuda-device-only", "-S", src, "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            pytest.fail(res.stdout + res.stderr)
        return open(out).read()


def _first_loop(asm, kernel):
    """Instructions of the kernel's K loop: the blocks the compiler marks as one
    depth-1 loop (its header, and the blocks noted as in that loop), for the
    loop with the most MFMAs."""
    body = asm.split("\n" + kernel + ":", 1)[1].split("s_endpgm", 1)[0]
    loops = {}
    # blocks start at a label line; its comment names the loop it belongs to
    parts = re.split(r"^(\.LBB\w+:[^\n]*)$", body, flags=re.M)
    for head, text in zip(parts[1::2], parts[2::2]):
        label = head.split(":", 1)[0][1:]  # without the leading '.'
        m = re.search(r"Header=(\w+) Depth=1", head)
        key = label if ("Loop Header" in head and "Depth=1" in head) else (m.group(1) if m else None)
        if key:
            loops[key] = loops.get(key, "") + text
    assert loops, kernel
    return max(loops.values(), key=lambda t: t.count("v_mfma"))


@pytest.mark.skipif(not os.path.exists(_build.HIPCC), reason="hipcc is not installed")
def test_m128_gemm_keeps_its_loop_in_registers():
    # gemm_kernel<MB=8, G, SZV=true, FMT> (the 128-row tile every M > 64
    # product with aligned scale rows runs): two waves per SIMD share 512
    # registers, so each has 256; a spill inside the K loop would add a
    # memory round trip (and a wait for every load in flight) per tile
    asm = _kernel_asm("wq_gemm.hip")
    meta = _kernel_metadata("wq_gemm.hip")
    for frag in ("gemm_kernelILi8ELi128ELb1ELi4E", "gemm_kernelILi8ELi32ELb1ELi4E", "gemm_kernelILi8ELi128ELb1ELi8E",
                 "gemm_kernelILi8ELi32ELb1ELi8E", "gemm_kernelILi8ELi32ELb1ELi2E", "gemm_kernelILi8ELi16ELb1ELi3E"):
        for name, (vgpr, scratch) in _find(meta, frag):
            assert vgpr <= 256, (name, vgpr)
            loop = _first_loop(asm, name)
            assert loop.count("v_mfma") >= 64, name  # the K loop: at least eight tiles of eight MFMAs
            assert "s_waitcnt vmcnt(0)" not in loop and "scratch_store" not in loop, name
            # no spill inside the loop, except a few reloads of loop-invariant
            # values per eight tiles where the registers are full: int8 codes at
            # g = 32 (a ring of 16-byte code slots), three; 4-bit codes at g = 32
            # (both steps' scales staged per tile), two
            allowed = {"gemm_kernelILi8ELi32ELb1ELi8E": 3, "gemm_kernelILi8ELi32ELb1ELi4E": 2}.get(frag, 0)
            assert loop.count("scratch_load") <= allowed, (name, loop.count("scratch_load"))
