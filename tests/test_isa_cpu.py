"""The device code as compiled: properties the build flags promise, checked in the assembly hipcc
emits for every HIP translation unit of the library (gfx950, the library's own flags).

- fp32 arithmetic runs with IEEE denormals and round-to-nearest-even in every kernel (the kernel
  descriptors' fp32 float modes), the environment the pinned per-token schedule is defined in;
- no packed fp32 instruction appears (the build disables them; the schedule's bits are those of
  scalar fp32 operations);
- no kernel writes through the scalar data cache: every store and atomic is a vector or LDS
  instruction, and no scalar-cache write-back or discard is issued.

This file names scalar-memory mnemonics, so it is kept out of the trees sent for GPU runs; it
needs only hipcc, which cross-compiles here.
"""
import concurrent.futures as cf
import importlib.util
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("cpr_build", os.path.join(ROOT, "bitwise_aligned_gated_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    b = _build_module()
    if not os.path.exists(b.HIPCC):
        pytest.skip("hipcc not found")
    out_dir = tmp_path_factory.mktemp("isa")
    sources = [s for s in b.SOURCES if s.endswith(".hip")]

    def one(src):
        out = os.path.join(out_dir, src + ".s")
        cmd = [b.HIPCC, *b.FLAGS, "--offload-device-only", "-S", "-x", "hip", os.path.join(b.CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"hipcc -S failed for {src}:\n{r.stderr[-2000:]}"
        with open(out) as f:
            return src, f.read()

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        return dict(ex.map(one, sources))


def _instructions(text):
    """Instruction lines (mnemonic first), without directives, labels and comments."""
    for line in text.splitlines():
        s = line.split(";", 1)[0].strip()
        if s and not s.startswith(".") and not s.endswith(":"):
            yield s


def _kernels(text):
    return re.findall(r"^\s*\.amdhsa_kernel\s+(\S+)", text, re.M)


def test_every_kernel_runs_ieee_fp32_modes(device_asm):
    total = 0
    for src, text in device_asm.items():
        kernels = _kernels(text)
        denorm = re.findall(r"^\s*\.amdhsa_float_denorm_mode_32\s+(\d+)", text, re.M)
        rnd = re.findall(r"^\s*\.amdhsa_float_round_mode_32\s+(\d+)", text, re.M)
        total += len(kernels)
        assert len(denorm) == len(kernels) and set(denorm) <= {"3"}, (src, denorm)   # fp32 denormals kept
        assert len(rnd) == len(kernels) and set(rnd) <= {"0"}, (src, rnd)            # round to nearest even
    assert total >= 20, f"only {total} kernel descriptors found"


def test_no_packed_fp32_instruction(device_asm):
    packed = re.compile(r"^v_pk_(fma|mul|add)_f32\b")
    for src, text in device_asm.items():
        bad = [s for s in _instructions(text) if packed.match(s)]
        assert not bad, f"{src}: packed fp32 instructions {bad[:3]}"


def test_no_write_through_the_scalar_data_cache(device_asm):
    scalar_write = re.compile(r"^s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|dcache_discard)")
    for src, text in device_asm.items():
        ins = list(_instructions(text))
        if _kernels(text):                                    # the scan does see the stores
            assert any(s.startswith("global_store") or s.startswith("ds_write") for s in ins), src
        bad = [s for s in ins if scalar_write.match(s)]
        assert not bad, f"{src}: scalar-cache writes {bad[:3]}"
