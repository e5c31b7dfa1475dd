"""Properties of the gfx950 code the kernels compile to (CPU only: hipcc emits the
device assembly without a GPU).

- M0 is written only by the direct-to-LDS load sequences, which declare it
  clobbered; that is sound only while no compiler-generated instruction reads M0,
  so the instructions that read it implicitly must be absent, apart from those loads.
- No scalar-cache writes (scalar stores, scalar atomics, write-back of that cache).
- No packed fp32 VALU instructions (the build disables their formation).
"""
import functools
import os
import re
import shutil
import subprocess

import pytest

from mla_latent_kv_41_amd import build

HIPCC = build.HIPCC


@functools.lru_cache(maxsize=None)
def device_asm(src, extra=()):
    flags = [f for f in build.FLAGS if f not in ("-fPIC", "-shared")]
    res = subprocess.run([HIPCC, *flags, *extra, "--cuda-device-only", "-S", src, "-o", "-"],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return res.stdout


def instructions(asm):
    for line in asm.splitlines():
        s = line.strip()
        if not s or s.startswith((";", ".", "_")) or s.endswith(":"):
            continue
        yield s.split(";")[0].strip()


# instructions that read M0 implicitly (LDS-direct and interpolation forms, GWS,
# messages, relative register moves, LDS "add TID" forms)
IMPLICIT_M0 = re.compile(r"^(s_sendmsg|s_movrel|v_movrel|v_interp|ds_gws|ds_\w*addtid|lds_direct|"
                         r"s_ttracedata)")
SCALAR_WRITE = re.compile(r"^(s_store|s_scratch_store|s_buffer_store|s_atomic|s_buffer_atomic|"
                          r"s_dcache_wb|s_dcache_discard)")
PACKED_F32 = re.compile(r"^v_pk_(add|mul|fma)_f32")


# every source as the library builds it, and the attention kernels' instrumented
# build (phase stamps) as the stamp tool builds it
CASES = [(os.path.basename(p)[:-4], ()) for p in sorted(build.sources())] + [("decode_bf16", ("-DMLA_STAMPS",))]


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not found")
@pytest.mark.parametrize("name,extra", CASES, ids=[n + ("-stamps" if e else "") for n, e in CASES])
def test_device_code_properties(name, extra):
    asm = device_asm(os.path.join(build.CSRC, name + ".hip"), extra)
    insts = list(instructions(asm))
    assert insts, "no instructions parsed"
    for k, s in enumerate(insts):
        mnem = s.split()[0]
        assert not IMPLICIT_M0.match(mnem), s
        assert not SCALAR_WRITE.match(mnem), s
        assert not PACKED_F32.match(mnem), s
        if re.search(r"\bm0\b", s):
            # only writes of M0 from an SGPR, each followed, after at least one address
            # add (the wait state M0 needs) and nothing else, by a direct-to-LDS load
            assert re.match(r"^s_mov_b32 m0, s\d+$", s), s
            j = k + 1
            while j < len(insts) and insts[j].startswith("v_add_u32"):
                j += 1
            assert j > k + 1 and j < len(insts) and insts[j].startswith("buffer_load") and \
                insts[j].endswith(" lds"), (s, insts[k + 1:j + 1])
        if mnem.startswith("buffer_load") and s.endswith(" lds"):
            # a run of direct-to-LDS loads and their address adds goes back to its M0 write
            j = k - 1
            while j >= 0 and (insts[j].startswith("v_add_u32") or
                              (insts[j].startswith("buffer_load") and insts[j].endswith(" lds"))):
                j -= 1
            assert j >= 0 and re.match(r"^s_mov_b32 m0, s\d+$", insts[j]), \
                ("direct-to-LDS load without its M0 write", s)


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not found")
@pytest.mark.parametrize("name", sorted(os.path.basename(p)[:-4] for p in build.sources()))
def test_kernels_use_no_scratch(name):
    """No kernel spills vector registers or uses scratch memory (SGPR spills go to
    VGPR lanes and are allowed). Each kernel's metadata map lists its keys in
    alphabetical order, .name among them, so a map is read as one block."""
    asm = device_asm(os.path.join(build.CSRC, name + ".hip"))
    meta = asm[asm.find("amdhsa.kernels:"):]
    blocks = re.split(r"\n\s+- \.", meta)
    kernels = {}
    for b in blocks:
        nm = re.search(r"(?:^|\n)\s*\.?name:\s+(_Z\S+)", "." + b)
        if not nm:
            continue
        vals = dict((k, int(v)) for k, v in re.findall(
            r"\.?(private_segment_fixed_size|vgpr_spill_count):\s+(\d+)", "." + b))
        kernels[nm.group(1)] = vals
    if name == "api":
        return  # host code only
    assert kernels, "no kernel metadata parsed"
    for k, v in kernels.items():
        assert set(v) == {"private_segment_fixed_size", "vgpr_spill_count"}, (k, v)  # both parsed
        assert v["private_segment_fixed_size"] == 0, (k, v)
        assert v["vgpr_spill_count"] == 0, (k, v)


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not found")
def test_rate_microbenchmark_builds():
    """The per-CU rate microbenchmark compiles for gfx950 under the library's flags,
    with the same device-code rules (its direct-to-LDS loads write M0 themselves)."""
    from mla_latent_kv_41_amd import rates
    asm = device_asm(rates.SRC)
    insts = list(instructions(asm))
    assert any(s.startswith("buffer_load_dwordx4") and s.endswith(" lds") for s in insts)
    assert any(s.startswith("v_mfma_f32_32x32x16_bf16") for s in insts)
    assert any(s.startswith("v_mfma_f32_16x16x32_bf16") for s in insts)
    for s in insts:
        mnem = s.split()[0]
        assert not IMPLICIT_M0.match(mnem), s
        assert not SCALAR_WRITE.match(mnem), s
        assert not PACKED_F32.match(mnem), s
    assert not re.search(r"(vgpr_spill_count|private_segment_fixed_size):\s+[1-9]", asm)
