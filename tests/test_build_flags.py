"""The library's compile commands: gfx950 code, with the packed fp32 VALU
forms (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32) kept out of the generated
code, for every source the library and the benchmark's probe are built from."""
import os

from coarse_grained_decode_amd import build as B


def _commands():
    objs = [(src, os.path.join(B.OBJDIR, name + ".o"), extra) for src, name, extra in B.UNITS]
    objs.append((B.PROBE_SOURCE, os.path.join(B.OBJDIR, "readprobe.o"), []))
    return [B.compile_command(src, obj, extra) for src, obj, extra in objs]


def test_every_source_is_compiled_for_gfx950_without_packed_fp32():
    cmds = _commands()
    sources = {os.path.basename(c[c.index("-c") + 1]) for c in cmds}
    assert set(B.SOURCES) <= sources and B.PROBE_SOURCE in sources
    for c in cmds:
        assert f"--offload-arch={B.ARCH}" in c
        i = c.index("-packed-fp32-ops")
        assert c[i - 3:i] == ["-Xclang", "-target-feature", "-Xclang"], c


def test_every_kernel_source_is_built():
    hip = {f for f in os.listdir(B.CSRC) if f.endswith(".hip")}
    assert hip == set(B.SOURCES) | {B.PROBE_SOURCE}


def test_default_architecture_is_gfx950():
    if "SPICY_OFFLOAD_ARCH" not in os.environ:
        assert B.ARCH == "gfx950"
