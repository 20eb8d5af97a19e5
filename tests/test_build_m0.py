"""The build's M0 check over the gfx950 disassembly of its own objects.

The buffer -> LDS tile loads are inline asm that write M0; the compiler cannot
be told M0 is clobbered, so the build refuses an object in which anything
else touches M0. CPU only: hipcc cross-compiles for gfx950 here."""
import os
import shutil
import subprocess

import pytest

from shared_prefix_packed_amd import build as B

HIPCC = shutil.which("hipcc") or os.path.join(B.ROCM, "bin", "hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


def _compile(tmp_path, body):
    src = tmp_path / "probe.hip"
    src.write_text("#include <hip/hip_runtime.h>\n" + body)
    obj = tmp_path / "probe.o"
    subprocess.run([HIPCC, *B.HIP_FLAGS, "-c", str(src), "-o", str(obj)], check=True,
                   stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    return str(obj)


LOAD_SEQ = r'''
__global__ void k(const int* __restrict__ p, int off) {
  __shared__ int s[256];
  typedef int i4 __attribute__((ext_vector_type(4)));
  i4 r = {0, 0, 64, 0x00020000};
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(off), "s"(r), "s"(__builtin_amdgcn_readfirstlane((int)(uintptr_t)s)) : "memory");
  %EXTRA%
}
'''


def test_library_objects_pass(tmp_path):
    """Every HIP object of the library: M0 appears only in the load sequences."""
    B.build()
    counts = {src: B.check_m0(os.path.join(B.BUILD_DIR, src + ".o")) for src in B.HIP_SOURCES}
    assert counts["pg_attn_mfma.hip"] > 0 and counts["pg_attn_bwd.hip"] > 0


def test_load_sequence_alone_passes(tmp_path):
    assert B.check_m0(_compile(tmp_path, LOAD_SEQ.replace("%EXTRA%", ""))) == 1


def test_other_m0_write_is_refused(tmp_path):
    """A planted M0 write outside a load sequence fails the build check."""
    obj = _compile(tmp_path, LOAD_SEQ.replace("%EXTRA%", 'asm volatile("s_mov_b32 m0, -1" ::: "memory");'))
    with pytest.raises(RuntimeError, match="M0 used outside"):
        B.check_m0(obj)
