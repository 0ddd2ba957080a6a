"""The gfx950 assembly of the library's kernels (built here from source, no
GPU needed) keeps the properties its memory ordering and numerics rely on:

- every L2 write-back of a release (buffer_wbl2) is followed by a wait for
  all outstanding vector memory operations (s_waitcnt with vmcnt(0)) before
  the next memory access, so the releasing store, atomic or CAS cannot reach
  memory ahead of the data it publishes. The compiler's own wait after the
  write-back can be merged away (a release atomic issued right after a load
  it needed was compiled to buffer_wbl2 followed directly by the atomic, and
  a tag written before it was then read back stale on another XCD), so the
  kernels put an explicit wait there;
- no packed fp32 instructions (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32);
- no MFMA (the reduction is adds, not a contraction).
"""
import os
import re
import subprocess

import pytest

from signal_pad_sync_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(B.CSRC, f) for f in ("arx_reduce.hip", "arx_sync.hip")] + \
          [os.path.join(ROOT, "tests", "devapi", "devapi_user.hip")]

MEM_OP = re.compile(r"^\s*(global_|buffer_(load|store|atomic)|flat_|scratch_)")


def assembly(src, tmp_path):
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path / (os.path.basename(src) + ".s")
    subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", str(out)], check=True,
                   capture_output=True, text=True, timeout=600)
    return out.read_text().splitlines()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    return {os.path.basename(s): assembly(s, d) for s in SOURCES}


def test_every_writeback_is_waited_for(asm):
    seen = 0
    for name, lines in asm.items():
        for i, ln in enumerate(lines):
            if "buffer_wbl2" not in ln:
                continue
            seen += 1
            waited = False
            for nxt in lines[i + 1:]:
                if re.match(r"^\s*s_waitcnt\b.*vmcnt\(0\)", nxt):
                    waited = True
                    break
                assert not MEM_OP.match(nxt) and "s_endpgm" not in nxt, \
                    f"{name}:{i + 1}: buffer_wbl2 followed by '{nxt.strip()}' before any vmcnt(0) wait"
            assert waited, f"{name}:{i + 1}: buffer_wbl2 never waited for"
    assert seen >= 10


def test_no_packed_fp32_and_no_mfma(asm):
    for name, lines in asm.items():
        for i, ln in enumerate(lines):
            assert not re.match(r"^\s*v_pk_(add|mul|fma)_f32", ln), f"{name}:{i + 1}: {ln.strip()}"
            assert not re.match(r"^\s*v_mfma", ln), f"{name}:{i + 1}: {ln.strip()}"
