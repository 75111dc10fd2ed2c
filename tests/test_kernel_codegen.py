"""Code-generation guards for the decode kernel (CPU only: hipcc cross-compiles
for gfx950 and the AMD assembly of this repository's own kernel is read).

The decode kernel keeps a ring of tiles in flight: when a slot is consumed,
only that slot's loads may be waited for.  Small register-allocation changes
can make the compiler insert a wait for *all* outstanding loads in the loop
(it then copies or reuses in-flight load destinations), which drains the
ring once per turn and costs a large part of the bandwidth.  This test fails
if a decode kernel's tile loop ever waits with less than one tile's K/V loads
still outstanding.
"""
import os
import re
import shutil
import subprocess

import pytest

from load_balanced_paged_step_amd import build as B

KV_LOADS_PER_TILE = 8   # 4 K + 4 V buffer loads per wave and tile (plus 4 Q loads, issued first)


def _asm(tmp_path) -> str:
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path / "decode_kernels.s"
    cmd = [hipcc, "-x", "hip", *B.DEVICE, *B.COMMON, "-S", "--offload-device-only",
           os.path.join(B.HERE, "csrc", "decode_kernels.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(asm: str):
    for m in re.finditer(r"^(_ZN4hpcd\w*decode_kernel\w*):", asm, re.M):
        end = asm.find("s_endpgm", m.end())
        yield m.group(1), asm[m.end():end]


def _ring_waits(asm: str):
    """(kernel name, every vmcnt wait inside the tile loop) for every decode
    kernel.  The tile loop is the outermost loop that holds the first score
    MFMA: its header and every block the compiler marks as belonging to it
    (directly or through an inner loop).  The VALU tile math's loop is found
    the same way from its first dot2."""
    for name, body in _kernels(asm):
        # the first score instruction: an MFMA, or a dot2 in the VALU tile math
        first_mfma = body.find("v_dot2c_f32_bf16" if _valu(name) else "v_mfma_f32_16x16x32_bf16")
        assert first_mfma > 0, name
        heads = list(re.finditer(r"^\.(LBB\w+):\s*;\s*=>\s*This (?:Inner )?Loop Header: Depth=1",
                                 body[:first_mfma], re.M))
        assert heads, name
        loop = heads[-1].group(1)            # "LBB1_71"; loop comments name it "BB1_71"
        loop_id = loop[1:]
        # split into basic blocks at labels and fall-through markers
        starts = [m.start() for m in re.finditer(r"^(?:\.LBB\w+:|; %bb\.\d+:)", body, re.M)] + [len(body)]
        waits = []
        for a, b in zip(starts, starts[1:]):
            block = body[a:b]
            first_line = block.split("\n", 1)[0]
            # the loop's label line is the header; later lines of the label comment name the parents
            head_comment = block[:block.find("\n\t")] if "\n\t" in block else first_line
            if first_line.startswith("." + loop + ":") or ("Header=" + loop_id + " ") in head_comment \
                    or ("Parent Loop " + loop_id + " ") in head_comment:
                waits += [int(x) for x in re.findall(r"s_waitcnt vmcnt\((\d+)\)", block)]
        assert waits, name
        yield name, waits


@pytest.fixture(scope="module")
def ring_waits(tmp_path_factory):
    return dict(_ring_waits(_asm(tmp_path_factory.mktemp("asm"))))


def _device_scheduled(name: str) -> bool:
    # decode_kernel<int KV, int PF, int NT, bool DEV, bool VALU, bool TRACE, bool FUSED>
    return re.search(r"decode_kernelI(?:Li\d+E)+Lb1E", name) is not None


def _valu(name: str) -> bool:
    return re.search(r"decode_kernelI(?:Li\d+E)+Lb[01]ELb1E", name) is not None


def _traced(name: str) -> bool:
    return re.search(r"decode_kernelI(?:Li\d+E)+Lb[01]ELb[01]ELb1E", name) is not None


def _fused(name: str) -> bool:
    return re.search(r"decode_kernelI(?:Li\d+E)+Lb[01]ELb[01]ELb[01]ELb1E", name) is not None


def test_decode_kernels_and_their_traced_twins(ring_waits):
    # bf16 / fp8 x host plan / device schedule x MFMA / VALU tile math, plus
    # the device-scheduled in-kernel-merge variants, each also as the
    # tracing-window instantiation
    plain = [n for n in ring_waits if not _traced(n)]
    assert len(plain) == 12 and len(ring_waits) == 24, list(ring_waits)
    assert sum(_device_scheduled(n) for n in plain) == 8
    assert sum(_valu(n) for n in plain) == 6
    assert sum(_fused(n) for n in plain) == 4 and all(_device_scheduled(n) for n in plain if _fused(n))


def test_device_scheduled_ring_keeps_a_tile_in_flight(ring_waits):
    bad = [(n, w) for n, w in ring_waits.items() if _device_scheduled(n) and min(w) < KV_LOADS_PER_TILE]
    assert not bad, bad


def test_host_planned_ring_keeps_a_tile_in_flight(ring_waits):
    # Two things once made this kernel wait for every load at its loop head:
    # a length read through a pointer that had lost its read-only provenance
    # (a vector load inside the loop), and the prologue issuing slot 0's Q
    # loads last (so the loop-entry path needed all loads done).
    bad = [(n, w) for n, w in ring_waits.items() if not _device_scheduled(n) and min(w) < KV_LOADS_PER_TILE]
    assert not bad, bad
