"""Properties of the compiled gfx950 code of the hot kernels (CPU only: hipcc emits the
assembly, nothing runs).

The kernels move their K and V tiles into LDS by DMA and read fragments of the other
buffer while the DMA is in flight.  The compiler waits for every outstanding load
(`s_waitcnt vmcnt`) before any LDS read it cannot tell apart from a pending DMA target,
which turns the double buffering into a full memory round trip per tile; each buffer
therefore lives in an LDS array of its own.  These tests hold that property: no
fragment read (`ds_read_b128`, `ds_read_b64_tr_b16`, `ds_read_b64_tr_b8`) follows a
vmcnt wait directly, and no kernel uses scratch memory.
"""

import os
import re
import subprocess

import pytest

from exact_attention_89_amd import build as B

KERNELS = {
    "attn_fwd_bf16_pp.hip": "attn_fwd_bf16_pp_kernel",
    "attn_fwd_bf16_4w.hip": "attn_fwd_bf16_4w_kernel",
    "attn_fwd_fp8.hip": "attn_fwd_fp8_kernel",
}
READ = re.compile(r"^\s*ds_read_(b128|b64_tr_b16|b64_tr_b8)\b")
VMWAIT = re.compile(r"^\s*s_waitcnt\b.*\bvmcnt\(")


def _asm(src, tmp_path):
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src),
           "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().splitlines()


def _functions(lines, name):
    """Instruction lists of every kernel whose symbol contains `name`."""
    funcs, cur = {}, None
    for ln in lines:
        m = re.match(r"^(_Z\S+):\s*(;.*)?$", ln)
        if m:
            cur = m.group(1) if name in m.group(1) else None
            if cur:
                funcs[cur] = []
            continue
        if cur is None:
            continue
        s = ln.strip()
        if not s or s.startswith(";") or s.startswith("."):
            continue
        funcs[cur].append(s)
        if s.startswith("s_endpgm"):
            cur = None
    return funcs


@pytest.mark.parametrize("src", sorted(KERNELS))
def test_no_fragment_read_waits_for_outstanding_loads(src, tmp_path):
    funcs = _functions(_asm(src, tmp_path), KERNELS[src])
    assert funcs, f"no {KERNELS[src]} in {src}"
    bad = []
    for fn, ins in funcs.items():
        reads = sum(1 for s in ins if READ.match(s))
        assert reads > 0, f"{fn}: no fragment reads found"
        for a, b in zip(ins, ins[1:]):
            if VMWAIT.match(a) and READ.match(b):
                bad.append(f"{fn}: {a} ; {b}")
    assert not bad, "fragment reads behind a vmcnt wait:\n" + "\n".join(bad[:10])


@pytest.mark.parametrize("src", sorted(KERNELS))
def test_no_scratch(src, tmp_path):
    lines = _asm(src, tmp_path)
    sizes = [int(m.group(1)) for ln in lines
             for m in [re.search(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", ln)] if m]
    assert sizes and all(s == 0 for s in sizes), sizes
