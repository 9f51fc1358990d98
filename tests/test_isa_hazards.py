"""The compiled kernels against two hazards the compiler leaves open on gfx950.

1. A store of more than 64 bits (dwordx3/x4) reads its data registers after
it issues; an instruction that writes one of those registers immediately
behind it can change the stored data.  The compiler inserts the wait state
for most forms but not for a buffer store with an SGPR scalar offset, and on
gfx950 that form lost data (two state rows of a pair in about one decode
launch of three).  No such store may be followed directly by a vector-ALU
(or matrix) instruction writing one of its data registers.

2. A matrix instruction that takes as its accumulator the result of a matrix
instruction of another form (a 16x16x16 step reading a 16x16x32 step's
result) gets no wait states from the compiler, and then reads the
accumulator from before the first step (measured: the chunk kernel's split
products lost their cross terms).  No such pair may stand closer than
MIXED_MFMA_WAIT_STATES wait states (counting each instruction between as one
and s_nop N as N + 1).

3. v_dot2c_f32_bf16 (and its other encodings) with a constant operand: the
compiler encodes the bf16 pair (-1, 0) as the inline constant -1.0, which the
instruction reads as the fp32 pattern, i.e. the pair (0, -1) (measured: half
of the values of x - bf16(x) came out wrong).  The kernels pass such pairs in
registers the compiler cannot see through; no dot2 may take an immediate.

The test compiles every kernel source for gfx950 with the library's own
flags.  Host-side only: it needs hipcc, not a GPU.
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from linear_attention_recurrence_token_amd import _build

STORE = re.compile(r'^(buffer_store_dwordx[34]|global_store_dwordx[34]|flat_store_dwordx[34])\s+(.*)$')
WRITE = re.compile(r'^(v_\S+)\s+(v\[\d+:\d+\]|v\d+)')
WAIT_STATES = 2    # what the compiler inserts for this hazard on gfx940-class chips
WIDE_SGPR_SOFFSET = re.compile(r'^buffer_store_dwordx[34]\s+\S+,\s*\S+,\s*s\[\d+:\d+\],\s*s\d+\b')
MFMA = re.compile(r'^(v_mfma_\w+)\s+(v\[\d+:\d+\]|a\[\d+:\d+\]),\s*[^,]+,\s*[^,]+,\s*(\S+)')
MIXED_MFMA_WAIT_STATES = 16
# a bf16 dot2 whose first source is an inline constant or a literal
DOT2_IMMEDIATE = re.compile(r'^v_dot2c?_f32_bf16\S*\s+v\d+,\s*(-?\d|0x|-?\d*\.\d)')


def _regs(spec):
    m = re.match(r'v\[(\d+):(\d+)\]$', spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r'v(\d+)$', spec)
    return {int(m.group(1))} if m else set()


def hazards(asm_text):
    """(function, store, next instruction) for each exposed wide store."""
    out = []
    func = None
    lines = [l.strip() for l in asm_text.splitlines()]
    code = [(i, l) for i, l in enumerate(lines) if l and not l.startswith((';', '.', '//'))]
    for k, (i, l) in enumerate(code):
        if re.match(r'^_Z\S*:', l) or re.match(r'^\w+:$', l) and not l.startswith('.'):
            if l.startswith('_Z'):
                func = l.split(':')[0]
            continue
        m = STORE.match(l)
        if not m:
            continue
        ops = [o.strip() for o in m.group(2).split(',')]
        # buffer stores: vdata first; global / flat stores: vaddr, vdata
        data = ops[0] if m.group(1).startswith('buffer') else ops[1]
        dregs = _regs(data)
        # the instructions within WAIT_STATES wait states of the store (one
        # per instruction, N + 1 for s_nop N) must not write its data
        waited = 0
        for _, nxt in code[k + 1:]:
            if waited >= WAIT_STATES or nxt.endswith(':') or nxt.startswith(('s_endpgm', 's_branch', 's_cbranch')):
                break
            w = WRITE.match(nxt)
            if w and not w.group(1).startswith(('v_cmp', 'v_readfirstlane', 'v_readlane')) and _regs(w.group(2)) & dregs:
                out.append((func, l, nxt))
                break
            m_nop = re.match(r'^s_nop\s+(\d+)', nxt)
            waited += int(m_nop.group(1)) + 1 if m_nop else 1
    return out


def _span(spec):
    m = re.match(r'[va]\[(\d+):(\d+)\]$', spec)
    return set(range(int(m.group(1)), int(m.group(2)) + 1)) if m else set()


def mixed_mfma_chains(asm_text):
    """(function, first, second) for each matrix instruction that takes as its
    accumulator, within MIXED_MFMA_WAIT_STATES wait states, the result of the
    matrix instruction of another form issued before it (tracked inside a
    basic block)."""
    out = []
    func = None
    prev = None          # (opcode, destination registers, line, wait states since)
    for raw in asm_text.splitlines():
        l = raw.strip()
        if not l or l.startswith((';', '//')):
            continue
        lab = re.match(r'^([\w.$]+):', l)
        if lab:
            if lab.group(1).startswith('_Z'):
                func = lab.group(1)
            prev = None
            continue
        if l.startswith('.'):
            continue
        m = MFMA.match(l)
        if m:
            if prev is not None and prev[0] != m.group(1) and prev[3] < MIXED_MFMA_WAIT_STATES \
                    and _span(m.group(3)) & prev[1]:
                out.append((func, prev[2], l))
            prev = (m.group(1), _span(m.group(2)), l, 0)
            continue
        if prev is not None:
            m_nop = re.match(r'^s_nop\s+(\d+)', l)
            prev = prev[:3] + (prev[3] + (int(m_nop.group(1)) + 1 if m_nop else 1),)
    return out


def test_mfma_scanner_finds_the_pattern():
    bad = ("_Zk:\n\tv_mfma_f32_16x16x32_bf16 v[28:31], v[22:25], v[26:29], 0\n"
           "\tv_mfma_f32_16x16x16_bf16 v[24:27], v[24:25], v[26:27], v[28:31]\n")
    spaced = ("_Zk:\n\tv_mfma_f32_16x16x32_bf16 v[28:31], v[22:25], v[26:29], 0\n"
              "\ts_nop 7\n\ts_nop 7\n\tv_mfma_f32_16x16x16_bf16 v[24:27], v[24:25], v[26:27], v[28:31]\n")
    same = ("_Zk:\n\tv_mfma_f32_16x16x32_bf16 v[28:31], v[22:25], v[26:29], 0\n"
            "\tv_mfma_f32_16x16x32_bf16 v[28:31], v[22:25], v[26:29], v[28:31]\n")
    other = ("_Zk:\n\tv_mfma_f32_16x16x32_bf16 v[28:31], v[22:25], v[26:29], 0\n"
             "\tv_mfma_f32_16x16x16_bf16 v[24:27], v[24:25], v[26:27], v[8:11]\n")
    assert len(mixed_mfma_chains(bad)) == 1
    assert mixed_mfma_chains(spaced) == [] and mixed_mfma_chains(same) == [] and mixed_mfma_chains(other) == []


def test_dot2_scanner_finds_the_pattern():
    assert DOT2_IMMEDIATE.match("v_dot2c_f32_bf16_e32 v0, -1.0, v3")
    assert DOT2_IMMEDIATE.match("v_dot2c_f32_bf16_e32 v1, 0xbf800000, v3")
    assert not DOT2_IMMEDIATE.match("v_dot2c_f32_bf16_e32 v93, s33, v95")
    assert not DOT2_IMMEDIATE.match("v_dot2c_f32_bf16_e32 v93, v12, v95")


def test_scanner_finds_the_pattern():
    bad = "_Zk:\n\tbuffer_store_dwordx4 v[2:5], v6, s[4:7], s0 offen nt\n\tv_add_f32_e32 v2, v70, v74\n"
    good = "_Zk:\n\tbuffer_store_dwordx4 v[2:5], v6, s[4:7], 0 offen nt\n\ts_nop 1\n\tv_add_f32_e32 v2, v70, v74\n"
    near = "_Zk:\n\tbuffer_store_dwordx4 v[2:5], v6, s[4:7], s0 offen\n\tv_mov_b32 v9, 0\n\tv_add_f32_e32 v3, v70, v74\n"
    assert len(hazards(near)) == 1
    assert WIDE_SGPR_SOFFSET.match("buffer_store_dwordx4 v[2:5], v86, s[4:7], s0 offen nt")
    assert not WIDE_SGPR_SOFFSET.match("buffer_store_dwordx4 v[2:5], v86, s[4:7], 0 offen nt")
    other = "_Zk:\n\tglobal_store_dwordx4 v[2:3], v[6:9], off\n\tv_add_co_u32_e32 v2, vcc, 16, v2\n"
    assert len(hazards(bad)) == 1
    assert hazards(good) == [] and hazards(other) == []


@pytest.fixture(scope="module")
def kernel_asm():
    """(source, gfx950 assembly) of every kernel source, built with the library's flags."""
    hipcc = _build.hipcc()
    tmp = tempfile.mkdtemp(prefix="kda_isa_")

    def asm(src):
        out = os.path.join(tmp, src + ".s")
        cmd = [hipcc, "--offload-arch=" + _build.ARCH, "-O3", "-std=c++17", "-w",
               "-I", os.path.join(_build.ROOT, "include")] + _build.DEVICE_FLAGS + \
              ["--offload-device-only", "-S", "-o", out, os.path.join(_build.CSRC, src)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        with open(out) as fh:
            return src, fh.read()

    try:
        with ThreadPoolExecutor(max_workers=min(8, len(_build.SOURCES))) as ex:
            return list(ex.map(asm, [s for s in _build.SOURCES if s != "kda_api.hip"]))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


NEEDS_HIPCC = pytest.mark.skipif(not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")),
                                 reason="needs hipcc")


@NEEDS_HIPCC
def test_no_mixed_form_mfma_accumulator_chain(kernel_asm):
    found = [(src,) + h for src, text in kernel_asm for h in mixed_mfma_chains(text)]
    assert not found, "\n".join("%s %s: %s -> %s" % f for f in found[:10])


@NEEDS_HIPCC
def test_no_wide_store_followed_by_a_write_to_its_data(kernel_asm):
    texts = kernel_asm
    found = [(src,) + h for src, text in texts for h in hazards(text)]
    assert not found, "\n".join("%s %s: %s -> %s" % f for f in found[:10])
    # and no wide buffer store takes an SGPR scalar offset, the form the
    # compiler does not guard at all
    sgpr = [(src, l.strip()) for src, text in texts for l in text.splitlines()
            if WIDE_SGPR_SOFFSET.match(l.strip())]
    assert not sgpr, "\n".join("%s: %s" % f for f in sgpr[:10])


@NEEDS_HIPCC
def test_no_bf16_dot2_with_an_immediate(kernel_asm):
    found = [(src, l.strip()) for src, text in kernel_asm for l in text.splitlines()
             if DOT2_IMMEDIATE.match(l.strip())]
    assert not found, "\n".join("%s: %s" % f for f in found[:10])
    # and the kernels that split with it do use it (the check is not vacuous)
    assert any(l.strip().startswith("v_dot2c_f32_bf16") for _, text in kernel_asm for l in text.splitlines())
