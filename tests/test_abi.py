"""The C ABI on the CPU: the library loads, exports every entry point that
include/gdn2.h declares, and rejects bad requests on the host before any
HIP call.  No test here launches a kernel; the device pointers below are
never dereferenced (validation only compares addresses)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_decay_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn2.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.library_path()):
        from gated_delta_rule_decay_amd.build import build_library
        build_library()
    return bd.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn2_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(bd.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.gdn2_abi_version() == 6
    for s in range(9):
        assert lib.gdn2_status_str(s) != b"unknown status"
    assert lib.gdn2_status_str(0) == b"ok"
    assert lib.gdn2_status_str(9) == b"unknown status"


def test_desc_layout_matches_header():
    # six int64, five int32, one float, four int32: 88 bytes
    assert ctypes.sizeof(bd.Gdn2Desc) == 88
    assert bd.Gdn2Desc.q_scale.offset == 68
    assert bd.Gdn2Desc.form.offset == 72
    assert bd.Gdn2Desc.gate_logits.offset == 76 and bd.Gdn2Desc.qk_l2norm.offset == 80
    assert bd.Gdn2Desc.o_dtype.offset == 84


def test_desc_layout_as_a_c_compiler_sees_it(tmp_path):
    # the header compiled by the host C compiler: size and every field offset
    # equal to the binding's ctypes structure
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    names = [f[0] for f in bd.Gdn2Desc._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "gdn2.h"\nint main(void) {\n'
                   '    printf("%zu\\n", sizeof(gdn2_desc));\n'
                   + "".join(f'    printf("%zu\\n", offsetof(gdn2_desc, {n}));\n' for n in names)
                   + "    return 0;\n}\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([cc, "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got == [ctypes.sizeof(bd.Gdn2Desc)] + [getattr(bd.Gdn2Desc, n).offset for n in names]


# Fake, well-separated device addresses for the inputs and outputs.
BASE = 1 << 40
SLOT = 1 << 32
Q, K, V, LA, EB, WR, S0, O, SO, WS = (BASE + i * SLOT for i in range(10))


def fwd(lib, desc, q=Q, k=K, v=V, la=LA, eb=EB, wr=WR, s0=S0, o=O, so=SO, ws=None, wsb=0):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gdn2_chunk_fwd(None if desc is None else ctypes.byref(desc), vp(q), vp(k), vp(v),
                              vp(la), vp(eb), vp(wr), vp(s0), vp(o), vp(so), vp(ws), wsb, None)


def step(lib, desc, q=Q, k=K, v=V, la=LA, eb=EB, wr=WR, st=S0, o=O):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gdn2_recurrent_step(None if desc is None else ctypes.byref(desc), vp(q), vp(k),
                                   vp(v), vp(la), vp(eb), vp(wr), vp(st), vp(o), None)


def good(**kw):
    base = dict(batch=2, seqlen=128, heads=4, dk=128, dv=128, chunk=64)
    base.update(kw)
    return bd.make_desc(**base)


def test_null_arguments(lib):
    assert fwd(lib, None) == 1
    assert fwd(lib, good(), q=None) == 1
    assert fwd(lib, good(), o=None) == 1
    assert fwd(lib, good(), la=None) == 1
    assert fwd(lib, good(tied=False), wr=None) == 1
    n = ctypes.c_size_t(0)
    assert lib.gdn2_chunk_fwd_workspace(None, ctypes.byref(n)) == 1
    assert lib.gdn2_chunk_fwd_workspace(ctypes.byref(good()), None) == 1
    assert step(lib, None) == 1
    assert step(lib, good(seqlen=1), st=None) == 1


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), 2), (dict(seqlen=-5), 2), (dict(heads=0), 2), (dict(dk=0), 2),
    (dict(dv=0), 2), (dict(dk=129), 4), (dict(dv=256), 4), (dict(chunk=8), 4),
    (dict(chunk=128), 4), (dict(qkv_dtype=7), 3), (dict(o_dtype=2), 3), (dict(o_dtype=-1), 3),
    (dict(decay_kind=2), 2),
    (dict(erase_kind=-1), 2), (dict(batch=1 << 40, seqlen=1 << 30), 2),
])
def test_bad_descriptors(lib, kw, status):
    assert fwd(lib, good(**kw)) == status


def test_write_kind_ignored_when_tied(lib):
    n = ctypes.c_size_t(99)
    d = good(tied=True, write_kind=9)
    assert lib.gdn2_chunk_fwd_workspace(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value == split_bytes(2, 4, 128)


def test_aliasing(lib):
    d = good()
    assert fwd(lib, d, o=Q + 16) == 5          # o inside q
    assert fwd(lib, d, so=V) == 5              # state_out on v
    assert fwd(lib, d, so=S0 + 64) == 5        # partial overlap with state0
    assert fwd(lib, d, o=SO) == 5              # o on state_out
    assert fwd(lib, d, o=S0 + 4) == 5          # o on state0
    d1 = good(seqlen=1)
    assert step(lib, d1, o=S0 + 8) == 5        # decode output inside the state
    assert step(lib, d1, st=K) == 5            # state on k


def test_bf16_output_span(lib):
    # a bf16 o is half as long as an fp32 one (only error paths are called
    # here: the addresses are not real)
    obytes = 2 * 128 * 4 * 128 * 2   # the bf16 o of good()
    assert fwd(lib, good(), q=O + obytes) == 5             # inside the fp32 o
    assert fwd(lib, good(o_dtype=1), q=O + obytes - 2) == 5  # on the bf16 o's last element
    assert step(lib, good(seqlen=1, o_dtype=3)) == 3
    d1 = good(seqlen=1, o_dtype=1)
    assert step(lib, d1, o=S0 - 2 * 4 * 128 * 2 + 2) == 5     # a bf16 decode output running into the state


def test_empty_calls_touch_nothing(lib):
    # T == 0 with the state updated in place: nothing to enqueue at all
    assert fwd(lib, good(seqlen=0), so=S0) == 0
    assert fwd(lib, good(seqlen=0), so=None) == 0
    assert fwd(lib, good(batch=0), so=None) == 0
    assert step(lib, good(batch=0, seqlen=1)) == 0


def test_decode_needs_one_token(lib):
    assert step(lib, good(seqlen=2)) == 2
    assert step(lib, good(seqlen=0)) == 2


def segments(chains, nc):
    """Segments per chain of the two-level scan: one unless the chains
    cannot fill 256 scan workgroups (two per chain and segment); then as
    many as fill them, each of at least 16 chunks, none empty."""
    if chains * 4 > 256:
        return 1
    n = min(256 // (2 * chains), nc // 16)
    if n < 2:
        return 1
    ln = -(-nc // n)
    return -(-nc // ln)


def split_bytes(B, H, T):
    """Two-pass workspace: per (chain, chunk) a 70 KiB fp16 record and 128
    fp32 chunk-end decays; with several segments per chain, two fp32 states
    per (chain, segment); each region 256-byte aligned."""
    a = lambda x: (x + 255) // 256 * 256
    nc = (T + 63) // 64
    n = B * H * nc
    ns = segments(B * H, nc)
    extra = 2 * a(B * H * ns * 128 * 128 * 4) if ns > 1 else 0
    return a(n * 71680) + a(n * 512) + extra


def test_segment_rule():
    assert segments(128, 64) == 1          # 8 x 16 heads, 4096 tokens: chip already full
    assert segments(16, 1024) == 8         # 1 x 16 heads, 65536 tokens
    assert segments(64, 64) == 2
    assert segments(2, 64) == 4            # capped by 16 chunks per segment
    assert segments(2, 31) == 1
    assert segments(1, 100) == 6           # 17-chunk segments, the last one 15


def query(lib, d):
    n = ctypes.c_size_t(123)
    assert lib.gdn2_chunk_fwd_workspace(ctypes.byref(d), ctypes.byref(n)) == 0
    return n.value


def test_workspace_query(lib):
    # the two-pass path covers bf16, dk = dv = 128, C = 64, gates of one kind or KDA's
    assert query(lib, good()) == split_bytes(2, 4, 128)
    assert query(lib, good(seqlen=100)) == split_bytes(2, 4, 100)
    assert query(lib, good(tied=True, decay_kind=0, erase_kind=0)) == split_bytes(2, 4, 128)
    # KDA's gates: the decay per key channel, the rates one per head
    assert query(lib, good(tied=True, erase_kind=0)) == split_bytes(2, 4, 128)
    assert query(lib, good(erase_kind=0, write_kind=0)) == split_bytes(2, 4, 128)
    assert query(lib, good(erase_kind=0, write_kind=1)) == 0          # rates of two kinds
    # long sequences on few chains add the segment states of the two-level scan
    assert query(lib, good(batch=1, seqlen=4096)) == split_bytes(1, 4, 4096) > split_bytes(1, 4, 64) * 64
    assert query(lib, good(batch=1, heads=16, seqlen=65536)) == split_bytes(1, 16, 65536)
    # everything else runs single-pass and needs none
    for d in (good(qkv_dtype=0, dk=32, dv=32, chunk=16), good(tied=True, decay_kind=0),
              good(dk=64), good(chunk=32), good(seqlen=0), good(batch=0)):
        assert query(lib, d) == 0


def test_workspace_checks(lib):
    d = good()
    need = split_bytes(2, 4, 128)
    assert fwd(lib, d, ws=WS, wsb=need - 1) == 6       # too small
    assert fwd(lib, d, ws=WS + 16, wsb=need) == 6      # not 256-byte aligned
    assert fwd(lib, d, ws=Q, wsb=need) == 5            # on top of q
    assert fwd(lib, d, ws=O - 256, wsb=need) == 5      # runs into o
    assert fwd(lib, d, ws=SO - need + 256, wsb=need) == 5  # runs into state_out


# ---- the backward ---------------------------------------------------------

DO, DST, DQ, DK, DV, DLA, DEB, DWR, DS0, BWS = (BASE + (20 + i) * SLOT for i in range(10))


def bwd(lib, desc, d_o=DO, dst=DST, dq=DQ, dk=DK, dv=DV, dla=DLA, deb=DEB, dwr=DWR, ds0=DS0,
        ws=BWS, wsb=None, q=Q, s0=S0):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    if wsb is None:
        wsb = bwd_bytes(desc) if desc is not None else 0
    return lib.gdn2_chunk_bwd(None if desc is None else ctypes.byref(desc), vp(q), vp(K), vp(V), vp(LA),
                              vp(EB), vp(WR), vp(s0), vp(d_o), vp(dst), vp(dq), vp(dk), vp(dv), vp(dla),
                              vp(deb), vp(dwr), vp(ds0), vp(ws), wsb, None)


def bwd_bytes(desc):
    """Two fp32 state records per (chain, internal chunk): 16 tokens for
    d = 128, 32 for d <= 32 at chunk 64 (whatever fits LDS)."""
    n = ctypes.c_size_t(0)
    assert bd.load_library().gdn2_chunk_bwd_workspace(ctypes.byref(desc), ctypes.byref(n)) == 0
    return n.value


def test_bwd_workspace_query(lib):
    a = lambda x: (x + 255) // 256 * 256
    # d = 128: two state records per 16-token chunk, then a per-chunk record of
    # the scans on the matrix cores (4 x 16x128 operands, 4 x 16x16 Grams/Tm,
    # 128 exit decays, fp32)
    rec = (4 * 16 * 128 + 4 * 16 * 16 + 128) * 4
    assert bwd_bytes(good()) == 2 * a(2 * 4 * (128 // 16) * 128 * 128 * 4) + a(2 * 4 * 8 * rec)
    assert bwd_bytes(good(seqlen=100)) == 2 * a(2 * 4 * 7 * 128 * 128 * 4) + a(2 * 4 * 7 * rec)
    assert bwd_bytes(good(dk=32, dv=32, chunk=64)) == 2 * a(2 * 4 * (128 // 32) * 32 * 32 * 4)
    assert bwd_bytes(good(seqlen=0)) == 0


def test_bwd_checks(lib):
    d = good()
    assert bwd(lib, None) == 1
    assert bwd(lib, d, d_o=None) == 1
    assert bwd(lib, d, dq=None) == 1
    assert bwd(lib, d, dwr=None) == 1
    assert bwd(lib, d, ws=None) == 6
    assert bwd(lib, d, wsb=bwd_bytes(d) - 1) == 6
    assert bwd(lib, d, ws=BWS + 16) == 6
    assert bwd(lib, d, dq=Q) == 5                    # gradient on top of an input
    assert bwd(lib, d, dk=DQ + 64) == 5              # two gradients overlap
    assert bwd(lib, d, ds0=BWS + 4096) == 5          # gradient inside the workspace
    assert bwd(lib, d, dv=DO) == 5                   # gradient on top of d_o
    assert bwd(lib, good(dk=129), wsb=0) == 4
    assert bwd(lib, good(chunk=8), wsb=0) == 4
    # d_o is fp32 whatever o_dtype says (a forward's descriptor reused with a
    # bf16 o): a gradient in the upper half of d_o still overlaps it
    dobytes = 2 * 128 * 4 * 128 * 4
    assert bwd(lib, good(o_dtype=1), dv=DO + dobytes // 2 + 256) == 5


def test_value_write_form_checks(lib):
    vw = dict(form=bd.GDN2_FORM_VALUE_WRITE)
    assert fwd(lib, good(form=2)) == 2                       # unknown form
    assert fwd(lib, good(tied=True, **vw)) == 2              # needs its own write gate
    assert fwd(lib, good(**vw), wr=None) == 1
    # the write gate has dv channels: its span is sized by dv, not dk
    d = good(dk=64, dv=128, **vw)
    wbytes = 2 * 128 * 4 * 128 * 4
    assert fwd(lib, d, wr=O - wbytes + 256) == 5             # runs into o
    # the two-pass kernels cover it, and the backward (same workspace as the key form)
    assert query(lib, good(**vw)) == split_bytes(2, 4, 128)
    assert bwd_bytes(good(**vw)) == bwd_bytes(good())


def test_fused_input_checks(lib):
    # bf16 logits take 2 bytes per gate element
    d = good(gate_logits=True)
    gbytes = 2 * 128 * 4 * 128 * 2
    assert fwd(lib, d, la=O - gbytes + 256) == 5        # a bf16 gate running into o
    assert fwd(lib, good(), la=O - gbytes + 256) == 5   # twice as long as fp32: also overlaps
    # the two-pass kernels cover it; the backward adds an fp32 copy of the
    # prepared inputs: q, k, v and two norms per token-head, the activated gates
    assert query(lib, good(gate_logits=True, qk_l2norm=True)) == split_bytes(2, 4, 128)
    a = lambda x: (x + 255) // 256 * 256
    rows = 2 * 128 * 4
    base = bwd_bytes(good())
    assert bwd_bytes(good(qk_l2norm=True)) == base + 3 * a(rows * 128 * 4) + 2 * a(rows * 4)
    assert bwd_bytes(good(gate_logits=True)) == base + 3 * a(rows * 128 * 4)
    assert bwd_bytes(good(gate_logits=True, tied=True, decay_kind=0, erase_kind=0)) == base + 2 * a(rows * 4)
    # gradients of bf16 logits are fp32: their spans are twice the logits'
    d = good(gate_logits=True)
    assert bwd(lib, d, dla=DO - gbytes - 256) == 5   # an fp32 d_log_decay running into d_o


# ---- packed sequences -----------------------------------------------------

CU = BASE + 40 * SLOT


def fwd_varlen(lib, desc, cu=CU, q=Q, k=K, v=V, la=LA, eb=EB, wr=WR, s0=S0, o=O, so=SO, ws=None, wsb=0):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gdn2_chunk_fwd_varlen(None if desc is None else ctypes.byref(desc), vp(cu), vp(q), vp(k),
                                     vp(v), vp(la), vp(eb), vp(wr), vp(s0), vp(o), vp(so), vp(ws), wsb,
                                     None)


def varlen_bytes(N, H, T):
    """Records and chunk-end decays for ceil(T/64) + N chunks per head (each
    sequence may end in a partial chunk); the plan: N token ranges (int32
    pairs), N+1 chunk prefix counts, one int32 pair per chunk; four N+1
    segment prefix counts; X and F slots for the segments of the sequences
    cut (segments of L chunks, L = max(16, ceil(H ceil(T/64) / 128)), at most
    ceil(T / 64 L) sequences cut), each a fp32 state per head."""
    a = lambda x: (x + 255) // 256 * 256
    ct = (T + 63) // 64
    nc = ct + N
    n = H * nc
    L = max(16, -(-H * ct // 128))
    long_max = -(-T // (64 * L))
    zb = (ct + long_max) // L + 1 + long_max
    return (a(n * 71680) + a(n * 512) + a(N * 8) + a((N + 1) * 4) + a(nc * 8) + 4 * a((N + 1) * 4)
            + 2 * a(zb * H * 128 * 128 * 4))


def query_varlen(lib, d):
    n = ctypes.c_size_t(123)
    assert lib.gdn2_chunk_fwd_varlen_workspace(ctypes.byref(d), ctypes.byref(n)) == 0
    return n.value


def test_varlen_workspace_query(lib):
    # batch = N sequences, seqlen = T packed tokens
    assert query_varlen(lib, good(batch=6, seqlen=430)) == varlen_bytes(6, 4, 430)
    assert query_varlen(lib, good(batch=1, seqlen=65536, heads=16)) == varlen_bytes(1, 16, 65536)
    vw = dict(form=bd.GDN2_FORM_VALUE_WRITE)
    assert query_varlen(lib, good(batch=3, seqlen=100, **vw)) == varlen_bytes(3, 4, 100)
    for d in (good(qkv_dtype=0), good(dk=64), good(chunk=32), good(seqlen=0), good(batch=0),
              good(tied=True, decay_kind=0)):
        assert query_varlen(lib, d) == 0


def test_varlen_checks(lib):
    d = good(batch=3, seqlen=200)
    n = ctypes.c_size_t(0)
    assert lib.gdn2_chunk_fwd_varlen_workspace(None, ctypes.byref(n)) == 1
    assert lib.gdn2_chunk_fwd_varlen_workspace(ctypes.byref(d), None) == 1
    assert fwd_varlen(lib, None) == 1
    assert fwd_varlen(lib, d, cu=None) == 1
    assert fwd_varlen(lib, d, q=None) == 1
    assert fwd_varlen(lib, d, wr=None) == 1
    assert fwd_varlen(lib, good(batch=0), cu=None, q=None) == 0   # no sequence: nothing to do
    assert fwd_varlen(lib, good(batch=3, seqlen=2 ** 31)) == 2    # offsets are int32
    assert fwd_varlen(lib, good(batch=-1)) == 2
    assert fwd_varlen(lib, good(chunk=8)) == 4
    assert fwd_varlen(lib, good(dk=129)) == 4
    # the offsets are an input; states are [N, H, dk, dv]
    assert fwd_varlen(lib, d, o=CU - 256) == 5
    assert fwd_varlen(lib, d, so=CU) == 5
    st = 3 * 4 * 128 * 128 * 4
    assert fwd_varlen(lib, d, so=S0 + st - 256) == 5
    need = varlen_bytes(3, 4, 200)
    assert fwd_varlen(lib, d, ws=WS, wsb=need - 1) == 6
    assert fwd_varlen(lib, d, ws=WS + 16, wsb=need) == 6
    assert fwd_varlen(lib, d, ws=CU - 256, wsb=need) == 5
    assert fwd_varlen(lib, d, ws=O - 256, wsb=need) == 5


def bwd_varlen(lib, desc, cu=CU, ws=BWS, wsb=None, d_o=DO, dq=DQ, ds0=DS0):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    if wsb is None:  # the size the library asks for (0 for a rejected descriptor)
        n = ctypes.c_size_t(0)
        if desc is not None:
            lib.gdn2_chunk_bwd_varlen_workspace(ctypes.byref(desc), ctypes.byref(n))
        wsb = n.value
    return lib.gdn2_chunk_bwd_varlen(None if desc is None else ctypes.byref(desc), vp(cu), vp(Q), vp(K), vp(V),
                                     vp(LA), vp(EB), vp(WR), vp(S0), vp(d_o), vp(DST), vp(dq), vp(DK), vp(DV),
                                     vp(DLA), vp(DEB), vp(DWR), vp(ds0), vp(ws), wsb, None)


def test_bwd_varlen_workspace_and_checks(lib):
    a = lambda x: (x + 255) // 256 * 256
    N, H, T = 3, 4, 200
    nc = (T + 15) // 16 + N  # 16-token chunks per head, bounded
    rec = (4 * 16 * 128 + 4 * 16 * 16 + 128) * 4
    plan = a(N * 8) + a((N + 1) * 4) + a(nc * 8)
    n = ctypes.c_size_t(0)
    d = good(batch=N, seqlen=T)
    assert lib.gdn2_chunk_bwd_varlen_workspace(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value == 2 * a(H * nc * 128 * 128 * 4) + a(H * nc * rec) + plan
    assert lib.gdn2_chunk_bwd_varlen_workspace(None, ctypes.byref(n)) == 1
    assert lib.gdn2_chunk_bwd_varlen_workspace(ctypes.byref(good(batch=3, seqlen=2 ** 31)), ctypes.byref(n)) == 2
    assert bwd_varlen(lib, None) == 1
    assert bwd_varlen(lib, d, cu=None) == 1
    assert bwd_varlen(lib, d, d_o=None) == 1
    assert bwd_varlen(lib, good(batch=0), cu=None) == 0        # no sequence: nothing to do
    assert bwd_varlen(lib, d, ws=None) == 6
    assert bwd_varlen(lib, d, dq=CU - 256) == 5                # a gradient over the offsets
    assert bwd_varlen(lib, d, ds0=S0 + 3 * 4 * 128 * 128 * 4 - 256) == 5  # d_state0 over state0 ([N,H,dk,dv])
    # d_o [T,H,dv] is fp32 whatever o_dtype says
    assert bwd_varlen(lib, good(batch=N, seqlen=T, o_dtype=1), dq=DO + T * H * 128 * 4 - 64) == 5


def fwd_static(lib, desc, q=Q, k=K, v=V, la=LA, eb=EB, wr=WR, s0=S0, o=O, so=SO):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gdn2_chunk_fwd_static(None if desc is None else ctypes.byref(desc), vp(q), vp(k), vp(v), vp(la),
                                     vp(eb), vp(wr), vp(s0), vp(o), vp(so), None)


def test_static_entry_point_checks(lib):
    # the allocation-free forward validates like gdn2_chunk_fwd, before any
    # HIP call (so before it looks up its scratch)
    assert fwd_static(lib, None) == 1
    assert fwd_static(lib, good(), q=None) == 1
    assert fwd_static(lib, good(), wr=None) == 1
    assert fwd_static(lib, good(form=2)) == 2
    assert fwd_static(lib, good(o_dtype=2)) == 3
    assert fwd_static(lib, good(dk=129)) == 4
    assert fwd_static(lib, good(), o=Q + 16) == 5
    assert fwd_static(lib, good(), so=S0 + 64) == 5
    assert fwd_static(lib, good(seqlen=0), so=S0) == 0   # nothing to enqueue
    # the 128 MiB scratch holds 1859 records of 70.5 KiB in one window, or
    # one chunk per chain beside the carried 64 KiB states of up to 974
    # chains; beyond both the check answers before any HIP call
    assert fwd_static(lib, good(batch=1860, heads=1, seqlen=64)) == 8
    assert fwd_static(lib, good(batch=975, heads=1, seqlen=128)) == 8
    assert fwd_static(lib, good(batch=244, heads=4, seqlen=65)) == 8
