"""The C-ABI library on the host: it loads, exports what include/gdn.h declares,
its struct layout matches, and every argument error is reported before any work
is enqueued (no GPU is touched by these tests)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def lib():
    from invariant_linear_attention_amd import gdn
    if not os.path.exists(gdn.LIBRARY):
        pytest.fail("libgdn.so is not built; run __graft_entry__.build()")
    return gdn.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdn_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == {"gdn_fwd_varlen", "gdn_fwd_varlen_train", "gdn_fwd_varlen_pool", "gdn_decode_step", "gdn_short_conv",
                          "gdn_query_plan", "gdn_bwd_workspace_size", "gdn_bwd_varlen", "gdn_bwd_varlen_noalloc",
                          "gdn_fwd_chunked", "gdn_chunked_workspace_size", "gdn_bwd_chunked_workspace_size",
                          "gdn_bwd_chunked", "gdn_preprocess", "gdn_preprocess_backward",
                          "gdn_short_conv_backward_workspace_size", "gdn_short_conv_backward", "gdn_status_string",
                          "gdn_abi_version"}
    for name in names:
        assert hasattr(lib, name), name


def test_abi_version(lib):
    text = open(HEADER).read()
    want = int(re.search(r"#define GDN_ABI_VERSION (\d+)", text).group(1))
    assert lib.gdn_abi_version() == want


def test_status_strings(lib):
    from invariant_linear_attention_amd import gdn
    for code, name in gdn.STATUS.items():
        assert gdn.status_string(code).startswith(name)


def test_struct_layout_matches_c(tmp_path):
    from invariant_linear_attention_amd.gdn import GdnDims
    src = tmp_path / "layout.c"
    fields = [f[0] for f in GdnDims._fields_]
    body = "".join('printf("%s %%zu\\n", offsetof(gdn_dims, %s));' % (f, f) for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "gdn.h"\n'
                   'int main(void){printf("size %%zu\\n", sizeof(gdn_dims));%s return 0;}\n' % body)
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.check_output([str(exe)]).decode().splitlines())
    assert int(out["size"]) == ctypes.sizeof(GdnDims)
    for f in fields:
        assert int(out[f]) == getattr(GdnDims, f).offset, f


# ------------------------------------------------------ argument errors (host)

def _dims(**kw):
    from invariant_linear_attention_amd.gdn import GdnDims
    d = dict(n_seqs=2, hk=2, hv=4, dk=128, dv=128, io_dtype=1, total_tokens=10, pool_size=0,
             plan_lanes=0, plan_rows=0, plan_waves=0, reserved=0)
    d.update(kw)
    return GdnDims(**d)


# Fake, well-separated, aligned addresses: the checks below fail before any launch.
BASE = 0x7F0000000000
MB = 1 << 24
P = {name: BASE + i * MB for i, name in enumerate(["q", "k", "v", "g", "b", "h0", "cu", "out", "hT",
                                                   "src", "dst", "pos0", "snap"])}


def call_fwd(lib, dims, **over):
    a = dict(P)
    a.update(over)
    return lib.gdn_fwd_varlen(ctypes.byref(dims) if dims is not None else None, a["q"], a["k"], a["v"], a["g"],
                              a["b"], a["h0"], a["cu"], a["out"], a["hT"], None)


def call_dec(lib, dims, **over):
    a = dict(P)
    a.update(over)
    return lib.gdn_decode_step(ctypes.byref(dims) if dims is not None else None, a["q"], a["k"], a["v"], a["g"],
                               a["b"], a.get("pool", a["h0"]), a.get("idx", a["cu"]), a["out"], None)


@pytest.mark.parametrize("case,code", [
    (dict(dims=None), 1),
    (dict(reserved=1), 2),
    (dict(n_seqs=-1), 2),
    (dict(total_tokens=-5), 2),
    (dict(hk=3), 2),
    (dict(dv=24), 2),
    (dict(io_dtype=7), 3),
    (dict(dk=48), 6),
    (dict(dk=256), 6),
    (dict(plan_rows=3, plan_waves=1), 6),
    (dict(plan_lanes=4, plan_rows=2, plan_waves=8), 6),
    (dict(plan_lanes=4, plan_rows=4, plan_waves=4), 6),
    (dict(plan_lanes=2), 6),
    (dict(plan_lanes=16, plan_rows=3), 6),
    (dict(plan_lanes=16, plan_rows=1, plan_waves=1), 6),
    (dict(dk=32, plan_lanes=8), 6),
    (dict(n_seqs=0, total_tokens=3), 2),
])
def test_fwd_rejects_bad_dims(lib, case, code):
    if case.get("dims", 0) is None:
        assert call_fwd(lib, None) == code
    else:
        assert call_fwd(lib, _dims(**case)) == code


def test_fwd_zero_sequences_is_a_noop(lib):
    assert call_fwd(lib, _dims(n_seqs=0, total_tokens=0)) == 0


@pytest.mark.parametrize("ptr", ["q", "k", "v", "g", "b", "cu", "out"])
def test_fwd_rejects_null(lib, ptr):
    assert call_fwd(lib, _dims(), **{ptr: None}) == 1


@pytest.mark.parametrize("ptr,off", [("q", 8), ("v", 4), ("out", 2), ("h0", 8), ("hT", 12), ("g", 2), ("cu", 1)])
def test_fwd_rejects_misaligned(lib, ptr, off):
    assert call_fwd(lib, _dims(), **{ptr: P[ptr] + off}) == 4


@pytest.mark.parametrize("over", [
    dict(out=P["q"]), dict(out=P["v"] + 256), dict(out=P["hT"]), dict(out=P["h0"]),
    dict(hT=P["k"]), dict(hT=P["h0"] + 4096),
])
def test_fwd_rejects_aliasing(lib, over):
    assert call_fwd(lib, _dims(), **over) == 5


@pytest.mark.parametrize("case,over,code", [
    (dict(total_tokens=3), {}, 2),              # decode needs T == B
    (dict(pool_size=-1, total_tokens=2), {}, 2),
    (dict(total_tokens=2, pool_size=4), dict(pool=None), 1),
    (dict(total_tokens=2, pool_size=4), dict(q=None), 1),
    (dict(total_tokens=2, pool_size=1), dict(idx=None), 2),  # identity map needs B entries
    (dict(total_tokens=2, pool_size=4), dict(out=P["q"]), 5),
    (dict(total_tokens=2, pool_size=4), dict(pool=P["v"]), 5),
    (dict(total_tokens=2, pool_size=4), dict(idx=P["cu"] + 2), 4),
    (dict(total_tokens=2, pool_size=4, dk=40), {}, 6),
])
def test_decode_rejects(lib, case, over, code):
    assert call_dec(lib, _dims(**case), **over) == code


def call_pool(lib, dims, snap_block=0, snap_per_seq=0, **over):
    a = dict(P)
    a.update(over)
    return lib.gdn_fwd_varlen_pool(ctypes.byref(dims) if dims is not None else None, a["q"], a["k"], a["v"],
                                   a["g"], a["b"], a["cu"], a.get("pool", a["h0"]), a["src"], a["dst"], a["pos0"],
                                   a["snap"], snap_block, snap_per_seq, a["out"], None)


@pytest.mark.parametrize("case,kw,code", [
    (dict(pool_size=0), {}, 2),                                       # a pool has slots
    (dict(pool_size=4), dict(snap_block=-16, snap_per_seq=1), 2),
    (dict(pool_size=4), dict(snap_block=24, snap_per_seq=1), 2),      # not a multiple of 16
    (dict(pool_size=4), dict(snap_block=32, snap_per_seq=0), 2),      # snapshots need slots
    (dict(pool_size=4), dict(snap_per_seq=-1), 2),
    (dict(pool_size=4), dict(snap_block=32, snap_per_seq=2, snap=None), 1),
    (dict(pool_size=4), dict(pool=None), 1),
    (dict(pool_size=4), dict(cu=None), 1),
    (dict(pool_size=4), dict(q=None), 1),
    (dict(pool_size=1), dict(src=None), 2),                          # identity slots need P >= N
    (dict(pool_size=1), dict(dst=None), 2),
    (dict(pool_size=4), dict(pool=P["h0"] + 8), 4),
    (dict(pool_size=4), dict(src=P["src"] + 2), 4),
    (dict(pool_size=4), dict(snap=P["snap"] + 1, snap_block=16, snap_per_seq=1), 4),
    (dict(pool_size=4), dict(out=P["h0"]), 5),                       # out overlaps the pool
    (dict(pool_size=4), dict(pool=P["v"]), 5),                       # pool overlaps an input
    (dict(pool_size=4), dict(out=P["pos0"]), 5),
    (dict(pool_size=4, dk=40), {}, 6),
    (dict(pool_size=4, plan_lanes=16, plan_rows=3), {}, 6),
    (dict(pool_size=4, n_seqs=0, total_tokens=3), {}, 2),
])
def test_pool_rejects(lib, case, kw, code):
    kw = dict(kw)
    sb, sp = kw.pop("snap_block", 0), kw.pop("snap_per_seq", 0)
    assert call_pool(lib, _dims(**case), snap_block=sb, snap_per_seq=sp, **kw) == code


def test_pool_null_dims(lib):
    assert call_pool(lib, None) == 1


def test_pool_zero_sequences_is_a_noop(lib):
    assert call_pool(lib, _dims(n_seqs=0, total_tokens=0, pool_size=4)) == 0


def test_decode_zero_batch_is_a_noop(lib):
    assert call_dec(lib, _dims(n_seqs=0, total_tokens=0, pool_size=4)) == 0


# ------------------------------------------------------------- launch planning

def _plan(decode=False, **kw):
    from invariant_linear_attention_amd import gdn
    return gdn.gdn_query_plan(_dims(**kw), decode)


def test_plan_benchmark_batch():
    # 8 sequences x 32 value heads x 128 rows: enough rows for 8 lanes x 1 row, 4 waves
    assert _plan(n_seqs=8, hk=16, hv=32, total_tokens=17459) == (8, 1, 4)


def test_plan_single_long_sequence():
    # one sequence, 32 heads: rows are scarce, 16 lanes per row spread them widest
    assert _plan(n_seqs=1, hk=16, hv=32, total_tokens=65536) == (16, 1, 4)


@pytest.mark.parametrize("B", [1, 8, 64, 256])
def test_plan_decode(B):
    assert _plan(decode=True, n_seqs=B, hk=16, hv=32, total_tokens=B, pool_size=B) == (4, 1, 1)


@pytest.mark.parametrize("dk,lanes", [(16, 4), (32, 4), (64, 8)])
def test_plan_smaller_heads(dk, lanes):
    # a lane holds at least 4 columns (dk = 16, 32: 4 lanes per row; dk = 64: 8)
    got = _plan(n_seqs=8, dk=dk, dv=64, total_tokens=100)
    assert got[0] == lanes and (64 // got[0]) * got[1] * got[2] <= 64


def test_plan_pinned_fields_are_kept():
    assert _plan(plan_lanes=16, plan_rows=2, plan_waves=8) == (16, 2, 8)
    assert _plan(plan_lanes=4)[0] == 4
    lanes, rows, waves = _plan(plan_waves=2)
    assert waves == 2
    assert _plan(decode=True, plan_rows=2, total_tokens=2, pool_size=2)[:2] == (4, 2)


def test_plan_rejects_like_the_entry_points():
    from invariant_linear_attention_amd import gdn
    with pytest.raises(gdn.GdnError) as e:
        _plan(plan_lanes=16, plan_rows=3)
    assert e.value.code == 6
    with pytest.raises(gdn.GdnError) as e:
        _plan(dk=48)
    assert e.value.code == 6
    with pytest.raises(gdn.GdnError) as e:
        _plan(reserved=1)
    assert e.value.code == 2


def test_plan_null_shape(lib):
    assert lib.gdn_query_plan(ctypes.byref(_dims()), 0, None) == 1


# ------------------------------------------------------ fused preprocessing

def test_preproc_layout_matches_c(tmp_path):
    from invariant_linear_attention_amd.gdn import GdnPreproc
    src = tmp_path / "pre.c"
    fields = [f[0] for f in GdnPreproc._fields_]
    body = "".join('printf("%s %%zu\\n", offsetof(gdn_preproc, %s));' % (f, f) for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "gdn.h"\n'
                   'int main(void){printf("size %%zu\\n", sizeof(gdn_preproc));%s return 0;}\n' % body)
    exe = tmp_path / "pre"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.check_output([str(exe)]).decode().splitlines())
    assert int(out["size"]) == ctypes.sizeof(GdnPreproc)
    for f in fields:
        assert int(out[f]) == getattr(GdnPreproc, f).offset, f


def _pre_dims(flags=3, eps=1e-6, A_log=BASE + 40 * MB, dt_bias=BASE + 41 * MB, **kw):
    from invariant_linear_attention_amd.gdn import GdnPreproc
    pre = GdnPreproc(flags=flags, eps=eps, A_log=A_log, dt_bias=dt_bias)
    d = _dims(**kw)
    d.pre = ctypes.pointer(pre)
    d._keep = pre
    return d


@pytest.mark.parametrize("kw,code", [
    (dict(flags=4), 6),                        # unknown flag
    (dict(flags=-1), 6),
    (dict(eps=-1.0), 2),
    (dict(eps=float("nan")), 2),
    (dict(eps=float("inf")), 2),
    (dict(A_log=None), 1),                     # the gate needs A_log
    (dict(A_log=BASE + 40 * MB + 2), 4),
    (dict(dt_bias=BASE + 41 * MB + 1), 4),
])
def test_preproc_rejected_everywhere(lib, kw, code):
    assert call_fwd(lib, _pre_dims(**kw)) == code
    assert call_dec(lib, _pre_dims(total_tokens=2, pool_size=4, **kw)) == code
    assert call_pool(lib, _pre_dims(pool_size=4, **kw)) == code
    from invariant_linear_attention_amd import gdn
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_query_plan(_pre_dims(**kw))
    assert e.value.code == code


def test_preproc_norm_only_needs_no_gate_arrays(lib):
    # flags = norm only: A_log NULL is fine; nothing launches because hk = 3 is bad
    assert call_fwd(lib, _pre_dims(flags=1, A_log=None, dt_bias=None, hk=3)) == 2
    from invariant_linear_attention_amd import gdn
    lanes, rows, waves = gdn.gdn_query_plan(_pre_dims(flags=1, A_log=None, dt_bias=None))
    assert lanes in (4, 8, 16) and rows in (1, 2, 4) and waves in (1, 2, 4, 8)


@pytest.mark.parametrize("over", [dict(out=BASE + 40 * MB), dict(hT=BASE + 41 * MB)])
def test_preproc_outputs_may_not_overlap_gate_arrays(lib, over):
    assert call_fwd(lib, _pre_dims(), **over) == 5


def test_preproc_pool_and_decode_alias(lib):
    assert call_pool(lib, _pre_dims(pool_size=4), out=BASE + 40 * MB) == 5
    assert call_pool(lib, _pre_dims(pool_size=4), pool=BASE + 41 * MB) == 5
    assert call_dec(lib, _pre_dims(total_tokens=2, pool_size=4), out=BASE + 41 * MB) == 5
    assert call_dec(lib, _pre_dims(total_tokens=2, pool_size=4), pool=BASE + 40 * MB) == 5



# ------------------------------------------------------------- short conv

def test_conv_dims_layout_matches_c(tmp_path):
    from invariant_linear_attention_amd.gdn import GdnConvDims
    src = tmp_path / "conv.c"
    fields = [f[0] for f in GdnConvDims._fields_]
    body = "".join('printf("%s %%zu\\n", offsetof(gdn_conv_dims, %s));' % (f, f) for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "gdn.h"\n'
                   'int main(void){printf("size %%zu\\n", sizeof(gdn_conv_dims));%s return 0;}\n' % body)
    exe = tmp_path / "conv"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.check_output([str(exe)]).decode().splitlines())
    assert int(out["size"]) == ctypes.sizeof(GdnConvDims)
    for f in fields:
        assert int(out[f]) == getattr(GdnConvDims, f).offset, f


def _cdims(**kw):
    from invariant_linear_attention_amd.gdn import GdnConvDims
    d = dict(n_seqs=2, channels=64, taps=4, io_dtype=1, total_tokens=10, pool_size=4, flags=1)
    d.update(kw)
    return GdnConvDims(**d)


CP = {name: BASE + (20 + i) * MB for i, name in enumerate(["x", "w", "b", "cu", "pool", "src", "dst", "y"])}


def call_conv(lib, dims, **over):
    a = dict(CP)
    a.update(over)
    return lib.gdn_short_conv(ctypes.byref(dims) if dims is not None else None, a["x"], a["w"], a["b"], a["cu"],
                              a["pool"], a["src"], a["dst"], a["y"], None)


@pytest.mark.parametrize("case,over,code", [
    (dict(taps=1), {}, 2), (dict(taps=9), {}, 2), (dict(channels=0), {}, 2), (dict(pool_size=0), {}, 2),
    (dict(n_seqs=-1), {}, 2), (dict(total_tokens=-1), {}, 2), (dict(flags=2), {}, 6), (dict(io_dtype=5), {}, 3),
    (dict(n_seqs=0, total_tokens=4), {}, 2),
    ({}, dict(cu=None), 1), ({}, dict(w=None), 1), ({}, dict(pool=None), 1), ({}, dict(x=None), 1),
    ({}, dict(y=None), 1),
    (dict(pool_size=1), dict(src=None), 2),
    ({}, dict(x=CP["x"] + 2), 4), ({}, dict(w=CP["w"] + 2), 4), ({}, dict(pool=CP["pool"] + 8), 4),
    (dict(io_dtype=0), dict(y=CP["y"] + 8), 4), (dict(channels=60), {}, 2), (dict(io_dtype=0, channels=62), {}, 2),
    ({}, dict(y=CP["x"]), 5), ({}, dict(y=CP["pool"]), 5), ({}, dict(pool=CP["w"]), 5),
    ({}, dict(pool=CP["x"] + 16), 5),
])
def test_conv_rejects(lib, case, over, code):
    assert call_conv(lib, _cdims(**case), **over) == code


def test_conv_null_dims_and_noop(lib):
    assert call_conv(lib, None) == 1
    assert call_conv(lib, _cdims(n_seqs=0, total_tokens=0)) == 0


# ------------------------------------------------------------------ backward

BP = {name: BASE + (40 + i) * MB for i, name in enumerate(
    ["q", "k", "v", "g", "b", "h0", "cu", "dout", "dhT", "dq", "dk", "dv", "dg", "db", "dh0", "ws", "sp", "hT"])}


def ws_size(lib, dims):
    n = ctypes.c_uint64(0)
    assert lib.gdn_bwd_workspace_size(ctypes.byref(dims), ctypes.byref(n)) == 0
    return int(n.value)


def call_bwd(lib, dims, ws_bytes=None, **over):
    a = dict(BP)
    a.update(over)
    if ws_bytes is None:
        ws_bytes = ws_size(lib, dims) if dims is not None else 0
    return lib.gdn_bwd_varlen(ctypes.byref(dims) if dims is not None else None, a["q"], a["k"], a["v"], a["g"],
                              a["b"], a["h0"], a["cu"], a["dout"], a["dhT"], a.get("sp"), a.get("hT"), a["dq"],
                              a["dk"], a["dv"], a["dg"], a["db"], a["dh0"], a["ws"], ctypes.c_uint64(ws_bytes), None)


def test_bwd_workspace_size(lib):
    """p, du (T hv dv), dk, dq (T hv dk), the gate term (T hv) and a final state
    per (sequence, head), each rounded up to 256 bytes."""
    up = lambda x: (x + 255) // 256 * 256
    T, N, hv, dk, dv = 10, 2, 4, 128, 64
    want = 2 * up(T * hv * dv * 4) + 2 * up(T * hv * dk * 4) + up(T * hv * 4) + up(N * hv * dv * dk * 4)
    assert ws_size(lib, _dims(dv=dv)) == want
    n = ctypes.c_uint64(0)
    assert lib.gdn_bwd_workspace_size(None, ctypes.byref(n)) == 1
    assert lib.gdn_bwd_workspace_size(ctypes.byref(_dims()), None) == 1
    assert lib.gdn_bwd_workspace_size(ctypes.byref(_dims(hv=3)), ctypes.byref(n)) == 2


@pytest.mark.parametrize("case,over,code", [
    (dict(dk=16), {}, 6), (dict(dv=16), {}, 6), (dict(dv=96), {}, 6), (dict(plan_lanes=8), {}, 6),
    (dict(hv=3), {}, 2), (dict(io_dtype=7), {}, 3), (dict(n_seqs=0, total_tokens=3), {}, 2),
    ({}, dict(cu=None), 1), ({}, dict(ws=None), 1), ({}, dict(q=None), 1), ({}, dict(dout=None), 1),
    ({}, dict(dq=None), 1), ({}, dict(dg=None), 1), ({}, dict(db=None), 1), ({}, dict(dv=None), 1),
    ({}, dict(q=BP["q"] + 8), 4), ({}, dict(dout=BP["dout"] + 8), 4), ({}, dict(ws=BP["ws"] + 4), 4),
    ({}, dict(dq=BP["dq"] + 4), 4), ({}, dict(g=BP["g"] + 2), 4),
    ({}, dict(dq=BP["q"]), 5), ({}, dict(dk=BP["dq"]), 5), ({}, dict(ws=BP["dout"]), 5),
    ({}, dict(dh0=BP["h0"]), 5), ({}, dict(dv=BP["ws"] + 256), 5), ({}, dict(dg=BP["db"]), 5),
    ({}, dict(hT=None), 1), ({}, dict(sp=BP["sp"] + 4), 4), ({}, dict(dq=BP["sp"]), 5), ({}, dict(ws=BP["hT"]), 5),
])
def test_bwd_rejects(lib, case, over, code):
    assert call_bwd(lib, _dims(**case), ws_bytes=(1 << 30), **over) == code


def test_bwd_small_workspace_and_noop(lib):
    d = _dims()
    assert call_bwd(lib, d, ws_bytes=ws_size(lib, d) - 1) == 2
    assert call_bwd(lib, None) == 1
    assert call_bwd(lib, _dims(n_seqs=0, total_tokens=0), ws_bytes=0) == 0


def test_bwd_rejects_preprocessing(lib):
    from invariant_linear_attention_amd import gdn
    pre = gdn.make_preproc(norm_qk=True)
    d = _dims()
    d.pre = ctypes.pointer(pre)
    assert call_bwd(lib, d, ws_bytes=1 << 30) == 6


# ------------------------------------------------------------- chunked backward

def cbwd_ws(lib, dims):
    n = ctypes.c_uint64(0)
    rc = lib.gdn_bwd_chunked_workspace_size(ctypes.byref(dims), ctypes.byref(n))
    return int(n.value) if rc == 0 else -rc


def call_cbwd(lib, dims, ws_bytes=None, **over):
    a = dict(BP)
    a.update(over)
    if ws_bytes is None:
        ws_bytes = cbwd_ws(lib, dims) if dims is not None else 0
    return lib.gdn_bwd_chunked(ctypes.byref(dims) if dims is not None else None, a["q"], a["k"], a["v"], a["g"],
                               a["b"], a["h0"], a["cu"], a["dout"], a["dhT"], a["dq"], a["dk"], a["dv"], a["dg"],
                               a["db"], a["dh0"], a["ws"], ctypes.c_uint64(ws_bytes), None)


def test_bwd_chunked_workspace_size(lib):
    """Records (1,088 floats per slot and value head), the chunk-start states (a dv x dk
    state per slot and value head), x = v - Gam P (a dv x 16 tile per slot and value
    head), the <dhT, hT> partials
    (N hv dv/16 x 4), then with P row parts (plan_rows; 0 = 2 for dv = 128, else 1):
    when value heads share key heads or P > 1, dq and dk per value head and part
    (P T hv dk each), and when P > 1 dbeta and dg per part (P T hv each); slots =
    T // 16 + 2 N + 2; every part rounded up to 256 bytes."""
    up = lambda x: (x + 255) // 256 * 256
    for T, N, hk, hv, dk, dv, rows in ((10, 2, 2, 4, 128, 64, 0), (100, 3, 2, 2, 64, 128, 0),
                                       (33, 1, 1, 1, 128, 32, 0), (100, 3, 2, 2, 64, 128, 1),
                                       (10, 2, 2, 4, 128, 64, 2), (21, 1, 1, 1, 64, 64, 2)):
        slots = T // 16 + 2 * N + 2
        ck = dv * dk
        P = rows or (2 if dv == 128 else 1)
        want = (up(slots * hv * 1088 * 4) + up(slots * hv * ck * 4) + up(slots * hv * dv * 16 * 4)
                + up(N * hv * (dv // 16) * 16) + (2 * up(P * T * hv * dk * 4) if hv > hk or P > 1 else 0)
                + (2 * up(P * T * hv * 4) if P > 1 else 0))
        d = _dims(total_tokens=T, n_seqs=N, hk=hk, hv=hv, dk=dk, dv=dv, plan_rows=rows)
        assert cbwd_ws(lib, d) == want, (T, N, hk, hv, dk, dv, rows)
    n = ctypes.c_uint64(0)
    assert lib.gdn_bwd_chunked_workspace_size(None, ctypes.byref(n)) == 1
    assert lib.gdn_bwd_chunked_workspace_size(ctypes.byref(_dims()), None) == 1
    assert cbwd_ws(lib, _dims(hv=3)) == -2
    assert cbwd_ws(lib, _dims(dk=32)) == -6


@pytest.mark.parametrize("case,over,code", [
    (dict(dk=32), {}, 6), (dict(dk=16), {}, 6), (dict(dv=16), {}, 6), (dict(dv=96), {}, 6),
    (dict(plan_lanes=8), {}, 6), (dict(plan_lanes=2), {}, 6), (dict(plan_rows=3), {}, 6),
    (dict(plan_rows=2, dv=32), {}, 6),
    (dict(plan_waves=3), {}, 6),
    (dict(hk=1, hv=32), {}, 6), (dict(hv=3), {}, 2), (dict(io_dtype=7), {}, 3),
    (dict(n_seqs=0, total_tokens=3), {}, 2),
    ({}, dict(cu=None), 1), ({}, dict(ws=None), 1), ({}, dict(q=None), 1), ({}, dict(dout=None), 1),
    ({}, dict(dq=None), 1), ({}, dict(dg=None), 1), ({}, dict(db=None), 1), ({}, dict(dv=None), 1),
    ({}, dict(q=BP["q"] + 8), 4), ({}, dict(dout=BP["dout"] + 8), 4), ({}, dict(ws=BP["ws"] + 4), 4),
    ({}, dict(dq=BP["dq"] + 4), 4), ({}, dict(g=BP["g"] + 2), 4), ({}, dict(dhT=BP["dhT"] + 4), 4),
    ({}, dict(dq=BP["q"]), 5), ({}, dict(dk=BP["dq"]), 5), ({}, dict(ws=BP["dout"]), 5),
    ({}, dict(dh0=BP["h0"]), 5), ({}, dict(dv=BP["ws"] + 256), 5), ({}, dict(dg=BP["db"]), 5),
    ({}, dict(ws=BP["dhT"]), 5),
])
def test_bwd_chunked_rejects(lib, case, over, code):
    assert call_cbwd(lib, _dims(**case), ws_bytes=(1 << 30), **over) == code


def test_bwd_chunked_small_workspace_preprocessing_and_noop(lib):
    from invariant_linear_attention_amd import gdn
    d = _dims()
    assert call_cbwd(lib, d, ws_bytes=cbwd_ws(lib, d) - 1) == 2
    assert call_cbwd(lib, None) == 1
    assert call_cbwd(lib, _dims(n_seqs=0, total_tokens=0), ws_bytes=0) == 0
    pre = gdn.make_preproc(norm_qk=True)
    d.pre = ctypes.pointer(pre)
    assert call_cbwd(lib, d, ws_bytes=1 << 30) == 6


# ------------------------------------------------------------------ chunked form

CH = {name: BASE + (80 + i) * MB for i, name in enumerate(
    ["q", "k", "v", "g", "b", "cu", "o", "iS", "ik", "ir", "ia", "ib", "ic", "oS", "ok", "or", "oa", "ob", "oc", "ws"])}


def ch_ws(lib, dims):
    """Workspace bytes for dims (0 where the dims themselves are refused)."""
    n = ctypes.c_uint64(0)
    return int(n.value) if lib.gdn_chunked_workspace_size(ctypes.byref(dims), ctypes.byref(n)) == 0 else 0


def call_chunked(lib, dims, with_in=True, ws_bytes=None, **over):
    from invariant_linear_attention_amd.gdn import GdnChunkState
    a = dict(CH)
    a.update(over)
    if ws_bytes is None:
        ws_bytes = ch_ws(lib, dims) if dims is not None else 0
    sin = GdnChunkState(a["iS"], a["ik"], a["ir"], a["ia"], a["ib"], a["ic"])
    sout = GdnChunkState(a["oS"], a["ok"], a["or"], a["oa"], a["ob"], a["oc"])
    return lib.gdn_fwd_chunked(ctypes.byref(dims) if dims is not None else None, a["q"], a["k"], a["v"], a["g"],
                               a["b"], a["cu"], ctypes.byref(sin) if with_in else None, ctypes.byref(sout), a["o"],
                               a["ws"], ctypes.c_uint64(ws_bytes), None)


def test_chunked_workspace_size(lib):
    """One record of 576 floats per (slot, value head), floor(T / 16) + 2 N + 2 slots."""
    d = _dims(n_seqs=3, total_tokens=100, hv=4)
    assert ch_ws(lib, d) == (100 // 16 + 2 * 3 + 2) * 4 * 576 * 4
    n = ctypes.c_uint64(0)
    assert lib.gdn_chunked_workspace_size(None, ctypes.byref(n)) == 1
    assert lib.gdn_chunked_workspace_size(ctypes.byref(d), None) == 1


# the five arrays an in-place update shares between in and out
SHARED = dict(oS=CH["iS"], ok=CH["ik"], oa=CH["ia"], ob=CH["ib"], **{"or": CH["ir"]})


@pytest.mark.parametrize("case,over,code", [
    (dict(dk=32), {}, 6), (dict(dk=16), {}, 6), (dict(plan_rows=1), {}, 6), (dict(plan_waves=3), {}, 6),
    (dict(hk=1, hv=32), {}, 6), (dict(hv=3), {}, 2), (dict(io_dtype=4), {}, 3), (dict(n_seqs=0, total_tokens=2), {}, 2),
    ({}, dict(cu=None), 1), ({}, dict(oS=None), 1), ({}, dict(oc=None), 1), ({}, dict(q=None), 1),
    ({}, dict(o=None), 1), ({}, dict(ik=None), 1), ({}, dict(ia=None), 1), ({}, dict(oa=None), 1),
    ({}, dict(ib=None), 1), ({}, dict(ob=None), 1), ({}, dict(ir=None), 1),
    ({}, dict(ws=None), 1),
    ({}, dict(q=CH["q"] + 8), 4), ({}, dict(oS=CH["oS"] + 4), 4), ({}, dict(oc=CH["oc"] + 2), 4),
    ({}, dict(ik=CH["ik"] + 4), 4), ({}, dict(ok=CH["ok"] + 8), 4), ({}, dict(ws=CH["ws"] + 4), 4),
    ({}, dict(oS=CH["iS"]), 5), ({}, {"or": CH["ir"] + 64}, 5), ({}, dict(o=CH["v"]), 5),
    ({}, dict(oa=CH["or"]), 5), ({}, dict(ob=CH["ia"]), 5), ({}, dict(oc=CH["q"]), 5), ({}, dict(ws=CH["oS"]), 5),
    ({}, dict(o=CH["ws"]), 5),
    # in place needs one token per sequence (T == N) and distinct count arrays
    ({}, SHARED, 5), (dict(total_tokens=2), dict(SHARED, oc=CH["ic"]), 5),
    (dict(total_tokens=2), dict(SHARED, oS=CH["oS"]), 5),
])
def test_chunked_rejects(lib, case, over, code):
    assert call_chunked(lib, _dims(**case), **over) == code


def test_chunked_small_workspace_null_in_and_noop(lib):
    d = _dims()
    assert call_chunked(lib, d, ws_bytes=ch_ws(lib, d) - 1) == 2
    # no cu_seqlens is allowed for one token per sequence (then the next check, the
    # workspace size, is what refuses) and refused otherwise
    one = _dims(total_tokens=2)
    assert call_chunked(lib, one, ws_bytes=ch_ws(lib, one) - 1, cu=None) == 2
    assert call_chunked(lib, d, cu=None) == 1
    assert call_chunked(lib, None) == 1
    assert call_chunked(lib, _dims(n_seqs=0, total_tokens=0)) == 0
    # no incoming state is allowed (empty states); a missing out array is not
    assert call_chunked(lib, _dims(n_seqs=0, total_tokens=0), with_in=False) == 0


def test_fwd_train_rejects(lib):
    def call(dims, **over):
        a = dict(P)
        a["sp"] = BASE + 70 * MB
        a.update(over)
        return lib.gdn_fwd_varlen_train(ctypes.byref(dims), a["q"], a["k"], a["v"], a["g"], a["b"], a["h0"], a["cu"],
                                        a["out"], a["hT"], a["sp"], None)
    from invariant_linear_attention_amd import gdn
    assert call(_dims(), sp=None) == 1
    assert call(_dims(), sp=P["q"]) == 5
    assert call(_dims(), sp=P["out"] + 64) == 5
    assert call(_dims(), sp=BASE + 70 * MB + 2) == 4
    d = _dims()
    d.pre = ctypes.pointer(gdn.make_preproc(norm_qk=True))
    assert call(d) == 6


# ------------------------------------------------- allocation-free backward

def call_bwd_noalloc(lib, dims, **over):
    a = dict(BP)
    a.update(over)
    return lib.gdn_bwd_varlen_noalloc(ctypes.byref(dims) if dims is not None else None, a["q"], a["k"], a["v"],
                                      a["g"], a["b"], a["h0"], a["cu"], a["dout"], a["dhT"], a.get("sp"), a.get("hT"),
                                      a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["dh0"], None)


def test_noalloc_scratch_constant_matches_header(lib):
    from invariant_linear_attention_amd import gdn
    text = open(HEADER).read()
    m = re.search(r"#define GDN_NOALLOC_SCRATCH_BYTES \((\d+)ull << (\d+)\)", text)
    assert int(m.group(1)) << int(m.group(2)) == gdn.GDN_NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("case,code", [
    (dict(hv=3), 2), (dict(dk=16), 6), (dict(io_dtype=7), 3), (dict(n_seqs=0, total_tokens=3), 2),
    (dict(n_seqs=0, total_tokens=0), 0),
    # 1100 tokens at hv = 32, dk = dv = 128 need about 72 MB: more than the 64 MiB scratch
    (dict(n_seqs=1, total_tokens=1100, hk=16, hv=32), 8),
    (dict(n_seqs=40, total_tokens=40, hk=16, hv=32), 8),   # 40 final states of 2 MiB each
])
def test_noalloc_refuses_on_the_host(lib, case, code):
    """Sizes are checked before any HIP call: these return without a GPU."""
    assert call_bwd_noalloc(lib, _dims(**case)) == code
    assert call_bwd_noalloc(lib, None) == 1


def test_noalloc_capacity_is_the_workspace_size(lib):
    from invariant_linear_attention_amd import gdn
    fits = _dims(n_seqs=1, total_tokens=990, hk=16, hv=32)
    over = _dims(n_seqs=1, total_tokens=993, hk=16, hv=32)
    assert ws_size(lib, fits) <= gdn.GDN_NOALLOC_SCRATCH_BYTES < ws_size(lib, over)
    assert call_bwd_noalloc(lib, over) == 8


# ------------------------------------------------- preprocessing and its gradients

PP = {name: BASE + (120 + i) * MB for i, name in enumerate(
    ["q", "k", "a", "b", "qn", "kn", "g", "beta", "dqn", "dkn", "dg", "dbeta", "dq", "dk", "da", "db", "dA", "dD",
     "Alog", "dtb"])}


def pre_dims(gated=True, norm=True, **kw):
    from invariant_linear_attention_amd import gdn
    d = _dims(**kw)
    if gated or norm:
        pre = gdn.GdnPreproc(flags=(gdn.GDN_PRE_QK_L2NORM if norm else 0) | (gdn.GDN_PRE_GATE_LOGITS if gated else 0),
                             eps=1e-6, A_log=PP["Alog"] if gated else None, dt_bias=PP["dtb"] if gated else None)
        d.pre = ctypes.pointer(pre)
        d._keep = pre
    return d


def call_pre(lib, dims, **over):
    a = dict(PP)
    a.update(over)
    return lib.gdn_preprocess(ctypes.byref(dims) if dims is not None else None, a["q"], a["k"], a["a"], a["b"],
                              a["qn"], a["kn"], a["g"], a["beta"], None)


def call_pre_bwd(lib, dims, **over):
    a = dict(PP)
    a.update(over)
    return lib.gdn_preprocess_backward(ctypes.byref(dims) if dims is not None else None, a["q"], a["k"], a["a"],
                                       a["b"], a["dqn"], a["dkn"], a["dg"], a["dbeta"], a["dq"], a["dk"], a["da"],
                                       a["db"], a["dA"], a["dD"], None)


@pytest.mark.parametrize("case,over,code", [
    (dict(dk=24), {}, 6), (dict(hv=3), {}, 2), (dict(io_dtype=5), {}, 3), (dict(reserved=1), {}, 2),
    ({}, dict(q=None), 1), ({}, dict(kn=None), 1), ({}, dict(beta=None), 1), ({}, dict(a=None), 1),
    ({}, dict(q=PP["q"] + 8), 4), ({}, dict(qn=PP["qn"] + 4), 4), ({}, dict(g=PP["g"] + 2), 4),
    ({}, dict(qn=PP["q"]), 5), ({}, dict(g=PP["a"]), 5), ({}, dict(beta=PP["g"]), 5), ({}, dict(kn=PP["qn"]), 5),
    ({}, dict(g=PP["Alog"]), 5), (dict(total_tokens=1 << 40), {}, 2),
])
def test_preprocess_rejects(lib, case, over, code):
    assert call_pre(lib, pre_dims(**case), **over) == code


@pytest.mark.parametrize("case,over,code", [
    (dict(dk=24), {}, 6), (dict(hv=3), {}, 2),
    ({}, dict(dqn=None), 1), ({}, dict(dq=None), 1), ({}, dict(da=None), 1), ({}, dict(db=None), 1),
    ({}, dict(dq=PP["dq"] + 4), 4), ({}, dict(dA=PP["dA"] + 2), 4),
    ({}, dict(dq=PP["q"]), 5), ({}, dict(da=PP["dg"]), 5), ({}, dict(dA=PP["Alog"]), 5), ({}, dict(dD=PP["dA"]), 5),
    ({}, dict(dk=PP["dq"]), 5), (dict(total_tokens=1 << 40), {}, 2),
])
def test_preprocess_backward_rejects(lib, case, over, code):
    assert call_pre_bwd(lib, pre_dims(**case), **over) == code


def test_preprocess_gate_needs_A_log_and_empty_calls(lib):
    from invariant_linear_attention_amd import gdn
    d = pre_dims()
    d.pre.contents.A_log = None
    assert call_pre(lib, d) == 1
    assert call_pre(lib, None) == 1
    # no tokens: nothing to do (the backward without gate logits launches nothing either)
    assert call_pre(lib, pre_dims(total_tokens=0), q=None, k=None, a=None, b=None, qn=None, kn=None, g=None,
                    beta=None) == 0
    assert call_pre_bwd(lib, pre_dims(gated=False, total_tokens=0), q=None, k=None, a=None, b=None, dqn=None,
                        dkn=None, dg=None, dbeta=None, dq=None, dk=None, da=None, db=None) == 0


# ------------------------------------------------------- convolution backward

CB = {name: BASE + (150 + i) * MB for i, name in enumerate(
    ["x", "w", "bias", "cu", "pool", "src", "dy", "dx", "dw", "db", "ds", "ws"])}


def conv_dims(**kw):
    from invariant_linear_attention_amd import gdn
    a = dict(n_seqs=3, channels=64, taps=4, io_dtype=1, total_tokens=100, pool_size=3, flags=1)
    a.update(kw)
    return gdn.GdnConvDims(**a)


def conv_ws(lib, dims):
    n = ctypes.c_uint64(0)
    rc = lib.gdn_short_conv_backward_workspace_size(ctypes.byref(dims), ctypes.byref(n))
    return int(n.value) if rc == 0 else -rc


def call_conv_bwd(lib, dims, ws_bytes=None, **over):
    a = dict(CB)
    a.update(over)
    if ws_bytes is None:
        ws_bytes = max(conv_ws(lib, dims), 0) if dims is not None else 0
    return lib.gdn_short_conv_backward(ctypes.byref(dims) if dims is not None else None, a["x"], a["w"], a["bias"],
                                       a["cu"], a["pool"], a["src"], a["dy"], a["dx"], a["dw"], a["db"], a["ds"],
                                       a["ws"], ctypes.c_uint64(ws_bytes), None)


def test_conv_backward_workspace_size(lib):
    """K + 1 partial sums per channel and block of 64 tokens."""
    for T, C, K in ((100, 64, 4), (64, 16, 2), (1, 8192, 8), (0, 32, 3)):
        assert conv_ws(lib, conv_dims(total_tokens=T, channels=C, taps=K, n_seqs=1 if T else 0)) == \
            (T + 63) // 64 * C * (K + 1) * 4
    assert conv_ws(lib, conv_dims(taps=9)) == -2
    assert lib.gdn_short_conv_backward_workspace_size(None, ctypes.byref(ctypes.c_uint64(0))) == 1


@pytest.mark.parametrize("case,over,code", [
    (dict(taps=1), {}, 2), (dict(taps=9), {}, 2), (dict(channels=0), {}, 2), (dict(pool_size=0), {}, 2),
    (dict(flags=2), {}, 6), (dict(io_dtype=3), {}, 3), (dict(n_seqs=0), {}, 2),
    (dict(pool_size=2), dict(src=None), 2),
    ({}, dict(w=None), 1), ({}, dict(dw=None), 1), ({}, dict(cu=None), 1), ({}, dict(pool=None), 1),
    ({}, dict(x=None), 1), ({}, dict(dy=None), 1), ({}, dict(dx=None), 1), ({}, dict(ws=None), 1),
    ({}, dict(x=CB["x"] + 1), 4), ({}, dict(dy=CB["dy"] + 2), 4), ({}, dict(ws=CB["ws"] + 2), 4),
    ({}, dict(dx=CB["x"]), 5), ({}, dict(dw=CB["w"]), 5), ({}, dict(ws=CB["dy"]), 5), ({}, dict(ds=CB["dx"]), 5),
    ({}, dict(db=CB["pool"]), 5), ({}, dict(dx=CB["src"]), 5),
])
def test_conv_backward_rejects(lib, case, over, code):
    assert call_conv_bwd(lib, conv_dims(**case), **over) == code


def test_conv_backward_small_workspace(lib):
    d = conv_dims()
    assert call_conv_bwd(lib, d, ws_bytes=conv_ws(lib, d) - 1) == 2
    assert call_conv_bwd(lib, None) == 1
