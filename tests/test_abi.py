"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before anything is enqueued
(no GPU is needed: validation never touches device memory)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hca.h")

hca = pytest.importorskip("long_context_attention_hca_amd", reason="libhca.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s*([A-Za-z_]\w*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"csa_compress", "hca_compress", "lightning_index_topk", "csa_sparse_mqa_attn",
            "hca_dense_mqa_attn"} <= set(names)
    lib = ctypes.CDLL(hca.library_path)
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_version_and_status_strings():
    assert hca.abi_version() == 3
    for code, text in [(0, b"ok"), (-1, b"invalid argument"), (-3, b"workspace too small")]:
        assert hca._status_string(code) == text


# fake, never-dereferenced device addresses (16-byte aligned)
P = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(16)]


def store(layout=2, d_nope=448, d_rope=64, n_rows=100, row_stride=448, rope_stride=64, data=None, reserved=0):
    return hca._StoreC(layout, d_nope, d_rope, reserved, n_rows, data if data is not None else 0x9000000,
                       row_stride, 0xA000000, 0xB000000, rope_stride)


def compress_call(**kw):
    a = dict(raw=P[0], dt=1, rs=512, n_rows=100, first_pos=0, logits=P[1], lrs=512, lcs=1, bias=P[2], m=4, w=8,
             fe=0, ne=24, out=store(), row0=0)
    a.update(kw)
    return hca._csa_compress(a["raw"], a["dt"], a["rs"], a["n_rows"], a["first_pos"], a["logits"], a["lrs"],
                             a["lcs"], a["bias"], a["m"], a["w"], a["fe"], a["ne"], ctypes.byref(a["out"]),
                             a["row0"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(raw=None), -1, "NULL"),
    (dict(dt=3), -2, "raw dtype"),
    (dict(m=0), -1, "m <= w"),
    (dict(w=2), -1, "m <= w"),
    (dict(ne=26), -1, "raw rows do not cover"),          # entries 0..25 need rows up to 103
    (dict(first_pos=1, fe=1, ne=2), -1, "raw rows do not cover"),   # entry 1 reads position 0
    (dict(out=store(n_rows=10)), -1, "output rows"),
    (dict(lcs=2), -1, "logit_col_stride"),
    (dict(raw=ctypes.c_void_p(0x100008)), -1, "aligned"),
    (dict(rs=500), -1, "raw_row_stride"),
    (dict(out=store(d_nope=444, d_rope=68, rope_stride=72)), -1, "multiples of 8"),
    (dict(out=store(reserved=1)), -1, "reserved"),
    (dict(out=store(layout=7)), -1, "unknown layout"),
    (dict(out=store(row_stride=440)), -1, "row_stride"),
])
def test_compress_rejects_bad_arguments(kw, status, msg):
    assert compress_call(**kw) == status
    assert msg in hca._last_error().decode()


def test_compress_offsets_with_halo_pass_validation_then_need_a_gpu():
    # entries 5..12 read positions 16..51: rows 16.. suffice; the call then fails only at launch time
    r = compress_call(first_pos=16, n_rows=36, fe=5, ne=8)
    if r == -4:
        assert "launch" in hca._last_error().decode()
    else:
        assert r == 0


def index_call(**kw):
    a = dict(q=P[0], qs=P[1], w=P[2], H=4, d=64, dt=3, k_idx=P[3], ks=P[4], k_rows=1000, krb=P[5], qseq=P[6],
             qpos=P[7], qlo=None, nq=4, mv=1000, m=4, cw=8, k=64, out=P[8], ws=P[9], wsb=1 << 30)
    a.update(kw)
    return hca._index(a["q"], a["qs"], a["w"], a["H"], a["d"], a["dt"], a["k_idx"], a["ks"], a["k_rows"], a["krb"],
                      a["qseq"], a["qpos"], a["qlo"], a["nq"], a["mv"], a["m"], a["cw"], a["k"], a["out"], a["ws"],
                      a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(qs=None), -1), (dict(d=128), -2), (dict(H=9), -2), (dict(H=0), -2),
    (dict(k=0), -1), (dict(k=4096), -1), (dict(m=0), -1), (dict(dt=2), -2), (dict(wsb=100), -3),
    (dict(ws=None), -3), (dict(k_idx=ctypes.c_void_p(0x100004)), -1), (dict(mv=(1 << 21) + 1), -2),
    (dict(cw=3), -1),                                        # the CSA window shorter than m
])
def test_index_rejects_bad_arguments(kw, status):
    assert index_call(**kw) == status


def test_index_workspace_is_monotone_and_batches():
    one = hca.lightning_index_topk_workspace(1, 262144, 1024)
    four = hca.lightning_index_topk_workspace(4, 262144, 1024)
    assert one > 262144 * 12 and four > 3 * one
    assert index_call(nq=0) == 0                    # nothing to do
    r = index_call(wsb=one)                         # enough for one query at a time
    assert r in (0, -4)


def attn_call(csa=True, **kw):
    a = dict(q=P[0], qdt=1, nq=4, H=64, cache=store(), crb=P[1], idx=P[2], k=64, mp=128, mv=100,
             win=store(), wrb=P[3], wp0=P[4], W=128, qseq=P[5], qpos=P[6], qlo=None, scale=0.04, o=P[7], odt=1,
             lse=P[8], ws=P[9], wsb=1 << 30)
    a.update(kw)
    if csa:
        return hca._csa_attn(a["q"], a["qdt"], a["nq"], a["H"], ctypes.byref(a["cache"]), a["crb"], a["idx"], a["k"],
                             ctypes.byref(a["win"]), a["wrb"], a["wp0"], a["W"], a["qseq"], a["qpos"], a["qlo"],
                             a["scale"], a["o"], a["odt"], a["lse"], a["ws"], a["wsb"], None)
    return hca._hca_attn(a["q"], a["qdt"], a["nq"], a["H"], ctypes.byref(a["cache"]), a["crb"], a["mp"], a["mv"],
                         ctypes.byref(a["win"]), a["wrb"], a["wp0"], a["W"], a["qseq"], a["qpos"], a["qlo"], a["scale"],
                         a["o"], a["odt"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("csa", [True, False])
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(H=0), -1), (dict(W=-1), -1), (dict(scale=float("inf")), -1),
    (dict(H=40), -2),                                        # MFMA path needs multiples of 16 heads
    (dict(qdt=0), -2),                                       # fp32 q with split stores
    (dict(cache=store(layout=0, d_nope=448, d_rope=64, row_stride=512)), -2),
    (dict(win=store(d_nope=384, d_rope=128, rope_stride=128)), -1),
    (dict(cache=store(d_nope=192, d_rope=64)), -1),           # widths differ from the window
    (dict(wsb=16), -3),
])
def test_attention_rejects_bad_arguments(csa, kw, status):
    assert attn_call(csa, **kw) == status


def test_attention_workspace_policy():
    # decode: few queries -> split-K partials; prefill: many queries -> no workspace
    assert hca.mqa_attn_workspace(1, 4, 64, 512, 8192 + 128) > 0
    assert hca.mqa_attn_workspace(1, 24576, 64, 512, 2048 + 128) == 0
    assert hca.mqa_attn_workspace(0, 16, 16, 192, 64 + 128) > 0


def test_mxfp4_output_store_validation():
    mx = lambda **k: store(**{**dict(layout=3, d_nope=64, d_rope=0, row_stride=32, rope_stride=2), **k})
    raw = dict(rs=64, lrs=64, out=mx())
    assert compress_call(**raw) in (0, -4)               # passes validation; launching needs a GPU
    for bad, msg in [(mx(d_rope=8), "d_rope == 0"), (mx(d_nope=48), "multiple of 32"),
                     (mx(row_stride=24), "row_stride"), (mx(rope_stride=1), "scale stride")]:
        assert compress_call(**{**raw, "out": bad}) == -1
        assert msg in hca._last_error().decode()


def test_decode_layer_struct_matches_the_header(tmp_path):
    src = tmp_path / "sz.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "hca.h"\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu\\n", sizeof(hca_decode_layer),'
                   ' offsetof(hca_decode_layer, window), offsetof(hca_decode_layer, csa),'
                   ' offsetof(hca_decode_layer, idx), offsetof(hca_decode_layer, idx_row_begin));return 0;}\n')
    exe = tmp_path / "sz"
    import subprocess
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    C = hca._DecodeLayerC
    assert got == [ctypes.sizeof(C), C.window.offset, C.csa.offset, C.idx.offset, C.idx_row_begin.offset]


def decode_call(B=2, d_idx=64, **kw):
    D = 512
    st = lambda layout=2: store(layout=layout, n_rows=1000)
    L = hca._DecodeLayerC(4, 8, 128, 128, 128, d_idx, P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[0],
                          st(), P[8], P[9], st(), P[10], st(), P[11],
                          store(layout=3, d_nope=64, d_rope=0, row_stride=32, rope_stride=2), P[12])
    for k, v in kw.items():
        setattr(L, k, v)
    return hca._decode_append(ctypes.byref(L), B, P[13], P[14], P[14], P[14], P[15], P[15], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(m=0), -1, "m <= w"), (dict(w=2), -1, "m <= w"), (dict(W=0), -1, "W >= 1"),
    (dict(R=100), -1, "ring rows"), (dict(B=0), -1, "B < 1"),
    (dict(window=store(layout=3, d_nope=64, d_rope=0, row_stride=32, rope_stride=2)), -2, "window layout"),
    (dict(window=store(d_nope=384, d_rope=64, row_stride=384)), -1, "widths differ"),
    (dict(hca=store(d_nope=384, d_rope=64, row_stride=384)), -1, "widths differ"),
    (dict(d_idx=48), -1, "idx width"), (dict(d_idx=12), -2, "d_idx"),
    (dict(bias_csa=None), -1, "NULL field"), (dict(hca_state=None), -1, "NULL field"),
    (dict(ring_x=0x100004), -1, "aligned"),
    (dict(idx_row_begin=None), -1, "NULL indexer"),
])
def test_decode_append_rejects_bad_arguments(kw, status, msg):
    B = kw.pop("B", 2)
    assert decode_call(B=B, **kw) == status
    assert msg in hca._last_error().decode()


def test_decode_append_valid_call_reaches_launch():
    assert decode_call() in (0, -4)
    assert decode_call(d_idx=0, idx_row_begin=None) in (0, -4)   # no indexer keys


@pytest.mark.parametrize("phase", ["scores", "select"])
def test_split_index_calls_need_the_whole_workspace(phase):
    one = hca.lightning_index_topk_workspace(1, 1000, 64)
    four = hca.lightning_index_topk_workspace(4, 1000, 64)
    a = dict(q=P[0], qs=P[1], w=P[2], H=4, d=64, dt=3, k_idx=P[3], ks=P[4], k_rows=1000, krb=P[5], qseq=P[6],
             qpos=P[7], qlo=None, nq=4, mv=1000, m=4, cw=8, k=64, out=P[8], ws=P[9])
    f = hca._index_phase[phase]
    call = lambda wsb: f(*[a[x] for x in ("q", "qs", "w", "H", "d", "dt", "k_idx", "ks", "k_rows", "krb", "qseq",
                                          "qpos", "qlo", "nq", "mv", "m", "cw", "k", "out", "ws")], wsb, None)
    assert call(one) == -3 and "all nq queries" in hca._last_error().decode()
    assert call(four) in (0, -4)
    assert index_call(wsb=one) in (0, -4)            # the one-call version batches instead


def proj_call(**kw):
    a = dict(x=P[0], n=4, ldx=32768, G=8, K=4096, w=P[1], N=1024, y=P[2], ydt=1, ldy=8192)
    a.update(kw)
    return hca._proj(a["x"], a["n"], a["ldx"], a["G"], a["K"], a["w"], a["N"], a["y"], a["ydt"], a["ldy"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(x=None), -1, "NULL"), (dict(n=-1), -1, "n out of range"), (dict(G=0), -1, "groups"),
    (dict(K=100), -2, "k_group"), (dict(N=40), -2, "n_group"), (dict(ydt=3), -2, "dtype"),
    (dict(ldx=1000), -1, "ldx"), (dict(ldx=32772), -1, "ldx"), (dict(ldy=100), -1, "ldy"),
    (dict(w=ctypes.c_void_p(0x100008)), -1, "aligned"),
])
def test_grouped_projection_rejects_bad_arguments(kw, status, msg):
    assert proj_call(**kw) == status
    assert msg in hca._last_error().decode()


def test_grouped_projection_valid_call_reaches_launch():
    assert proj_call() in (0, -4)
    assert proj_call(n=0) == 0


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: any --gpus other than 1 exits with status 2 and says why,
    before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_binding_fails_loudly_without_the_library(tmp_path):
    """The binding has no CPU fallback: importing it from a folder without libhca.so raises
    ImportError naming the missing library."""
    import importlib.util
    import shutil
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = tmp_path / "hca_without_lib"
    pkg.mkdir()
    shutil.copy(os.path.join(root, "long_context_attention_hca_amd", "__init__.py"), pkg / "__init__.py")
    spec = importlib.util.spec_from_file_location("hca_without_lib", pkg / "__init__.py",
                                                  submodule_search_locations=[str(pkg)])
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError, match="libhca.so"):
        spec.loader.exec_module(mod)
    sys.modules.pop("hca_without_lib", None)


def test_noalloc_attention_rejects_calls_beyond_its_scratch():
    """hca_dense_mqa_attn_noalloc checks on the host that the split-K partials fit its 16 MiB static
    scratch: 16 fp32 heads of 512 over a million entries need 512 splits of 16 x 513 floats."""
    f32 = store(layout=0, d_nope=448, d_rope=64, row_stride=512)
    args = lambda nq, mv: (P[0], 0, nq, 16, ctypes.byref(f32), P[1], 1, mv, ctypes.byref(f32), P[3], P[4], 0, P[5],
                           P[6], None, 0.04, P[7], 0, P[8], None)
    assert hca.mqa_attn_workspace(0, 1, 16, 512, 1 << 20) > 16 << 20
    assert hca._hca_attn_noalloc(*args(1, 1 << 20)) == -3
    assert "16 MiB" in hca._last_error().decode()
    assert hca._hca_attn_noalloc(*args(0, 1 << 20)) == 0          # nothing to do
    bad = hca._StoreC(7, 448, 64, 0, 100, 0x9000000, 512, 0, 0, 0)
    assert hca._hca_attn_noalloc(P[0], 0, 1, 16, ctypes.byref(bad), P[1], 1, 100, ctypes.byref(f32), P[3], P[4], 0,
                                 P[5], P[6], None, 0.04, P[7], 0, P[8], None) == -1


def test_deferred_merge_validation():
    """mqa_attn_merge rejects NULL or malformed partial records on the host; records of calls that
    were not split (or had no queries) need no launch, so they succeed without a GPU; the partial
    calls validate their arguments as the undeferred calls do and need an output record."""
    AP = hca.AttnPartials
    assert hca._attn_merge(None, None, None) == -1
    assert hca._attn_merge(ctypes.byref(AP(None, None, P[7], P[8], 4, 0, 512, 2, 1)), None, None) == -1
    assert hca._attn_merge(ctypes.byref(AP(None, None, P[7], P[8], 4, 64, 512, 2, 1)), None, None) == -1  # no partials
    assert hca._attn_merge(ctypes.byref(AP(P[9], P[9], P[7], P[8], 4, 64, 512, 2, 9)), None, None) == -1  # o dtype
    assert hca._attn_merge(ctypes.byref(AP(P[9], P[9], None, P[8], 4, 64, 512, 2, 1)), None, None) == -1  # no output
    done = AP(None, None, P[7], P[8], 4, 64, 512, 1, 1)  # one split: the call wrote its output itself
    empty = AP(None, None, None, None, 0, 64, 512, 1, 1)
    assert hca._attn_merge(ctypes.byref(done), ctypes.byref(empty), None) == 0
    bad = AP(P[9], P[9], P[7], P[8], -1, 64, 512, 2, 1)
    assert hca._attn_merge(ctypes.byref(done), ctypes.byref(bad), None) == -1
    a = dict(q=P[0], qdt=1, nq=4, H=64, crb=P[1], idx=P[2], k=64, wrb=P[3], wp0=P[4], W=128, qseq=P[5],
             qpos=P[6], o=P[7], lse=P[8], ws=P[9])
    out = AP()
    c, w = store(), store()
    args = (a["q"], a["qdt"], a["nq"], 40, ctypes.byref(c), a["crb"], a["idx"], a["k"], ctypes.byref(w), a["wrb"],
            a["wp0"], a["W"], a["qseq"], a["qpos"], None, 0.04, a["o"], 1, a["lse"], a["ws"], 1 << 30, None)
    assert hca._csa_attn_partials(*args, ctypes.byref(out)) == -2          # 40 heads: unsupported, as undeferred
    assert hca._csa_attn_partials(*args, None) == -1                       # no record
    hargs = (a["q"], a["qdt"], a["nq"], 64, ctypes.byref(c), a["crb"], 128, 100, ctypes.byref(w), a["wrb"],
             a["wp0"], a["W"], a["qseq"], a["qpos"], None, 0.04, a["o"], 1, a["lse"], a["ws"], 16, None)
    assert hca._hca_attn_partials(*hargs, ctypes.byref(out)) == -3         # workspace too small


def pending_call(out, **kw):
    a = dict(q=P[0], qs=P[1], w=P[2], H=4, d=64, dt=3, k_idx=P[3], ks=P[4], k_rows=1000, krb=P[5], qseq=P[6],
             qpos=P[7], qlo=None, nq=4, mv=1000, m=4, cw=8, k=64, out=P[8], ws=P[9], wsb=1 << 30)
    a.update(kw)
    return hca._index_pending(a["q"], a["qs"], a["w"], a["H"], a["d"], a["dt"], a["k_idx"], a["ks"], a["k_rows"],
                              a["krb"], a["qseq"], a["qpos"], a["qlo"], a["nq"], a["mv"], a["m"], a["cw"], a["k"],
                              a["out"], a["ws"], a["wsb"], None, out)


def test_pending_select_records_and_validates():
    """lightning_index_select_pending validates as lightning_index_select (the split calls' whole-
    workspace rule included) and records without touching a device; the combined HCA call rejects
    a missing record or one the library did not fill before anything is enqueued."""
    sel = hca.PendingSelect()
    assert pending_call(None) == -1                                  # no record
    assert pending_call(ctypes.byref(sel), k=0) == -1
    assert pending_call(ctypes.byref(sel), dt=2) == -2
    one = hca._index_ws(1, 1000, 64)
    assert pending_call(ctypes.byref(sel), wsb=one) == -3            # not the workspace of all 4 queries
    assert not any(sel.opaque)                                        # untouched on error
    assert pending_call(ctypes.byref(sel)) == 0                       # recorded on the host
    assert any(sel.opaque)
    empty = hca.PendingSelect()
    assert pending_call(ctypes.byref(empty), nq=0) == 0               # nothing to select: an inactive record
    c, w = store(), store()
    out = hca.AttnPartials()
    hargs = (P[0], 1, 4, 64, ctypes.byref(c), P[1], 128, 100, ctypes.byref(w), P[3], P[4], 128, P[5], P[6], None,
             0.04, P[7], 1, P[8], P[9], 1 << 30, None)
    assert hca._hca_attn_partials_select(*hargs, None, ctypes.byref(out)) == -1
    assert hca._hca_attn_partials_select(*hargs, ctypes.byref(sel), None) == -1
    assert hca._hca_attn_partials_select(*hargs, ctypes.byref(hca.PendingSelect()), ctypes.byref(out)) == -1
    assert "lightning_index_select_pending" in hca._last_error().decode()
    bad_heads = (P[0], 1, 4, 40) + hargs[4:]
    assert hca._hca_attn_partials_select(*bad_heads, ctypes.byref(sel), ctypes.byref(out)) == -2
