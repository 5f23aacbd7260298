"""The C-ABI library loads, exports every symbol the header declares, and rejects bad
arguments on the host before launching anything (no GPU needed: every call here fails
its checks, so nothing reaches the HIP runtime)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "s2a.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4
A = 0x10000           # a fake 16-byte-aligned address; never dereferenced
MIS = 0x10002         # misaligned


@pytest.fixture(scope="module")
def lib():
    from block_sparse_attention_41_amd import build_lib, ops
    if not os.path.exists(ops.LIB_PATH):
        build_lib.build(verbose=False)
    return ops.lib()


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"if", "sizeof"})


def test_header_declares_the_six_entry_points():
    names = _declared_functions()
    for n in ("s2attn_fwd", "s2attn_bwd", "hga_summarize", "hga_select_topk", "hga_fwd", "hga_bwd_active"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    from block_sparse_attention_41_amd import ops
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r" T (\w+)$", out.stdout, flags=re.M))
    for n in _declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(ops.EXPORTED) == set(_declared_functions())


def test_status_strings(lib):
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR):
        assert lib.s2a_status_string(code)
    assert lib.s2a_status_string(99) == b"unknown status"


def _s2fwd(lib, **kw):
    a = dict(q=A, k=A, v=A, o=A, lse=A, B=1, N=1024, H=4, Hkv=4, d=64, G=256, shift=1, scale=0.125)
    a.update(kw)
    return lib.s2attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["N"], a["H"], a["Hkv"], a["d"],
                          a["G"], a["shift"], a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(lse=MIS), INVALID), (dict(B=0), INVALID), (dict(N=-64), INVALID),
    (dict(H=6, Hkv=4), INVALID), (dict(N=1000), INVALID), (dict(G=0), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(H=4, Hkv=1, shift=1), INVALID),                 # odd Hkv with shifting
    (dict(d=96), UNSUPPORTED), (dict(N=960, G=96, shift=0), UNSUPPORTED),   # G % 64
    (dict(N=768, G=192, shift=1), UNSUPPORTED),           # G/2 % 64 when shifting
])
def test_s2attn_fwd_rejects(lib, kw, code):
    assert _s2fwd(lib, **kw) == code


def test_s2attn_bwd_workspace_sizes(lib):
    # the stored-dS workspace: the statistics padded to 256 bytes, then bf16 dS of every
    # lower-triangle 64 x 64 tile of every (batch, head, group)
    stats = 2 * 2 * 4 * 1024 * 4
    tiles = 2 * 4 * (1024 // 256) * (4 * 5 // 2) * 64 * 64 * 2
    assert lib.s2attn_bwd_workspace_bytes_dsq(2, 1024, 4, 4, 64, 256) == stats + tiles
    assert lib.s2attn_bwd_workspace_bytes_dsq(1, 8192, 32, 32, 128, 2048) == 2 * 32 * 8192 * 4 + 128 * 528 * 8192
    stats_odd = 1 * 4 * 192 * 2 * 4                          # 6144 bytes, padded to 6144 (a 256 multiple)
    assert lib.s2attn_bwd_workspace_bytes_dsq(1, 192, 4, 4, 64, 192) == stats_odd + 4 * 6 * 64 * 64 * 2
    for bad in ((0, 1024, 4, 4, 64, 256), (1, 1024, 0, 4, 64, 256), (1, 1024, 4, 4, 64, 0),
                (1, 1000, 4, 4, 64, 250), (1, 1024, 4, 4, 64, 96), (1, 1024, 4, 4, 64, 384)):
        assert lib.s2attn_bwd_workspace_bytes_dsq(*bad) == 0, bad


def test_s2attn_bwd_rejects(lib):
    ws = lib.s2attn_bwd_workspace_bytes(1, 1024, 4, 4, 64)
    assert ws == 2 * 1 * 4 * 1024 * 4          # D and LSE*log2(e), float32 [B, H, N] each

    def call(wsp=A, wsb=ws, **kw):
        a = dict(B=1, N=1024, H=4, Hkv=4, d=64, G=256, shift=1, scale=0.125)
        a.update(kw)
        return lib.s2attn_bwd(A, A, A, A, A, A, A, A, A, wsp, wsb, a["B"], a["N"], a["H"], a["Hkv"], a["d"],
                              a["G"], a["shift"], a["scale"], None)
    assert call(wsb=ws - 1) == WORKSPACE
    assert call(wsp=None) == WORKSPACE
    assert call(N=1000) == INVALID
    assert call(d=32) == UNSUPPORTED
    assert lib.s2attn_bwd(None, A, A, A, A, A, A, A, A, A, ws, 1, 1024, 4, 4, 64, 256, 1, 0.125, None) == INVALID
    # the stage entry points share the checks
    assert lib.s2attn_bwd_prep(A, A, A, A, ws - 1, 1, 1024, 4, 4, 64, 256, 1, 0.125, None) == WORKSPACE
    assert lib.s2attn_bwd_prep(None, A, A, A, ws, 1, 1024, 4, 4, 64, 256, 1, 0.125, None) == INVALID
    assert lib.s2attn_bwd_dq(A, A, A, A, None, A, ws, 1, 1024, 4, 4, 64, 256, 1, 0.125, None) == INVALID
    assert lib.s2attn_bwd_dq_prep(A, A, A, None, A, A, A, A, ws, 1, 1024, 4, 4, 64, 256, 1, 0.125, None) == INVALID
    assert lib.s2attn_bwd_dq_prep(A, A, A, A, A, A, A, A, ws - 1, 1, 1024, 4, 4, 64, 256, 1, 0.125, None) == WORKSPACE
    assert lib.s2attn_bwd_dq(A, A, A, A, A, A, ws, 1, 1000, 4, 4, 64, 256, 1, 0.125, None) == INVALID
    assert lib.s2attn_bwd_dkdv(A, A, A, A, A, MIS, A, ws, 1, 1024, 4, 4, 64, 256, 1, 0.125, None) == INVALID
    assert lib.s2attn_bwd_dkdv(A, A, A, A, A, A, A, ws, 1, 1024, 4, 4, 96, 256, 1, 0.125, None) == UNSUPPORTED


def test_hga_entry_points_reject(lib):
    # summaries
    assert lib.hga_summarize(A, 0, A, 0, 1, 1000, 8, 128, 128, None) == INVALID      # T % chunk
    assert lib.hga_summarize(A, 0, A, 0, 1, 1024, 8, 128, 96, None) == INVALID       # T % chunk
    assert lib.hga_summarize(A, 0, A, 0, 1, 960, 8, 128, 96, None) == UNSUPPORTED    # chunk % 64
    assert lib.hga_summarize(None, 0, A, 0, 1, 1024, 8, 128, 128, None) == INVALID
    assert lib.hga_summarize(A, 0, A, 0, 1, 0, 8, 128, 128, None) == OK              # empty history: no-op
    assert lib.hga_summarize(A, 100, A, 0, 2, 1024, 8, 128, 128, None) == INVALID    # batch stride too small
    # selection
    assert lib.hga_select_topk(A, A, 0, A, 1, 2048, 32, 8, 128, 112, 64, 0, None) == INVALID   # topk < 1
    assert lib.hga_select_topk(A, A, 0, A, 1, 2048, 32, 8, 128, 112, 64, 65, None) == UNSUPPORTED
    assert lib.hga_select_topk(A, A, 0, A, 1, 2048, 32, 8, 128, 112, 32, 8, None) == UNSUPPORTED  # qblock
    assert lib.hga_select_topk(A, A, 0, A, 1, 2000, 32, 8, 128, 112, 64, 8, None) == INVALID  # S % qblock
    assert lib.hga_select_topk(A, A, 0, A, 1, 2048, 30, 8, 128, 112, 64, 8, None) == INVALID  # H % Hkv
    # forward / backward
    args = [A, A, A, 0, A, A, 0, A, A, A, 1, 2048, 32, 8, 128, 14336, 128, 64, 8, 0.088]
    assert lib.hga_fwd(*args[:-1], 0.0, None) == INVALID
    bad = list(args)
    bad[15] = 14300                                  # T % chunk
    assert lib.hga_fwd(*bad, None) == INVALID
    bad = list(args)
    bad[17] = 128                                    # qblock
    assert lib.hga_fwd(*bad, None) == UNSUPPORTED
    bad = list(args)
    bad[4] = None                                    # history pointer with T > 0
    assert lib.hga_fwd(*bad, None) == INVALID
    ws = lib.hga_bwd_workspace_bytes(1, 2048, 32, 8, 128)
    assert ws >= 2 * 32 * 2048 * 4                   # two row statistics (+ split partial sums)
    assert ws % 16 == 0
    assert lib.hga_bwd_workspace_bytes(1, 2048, 30, 8, 128) == 0   # H % Hkv: no valid size
    # stored dS: the above padded to 256 bytes, then bf16 dS of each (batch, q head)'s
    # lower-triangle 64 x 64 tiles over the segment
    assert lib.hga_bwd_workspace_bytes_dsq(1, 2048, 32, 8, 128) == (ws + 255) // 256 * 256 + 32 * 528 * 64 * 64 * 2
    ws2 = lib.hga_bwd_workspace_bytes(2, 192, 4, 2, 64)
    assert lib.hga_bwd_workspace_bytes_dsq(2, 192, 4, 2, 64) == (ws2 + 255) // 256 * 256 + 2 * 4 * 6 * 64 * 64 * 2
    for bad in ((0, 2048, 32, 8, 128), (1, 2048, 30, 8, 128), (1, 2000, 32, 8, 128), (1, 2048, 0, 8, 128)):
        assert lib.hga_bwd_workspace_bytes_dsq(*bad) == 0, bad
    bargs = [A, A, A, 0, A, A, 0, A, A, A, A, A, A, A, A, ws - 4, 1, 2048, 32, 8, 128, 14336, 128, 64, 8, 0.088]
    assert lib.hga_bwd_active(*bargs, None) == WORKSPACE
    bargs[15] = ws
    bargs[19] = 7                                    # H % Hkv
    assert lib.hga_bwd_active(*bargs, None) == INVALID


def test_hga_shared_and_decode_entry_points_reject(lib):
    args = [A, A, A, 0, A, A, 0, A, A, A, 1, 2048, 32, 8, 128, 14336, 128, 64, 8, 0.088]
    bad = list(args)
    bad[17] = 128                                    # qblock
    assert lib.hga_fwd_shared(*bad, None) == UNSUPPORTED
    assert lib.hga_select_topk_shared(A, A, 0, A, 1, 2048, 32, 8, 128, 112, 64, 65, None) == UNSUPPORTED
    # decode: workspace covers 32 rows x (d + 4) floats per (batch, head, split); the 48
    # tiles of each of 32 heads are cut into splits of 1 (about 2048 splits in all)
    ws = lib.hga_decode_workspace_bytes(1, 1, 2048, 32, 128, 128, 8)
    assert ws == 32 * 48 * 32 * 132 * 4
    assert lib.hga_decode_workspace_bytes(4, 1, 2048, 32, 128, 128, 8) == 4 * 32 * 16 * 32 * 132 * 4  # 3 each
    assert lib.hga_decode_workspace_bytes(1, 33, 2048, 32, 128, 128, 8) == 0
    dargs = [A, A, A, 0, A, A, 0, A, A, A, A, ws, 1, 1, 2048, 32, 8, 128, 14336, 128, 8, 0.088]
    assert lib.hga_decode(*dargs[:11], ws - 16, *dargs[12:], None) == WORKSPACE
    bad = list(dargs)
    bad[13] = 33                                     # nq > 32
    assert lib.hga_decode(*bad, None) == UNSUPPORTED
    bad = list(dargs)
    bad[13], bad[14] = 5, 4                          # nq > Sa
    assert lib.hga_decode(*bad, None) == INVALID
    bad = list(dargs)
    bad[18] = 14300                                  # T % chunk
    assert lib.hga_decode(*bad, None) == INVALID
    bad = list(dargs)
    bad[4] = None                                    # history pointer with T > 0
    assert lib.hga_decode(*bad, None) == INVALID


@pytest.mark.parametrize("B,S,H,Hkv,d", [(1, 2048, 32, 8, 128), (1, 2048, 32, 8, 64), (2, 1024, 16, 4, 128),
                                         (1, 4096, 32, 8, 128)])
def test_hga_split_parts_fit_one_round(lib, B, S, H, Hkv, d):
    """The split dK/dV plan of the HGA backward never makes more than one round of parts
    (256 CUs, one fused workgroup each): its float32 partials (dK and dV, 128 keys x 128
    floats per part) are what the workspace holds beyond the two row statistics."""
    ws = lib.hga_bwd_workspace_bytes(B, S, H, Hkv, d)
    stats = 2 * B * H * S * 4
    parts, rem = divmod(ws - stats, 4 * 2 * 128 * 128)
    assert rem == 0
    blocks = B * Hkv * (S // 128)          # key blocks of 128 in the segment
    if blocks >= 256:
        assert parts == 0                  # enough blocks: no split
    else:
        assert blocks < parts <= 256


def test_hga_append_history_rejects(lib):
    def call(**kw):
        a = dict(ks=A, vs=A, sbs=0, kh=A, vh=A, hbs=0, summ=A, smbs=0, B=1, S=256, Hkv=2, d=128, T=512, chunk=128)
        a.update(kw)
        return lib.hga_append_history(a["ks"], a["vs"], a["sbs"], a["kh"], a["vh"], a["hbs"], a["summ"], a["smbs"],
                                      a["B"], a["S"], a["Hkv"], a["d"], a["T"], a["chunk"], None)
    assert call(S=0) == OK                          # nothing to append: no launch
    assert call(ks=None) == INVALID
    assert call(summ=MIS) == INVALID
    assert call(S=200) == INVALID                   # S % chunk
    assert call(T=100) == INVALID                   # T % chunk
    assert call(T=-128) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(chunk=96, S=192, T=96) == UNSUPPORTED
    assert call(B=2, hbs=(512 + 256) * 2 * 128 - 8, sbs=256 * 2 * 128, smbs=6 * 2 * 128) == INVALID   # history too short
    assert call(B=2, hbs=(512 + 256) * 2 * 128, sbs=256 * 2 * 128, smbs=5 * 2 * 128) == INVALID       # summaries too short


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from block_sparse_attention_41_amd import ops
    monkeypatch.setattr(ops, "_lib", None)
    monkeypatch.setattr(ops, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        ops.lib()


@pytest.mark.parametrize("which", ["batch", "head_dim", "row_stride"])
def test_select_binding_rejects_mismatched_summaries(which):
    """The selection binding checks the summaries against q before any launch: a summary
    table of another batch size or head dim, or with rows that are not contiguous, would
    make the kernel read outside it or score the wrong rows."""
    import torch
    from block_sparse_attention_41_amd import ops
    q = torch.zeros((2, 128, 4, 64), dtype=torch.bfloat16)
    if which == "batch":
        summ = torch.zeros((1, 8, 2, 64))
    elif which == "head_dim":
        summ = torch.zeros((2, 8, 2, 32))
    else:
        summ = torch.zeros((2, 8, 4, 64))[:, :, ::2]       # kv heads two rows apart
    for fn in (ops.hga_select_topk, ops.hga_select_topk_shared):
        with pytest.raises(ValueError):
            fn(q, summ, 64, 4)


def test_s2attn_bwd_noalloc_rejects_on_the_host(lib):
    """The no-workspace backward checks everything before touching the runtime: bad
    arguments, and sizes whose row statistics exceed its static array (8 MiB:
    B * H * N <= 2^20 rows)."""
    def call(B=1, N=1024, H=4, Hkv=4, d=64, G=256, ptr=A):
        return lib.s2attn_bwd_noalloc(ptr, A, A, A, A, A, A, A, A, B, N, H, Hkv, d, G, 1, 0.125, None)
    assert call(ptr=None) == INVALID
    assert call(ptr=MIS) == INVALID
    assert call(N=1000) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert lib.s2attn_bwd_workspace_bytes(1, 65536, 32, 8, 128) == 2 * 65536 * 32 * 4      # 16 MiB
    assert call(B=1, N=65536, H=32, Hkv=8, d=128, G=8192) == WORKSPACE      # 16 MiB of statistics
    assert call(B=2, N=32768, H=32, Hkv=32, d=128, G=8192) == WORKSPACE


def test_hga_fwd_select_shared_rejects(lib):
    def call(summ=A, sbs=1 << 20, B=1, S=256, T=1024, H=8, Hkv=2, d=128, chunk=128, topk=4, qptr=A):
        return lib.hga_fwd_select_shared(qptr, A, A, 1 << 20, A, A, 1 << 22, summ, sbs, A, A, A, B, S, H, Hkv, d, T,
                                         chunk, 64, topk, 0.088, None)
    assert call(qptr=None) == INVALID
    assert call(summ=None) == INVALID                 # history present, no summaries
    assert call(summ=MIS) == INVALID
    assert call(B=2, sbs=8) == INVALID                # summaries of two batches overlap
    assert call(T=1000) == INVALID                    # T % chunk
    assert call(topk=65) == UNSUPPORTED
    assert call(d=96) == UNSUPPORTED


def test_hga_stage_selected_rejects(lib):
    text = open(HEADER, encoding="utf-8").read()
    S2A_STAGE_MAX_CHUNKS = int(re.search(r"#define S2A_STAGE_MAX_CHUNKS (\d+)", text).group(1))
    def call(idx=A, lists=8, nqb=4, topk=4, T=2048, chunk=128, max_slots=16, B=1, Hkv=2, d=128, hbs=1 << 20,
             sbs=1 << 20, out=A):
        return lib.hga_stage_selected(idx, lists, nqb, topk, A, A, hbs, T, out, out, out, A, A, sbs, max_slots, B,
                                      Hkv, d, chunk, None)
    assert call(idx=None) == INVALID
    assert call(out=MIS) == INVALID
    assert call(lists=7) == INVALID                   # lists % Hkv
    assert call(T=2000) == INVALID                    # T % chunk
    assert call(max_slots=15) == INVALID              # C = 16 chunks, 4 lists x 4 blocks x 4 can name all
    assert call(lists=2, max_slots=15) == INVALID     # shared lists name at most 16 too
    assert call(lists=2, nqb=1, max_slots=3) == INVALID
    assert call(B=2, hbs=8) == INVALID                # host batches overlap
    assert call(chunk=96, T=1920) == UNSUPPORTED
    assert call(topk=65) == UNSUPPORTED
    assert call(d=96) == UNSUPPORTED
    assert call(T=128 * (S2A_STAGE_MAX_CHUNKS + 1), max_slots=64) == UNSUPPORTED


def test_hga_detach_segment_rejects(lib):
    def call(seg=A, host=A, summ=A, S=256, T=512, chunk=128, d=128):
        return lib.hga_detach_segment(seg, seg, 1 << 20, host, host, 1 << 20, summ, 1 << 20, 1, S, 2, d, T, chunk,
                                      None)
    assert call(seg=None) == INVALID
    assert call(host=None) == INVALID
    assert call(summ=MIS) == INVALID
    assert call(S=200) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(S=0) == 0                             # nothing to detach


def test_hga_stage_update_rejects(lib):
    text = open(HEADER, encoding="utf-8").read()
    max_slots_cap = int(re.search(r"#define S2A_STAGE_MAX_SLOTS (\d+)", text).group(1))

    def call(idx=A, lists=8, T=2048, max_slots=16, out=A, chunk=128):
        return lib.hga_stage_update(idx, lists, 4, 4, A, A, 1 << 20, T, out, out, out, out, out, A, A, 1 << 20,
                                    max_slots, 1, 2, 128, chunk, None)
    assert call(idx=None) == INVALID
    assert call(out=MIS) == INVALID
    assert call(lists=7) == INVALID
    assert call(max_slots=15) == INVALID
    assert call(max_slots=max_slots_cap + 1) == UNSUPPORTED
    assert call(chunk=96, T=1920) == UNSUPPORTED
