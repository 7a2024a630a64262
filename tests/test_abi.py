"""The C ABI of libwkv7 on the host: it loads, exports every declared symbol,
and rejects bad arguments before anything reaches the GPU (CPU only).

The rejection tests pass made-up device addresses; every case is built to
fail a host-side check, so no kernel is ever launched.  They are skipped
where a GPU is present (the GPU suite repeats them with real allocations).
"""
import ctypes
import os
import re

import pytest

import linear_rnn_lm_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wkv7.h")

OK, ERR_ARG, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_ALIAS, ERR_HIP, ERR_WS = range(8)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wkv7_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = L.lib()
    names = declared_functions()
    assert {"wkv7_fwd", "wkv7_bwd", "wkv7_fwd_sequential", "wkv7_bwd_workspace_bytes", "wkv7_chunk_prepare",
            "wkv7_fwd_scan", "wkv7_bwd_scan", "wkv7_bwd_inputs", "wkv7_chunk_ops_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in wkv7.h but not exported"


def test_library_has_no_unexpected_exports():
    out = os.popen(f"nm -D --defined-only {L.LIB_PATH}").read()
    exported = set(re.findall(r"\bT (wkv7_[a-z0-9_]+)\b", out))
    assert exported == set(declared_functions())


def test_queries():
    lib = L.lib()
    assert lib.wkv7_version() >= 100
    assert lib.wkv7_chunk_len() == 32
    assert [L.num_chunks(t) for t in (0, 1, 31, 32, 33, 64, 1024)] == [0, 1, 1, 1, 2, 2, 32]
    per_chunk = 32 * 32 * 4 + 36864          # (I - L)^-1 in fp32 + the transition operands
    assert L.chunk_ops_bytes(12, 1024, 6) == 12 * 6 * 32 * per_chunk
    assert L.workspace_bytes(12, 1024, 6) == 12 * 6 * 32 * 64 * 64 * 4 + L.chunk_ops_bytes(12, 1024, 6)
    assert L.workspace_bytes(1, 1, 1) == 64 * 64 * 4 + per_chunk
    assert L.fwd_workspace_bytes(1, 1, 1) == 0
    assert L.fwd_workspace_bytes(2, 33, 3) == 2 * 3 * 2 * per_chunk
    assert L.chunk_ops_bytes(1, 10, 1, 32) == 0
    assert L.workspace_bytes(1, 0, 1) == 0
    assert L.workspace_bytes(1, 10, 1, 32) == 0
    for s in range(8):
        assert lib.wkv7_status_str(s).startswith(b"WKV7")
    assert b"unknown" in lib.wkv7_status_str(99)


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


needs_no_gpu = pytest.mark.skipif(_gpu_present(), reason="made-up device pointers are only used without a GPU")

BASE = 1 << 40          # a made-up, 16-byte-aligned device address
MB = 1 << 20


def fake(n):            # distinct non-overlapping fake buffers, 64 MiB apart
    return BASE + n * 64 * MB


def fwd_args(**over):
    a = dict(B=1, T=64, H=1, D=64, dt=1, r=fake(0), w=fake(1), k=fake(2), v=fake(3), a=fake(4),
             b=fake(5), h0=None, y=fake(6), ck=fake(7), hT=fake(8), ops=fake(10), ws=fake(11), wsb=1 << 20)
    a.update(over)
    return a


def call_fwd(fn="wkv7_fwd", **over):
    a = fwd_args(**over)
    f = getattr(L.lib(), fn)
    head = (a["B"], a["T"], a["H"], a["D"], a["dt"], a["r"], a["w"], a["k"], a["v"], a["a"], a["b"])
    if fn in ("wkv7_fwd", "wkv7_fwd_proj"):
        return f(*head, a["h0"], a["y"], a["ck"], a["hT"], a["ws"], a["wsb"], None)
    if fn == "wkv7_fwd_scan":
        return f(*head[:5], a["v"], a["ops"], a["h0"], a["y"], a["ck"], a["hT"], None)
    return f(*head, a["h0"], a["y"], a["ck"], a["hT"], None)


@needs_no_gpu
@pytest.mark.parametrize("fn", ["wkv7_fwd", "wkv7_fwd_proj", "wkv7_fwd_sequential", "wkv7_fwd_scan"])
def test_fwd_rejects_bad_arguments(fn):
    c = lambda **o: call_fwd(fn, **o)
    assert c(D=32) == ERR_SHAPE
    assert c(T=0) == ERR_SHAPE
    assert c(B=0) == ERR_SHAPE
    assert c(H=-1) == ERR_SHAPE
    assert c(T=1 << 20, H=16) == ERR_SHAPE           # a 4 GiB fp32 token tensor
    assert c(dt=7) == ERR_DTYPE
    assert c(v=None) == ERR_ARG
    assert c(y=None, ck=None, hT=None) == ERR_ARG
    assert c(v=fake(3) + 4) == ERR_ALIGN
    assert c(h0=fake(9) + 8) == ERR_ALIGN
    assert c(y=fake(3)) == ERR_ALIAS                 # y on top of v
    assert c(y=fake(3) + 4096) == ERR_ALIAS          # y overlapping the tail of v
    assert c(hT=fake(6)) == ERR_ALIAS                # hT inside y
    assert c(ck=fake(6) + 16) == ERR_ALIAS           # ckpt overlapping y
    assert c(h0=fake(9), hT=fake(9) + 64) == ERR_ALIAS  # hT overlapping h0 but not equal
    if fn != "wkv7_fwd_scan":
        assert c(r=None) == ERR_ARG
        assert c(b=None) == ERR_ARG
        assert c(w=fake(1) + 4) == ERR_ALIGN
        assert c(y=fake(0)) == ERR_ALIAS             # y on top of r
        assert c(y=fake(5) + 4096) == ERR_ALIAS      # y overlapping the tail of b
    if fn in ("wkv7_fwd", "wkv7_fwd_proj"):
        assert c(ws=None) == ERR_WS
        assert c(wsb=1000) == ERR_WS
        assert c(ws=fake(11) + 4) == ERR_ALIGN
        assert c(ws=fake(6)) == ERR_ALIAS                # workspace on top of y
    if fn == "wkv7_fwd_scan":
        assert c(ops=None) == ERR_ARG
        assert c(ops=fake(10) + 8) == ERR_ALIGN
        assert c(y=fake(10)) == ERR_ALIAS                # y on top of the chunk operands


@needs_no_gpu
def test_bwd_division_rejects_bad_arguments():
    lib = L.lib()

    def c(**o):
        a = dict(B=1, T=64, H=1, D=64, dt=1, dy=fake(0), dhT=None, r=fake(1), w=fake(2), k=fake(3), v=fake(4),
                 a=fake(5), b=fake(6), ck=fake(7), hT=fake(16), restart=1, dr=fake(8), dw=fake(9), dk=fake(10),
                 dv=fake(11), da=fake(12), db=fake(13), dh0=fake(14))
        a.update(o)
        return lib.wkv7_bwd_division(a["B"], a["T"], a["H"], a["D"], a["dt"], a["dy"], a["dhT"], a["r"], a["w"],
                                     a["k"], a["v"], a["a"], a["b"], a["ck"], a["hT"], a["restart"], a["dr"],
                                     a["dw"], a["dk"], a["dv"], a["da"], a["db"], a["dh0"], None)

    assert c(D=16) == ERR_SHAPE
    assert c(T=0) == ERR_SHAPE
    assert c(dt=3) == ERR_DTYPE
    assert c(restart=2) == ERR_ARG
    assert c(ck=None) == ERR_ARG                      # restarting needs the checkpoints
    assert c(hT=None) == ERR_ARG
    assert c(dy=None) == ERR_ARG
    assert c(da=None) == ERR_ARG
    assert c(dv=fake(11) + 4) == ERR_ALIGN
    assert c(dr=fake(0)) == ERR_ALIAS                 # dr on dy
    assert c(dh0=fake(16)) == ERR_ALIAS               # dh0 on hT


@needs_no_gpu
def test_chunk_prepare_rejects_bad_arguments():
    lib = L.lib()
    c = lambda B=1, T=64, H=1, D=64, dt=1, r=fake(4), w=fake(0), k=fake(5), a=fake(1), b=fake(2), out=fake(3): \
        lib.wkv7_chunk_prepare(B, T, H, D, dt, r, w, k, a, b, out, None)
    assert c(D=48) == ERR_SHAPE
    assert c(T=0) == ERR_SHAPE
    assert c(dt=5) == ERR_DTYPE
    assert c(out=None) == ERR_ARG
    assert c(a=None) == ERR_ARG
    assert c(k=None) == ERR_ARG
    assert c(out=fake(3) + 2) == ERR_ALIGN
    assert c(out=fake(1)) == ERR_ALIAS
    assert c(out=fake(5) - 64) == ERR_ALIAS          # operands running into k


@needs_no_gpu
@pytest.mark.parametrize("fn", ["wkv7_bwd", "wkv7_bwd_proj"])
def test_bwd_rejects_bad_arguments(fn):
    lib = L.lib()
    B, T, H, D = 1, 64, 1, 64
    ws = L.workspace_bytes(B, T, H)

    def c(**o):
        a = dict(B=B, T=T, H=H, D=D, dt=1, dy=fake(0), dhT=None, r=fake(1), w=fake(2), k=fake(3),
                 v=fake(4), a=fake(5), b=fake(6), ck=fake(7), dr=fake(8), dw=fake(9), dk=fake(10),
                 dv=fake(11), da=fake(12), db=fake(13), dh0=fake(14), ws=fake(15), wsb=ws)
        a.update(o)
        return getattr(lib, fn)(a["B"], a["T"], a["H"], a["D"], a["dt"], a["dy"], a["dhT"], a["r"], a["w"],
                            a["k"], a["v"], a["a"], a["b"], a["ck"], a["dr"], a["dw"], a["dk"], a["dv"],
                            a["da"], a["db"], a["dh0"], a["ws"], a["wsb"], None)

    def cs(**o):
        a = dict(dt=1, dy=fake(0), dhT=None, inv=fake(16), dck=fake(17), dv=fake(11), dh0=None, T=T)
        a.update(o)
        return lib.wkv7_bwd_scan(B, a["T"], H, D, a["dt"], a["dy"], a["dhT"], a["inv"], a["dck"], a["dv"],
                                 a["dh0"], None)

    def ci(**o):
        a = dict(dt=1, dy=fake(0), dhT=None, r=fake(1), w=fake(2), k=fake(3), v=fake(4), a=fake(5), b=fake(6),
                 inv=fake(16), ck=fake(7), dck=fake(17), dr=fake(8), dw=fake(9), dk=fake(10), da=fake(12),
                 db=fake(13))
        a.update(o)
        return lib.wkv7_bwd_inputs(B, T, H, D, a["dt"], a["dy"], a["dhT"], a["r"], a["w"], a["k"], a["v"],
                                   a["a"], a["b"], a["inv"], a["ck"], a["dck"], a["dr"], a["dw"], a["dk"],
                                   a["da"], a["db"], None)

    assert cs(T=0) == ERR_SHAPE
    assert cs(dt=9) == ERR_DTYPE
    assert cs(inv=None) == ERR_ARG
    assert cs(dck=None) == ERR_ARG
    assert cs(dv=fake(11) + 4) == ERR_ALIGN
    assert cs(dck=fake(16)) == ERR_ALIAS              # dh_ckpt on the chunk operands
    assert cs(dh0=fake(0) + 64) == ERR_ALIAS          # dh0 inside dy
    assert cs(dv=fake(0)) == ERR_ALIAS                # dv on dy
    assert ci(inv=None) == ERR_ARG
    assert ci(dck=None) == ERR_ARG
    assert ci(dr=fake(17)) == ERR_ALIAS               # dr on dh_ckpt
    assert ci(db=fake(7) + 16) == ERR_ALIAS           # db inside the checkpoints

    assert c(D=16) == ERR_SHAPE
    assert c(T=0) == ERR_SHAPE
    assert c(T=1 << 24) == ERR_SHAPE                  # token tensors past 4 GiB (fp32)
    assert cs(T=1 << 24) == ERR_SHAPE
    assert c(dt=2) == ERR_DTYPE
    assert c(dy=None) == ERR_ARG
    assert c(ck=None) == ERR_ARG
    assert c(db=None) == ERR_ARG
    assert c(ws=None) == ERR_WS
    assert c(wsb=ws - 4) == ERR_WS
    assert c(dv=fake(11) + 2) == ERR_ALIGN
    assert c(ws=fake(15) + 8) == ERR_ALIGN
    assert c(dr=fake(0)) == ERR_ALIAS                # dr on dy
    assert c(dw=fake(8) + 64) == ERR_ALIAS           # dw overlapping dr
    assert c(ws=fake(7)) == ERR_ALIAS                # workspace on the checkpoints
    assert c(dh0=fake(16), dhT=fake(16)) == ERR_ALIAS


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        L.lib()


def test_segment_spans():
    from linear_rnn_lm_amd.segments import _segments
    assert _segments(100, 32) == [(0, 32), (32, 64), (64, 96), (96, 100)]
    assert _segments(64, 64) == [(0, 64)]
    assert _segments(5, 100) == [(0, 5)]
    with pytest.raises(ValueError):
        _segments(10, 0)


def test_checkpoint_addressing_has_no_32_bit_limit():
    """Checkpoints and state gradients are addressed per chunk with 64-bit
    bases: one head of 16,777,215 tokens (524,288 chunks, 8 GiB of
    checkpoints) is a valid shape; only the token tensors' 32-bit byte
    offsets bound T (the next token past 2^24 per head is refused)."""
    T = (1 << 24) - 1
    nc = L.num_chunks(T)
    per_chunk = 32 * 32 * 4 + 36864
    assert nc == 1 << 19
    assert L.chunk_ops_bytes(1, T, 1) == nc * per_chunk
    assert L.workspace_bytes(1, T, 1) == nc * 64 * 64 * 4 + nc * per_chunk
    assert L.workspace_bytes(1, T + 1, 1) == 0          # 4 GiB fp32 token tensor: refused
    assert L.workspace_bytes(1, (1 << 23) + 40, 1) > (1 << 32)


@needs_no_gpu
def test_fwd_accepts_long_single_head_on_the_host():
    """B = H = 1 with T above 2^23 passes every host check of wkv7_fwd (made-up
    buffers of the right sizes, 64 GiB apart); without a GPU the launch then
    fails, never the shape check."""
    T = (1 << 23) + 40
    big = lambda n: BASE + n * (64 << 30)
    ws = L.fwd_workspace_bytes(1, T, 1)
    st = call_fwd("wkv7_fwd", T=T, r=big(0), w=big(1), k=big(2), v=big(3), a=big(4), b=big(5), y=big(6),
                  ck=big(7), hT=big(8), ws=big(9), wsb=ws)
    assert st == ERR_HIP


@needs_no_gpu
def test_entry_points_from_two_threads():
    """Queries and launch paths called from two host threads at once (ctypes
    releases the GIL): every call returns the same status it returns alone
    (the launch fails for want of a GPU, after the host checks)."""
    import threading
    lib = L.lib()
    alone = (call_fwd("wkv7_fwd"), call_fwd("wkv7_fwd_sequential"), call_fwd("wkv7_fwd_scan"))
    assert alone == (ERR_HIP, ERR_HIP, ERR_HIP)
    results, errors = [], []

    def worker():
        try:
            for _ in range(200):
                got = (lib.wkv7_num_chunks(1000), lib.wkv7_bwd_workspace_bytes(2, 100, 3, 64),
                       lib.wkv7_status_str(6), call_fwd("wkv7_fwd"), call_fwd("wkv7_fwd_sequential"),
                       call_fwd("wkv7_fwd_scan"), call_fwd("wkv7_fwd", D=32))
                results.append(got)
        except Exception as e:  # pragma: no cover
            errors.append(e)

    ts = [threading.Thread(target=worker) for _ in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors
    expect = (32, lib.wkv7_bwd_workspace_bytes(2, 100, 3, 64), lib.wkv7_status_str(6), ERR_HIP, ERR_HIP, ERR_HIP,
              ERR_SHAPE)
    assert len(results) == 400 and all(r == expect for r in results)


@needs_no_gpu
def test_fwd_noalloc_host_checks():
    """wkv7_fwd_noalloc: wkv7_fwd's checks, then a refusal of operands larger
    than the library's static scratch, both before any launch."""
    lib = L.lib()
    cap = lib.wkv7_fwd_noalloc_max_bytes()
    assert cap == 128 << 20

    def c(**o):
        a = fwd_args(**o)
        return lib.wkv7_fwd_noalloc(a["B"], a["T"], a["H"], a["D"], a["dt"], a["r"], a["w"], a["k"], a["v"],
                                    a["a"], a["b"], a["h0"], a["y"], a["ck"], a["hT"], None)

    assert c(D=32) == ERR_SHAPE
    assert c(v=None) == ERR_ARG
    assert c(y=fake(3)) == ERR_ALIAS
    assert L.fwd_workspace_bytes(16, 1024, 8) > cap
    big = lambda n: BASE + n * (1 << 30)
    assert c(B=16, T=1024, H=8, r=big(0), w=big(1), k=big(2), v=big(3), a=big(4), b=big(5), y=big(6),
             ck=big(7), hT=big(8)) == ERR_WS
    assert c() == ERR_HIP           # fits: passes the host checks, then no GPU to launch on
