"""The C-ABI library on the host (no GPU): exports, the host container codec
against the oracle codec, and every argument/format/code error path, all of
which are decided before any launch."""
import ctypes
import re

import numpy as np
import pytest

import ternary_quantized_moe_amd as tq
from ternary_quantized_moe_amd import binding
from golden_io import read_block_fixture
from oracle import codec
from synthetic import CONFIGS, LayerGen

PQ2_0, PTQ1_0 = 142, 143


def test_library_exports_every_declared_symbol():
    header = open(binding.__file__.replace("ternary_quantized_moe_amd/binding.py", "include/moe_ternary.h")).read()
    declared = set(re.findall(r"^\s*(?:int64_t|int32_t|const char\*)\s+(moe_\w+)\(", header, re.M))
    assert declared == set(binding.EXPORTS)
    L = tq.lib()
    for name in declared:
        assert hasattr(L, name)


def test_block_sizes():
    assert tq.block_bytes(PQ2_0) == 34 and tq.block_bytes(PTQ1_0) == 28
    assert tq.block_bytes(42) == -1
    assert tq.packed_bytes(PQ2_0, 256) == 68 and tq.packed_bytes(PTQ1_0, 100) == -1


@pytest.mark.parametrize("fmt,name", [(PQ2_0, "pq2_0_block.txt"), (PTQ1_0, "ptq1_0_block.txt")])
def test_golden_blocks(fmt, name):
    trits, scale, data = read_block_fixture(name)
    assert tq.pack(fmt, trits, np.array([scale], np.uint16)).tobytes() == data.tobytes()
    t2, s2 = tq.unpack(fmt, data, 128)
    assert np.array_equal(t2, trits) and int(s2[0]) == scale


@pytest.mark.parametrize("fmt", [PQ2_0, PTQ1_0])
def test_pack_matches_oracle_codec_bitwise(fmt):
    g = LayerGen(CONFIGS["olmoe"])
    for e in (0, 17):
        for t, s in zip(g.expert_trits(e), g.expert_scales(e)):
            mine = tq.pack(fmt, t, s)
            ref = codec.pack(fmt, t, s)
            assert mine.tobytes() == ref.tobytes()
            tt, ss = tq.unpack(fmt, mine, t.size)
            assert np.array_equal(tt, t.reshape(-1)) and np.array_equal(ss, s.reshape(-1))


def test_unpack_exhaustive_pq2_bytes():
    blocks = np.zeros((256, 34), np.uint8)
    blocks[:, 5] = np.arange(256)
    for v in range(256):
        raw = blocks[v]
        valid = all(((v >> (2 * i)) & 3) != 2 for i in range(4))
        if valid:
            t, s = tq.unpack(PQ2_0, raw, 128)
            t2, s2 = codec.unpack(PQ2_0, raw, 128)
            assert np.array_equal(t, t2)
        else:
            with pytest.raises(tq.MoeError) as ei:
                tq.unpack(PQ2_0, raw, 128)
            assert ei.value.name == "MOE_E_CODE" and "group 0, byte 5" in str(ei.value)


def test_unpack_exhaustive_ptq1_bytes():
    for pos, lim in ((3, 243), (25, 81)):
        for v in range(256):
            raw = np.zeros(56, np.uint8)
            raw[28 + pos] = v
            if v < lim:
                t, _ = tq.unpack(PTQ1_0, raw, 256)
                t2, _ = codec.unpack(PTQ1_0, raw, 256)
                assert np.array_equal(t, t2)
            else:
                with pytest.raises(tq.MoeError) as ei:
                    tq.unpack(PTQ1_0, raw, 256)
                assert ei.value.name == "MOE_E_CODE" and f"group 1, byte {pos}" in str(ei.value)


def test_codec_error_codes():
    t = np.zeros(256, np.int8)
    s = np.full(2, 0x3C00, np.uint16)
    with pytest.raises(tq.MoeError) as ei:
        tq.pack(42, t, s)
    assert ei.value.name == "MOE_E_FORMAT" and "142" in str(ei.value) and "143" in str(ei.value)
    with pytest.raises(tq.MoeError) as ei:
        tq.pack(PQ2_0, np.zeros(100, np.int8), s[:0])
    assert ei.value.name == "MOE_E_SHAPE"
    bad = t.copy()
    bad[7] = 3
    with pytest.raises(tq.MoeError) as ei:
        tq.pack(PTQ1_0, bad, s)
    assert ei.value.name == "MOE_E_ARG"
    for nf in (0x7C00, 0xFE00):
        with pytest.raises(tq.MoeError) as ei:
            tq.pack(PQ2_0, t, np.array([0x3C00, nf], np.uint16))
        assert ei.value.name == "MOE_E_NONFINITE"
    L = tq.lib()
    out = np.zeros(10, np.uint8)
    rc = L.moe_pack(PQ2_0, t.ctypes.data, s.ctypes.data, 256, out.ctypes.data, 10)
    assert rc == -6
    raw = np.zeros(28, np.uint8)
    raw[27] = 0x7C
    with pytest.raises(tq.MoeError) as ei:
        tq.unpack(PTQ1_0, raw, 128)
    assert ei.value.name == "MOE_E_NONFINITE"


def _fake_banks(d=256, f=128, E=8, S=0, fmts=None, offsets=None, nbytes=None, layout=binding.BANKS_TILE_MAJOR):
    fmts = np.full(E + S, PQ2_0, np.uint8) if fmts is None else np.asarray(fmts, np.uint8)
    size = 3 * d * f // 128 * 34
    offsets = np.arange(E + S, dtype=np.int64) * size if offsets is None else np.asarray(offsets, np.int64)
    keep = (fmts, offsets)
    c = binding.ExpertBanksC(d, f, E, S, 0x1000, nbytes if nbytes is not None else size * (E + S) + 16, 0x2000,
                             0x3000, offsets.ctypes.data, fmts.ctypes.data, layout)
    return c, keep


def _forward_rc(c, T=4, k=2, r=16, x=0x10000, y=0x20000, ws=0x40000, ws_bytes=1 << 40, A=0x50000, B=0x60000,
                router=0x70000):
    L = tq.lib()
    return L.moe_ternary_forward(x, T, router, None, ctypes.byref(c), A, B, r, k, y, ws, ws_bytes, None)


def test_forward_validation_happens_before_launch():
    L = tq.lib()
    c, keep = _fake_banks()
    assert _forward_rc(c, k=9) == -3                   # k > E
    assert _forward_rc(c, k=0) == -3
    assert _forward_rc(c, r=12) == -3                  # rank not a multiple of 8
    assert _forward_rc(c, A=None) == -1                # A without B
    assert _forward_rc(c, x=0x10000, y=0x10000) == -1  # aliasing
    assert _forward_rc(c, ws_bytes=10) == -6
    assert _forward_rc(c, ws=0x40010) == -1            # misaligned workspace
    assert _forward_rc(c, T=0) == 0                    # no-op, nothing launched
    assert "" == L.moe_last_error().decode()
    c2, keep2 = _fake_banks(d=200)
    assert _forward_rc(c2) == -3
    c3, keep3 = _fake_banks(fmts=[142] * 7 + [99])
    assert _forward_rc(c3) == -2
    assert "bank 7" in L.moe_last_error().decode()
    c4, keep4 = _fake_banks(nbytes=100)
    assert _forward_rc(c4) == -6
    c6, keep6 = _fake_banks(nbytes=8 * 3 * 256 * 128 // 128 * 34 + 15)  # one byte short of the slack
    assert _forward_rc(c6) == -6 and "slack" in L.moe_last_error().decode()
    c5, keep5 = _fake_banks(offsets=np.arange(8) * 2)
    assert _forward_rc(c5) == -1                      # offsets not multiples of 16
    c7, keep7 = _fake_banks(offsets=np.arange(8) * (3 * 256 * 128 // 128 * 34) + 4, nbytes=8 * 3 * 256 * 128 // 128 * 34 + 20)
    assert _forward_rc(c7) == -1 and "multiple of 16" in L.moe_last_error().decode()
    assert L.moe_workspace_bytes(ctypes.byref(c), 16, 2, 16) > 0
    assert L.moe_workspace_bytes(None, 16, 2, 16) == -1


def test_banks_must_declare_the_tile_major_order():
    """Banks in moe_pack's row-major block order, or with no declared order,
    are refused before any launch."""
    L = tq.lib()
    c, keep = _fake_banks(layout=binding.BANKS_ROW_MAJOR)
    assert _forward_rc(c) == -1 and "moe_tile_container" in L.moe_last_error().decode()
    c, keep = _fake_banks(layout=0)
    assert _forward_rc(c) == -1 and "MOE_BANKS_TILE_MAJOR" in L.moe_last_error().decode()
    assert L.moe_ternary_forward_noalloc(0x10000, 4, 0x70000, None, ctypes.byref(c), None, None, 0, 2, 0x20000,
                                         None) == -1
    c, keep = _fake_banks()
    assert _forward_rc(c, T=0) == 0



def test_noalloc_forward_validation():
    """moe_ternary_forward_noalloc checks its arguments and the size of its
    scratch on the host, before it touches the device."""
    L = tq.lib()
    c, keep = _fake_banks()

    def rc(T=4, k=2, r=16, A=0x50000, B=0x60000):
        return L.moe_ternary_forward_noalloc(0x10000, T, 0x70000, None, ctypes.byref(c), A, B, r, k, 0x20000, None)
    assert rc(k=9) == -3 and rc(k=0) == -3
    assert rc(r=-8) == -1
    assert rc(T=0) == 0
    need = L.moe_workspace_bytes(ctypes.byref(c), 1 << 20, 2, 16)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    assert rc(T=1 << 20) == -6 and "scratch" in L.moe_last_error().decode()
    assert L.moe_ternary_forward_noalloc(0x10000, 4, 0x70000, None, None, None, None, 0, 2, 0x20000, None) == -1


def test_ternary_forward_validation():
    """moe_ternary_forward_q checks on the host, before any launch."""
    L = tq.lib()
    c, keep = _fake_banks()

    def rc(r=128, A=0x50000, B=0x60000, delta=None, k=2):
        return L.moe_ternary_forward_q(0x10000, 4, 0x70000, delta, ctypes.byref(c), A, B, r, k, 0x20000, 0x40000,
                                       1 << 40, None)
    assert rc(r=16) == -3 and "multiple of 128" in L.moe_last_error().decode()   # B rows of 16
    assert rc(B=None) == -1                                                        # A without B
    assert rc(r=0) == -1                                                           # rank 0 with A, B
    assert rc(A=0x50001) == -1 and "2-byte" in L.moe_last_error().decode()
    assert rc(delta=0x30001, A=None, B=None, r=0) == -1
    assert rc(k=9) == -3


def test_factored_forward_validation():
    """moe_ternary_forward_factored checks on the host, before any launch."""
    L = tq.lib()
    c, keep = _fake_banks()

    def rc(rd=64, U=0x50000, V=0x60000, T=4, ws_bytes=1 << 40):
        return L.moe_ternary_forward_factored(0x10000, T, 0x70000, U, V, rd, ctypes.byref(c), None, None, 0, 2,
                                              0x20000, 0x40000, ws_bytes, None)
    assert rc(rd=12) == -3 and rc(rd=0) == -3 and rc(rd=2048) == -3
    assert rc(U=None) == -1 and rc(V=None) == -1
    assert rc(U=0x50008) == -1 and rc(V=0x60002) == -1     # U 16-byte, V 4-byte aligned
    assert rc(ws_bytes=4096) == -6
    assert rc(T=0) == 0
    assert L.moe_workspace_bytes_factored(ctypes.byref(c), 16, 2, 0, 64) > L.moe_workspace_bytes(ctypes.byref(c), 16, 2, 0)
    assert L.moe_workspace_bytes_factored(ctypes.byref(c), 16, 2, 0, 0) == -1


def test_draft_head_validation():
    """moe_draft_head checks on the host, before any launch."""
    L = tq.lib()
    args = dict(hid=0x10000, emb=0x20000, T=4, h=256, m=512, w1=0x30000, b1=None, w2=0x40000, b2=None, y=0x50000,
                ws=0x60000, ws_bytes=1 << 40)

    def rc(**kw):
        a = dict(args, **kw)
        return L.moe_draft_head(a["hid"], a["emb"], a["T"], a["h"], a["m"], a["w1"], a["b1"], a["w2"], a["b2"], a["y"],
                                a["ws"], a["ws_bytes"], None)
    assert rc(h=200) == -3 and rc(m=100) == -3 and rc(T=-1) == -3
    assert rc(w2=None) == -1 and rc(emb=None) == -1
    assert rc(ws=0x60010) == -1                        # workspace not 256-byte aligned
    assert rc(w1=0x30002) == -1                        # weights not 4-byte aligned
    assert rc(hid=0x10008) == -1                       # inputs not 16-byte aligned
    assert rc(ws_bytes=1024) == -6
    assert rc(T=0) == 0
    assert L.moe_draft_head_workspace_bytes(4, 256, 512) > 0
    assert L.moe_draft_head_workspace_bytes(-1, 256, 512) == -1

def test_lowrank_validation():
    """moe_lowrank_apply checks on the host, before any launch."""
    L = tq.lib()
    args = dict(x=0x10000, yin=None, T=4, d=256, A=0x30000, Aq=None, B=0x40000, Bq=None, r=64, y=0x50000,
                ws=0x60000, ws_bytes=1 << 40)

    def rc(**kw):
        a = dict(args, **kw)
        return L.moe_lowrank_apply(a["x"], a["yin"], a["T"], a["d"], a["A"], a["Aq"], a["B"], a["Bq"], a["r"],
                                   a["y"], a["ws"], a["ws_bytes"], None)
    assert rc(d=200) == -3 and rc(r=12) == -3 and rc(r=8192) == -3 and rc(T=-1) == -3
    assert rc(B=None, Bq=0x70000) == -3                # a ternary B needs r % 128 == 0
    assert rc(A=None) == -1 and rc(Aq=0x70000) == -1   # exactly one form of each
    assert rc(x=None) == -1 and rc(y=0x10000) == -1    # y aliasing x
    assert rc(ws=0x60010) == -1
    assert rc(yin=0x20008) == -1 and rc(A=0x30002) == -1
    assert rc(ws_bytes=1024) == -6
    assert rc(T=0) == 0
    assert L.moe_lowrank_workspace_bytes(4, 256, 64) > 0
    assert L.moe_lowrank_workspace_bytes(4, 0, 64) == -1


def test_route_validation():
    L = tq.lib()
    assert L.moe_route(0x1000, 4, 100, 8, 0x2000, None, 2, 1, 1, 1, 1, 1, 1, 0x4000, 1 << 30, None) == -3
    assert L.moe_route(0x1000, 4, 256, 8, 0x2000, None, 9, 1, 1, 1, 1, 1, 1, 0x4000, 1 << 30, None) == -3
    assert L.moe_route(0x1000, 4, 256, 2000, 0x2000, None, 2, 1, 1, 1, 1, 1, 1, 0x4000, 1 << 30, None) == -3
    assert L.moe_route(0x1000, 4, 256, 8, 0x2000, None, 2, 1, 1, 1, 1, 1, 1, 0x4000, 16, None) == -6
    assert L.moe_route(0x1000, 0, 256, 8, 0x2000, None, 2, 1, 1, 1, 1, 1, 1, 0x4000, 0, None) == 0
    assert L.moe_unpack_device(99, 1, 128, 1, 1, None) == -2
    assert L.moe_unpack_device(142, 1, 100, 1, 1, None) == -3


def test_route_factored_validation():
    """moe_route_factored checks on the host, before any launch."""
    L = tq.lib()

    def rc(T=4, d=256, E=8, U=0x50000, V=0x60000, rd=64, k=2, ws_bytes=1 << 30):
        return L.moe_route_factored(0x1000, T, d, E, 0x2000, U, V, rd, k, 1, 1, 1, 1, 1, 1, 0x4000, ws_bytes, None)
    assert rc(d=100) == -3 and rc(k=9) == -3
    assert rc(rd=12) == -3 and rc(rd=0) == -3 and rc(rd=2048) == -3
    assert rc(U=None) == -1 and rc(V=None) == -1
    assert rc(U=0x50008) == -1 and rc(V=0x60002) == -1
    assert rc(ws_bytes=16) == -6
    assert rc(T=0) == 0
    assert L.moe_route_workspace_bytes_factored(16, 256, 8, 2, 64) > L.moe_route_workspace_bytes(16, 256, 8, 2)
    assert L.moe_route_workspace_bytes_factored(16, 256, 8, 2, 0) == -1


def test_quantize_validation():
    """Argument checks of moe_quantize_device happen on the host, before any launch."""
    L = tq.lib()
    w, out = 0x10000, 0x40000
    assert L.moe_quantize_device(99, 0, w, 256, out, None, None) == -2
    assert L.moe_quantize_device(142, 2, w, 256, out, None, None) == -1          # unknown method
    assert L.moe_quantize_device(142, 0, w, 100, out, None, None) == -3          # not a multiple of 128
    assert L.moe_quantize_device(143, 1, w, -128, out, None, None) == -3
    assert L.moe_quantize_device(142, 0, w, 1 << 62, out, None, None) == -3      # beyond one launch
    assert L.moe_quantize_device(142, 0, None, 128, out, None, None) == -1
    assert L.moe_quantize_device(142, 0, w + 2, 128, out, None, None) == -1      # d_w not 16-byte aligned
    assert L.moe_quantize_device(143, 0, w, 128, out + 2, None, None) == -1      # d_dst not 4-byte aligned
    assert L.moe_quantize_device(142, 0, w, 256, w + 256, None, None) == -1      # overlap
    assert "overlap" in L.moe_last_error().decode()
    assert L.moe_quantize_device(142, 0, w, 256, out, out + 8, None) == -1       # rounds overlap dst
    assert L.moe_quantize_device(142, 0, w, 256, out, w + 2, None) == -1         # rounds overlap w
    assert L.moe_quantize_device(142, 0, w, 0, out, None, None) == 0


def test_ple_gather_validation():
    """Argument checks of moe_ple_gather_q4_0 happen on the host, before any launch."""
    L = tq.lib()
    t, i, o = 0x10000, 0x20000, 0x40000
    assert L.moe_ple_gather_q4_0(t, 10, 100, i, 4, o, None) == -3          # row length not a multiple of 32
    assert L.moe_ple_gather_q4_0(t, 10, 0, i, 4, o, None) == -3
    assert L.moe_ple_gather_q4_0(t, -1, 64, i, 4, o, None) == -3
    assert L.moe_ple_gather_q4_0(t, 10, 64, i, -4, o, None) == -3
    assert L.moe_ple_gather_q4_0(t, 10, 64, None, 4, o, None) == -1
    assert L.moe_ple_gather_q4_0(t + 1, 10, 64, i, 4, o, None) == -1      # table not 2-byte aligned
    assert L.moe_ple_gather_q4_0(t, 10, 64, i + 4, 4, o, None) == -1      # indices not 8-byte aligned
    assert L.moe_ple_gather_q4_0(t, 10, 64, i, 4, o + 8, None) == -1      # output not 16-byte aligned
    assert L.moe_ple_gather_q4_0(t, 10, 64, i, 0, o, None) == 0           # nothing to do


def _plain_to_tiles(data, rows, cols, bb):
    """The tile-major order written as a numpy reshape: [row tile][group][row in tile]."""
    G = cols // 128
    return data.reshape(rows // 16, 16, G, bb).transpose(0, 2, 1, 3).reshape(-1)


@pytest.mark.parametrize("fmt", [PQ2_0, PTQ1_0])
def test_tile_container_is_the_tile_major_permutation(fmt):
    rng = np.random.default_rng(5)
    rows, cols = 48, 384
    t = rng.integers(-1, 2, size=(rows, cols)).astype(np.int8)
    s = (rng.integers(0, 0x3C00, size=rows * cols // 128)).astype(np.uint16)
    plain = tq.pack(fmt, t, s)
    tiled = tq.tile_container(fmt, plain, rows, cols)
    assert np.array_equal(tiled, _plain_to_tiles(plain, rows, cols, tq.block_bytes(fmt)))
    assert np.array_equal(tq.untile_container(fmt, tiled, rows, cols), plain)
    # every block keeps its bytes: block (n, g) of the tiled order decodes to row n, group g
    bb, G = tq.block_bytes(fmt), cols // 128
    n, g = 37, 2
    blk = tiled[(((n // 16) * G + g) * 16 + n % 16) * bb:][:bb]
    tr, sc = tq.unpack(fmt, blk, 128)
    assert np.array_equal(tr, t[n, 128 * g:128 * (g + 1)]) and int(sc[0]) == int(s[n * G + g])


def test_tile_container_errors():
    L = tq.lib()
    src = np.zeros(34 * 3 * 16, np.uint8)
    dst = np.zeros_like(src)
    assert L.moe_tile_container(42, src.ctypes.data, 16, 384, dst.ctypes.data, dst.size) == -2
    assert L.moe_tile_container(PQ2_0, src.ctypes.data, 8, 384, dst.ctypes.data, dst.size) == -3
    assert L.moe_tile_container(PQ2_0, src.ctypes.data, 16, 200, dst.ctypes.data, dst.size) == -3
    assert L.moe_tile_container(PQ2_0, src.ctypes.data, 16, 384, dst.ctypes.data, dst.size - 1) == -6
    assert L.moe_untile_container(PQ2_0, src.ctypes.data, 16, 384, src.ctypes.data, src.size) == -1
    assert L.moe_tile_container(PQ2_0, None, 16, 384, dst.ctypes.data, dst.size) == -1
    assert L.moe_tile_container(PQ2_0, src.ctypes.data, 16, 384, dst.ctypes.data, dst.size) == 0
