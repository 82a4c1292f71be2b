"""CPU model of the LDS for every fragment read the kernels make.

The offsets come from `attention_flash_sdpa_amd/csrc/lds_layout.h`, the one
definition the kernels use, built here for the host (`lds_layout_dump.cpp`).
Two properties are checked for each read pattern:

* layout: through the fill mapping (slot s of a block holds chunk
  (s % SLOTS) ^ f(row) of row s / SLOTS), every lane reads exactly the key
  row and bytes its MFMA operand needs, including the transposed reads'
  cross-lane exchange and the row offsets the kernels add per score tile or
  key chunk;
* banks: the lanes the LDS serves together address distinct banks.

The bank model (64 banks of 4 bytes; 8-byte reads, plain or transposed, served
32 consecutive lanes at a time; 16-byte reads 16 lanes at a time in the groups
{0-3, 12-15, 20-23, 24-27} and {4-7, 8-11, 16-19, 28-31} of each half-wave)
was measured on MI355X with rocprofv3's SQ_LDS_BANK_CONFLICT counter: one
wave reading with two lanes on one bank and all others on a broadcast address
shows a conflict exactly when the two lanes share a group.  The model also
reproduces the kernels' own counts: 0 for the prefill kernels, and 32 cycles
per 32-key block for the decode K reads under the prefill swizzle they used
before (`test_model_reproduces_measured_decode_conflicts`).

The mask values of the masked prefill go from global memory straight into
registers, so that kernel adds no LDS read pattern of its own.
"""
import json
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_flash_sdpa_amd", "csrc")
BANKS = 64


@pytest.fixture(scope="module")
def lay(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("lds") / "lds_layout_dump")
    src = os.path.join(ROOT, "tests", "lds_layout_dump.cpp")
    subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC, src, "-o", exe], check=True)
    return json.loads(subprocess.run([exe], check=True, capture_output=True, text=True).stdout)


# ------------------------------------------------------------------ the model
_B128_HALF = ([0, 1, 2, 3, 12, 13, 14, 15, 20, 21, 22, 23, 24, 25, 26, 27],
              [4, 5, 6, 7, 8, 9, 10, 11, 16, 17, 18, 19, 28, 29, 30, 31])
LANE_GROUPS = {
    16: [[h + lane for lane in g] for h in (0, 32) for g in _B128_HALF],
    8: [list(range(0, 32)), list(range(32, 64))],
}


def bank_conflicts(addrs, width):
    """Extra LDS cycles of one read instruction: `addrs` are the 64 lanes'
    byte addresses, each lane reads `width` bytes.  Within a group of lanes
    served together, k different dwords on one bank cost k - 1 extra cycles
    (the same dword is a broadcast)."""
    extra = 0
    for group in LANE_GROUPS[width]:
        assert sorted(group) == sorted(set(group)) and len(group) * width == 256
        banks = {}
        for lane in group:
            for k in range(width // 4):
                dw = addrs[lane] // 4 + k
                banks.setdefault(dw % BANKS, set()).add(dw)
        extra += max(len(v) for v in banks.values()) - 1
    return extra


def inverse_fill(chunks, slots):
    """LDS byte of a block -> (key row, byte within the row), from the fill
    mapping; asserts that every row holds each of its chunks exactly once."""
    inv = {}
    for slot, ch in enumerate(chunks):
        row = slot // slots
        assert 0 <= ch < slots
        for b in range(16):
            inv[slot * 16 + b] = (row, ch * 16 + b)
    rows = len(chunks) // slots
    for r in range(rows):
        assert sorted(chunks[r * slots:(r + 1) * slots]) == list(range(slots)), f"row {r} is not a permutation"
    return inv


def direct(addrs, inv, width):
    """What each lane of a plain read receives: a list of (row, byte) per lane."""
    return [[inv[a + b] for b in range(width)] for a in addrs]


def transposed(addrs, inv, elem):
    """What each lane of ds_read_b64_tr_b16 (elem = 2) or _tr_b8 (elem = 1)
    receives, as a list of (row, element index) per lane.  Within each group of
    16 lanes, lane i gets element r (r < 8 / elem) of the 8-byte row that
    another group lane addresses: for 16-bit elements lane 4r + i/4 at
    position i%4, for 8-bit elements lane 2r + i/8 at position i%8."""
    n = 8 // elem
    per = 16 // n            # group lanes that address one output row slot
    out = []
    for lane in range(64):
        g0, i = lane - lane % 16, lane % 16
        vals = []
        for r in range(n):
            src = g0 + per * r + i // n
            row, byte = inv[addrs[src] + elem * (i % n)]
            assert byte % elem == 0
            vals.append((row, byte // elem))
        out.append(vals)
    return out


# P's key order.  The scores of a 32x32 tile sit in lane l, register r at key
# 8(r/4) + 4(l/32) + r%4; packed 16 keys (8 registers) per MFMA step, element j
# of key chunk c is key 16c + 8(j/4) + 4(l/32) + j%4.  The 16x16 decode tiles
# hold key 4(l/16) + r of tile t; the B operand takes tile j/4, register j%4:
# key 16(j/4) + 4(l/16) + j%4.  The V^T operand must use the same order.
def key32(lane, c, j):
    return 16 * c + 8 * (j // 4) + 4 * (lane // 32) + j % 4


def key16(lane, j):
    return 16 * (j // 4) + 4 * (lane // 16) + j % 4


# ------------------------------------------------------------------ fills
@pytest.mark.parametrize("name,slots", [("fill_prefill16", 16), ("fill_prefill8", 8), ("fill_quarter", 4),
                                        ("fill_decode16", 16), ("fill_decode8", 8)])
def test_fill_places_every_chunk_once(lay, name, slots):
    inv = inverse_fill(lay[name], slots)
    assert len(inv) == 16 * len(lay[name])


# ------------------------------------------------------------------ 16-bit prefill
@pytest.mark.parametrize("slots", [16, 8])
def test_prefill_k_fragments(lay, slots):
    """32x32x16 K fragment, k-step s, score tile t (+32 rows): lane l gets key
    row 32t + l%32, head dims 16s + 8(l/32) .. +7 (bytes 32s + 16(l/32) ..)."""
    inv = inverse_fill(lay[f"fill_prefill{slots}"], slots)
    row_bytes = 16 * slots
    for s, addrs in enumerate(lay[f"prefill_k{slots}"]):
        for t in range(2):
            a = [x + 32 * t * row_bytes for x in addrs]
            assert bank_conflicts(a, 16) == 0, (s, t)
            for lane, got in enumerate(direct(a, inv, 16)):
                want = [(32 * t + lane % 32, 32 * s + 16 * (lane // 32) + b) for b in range(16)]
                assert got == want, (s, t, lane)


@pytest.mark.parametrize("slots", [16, 8])
def test_prefill_vt_fragments(lay, slots):
    """V^T fragment by ds_read_b64_tr_b16, halves hf = 0, 1 (elements j = 4hf ..
    4hf+3), value tile t, key chunk c (+16 rows): lane l gets value column
    32t + l%32 of the keys P's element j holds."""
    inv = inverse_fill(lay[f"fill_prefill{slots}"], slots)
    row_bytes = 16 * slots
    for hf, per_t in enumerate(lay[f"prefill_vt{slots}"]):
        for t, addrs in enumerate(per_t):
            for c in range(4):
                a = [x + 16 * c * row_bytes for x in addrs]
                assert bank_conflicts(a, 8) == 0, (hf, t, c)
                for lane, got in enumerate(transposed(a, inv, 2)):
                    want = [(key32(lane, c, 4 * hf + r), 32 * t + lane % 32) for r in range(4)]
                    assert got == want, (hf, t, c, lane)


# ------------------------------------------------------------------ fp8 prefill
def test_fp8_k_fragments(lay):
    """32x32x64 fp8 K fragment: lane l gets key row 32t + l%32 and the 32 bytes
    of dims 64s + 32(l/32) .. in two 16-byte halves c; s = 0, 1 from the
    128-byte part A, s = 2 from the 64-byte part B (dims 128 ..)."""
    inv_a = inverse_fill(lay["fill_prefill8"], 8)
    inv_b = inverse_fill(lay["fill_quarter"], 4)
    for t in range(2):
        for s in range(2):
            for c in range(2):
                a = [x + 32 * t * 128 for x in lay["fp8_ka"][s][c]]
                assert bank_conflicts(a, 16) == 0, (s, c, t)
                for lane, got in enumerate(direct(a, inv_a, 16)):
                    assert got == [(32 * t + lane % 32, 64 * s + 32 * (lane // 32) + 16 * c + b)
                                   for b in range(16)], (s, c, t, lane)
        for c in range(2):
            a = [x + 32 * t * 64 for x in lay["fp8_kb"][c]]
            assert bank_conflicts(a, 16) == 0, (c, t)
            for lane, got in enumerate(direct(a, inv_b, 16)):
                assert got == [(32 * t + lane % 32, 32 * (lane // 32) + 16 * c + b) for b in range(16)], (c, t, lane)


def test_fp8_vt_fragments(lay):
    """V^T fragment by ds_read_b64_tr_b8, value tile t, key chunk c (+16 rows):
    byte j of lane l is value column 32t + l%32 of the key P's element j of
    chunk c holds (the same order for the bf16 and the fp8 P·V)."""
    inv = inverse_fill(lay["fill_prefill8"], 8)
    for t, addrs in enumerate(lay["fp8_vt"]):
        for c in range(4):
            a = [x + 16 * c * 128 for x in addrs]
            assert bank_conflicts(a, 8) == 0, (t, c)
            for lane, got in enumerate(transposed(a, inv, 1)):
                assert got == [(key32(lane, c, j), 32 * t + lane % 32) for j in range(8)], (t, c, lane)


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("slots", [16, 8])
def test_decode_k_fragments(lay, slots):
    """16x16x32 K fragment, k-step s, score tile t (+16 rows): lane l gets key
    row 16t + l%16, head dims 32s + 8(l/16) .. +7."""
    inv = inverse_fill(lay[f"fill_decode_k{slots}"], slots)
    row_bytes = 16 * slots
    for s, addrs in enumerate(lay[f"decode_k{slots}"]):
        for t in range(2):
            a = [x + 16 * t * row_bytes for x in addrs]
            assert bank_conflicts(a, 16) == 0, (s, t)
            for lane, got in enumerate(direct(a, inv, 16)):
                assert got == [(16 * t + lane % 16, 64 * s + 16 * (lane // 16) + b) for b in range(16)], (s, t, lane)


@pytest.mark.parametrize("slots", [16, 8])
def test_decode_vt_fragments(lay, slots):
    """Decode V^T by ds_read_b64_tr_b16, halves hf, value tile t: lane l gets
    value column 16t + l%16 of the keys of P's elements 4hf .. 4hf+3."""
    inv = inverse_fill(lay[f"fill_decode{slots}"], slots)
    for hf, per_t in enumerate(lay[f"decode_vt{slots}"]):
        for t, addrs in enumerate(per_t):
            assert bank_conflicts(addrs, 8) == 0, (hf, t)
            for lane, got in enumerate(transposed(addrs, inv, 2)):
                assert got == [(key16(lane, 4 * hf + r), 16 * t + lane % 16) for r in range(4)], (hf, t, lane)


# ------------------------------------------------------------------ the model itself
def _old_decode_k_addrs(slots, s, t):
    """The decode K reads as they were laid out with the prefill swizzle."""
    def swz(r):
        if slots == 16:
            return ((r & 3) << 2) | ((r >> 2) & 3)
        x = r >> 1
        return ((x & 1) << 2) | ((x >> 1) & 3)
    return [(16 * t + lane % 16) * 16 * slots + (((4 * s + lane // 16) ^ swz(16 * t + lane % 16)) << 4)
            for lane in range(64)]


def test_model_reproduces_measured_decode_conflicts():
    """rocprofv3 on MI355X gave the decode kernel at d = 128 (C4: 1,024 waves x
    32 blocks) 1,048,576 SQ_LDS_BANK_CONFLICT cycles per launch with the
    prefill swizzle on its K rows: 32 per block, all from the 8 K reads (a
    single-wave probe of one such read gave 4 cycles per instruction)."""
    per_block = sum(bank_conflicts(_old_decode_k_addrs(16, s, t), 16) for s in range(4) for t in range(2))
    assert per_block == 32
    assert bank_conflicts(_old_decode_k_addrs(16, 0, 0), 16) == 4
    assert 1024 * 32 * per_block == 1048576


def test_model_flags_unswizzled_k_reads():
    """Without the swizzle, 16 lanes reading one 16-byte chunk of 16 rows of
    256 bytes all land on the same four banks: 15 extra cycles per group (a
    single-wave probe measured 60 per instruction)."""
    addrs = [(lane % 32) * 256 + 16 * (lane // 32) for lane in range(64)]
    assert bank_conflicts(addrs, 16) == 4 * 15
    # 128-byte rows: two rows per bank line, 8-way
    addrs = [(lane % 32) * 128 + 16 * (lane // 32) for lane in range(64)]
    assert bank_conflicts(addrs, 16) == 4 * 7


def test_model_broadcast_is_free():
    assert bank_conflicts([0] * 64, 16) == 0
    assert bank_conflicts([8 * (lane % 32) for lane in range(64)], 8) == 0
