"""Host-side checks of the grouped decode plan (no GPU): the image that
bitlinear_fwd_group_plan uploads, built into host memory with stand-in
device addresses (low words with bit 31 set, as real device addresses
often have), is replayed against every read the contraction kernel makes:
header, activation rows, items, each workgroup's strip list and the 16
wavefront start records that cut it into ranges.  Every strip of every item
must be covered exactly once, in whole k blocks, and the ranges must tile
each workgroup's steps in the documented 19 : 17 : 15 : 13 proportions.
For one-launch runs, each wavefront's activation segments must cover every
row of the workgroup's items exactly once, land in the LDS room the strips
point at, and name the slots of their row's absmax; each item's x_q and
x_scale must be written by exactly one workgroup."""
import numpy as np
import pytest

from sparse_linear_layers_group_amd import bitlinear as bl

QWEN05 = [(896, 896), (128, 896), (128, 896), (896, 896), (4864, 896), (4864, 896), (896, 4864)]
S_OF = {(8, 8): 8, (6, 8): 6, (4, 8): 4, (2, 4): 4, (3, 8): 4, (2, 8): 2}
WEIGHTS = (19, 17, 15, 13)  # per group of four wavefronts (w // 4)

# plan image: header 64 B | 256 x 16 wavefront starts (80 B) | 256 x 16 x 4
# fused segments (48 B) | row descriptors (32 B, at least 1024) | strip
# descriptors (64 B) | items (64 B)
HDR, WAVE, FSEG, ROW, DESC, ITEM = 64, 80, 48, 32, 64, 64
SEGS_PER_WAVE, SEG_VALS = 4, 1024
FUSED_CODES = 160 * 1024 - 512 * 4 * 32 - 4 * 64  # LDS after the code tables, before the 64 segment maxima


def _wave_split(n, w):
    c = sum(WEIGHTS[g] * min(max(w - 4 * g, 0), 4) for g in range(4))
    return n * c // 256


def _items(shapes):
    arr = (bl.bitlinear_fwd_item * len(shapes))()
    info = []
    for i, (n_out, k) in enumerate(shapes):
        base = 0x7f0000000000 + 0x100000000 * i + 0x80000000
        p = dict(X=base, packed=base + 0x10000000, gamma=base + 0x20000000, Y=base + 0x30000000,
                 xq=base + 0x40000000, x_scale=base + 0x50000000)
        arr[i] = bl.bitlinear_fwd_item(p["X"], p["packed"], p["gamma"], p["Y"], p["xq"], p["x_scale"], k, n_out)
        info.append(dict(p, k=k, n_out=n_out))
    return arr, info


class _Img:
    def __init__(self, img):
        self.b = img

    def i32(self, o):
        return int(self.b[o:o + 4].view(np.int32)[0])

    def i64(self, o):
        return int(self.b[o:o + 8].view(np.int64)[0])

    def u64(self, o):
        return int(self.b[o:o + 8].view(np.uint64)[0])

    def desc(self, o):
        return dict(packed=self.u64(o), xq=self.u64(o + 8), Y=self.u64(o + 16), scale=self.u64(o + 24),
                    gamma=self.u64(o + 32), n_out=self.i64(o + 40), k=self.i32(o + 48), row0=self.i32(o + 52),
                    lds_x=self.i32(o + 56), lds_s=self.i32(o + 60))


def _replay(shapes, tokens, n=6, m=8):
    items, info = _items(shapes)
    nbytes = bl.bitlinear_fwd_group_plan_bytes(items, len(shapes), tokens)
    img = np.zeros(nbytes, np.uint8)
    bl.bitlinear_fwd_group_plan_host(items, len(shapes), tokens, n, m, img)
    P = _Img(img)
    bb = 2 * (8 + S_OF[(n, m)])
    count, tok, s_hdr, blocks = P.i32(0), P.i32(4), P.i32(8), P.i32(12)
    rows, steps, strips, fused = P.i64(16), P.i64(24), P.i64(32), P.i32(40)
    assert (count, tok, s_hdr, rows) == (len(shapes), tokens, S_OF[(n, m)], len(shapes) * tokens)
    assert steps == sum(-(-no // 64) * (k // 128) for no, k in shapes)
    assert strips == sum(-(-no // 64) for no, _ in shapes)
    assert 1 <= blocks <= 256
    waves = HDR
    fseg_off = waves + 4096 * WAVE
    rows_off = fseg_off + 4096 * SEGS_PER_WAVE * FSEG
    strips_off = rows_off + max(rows, 1024) * ROW
    items_off = strips_off + strips * DESC
    assert items_off + count * ITEM == nbytes
    r = 0
    for it in info:
        for t in range(tokens):
            o = rows_off + r * ROW
            assert (P.u64(o), P.u64(o + 8), P.u64(o + 16), P.i64(o + 24)) == (
                it["X"] + 2 * t * it["k"], it["xq"] + t * it["k"], it["x_scale"] + 4 * t, it["k"])
            r += 1
    for i, it in enumerate(info):
        o = items_off + i * ITEM
        assert [P.u64(o + 8 * f) for f in range(6)] == [it[x] for x in ("X", "packed", "gamma", "Y", "xq", "x_scale")]
        assert (P.i64(o + 48), P.i64(o + 56)) == (it["k"], it["n_out"])
    want = {}
    for it in info:
        for st in range(-(-it["n_out"] // 64)):
            want[it["packed"] + st * (it["k"] // 128) * 64 * bb] = (it, st)
    owner = {}
    next_desc = 0
    writers = {}
    fits = True
    item_of = {it["packed"]: i for i, it in enumerate(info)}
    for b in range(256):
        first = waves + b * 16 * WAVE
        if b >= blocks:
            assert all(P.i32(first + w * WAVE + 76) == 0 for w in range(16))
            continue
        # the workgroup's strip list: contiguous descriptors from next_desc
        rec0 = P.i32(first + 64)
        assert rec0 == next_desc and P.i32(first + 68) == 0
        n_b = sum(P.i32(first + w * WAVE + 72) for w in range(16))
        steps_of = []
        j, cum = rec0, 0
        while cum < n_b:
            d = P.desc(strips_off + j * DESC)
            it, st = want[d["packed"]]
            assert (d["xq"], d["Y"], d["scale"], d["gamma"]) == (it["xq"], it["Y"], it["x_scale"], it["gamma"])
            assert (d["n_out"], d["k"], d["row0"]) == (it["n_out"], it["k"], 64 * st)
            assert d["packed"] not in owner
            owner[d["packed"]] = b
            steps_of.append((j, cum, d["k"] // 128))
            cum += d["k"] // 128
            j += 1
        assert cum == n_b
        # fused item list: the distinct items of the strips, in order, codes
        # then scales in LDS; the strips carry their item's offsets
        its = []
        for jj in range(rec0, j):
            d = P.desc(strips_off + jj * DESC)
            i = item_of[want[d["packed"]][0]["packed"]]
            if not its or its[-1] != i:
                its.append(i)
        off = 0
        offs = {}
        for i in its:
            offs[i] = [off, None]
            off += -(-tokens * info[i]["k"] // 16) * 16
        for i in its:
            offs[i][1] = off
            off += -(-tokens * 4 // 16) * 16
        room = off <= FUSED_CODES
        for jj in range(rec0, j):
            d = P.desc(strips_off + jj * DESC)
            i = item_of[want[d["packed"]][0]["packed"]]
            assert [d["lds_x"], d["lds_s"]] == offs[i]
        # the segments as the wavefronts read them: slot j of wavefront w
        segs = []
        for w in range(16):
            for sj in range(SEGS_PER_WAVE):
                o = fseg_off + ((b * 16 + w) * SEGS_PER_WAVE + sj) * FSEG
                f = dict(x=P.u64(o), xq=P.u64(o + 8), scale=P.u64(o + 16), lds_q=P.i32(o + 24),
                         lds_s=P.i32(o + 28), nvals=P.i32(o + 32),
                         slot=int(img[o + 36:o + 38].view(np.int16)[0]),
                         row_slot=int(img[o + 38:o + 40].view(np.int16)[0]),
                         row_slots=int(img[o + 40:o + 42].view(np.int16)[0]),
                         first=int(img[o + 42:o + 44].view(np.int16)[0]))
                if f["nvals"]:
                    assert f["slot"] % 16 == w and f["slot"] // 16 == sj  # dealt round-robin
                    segs.append(f)
                else:
                    assert f == dict.fromkeys(f, 0)
        need = sum(tokens * -(-info[i]["k"] // SEG_VALS) for i in its)
        fits = fits and room and need <= 16 * SEGS_PER_WAVE
        if fused:
            assert sorted(f["slot"] for f in segs) == list(range(need))
            slot_of = {f["slot"]: f for f in segs}
            for i in its:
                it = info[i]
                writer = i not in writers
                if writer:
                    writers[i] = b
                for t in range(tokens):
                    row = [f for f in segs if it["X"] + 2 * t * it["k"] <= f["x"] < it["X"] + 2 * (t + 1) * it["k"]]
                    row.sort(key=lambda f: f["x"])
                    # the row's values, each once, in segments of at most 1024
                    v = 0
                    for f in row:
                        assert f["x"] == it["X"] + 2 * (t * it["k"] + v)
                        assert f["nvals"] == min(SEG_VALS, it["k"] - v) and f["nvals"] % 8 == 0
                        assert f["lds_q"] == offs[i][0] + t * it["k"] + v
                        assert f["lds_s"] == offs[i][1] + 4 * t
                        assert f["xq"] == (it["xq"] + t * it["k"] + v if writer else 0)
                        assert f["scale"] == (it["x_scale"] + 4 * t if writer and v == 0 else 0)
                        assert f["first"] == (1 if v == 0 else 0)
                        v += f["nvals"]
                    assert v == it["k"]
                    # each segment names exactly its row's slots
                    slots = sorted(f["slot"] for f in row)
                    for f in row:
                        assert list(range(f["row_slot"], f["row_slot"] + f["row_slots"])) == slots
                        assert all(slot_of[q] in row for q in slots)
        else:
            assert not segs  # a plan that does not fuse carries no segments
        next_desc = j
        # wavefront w: steps [split(w), split(w+1)) of the list, from its record
        for w in range(16):
            o = first + w * WAVE
            rec, kb, cnt, act = P.i32(o + 64), P.i32(o + 68), P.i32(o + 72), P.i32(o + 76)
            assert act == 1
            s0, s1 = _wave_split(n_b, w), _wave_split(n_b, w + 1)
            assert cnt == s1 - s0
            jj, c0, nk = next((x for x in steps_of if x[1] <= s0 < x[1] + x[2]), steps_of[-1])
            assert (rec, kb) == (jj, s0 - c0) or (cnt == 0 and s0 == n_b)
            assert P.desc(o) == P.desc(strips_off + rec * DESC)
    assert next_desc == strips and len(owner) == len(want)
    if fused:
        assert sorted(writers) == list(range(count))  # every item written by exactly one workgroup
    assert fused == (1 if fits else 0)
    assert bl.bitlinear_fwd_group_plan_fuses(items, len(shapes), tokens, n, m) == bool(fused)
    return fused


@pytest.mark.parametrize("shapes,tokens,fuses", [
    (QWEN05 * 2, 1, 1),
    (QWEN05 * 24, 1, 1),
    (QWEN05 * 24, 4, 0),  # codes fit LDS, but ~160 segments per workgroup (64 slots)
    (QWEN05 * 24, 16, 0),  # up to ~150 KB of codes in some workgroups
    ([(48, 256), (128, 896), (40, 384), (896, 4864), (200, 1152)], 1, 1),
    ([(48, 256), (128, 896), (40, 384), (896, 4864), (200, 1152)], 16, 0),  # segments
    ([(64, 128), (128, 256)], 1, 1),
    ([(11008, 2048)] * 16, 1, 1),
    ([(2048, 11008)] * 16, 16, 0),  # 176 KB of codes per item
    ([(64000, 128)] * 8, 16, 0),  # 16 rows per item, one segment each: over 64 slots
    ([(64000, 128)] * 3, 16, 1),
    # ~40 distinct 2048-wide items per workgroup at 16 tokens: 1.3 MB of
    # activation codes per workgroup, far past its LDS
    ([(64, 2048)] * 10000, 16, 0),
])
def test_group_plan_replay(shapes, tokens, fuses):
    assert _replay(shapes, tokens) == fuses


@pytest.mark.parametrize("n,m", [(8, 8), (4, 8), (2, 4), (2, 8)])
def test_group_plan_replay_patterns(n, m):
    _replay(QWEN05 * 3, 2, n, m)


def test_group_plan_host_rejects_short_image():
    items, _ = _items(QWEN05)
    nbytes = bl.bitlinear_fwd_group_plan_bytes(items, len(QWEN05), 1)
    img = np.zeros(nbytes - 16, np.uint8)
    with pytest.raises(bl.BitLinearError) as e:
        bl.bitlinear_fwd_group_plan_host(items, len(QWEN05), 1, 6, 8, img)
    assert e.value.status == bl.BL_EWORKSPACE


def test_group_plan_fuses_reports_errors():
    """bitlinear_fwd_group_plan_fuses answers 1 or 0, and turns invalid
    items into the same errors the plan builder reports (negated on the C
    side, raised by the binding)."""
    items, _ = _items(QWEN05)
    assert bl.bitlinear_fwd_group_plan_fuses(items, len(QWEN05), 1, 6, 8) is True
    with pytest.raises(bl.BitLinearError) as e:
        bl.bitlinear_fwd_group_plan_fuses(items, len(QWEN05), 1, 5, 8)
    assert e.value.status == bl.BL_EUNSUPPORTED
    bad, _ = _items([(64, 200)])  # k not a multiple of 128
    with pytest.raises(bl.BitLinearError) as e:
        bl.bitlinear_fwd_group_plan_fuses(bad, 1, 1, 6, 8)
    assert e.value.status == bl.BL_ESHAPE
