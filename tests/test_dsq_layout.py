"""Host model of the stored-dS tile layout (csrc/dsq.h, csrc/attn_dsq.hip, and the local
half tiles of hga_dqw_kernel in csrc/attn_bwd.hip).

The key-major kernel stores each 64x64 dS tile as its registers hold it; the dQ kernel
copies the tile's 16-byte chunks into LDS in a permuted slot order and reads B fragments
with ds_read_b64_tr_b16.  This model replays the three steps with the formulas of the
kernels and the instruction's documented lane exchange (output lane i of a 16-lane group
gets element i % 4 of the 8 bytes addressed by source lane 4 j + i / 4, for j = 0..3), and
checks that every lane receives the keys and query the MFMA expects, that the slot order is
a permutation, and that the 32 lanes served together hit 64 distinct banks."""
import numpy as np


def chunk_of_slot(s):
    return (s & 0x180) | (((s >> 3) & 1) << 6) | (((s >> 2) & 1) << 5) | (((s >> 4) & 7) << 2) | (s & 3)


def tr_offset(lane, mq):
    lq, g = lane % 32, lane // 32
    t = lq & 15
    slot = (t >> 2) | ((t & 1) << 2) | ((lq >> 4) << 3) | (g << 4) | (mq << 7)
    return 8 * slot + 4 * ((t >> 1) & 1)


def stored_tile():
    """Element e of the 4096-element tile holds key * 64 + query (the store of dsq.h)."""
    tile = np.full(4096, -1, dtype=np.int64)
    for p in range(2):
        for mq in range(2):
            for h in range(2):
                for lane in range(64):
                    l, g = lane % 32, lane // 32
                    qs = [32 * mq + 16 * h + 4 * g + j for j in range(4)] + \
                         [32 * mq + 16 * h + 8 + 4 * g + j for j in range(4)]
                    base = p * 2048 + ((mq * 2 + h) * 64 + lane) * 8
                    tile[base:base + 8] = [(32 * p + l) * 64 + q for q in qs]
    return tile


def lds_tile(tile, waves):
    lds = np.full(4096, -1, dtype=np.int64)
    per = 8 // waves
    for w in range(waves):
        for i in range(per):
            for lane in range(64):
                src = 8 * chunk_of_slot((per * w + i) * 64 + lane)
                dst = (per * w + i) * 512 + lane * 8
                lds[dst:dst + 8] = tile[src:src + 8]
    return lds


def tr_read(lds, addrs):
    out = np.zeros((64, 4), dtype=np.int64)
    for grp in range(4):
        for i in range(16):
            for j in range(4):
                out[grp * 16 + i, j] = lds[addrs[grp * 16 + 4 * j + i // 4] + i % 4]
    return out


def test_store_covers_the_tile_once():
    tile = stored_tile()
    assert (tile >= 0).all() and len(set(tile.tolist())) == 4096


def test_slot_order_is_a_permutation():
    assert sorted(chunk_of_slot(s) for s in range(512)) == list(range(512))


def test_transposed_reads_give_each_lane_its_fragment():
    tile = stored_tile()
    for waves in (4, 8):
        lds = lds_tile(tile, waves)
        assert (lds >= 0).all()
        for mq in range(2):
            for kb in range(4):
                base = [tr_offset(lane, mq) + 512 * (kb & 1) + 2048 * (kb >> 1) for lane in range(64)]
                x, y = tr_read(lds, base), tr_read(lds, [a + 256 for a in base])
                for lane in range(64):
                    lq, g = lane % 32, lane // 32
                    keys = [16 * kb + 4 * g + r for r in range(4)] + [16 * kb + 8 + 4 * g + r for r in range(4)]
                    want = [k * 64 + 32 * mq + lq for k in keys]
                    assert list(x[lane]) + list(y[lane]) == want


def test_half_tile_staging_gives_each_lane_its_fragment():
    """The HGA dQ kernel stages one 32-key pair p of a tile (4 KB): LDS slot 64 i + lane,
    i < 4, gets chunk p * 256 + chunk_of_slot(64 i + lane); K-step kb in {0, 1} of the pair
    then reads at tr_offset(lane, mq) + 512 kb (and + 256)."""
    tile = stored_tile()
    for p in range(2):
        lds = np.full(2048, -1, dtype=np.int64)
        for i in range(4):
            for lane in range(64):
                c = chunk_of_slot(64 * i + lane)
                assert c < 256
                src = p * 2048 + 8 * c
                lds[i * 512 + lane * 8:i * 512 + lane * 8 + 8] = tile[src:src + 8]
        assert (lds >= 0).all()
        for mq in range(2):
            for kb in range(2):
                base = [tr_offset(lane, mq) + 512 * kb for lane in range(64)]
                assert max(base) + 256 + 4 <= 2048
                x, y = tr_read(lds, base), tr_read(lds, [a + 256 for a in base])
                for lane in range(64):
                    lq, g = lane % 32, lane // 32
                    keys = [32 * p + 16 * kb + 4 * g + r for r in range(4)] + \
                           [32 * p + 16 * kb + 8 + 4 * g + r for r in range(4)]
                    want = [k * 64 + 32 * mq + lq for k in keys]
                    assert list(x[lane]) + list(y[lane]) == want


def test_transposed_reads_are_bank_conflict_free():
    # 64 banks of 4 bytes; an 8-byte read by 32 lanes must touch every bank exactly once
    for mq in range(2):
        for kb in range(4):
            for second in (0, 256):
                base = [tr_offset(lane, mq) + 512 * (kb & 1) + 2048 * (kb >> 1) + second for lane in range(64)]
                for half in range(2):
                    banks = []
                    for lane in range(32 * half, 32 * half + 32):
                        word = base[lane] * 2 // 4
                        banks += [word % 64, (word + 1) % 64]
                    assert sorted(banks) == list(range(64))


# ---------------------------------------------------------------------------------------
# The dQ kernel's unit stream (dqs_unit / launch_dqs in csrc/attn_dsq.hip): every
# (batch-head-group, query tile, key tile <= query tile) exactly once over the grid.
QT = 4


def _plan(B, N, H, G, cus_per_xcd=32):
    ntl = G // 64
    np_ = (ntl + QT - 1) // QT
    nsu = (np_ + 1) // 2
    tsu = B * H * (N // G) * nsu
    per = (tsu + 7) // 8
    return dict(ntl=ntl, np=np_, nsu=nsu, tsu=tsu, per=per, slots=min(per, cus_per_xcd))


def _unit(P, k, xcd, slot):
    nr = (P["per"] + P["slots"] - 1) // P["slots"]
    while True:
        if (k >> 1) >= nr:
            return None
        r = (nr - 1 - (k >> 1)) * P["slots"] + slot
        su = xcd * P["per"] + r
        if r >= P["per"] or su >= P["tsu"]:
            k = (k | 1) + 1
            continue
        si, bhg = su % P["nsu"], su // P["nsu"]
        pair = si if k & 1 else P["np"] - 1 - si
        if (k & 1) and si >= P["np"] - 1 - si:
            k += 1
            continue
        qa = QT * pair
        nt = min(QT, P["ntl"] - qa)
        return dict(k=k, t=0, qa=qa, nt=nt, n=qa + nt, bhg=bhg)


def test_dq_unit_stream_covers_every_tile_once():
    for B, N, H, G in [(1, 8192, 32, 2048), (1, 1024, 4, 256), (2, 768, 4, 192), (3, 512, 8, 128),
                       (1, 512, 4, 512), (1, 256, 2, 64), (2, 2048, 8, 512), (1, 1024, 1, 1024),
                       (5, 4096, 12, 2048), (1, 2048, 33, 2048), (1, 1344, 2, 448), (2, 640, 3, 320)]:
        P = _plan(B, N, H, G)
        seen, steps = set(), []
        for xcd in range(8):
            for slot in range(P["slots"]):
                c, n = _unit(P, 0, xcd, slot), 0
                while c:
                    for j in range(QT):
                        if j < c["nt"] and c["t"] <= c["qa"] + j:
                            key = (c["bhg"], c["qa"] + j, c["t"])
                            assert key not in seen
                            seen.add(key)
                    n += 1
                    c["t"] += 1
                    if c["t"] >= c["n"]:
                        c = _unit(P, c["k"] + 1, xcd, slot)
                steps.append(n)
        ntl = P["ntl"]
        assert len(seen) == B * H * (N // G) * ntl * (ntl + 1) // 2
        if (B, N, H, G) == (1, 8192, 32, 2048):
            assert min(steps) == max(steps) == 72   # the 8K step: every workgroup 72 steps
