"""Host-side check of the stored-dS chunk layout (CPU only).

The dK/dV kernel stores each wave's 32 x 32 block of dS as a 2 KB chunk: lane
h*32 + k (key k of the wave, row half h) holds, for row chunk kc, the dS of
rows kc*16 + (e/4)*8 + h*4 + e%4 (e = 0..7) -- its MFMA operand -- and writes
those 16 bytes to slot byte kc*1024 + h*512 + (k XOR 4(2kc + h))*16
(ds_chunk_off in csrc/fa_bwd.hip).  The dQ kernel reads the chunk back from
LDS with ds_read_b64_tr_b16, which within each group of 16 lanes hands lane s
element s%4 of the 8 bytes that lane 4*i + s/4 loaded (i = 0..3): lane
4r + c of group g points at key 4(g/2) + r (+8 for the second read, +16h for
key half h) and rows 16(g%2) + 4c .. +3.  This test restates both sides,
checks that the reads deliver the dQ MFMA's operand (row l%32 and keys
16h + (e/4)*8 + (l/32)*4 + e%4 in lane l), and that each half-wave read
touches 64 distinct 4-byte LDS banks.
"""

import numpy as np


def chunk_off(kc, h, k):
    return kc * 1024 + h * 512 + ((k ^ (4 * (2 * kc + h))) * 16)


def store_block(ds):
    mem = np.full(1024, -1, dtype=np.int64)  # 16-bit elements of one chunk
    for lane in range(64):
        h, key = lane // 32, lane % 32
        for kc in range(2):
            base = chunk_off(kc, h, key) // 2
            for e in range(8):
                row = kc * 16 + (e // 4) * 8 + h * 4 + e % 4
                assert mem[base + e] == -1
                mem[base + e] = ds[row, key]
    return mem


def read_addr(lane, hk, second):
    g, s16 = lane >> 4, lane & 15
    r4, cc = s16 >> 2, s16 & 3
    a = chunk_off(g & 1, cc & 1, (g >> 1) * 4 + r4) + (cc >> 1) * 8 + hk * 256
    return a ^ 128 if second else a


def tr_read(mem, addr):
    out = np.zeros((64, 4), dtype=np.int64)
    for g in range(4):
        loaded = [mem[addr(16 * g + t) // 2: addr(16 * g + t) // 2 + 4] for t in range(16)]
        for s in range(16):
            for i in range(4):
                out[16 * g + s, i] = loaded[4 * i + s // 4][s % 4]
    return out


def test_chunk_is_filled_once_and_reads_give_the_dq_operand():
    ds = np.random.default_rng(0).integers(0, 1 << 16, size=(32, 32))
    mem = store_block(ds)
    assert (mem >= 0).all()
    for hk in range(2):
        frag = np.concatenate([tr_read(mem, lambda l: read_addr(l, hk, False)),
                               tr_read(mem, lambda l: read_addr(l, hk, True))], axis=1)
        for lane in range(64):
            for e in range(8):
                key = hk * 16 + (e // 4) * 8 + (lane // 32) * 4 + e % 4
                assert frag[lane, e] == ds[lane % 32, key], (hk, lane, e)


def test_transposed_reads_hit_distinct_banks():
    for hk in range(2):
        for second in (False, True):
            for half in range(2):
                banks = set()
                for lane in range(32 * half, 32 * half + 32):
                    a = read_addr(lane, hk, second)
                    banks.update({(a // 4) % 64, (a // 4 + 1) % 64})
                assert len(banks) == 64, (hk, second, half)


def test_each_store_instruction_fills_one_kilobyte():
    for kc in range(2):
        offs = sorted(chunk_off(kc, lane // 32, lane % 32) for lane in range(64))
        assert offs == list(range(kc * 1024, kc * 1024 + 1024, 16))
