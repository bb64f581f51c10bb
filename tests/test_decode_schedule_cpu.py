"""The decode kernel's load schedule, emulated on the CPU.

decode_kernel (gemm_decode.hpp) gives each wave the K units
kb0 + wave + i*NW, i < n_w, of its split (a unit is U consecutive K blocks:
U = 4 for the 2:4 weight loaded four blocks at a time, else 1), and cycles
them through D register slots: the first D slots are filled up front, full rounds refill every slot
while two more rounds remain, the last full round refills only blocks that
exist, and a remainder consumes what is left.  This test mirrors that control
flow (it must change with the kernel) and checks, over every small
configuration and the ones the library launches, that

  * every load stays inside the wave's K range (so inside the row), also
    when a wave has fewer units than slots or none at all (a split with fewer
    units than waves);
  * the blocks consumed are exactly the wave's blocks, each once, in order,
    and over all waves and splits every K block of the row exactly once.

A schedule that filled the first slots with their own block indices, as an
earlier form did, fails the first check."""
from __future__ import annotations

import pytest


def schedule(KB: int, NW: int, D: int, S: int, split: int, wave: int, clamp_first: bool = True, U: int = 1):
    """(loaded blocks, consumed blocks, the wave's blocks, its split's block range)
    for one wave; KB must be a multiple of U."""
    KU = KB // U
    KBs = (KU + S - 1) // S
    kb0 = split * KBs if S > 1 else 0
    KBr = max(0, min(KU, kb0 + KBs) - kb0) if S > 1 else KU
    n_w = (KBr - wave + NW - 1) // NW if wave < KBr else 0
    slot = [None] * D
    loads, consumed = [], []

    def blocks(i):
        unit = kb0 + wave + i * NW
        return [unit * U + u for u in range(U)]

    def load(d, i):
        loads.extend(blocks(i))
        slot[d] = blocks(i)

    if n_w > 0:
        for d in range(D):
            load(d, min(d, n_w - 1) if clamp_first else d)
    i0 = 0
    while i0 + 2 * D <= n_w:
        for d in range(D):
            consumed.extend(slot[d])
            load(d, i0 + d + D)
        i0 += D
    if i0 + D <= n_w:
        for d in range(D):
            consumed.extend(slot[d])
            if i0 + d + D < n_w:
                load(d, i0 + d + D)
        i0 += D
    for d in range(D - 1):
        if i0 + d < n_w:
            consumed.extend(slot[d])
    mine = [b for i in range(n_w) for b in blocks(i)]
    return loads, consumed, mine, (kb0 * U, (kb0 + KBr) * U)


def violations(KB, NW, D, S, clamp_first=True, U=1):
    bad = []
    every = []
    for split in range(S):
        for wave in range(NW):
            loads, consumed, mine, (lo, hi) = schedule(KB, NW, D, S, split, wave, clamp_first, U)
            if any(not (lo <= kb < hi and kb < KB) for kb in loads) or consumed != mine:
                bad.append((split, wave))
            every.extend(consumed)
    if sorted(every) != list(range(KB)):
        bad.append("coverage")
    return bad


@pytest.mark.parametrize("S", [1, 2, 4])
@pytest.mark.parametrize("D", [1, 2, 3, 4])
@pytest.mark.parametrize("NW", [1, 4, 8, 16])
def test_schedule_in_range_and_complete(NW, D, S):
    for KB in list(range(1, 70)) + [112, 144, 224]:
        assert not violations(KB, NW, D, S), (KB, NW, D, S)


def test_unclamped_first_slots_read_out_of_range():
    """Without the clamp, a wave with fewer blocks than slots loads past its
    range (e.g. two K blocks over 16 waves with two slots)."""
    assert violations(2, 16, 2, 1, clamp_first=False)
    assert not violations(2, 16, 2, 1)


@pytest.mark.parametrize("S", [1, 2, 4])
@pytest.mark.parametrize("NW", [8, 16])
def test_four_block_units_in_range_and_complete(NW, S):
    """The 2:4 weight loaded four K blocks at a time (D = 1 slot of one unit), with
    splits that leave some waves without a unit: e.g. the 4096 x 14336 weight (112
    blocks = 28 units) split four ways gives 7 units per split over 8 waves, and
    K = 12800 (25 units) gives 7/7/7/4."""
    for KB in [4 * u for u in range(1, 40)] + [112, 100, 144, 224]:
        assert not violations(KB, NW, 1, S, U=4), (KB, NW, S)


def test_idle_waves_with_units():
    """Waves past a split's unit count load nothing."""
    loads, consumed, mine, _ = schedule(112, 8, 1, 4, split=0, wave=7, U=4)
    assert loads == [] and consumed == [] and mine == []
    loads, _, _, (lo, hi) = schedule(100, 8, 1, 4, split=3, wave=3, U=4)
    assert loads == list(range(96, 100)) and (lo, hi) == (84, 100)


# ------------------------------------------------------- shared-token form --
#
# decode_shared_kernel (gemm_decode.hpp): workgroup b0 of a grid of G (G a
# multiple of the K split count S) takes split b0 % S and row bands
# b0 / S + j * (G / S); its waves split each band's US units round-robin (a
# wave with n_w units per band), run their items t = j * n_w + i through the
# D-slot schedule of decode_kernel, and after the last unit of a band meet at
# a barrier, so every wave must close the same bands in the same order.

def shared_schedule(bands: int, S: int, G: int, b0: int, US: int, NW: int, D: int, wave: int):
    first, stride = b0 // S, G // S
    nbj = (bands - first + stride - 1) // stride if first < bands else 0
    n_w = (US - wave + NW - 1) // NW
    T = nbj * n_w
    item = lambda t: (first + (t // n_w) * stride, b0 % S, wave + (t % n_w) * NW)
    slot = [None] * D
    loads, consumed, closed = [], [], []

    def load(d, t):
        loads.append(item(t))
        slot[d] = item(t)

    def consume(d, t):
        assert slot[d] == item(t)
        consumed.append(slot[d])
        if t % n_w == n_w - 1:
            closed.append(item(t)[0])

    if T > 0:
        for d in range(D):
            load(d, min(d, T - 1))
    t0 = 0
    while t0 + 2 * D <= T:
        for d in range(D):
            consume(d, t0 + d)
            load(d, t0 + d + D)
        t0 += D
    if t0 + D <= T:
        for d in range(D):
            consume(d, t0 + d)
            if t0 + d + D < T:
                load(d, t0 + d + D)
        t0 += D
    for d in range(D - 1):
        if t0 + d < T:
            consume(d, t0 + d)
    return loads, consumed, closed, [item(t) for t in range(T)], nbj


@pytest.mark.parametrize("bands,S,G,US,NW", [
    (1792, 1, 256, 32, 16), (1792, 1, 512, 32, 16), (256, 1, 256, 32, 16), (8, 1, 8, 8, 8),
    (1792, 1, 512, 8, 8), (1024, 1, 256, 2, 2), (100, 1, 64, 5, 4), (256, 4, 256, 28, 16),
    (256, 4, 512, 7, 4), (256, 2, 256, 56, 16), (37, 1, 16, 3, 3), (5, 1, 8, 4, 4)])
@pytest.mark.parametrize("D", [1, 2, 3])
def test_shared_schedule_covers_every_unit_once(bands, S, G, US, NW, D):
    every = []
    for b0 in range(G):
        per_wave_closed = []
        for wave in range(NW):
            loads, consumed, closed, items, nbj = shared_schedule(bands, S, G, b0, US, NW, D, wave)
            assert all(b < bands and u < US for b, _, u in loads), (b0, wave)
            assert consumed == items
            per_wave_closed.append(closed)
            every.extend(consumed)
        # every wave meets the others at the same band barriers, in order
        assert all(c == per_wave_closed[0] for c in per_wave_closed), b0
        assert per_wave_closed[0] == [b0 // S + j * (G // S) for j in range(len(per_wave_closed[0]))]
    assert sorted(every) == sorted((b, s, u) for b in range(bands) for s in range(S) for u in range(US))


def test_shared_schedule_needs_a_unit_per_wave():
    """With fewer units than waves a wave would close no band and miss the
    barriers, which is why the host requires at least NW units per split."""
    _, _, closed, _, nbj = shared_schedule(64, 1, 16, 0, 3, 4, 2, 3)
    assert nbj > 0 and closed == []


def test_shared_staging_split_is_exact():
    """The staging loop of decode_shared_kernel splits a chunk index q into
    (row, rest) by d with a float reciprocal and one correction step instead
    of an integer division.  Emulated in float32 for every divisor the kernel
    can use (chunks per row 8 * KBs for 16 <= KBs < 64, and KBs itself) and
    every index below 16 rows: always equal to divmod."""
    import numpy as np

    def split(q, d):
        inv = np.float32(1.0) / np.float32(d)
        row = (np.float32(q) * inv).astype(np.int64)  # truncation, as the float -> int conversion
        rem = q - row * d
        lo, hi = rem < 0, rem >= d
        row = np.where(lo, row - 1, np.where(hi, row + 1, row))
        rem = np.where(lo, rem + d, np.where(hi, rem - d, rem))
        return row, rem

    for d in sorted(set(range(16, 64)) | {8 * k for k in range(16, 64)}):
        q = np.arange(16 * d, dtype=np.int64)
        row, rem = split(q, d)
        assert np.array_equal(row, q // d) and np.array_equal(rem, q % d), d


def wave_band_schedule(bands: int, G: int, b0: int, US: int, NW: int, D: int, wave: int):
    """decode_shared_kernel with whole bands per wave (WB, S = 1): wave v of
    workgroup b0 takes the workgroup's bands v, v + NW, ... (its j-th band is
    b0 + (v + j NW) G) and all US units of each, through the D-slot schedule."""
    nbj = (bands - b0 + G - 1) // G if b0 < bands else 0
    nbw = (nbj - wave + NW - 1) // NW if nbj > wave else 0
    T = nbw * US
    item = lambda t: (b0 + (wave + (t // US) * NW) * G, t % US)
    slot = [None] * D
    loads, consumed, stored = [], [], []

    def load(d, t):
        loads.append(item(t))
        slot[d] = item(t)

    def consume(d, t):
        assert slot[d] == item(t)
        consumed.append(slot[d])
        if t % US == US - 1:
            stored.append(item(t)[0])

    if T > 0:
        for d in range(D):
            load(d, min(d, T - 1))
    t0 = 0
    while t0 + 2 * D <= T:
        for d in range(D):
            consume(d, t0 + d)
            load(d, t0 + d + D)
        t0 += D
    if t0 + D <= T:
        for d in range(D):
            consume(d, t0 + d)
            if t0 + d + D < T:
                load(d, t0 + d + D)
        t0 += D
    for d in range(D - 1):
        if t0 + d < T:
            consume(d, t0 + d)
    return loads, consumed, stored, [item(t) for t in range(T)]


@pytest.mark.parametrize("bands,G,US,NW", [(1792, 256, 8, 16), (1792, 256, 8, 8), (1024, 256, 8, 16), (37, 8, 3, 4),
                                           (5, 8, 8, 16), (300, 64, 1, 3)])
@pytest.mark.parametrize("D", [1, 2, 3])
def test_wave_band_schedule_covers_every_band_once(bands, G, US, NW, D):
    every, bands_stored = [], []
    for b0 in range(G):
        for wave in range(NW):
            loads, consumed, stored, items = wave_band_schedule(bands, G, b0, US, NW, D, wave)
            assert all(b < bands and u < US for b, u in loads), (b0, wave)
            assert consumed == items
            every.extend(consumed)
            bands_stored.extend(stored)
    assert sorted(every) == sorted((b, u) for b in range(bands) for u in range(US))
    assert sorted(bands_stored) == list(range(bands))  # each band stored once, by the wave that summed it


def scale_stride(blocks: int) -> int:
    """QuantTokens::scale_stride: rows of an odd number of floats."""
    return blocks | 1


def stage_scales(xs, M: int, KB: int, kb_lo: int, blocks: int, nthreads: int, k_pass: int = 4):
    """QuantTokens::stage_scales over all threads of a workgroup: (LDS contents by
    index, global indices read).  Mirrors the kernel's passes: every thread loads
    k_pass words (past the end: the last word again), then writes those in range."""
    ss = scale_stride(blocks)
    lds, reads = {}, []
    total = M * blocks
    for q0 in range(0, total, k_pass * nthreads):
        for tid in range(nthreads):
            vals = []
            for u in range(k_pass):
                q = min(q0 + u * nthreads + tid, total - 1)
                m = q // blocks
                g = m * KB + kb_lo + (q - m * blocks)
                reads.append(g)
                vals.append(xs[g])
            for u in range(k_pass):
                q = q0 + u * nthreads + tid
                if q < total:
                    m = q // blocks
                    idx = m * ss + (q - m * blocks)
                    assert idx not in lds, "an LDS word written twice"
                    lds[idx] = vals[u]
    return lds, reads


# (M, K blocks, S, U, waves): every launched decode configuration on quantized
# tokens (the Llama-3-8B and DeepSeek-V3 shapes, dense and 2:4) plus ragged ones
@pytest.mark.parametrize("M,KB,S,U,NW", [
    (1, 32, 1, 1, 16), (3, 32, 1, 1, 16), (16, 32, 1, 4, 8), (16, 32, 1, 1, 8), (32, 32, 1, 1, 8), (64, 32, 2, 1, 8),
    (16, 112, 4, 1, 8), (32, 112, 4, 4, 8), (20, 112, 4, 1, 8), (1, 112, 1, 1, 4), (64, 56, 1, 1, 8),
    (13, 65, 4, 1, 8), (7, 9, 4, 1, 8), (5, 3, 4, 1, 8), (64, 144, 1, 4, 8), (64, 33, 2, 1, 16)])
def test_token_scale_staging_and_indices(M, KB, S, U, NW):
    """Each split's workgroup stages exactly the scales of its K range: every
    global read is inside xs and inside the split's blocks, every LDS word of
    the range is written once with the right value, and the LDS index each
    load records (m * ss + kb - kb_lo) points at xs[m][kb] for every block the
    split's waves load, within the bytes the host allocates for the launch."""
    KU = KB // U
    KBs = (KU + S - 1) // S
    xs = list(range(M * KB))  # distinct values: the LDS word names its source
    alloc_words = M * scale_stride(KBs * U)
    for split in range(S):
        kb0 = split * KBs if S > 1 else 0
        KBr = max(0, min(KU, kb0 + KBs) - kb0) if S > 1 else KU
        lo, blocks = kb0 * U, KBr * U
        lds, reads = stage_scales(xs, M, KB, lo, blocks, NW * 64)
        ss = scale_stride(blocks)
        assert len(lds) == M * blocks
        for g in reads:
            assert 0 <= g < M * KB and lo <= g % KB < lo + blocks
        for wave in range(NW):
            loads, _, _, (r0, r1) = schedule(KB, NW, 2, S, split, wave, U=U)
            for kb in loads:
                assert r0 <= kb < r1
                for m in range(M):
                    idx = m * ss + (kb - lo)
                    assert idx < alloc_words
                    assert lds[idx] == xs[m * KB + kb]


def test_token_scale_rows_hit_distinct_banks():
    """The 16 tokens of a fragment read their scales from 16 different LDS banks
    (32-bit banks, 64 of them) for every K range the launches stage."""
    for blocks in (1, 3, 7, 8, 14, 16, 28, 32, 56, 112):
        ss = scale_stride(blocks)
        for kb in range(blocks):
            banks = {(m * ss + kb) % 64 for m in range(16)}
            assert len(banks) == 16, (blocks, kb)


def swz(r: int) -> int:
    """The tile kernels' 16-byte chunk swizzle of row r (gemm_common.hpp)."""
    return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r >> 2) & 1) << 2)


@pytest.mark.parametrize("M,c", [(64, 0), (64, 3), (17, 1), (23, 1), (40, 2)])
def test_linear_code_tile_round_trip(M, c):
    """load_row_runs / row_runs_to_frag (the token code tiles of
    QuantTokensT (modes 1 and 2) and the weight tiles of DenseWeightRows, whose rows are
    never clamped): each lane loads 16 bytes of a
    whole-row run (8 rows of 128 bytes per load, rows past M clamped to M - 1),
    writes them to the wave's LDS tile at 16 * lane (and 1024 + 16 * lane), and
    reads back the MFMA fragment: lane (g, lr) must get bytes 16g .. 16g + 15
    and 64 + 16g .. 64 + 16g + 15 of token min(16c + lr, M - 1)'s K block."""
    K = 4096
    kb = 5
    x = [[(m * 131 + b * 7) % 251 for b in range(K)] for m in range(M)]
    tile = [None] * 2048
    for lane in range(64):
        r, p = lane >> 3, lane & 7
        for h in (0, 1):
            row = min(16 * c + 8 * h + r, M - 1)
            chunk = p ^ swz(8 * h + r)
            for j in range(16):
                tile[1024 * h + 16 * lane + j] = x[row][kb * 128 + 16 * chunk + j]
    assert None not in tile
    for lane in range(64):
        g, lr = lane >> 4, lane & 15
        m = min(16 * c + lr, M - 1)
        lo = tile[lr * 128 + ((g ^ swz(lr)) << 4):][:16]
        hi = tile[lr * 128 + (((g + 4) ^ swz(lr)) << 4):][:16]
        assert lo == x[m][kb * 128 + 16 * g:][:16]
        assert hi == x[m][kb * 128 + 64 + 16 * g:][:16]


def vswz(r: int) -> int:
    """The 2:4 tile kernel's chunk swizzle of a 64-byte value row (gemm_sparse.hip)."""
    return (((r >> 2) & 1) * 3) ^ (((r >> 3) & 1) << 1)


def test_sparse_value_tile_round_trip():
    """SparseWeight4Rows: four runs of 4 rows x 256 bytes (lane l: row 4i + l / 16,
    16-byte chunk l % 16, i.e. block (l / 4) % 4, chunk l % 4), written to four
    16 x 64-byte blocks with chunk c of row r at position c ^ vswz(r), read back
    as lane (g, lr)'s fragment of block b: bytes 16g .. 16g + 15 of row lr's block
    b values, as SparseWeight4 loads them."""
    vals = [[(r * 37 + b * 11) % 253 for b in range(256)] for r in range(16)]  # one unit: 4 blocks x 64 B
    tile = [None] * 4096
    for i in range(4):
        for lane in range(64):
            r = 4 * i + (lane >> 4)
            u, c = (lane >> 2) & 3, lane & 3
            data = vals[r][16 * (lane & 15):][:16]
            off = u * 1024 + r * 64 + 16 * (c ^ vswz(r))
            for j in range(16):
                assert tile[off + j] is None, "a byte written twice"
                tile[off + j] = data[j]
    assert None not in tile
    for lane in range(64):
        g, lr = lane >> 4, lane & 15
        for b in range(4):
            off = b * 1024 + lr * 64 + 16 * (g ^ vswz(lr))
            assert tile[off:off + 16] == vals[lr][64 * b + 16 * g:][:16]
