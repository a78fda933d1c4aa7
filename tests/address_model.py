"""Host-side model of every memory access the decode kernels make (and, at
the end, the absorb_q / expand_v projection kernels).

For a launch description (the kernel arguments) this module enumerates, per
workgroup, wave and lane, the address arithmetic of the kernels as written in
csrc/decode_latent_wide.hip (128 heads, bf16 cache), csrc/decode_latent_fp8.hip
(128 heads, E4M3 cache) and csrc/decode_latent.hip (16, 32 and 64 heads):

  * every direct-to-LDS copy (global_load_lds_dword[x4]): its global source
    bytes and its LDS destination bytes, including the copies issued past the
    last tile and the clamped rows of ragged tiles;
  * the query loads / query staging copies;
  * every store of o_lat / o_part (bf16 rows) and lse / lse_part.

and checks them against the buffers: a cache read must land inside the row
of a token of the workgroup's own token range (and, paged, inside that
token's block), query reads inside the workgroup's query rows, LDS bytes
inside the kernel's LDS allocation, stores inside the workgroup's own output
rows.  The model is plain integer arithmetic on the host; nothing here runs
on a GPU.  A mismatch between the model and the kernels' source is a bug of
the model; the tests keep them side by side (same names, same formulas).
"""
import numpy as np

TILE = 32
KV_ROW_BF16 = 1024
PE_ROW_BF16 = 128


def lat_swz(r):
    r = np.asarray(r)
    return (((r >> 1) & 1) * 6) ^ (((r >> 2) & 1) * 4) ^ (((r >> 3) & 1) * 3)


def kv_swizzle(r):
    r = np.asarray(r)
    return ((r & 7) << 1) | ((r >> 3) & 1)


def pe_swizzle(r):
    return (np.asarray(r) >> 1) & 7


class Launch:
    """The arguments of one decode-kernel launch (what DecodeArgs holds).

    lens: device lengths per sequence (clamped like the kernels do);
    kv_sb / pe_sb: bytes between slots; seq_stride (contiguous) or
    block_table [B, max_blocks] + block_size (paged); num_slots: slots the
    cache allocation holds; items: planned (seq, first_tile, count, partial row) rows or
    None; q_start / q_per_seq / q_group: prefill.
    """

    def __init__(self, heads, lens, max_seq_len, num_splits=1, fp8=False, kv_sb=None, pe_sb=None,
                 seq_stride=None, block_table=None, block_size=0, num_slots=None, items=None,
                 q_start=None, q_per_seq=1, q_group=1):
        self.H = heads
        self.lens = np.asarray(lens, dtype=np.int64)
        self.max_seq_len = int(max_seq_len)
        self.P = int(num_splits)
        self.fp8 = bool(fp8)
        self.kv_sb = kv_sb if kv_sb is not None else (1152 if not fp8 else 576)
        self.pe_sb = pe_sb if pe_sb is not None else self.kv_sb
        self.seq_stride = seq_stride
        self.block_table = None if block_table is None else np.asarray(block_table, dtype=np.int64)
        self.block_size = int(block_size)
        self.num_slots = num_slots
        self.items = None if items is None else np.asarray(items, dtype=np.int64)
        self.q_start = None if q_start is None else np.asarray(q_start, dtype=np.int64)
        self.q_per_seq = int(q_per_seq)
        self.q_group = int(q_group)
        per = -(-self.max_seq_len // self.P)
        self.chunk = 32 * (-(-per // 32))
        self.kv_row = KV_ROW_BF16 // (2 if fp8 else 1)
        self.pe_row = PE_ROW_BF16 // (2 if fp8 else 1)

    # -- the cache slot of token t of sequence cb --
    def slot(self, cb, t):
        t = np.asarray(t)
        if self.block_table is None:
            return cb * self.seq_stride + t
        return self.block_table[cb, t // self.block_size] * self.block_size + t % self.block_size


# The kernels clamp the rows of a ragged tile to its last valid row; a test
# turns this off to show the model reports the reads it would cause.
CLAMP_RAGGED_ROWS = True


class Violation(AssertionError):
    pass


def _need(cond, msg):
    if not np.all(cond):
        raise Violation(msg)


# ---------------------------------------------------------------------------
# 128-head kernel (decode_latent_wide_kernel<4, PAGED, FP8>)
# ---------------------------------------------------------------------------

def wide_lds_layout():
    NW, H = 4, 128
    NLAT, NPE = 4, 3
    kLatBytes, kPeBytes = TILE * 1024, TILE * 128
    kPeRing = 0
    kLatRing = kPeRing + NPE * kPeBytes
    kPOff = kLatRing + NLAT * kLatBytes
    kPBuf = NW * 2048
    kAlphaOff = kPOff + 2 * kPBuf
    kFlagOff = kAlphaOff + 2 * H * 4
    kSmem = kFlagOff + 64
    kQStage = kLatRing + 2 * kLatBytes
    return dict(NLAT=NLAT, NPE=NPE, kLatBytes=kLatBytes, kPeBytes=kPeBytes, kLatRing=kLatRing,
                kPeRing=kPeRing, kSmem=kSmem, kQStage=kQStage, kQWave=16 * 1024 + 2048)


def wide_items(L):
    """(item, b, cb, row0, i0, nq, t_begin, t_end, part, final, rot) per workgroup."""
    H = L.H
    QG = L.q_group
    out = []
    if L.items is not None:
        n_wg = len(L.items)
    else:
        groups = -(-L.q_per_seq // QG)
        n_rows_wg = (len(L.lens) if L.q_start is None else (len(L.q_start) * groups))
        n_wg = n_rows_wg * L.P
    max_tiles = -(-L.max_seq_len // 32)
    for item in range(n_wg):
        planned = L.items is not None
        if planned:
            s, f, n, slot = L.items[item]
            if not 0 <= slot < len(L.items):
                continue  # no partial row: the workgroup returns at once
            ok = 0 <= s < len(L.lens) and 0 <= f < max_tiles and n >= 1
            pl = (s, 32 * f, 32 * (f + min(n, max_tiles - f))) if ok else (0, 0, 0)
            qrow, split = pl[0], item
        else:
            qrow, split = item // L.P, item % L.P
        groups = -(-L.q_per_seq // QG)
        batch_rows = len(L.lens) if L.q_start is None else len(L.q_start) * L.q_per_seq
        n_wg_rows = (batch_rows // L.q_per_seq) * groups if QG > 1 else batch_rows
        b = qrow if L.q_start is None else n_wg_rows - 1 - qrow
        cb = b // groups
        i0 = (b - cb * groups) * QG
        nq = min(QG, L.q_per_seq - i0)
        row0 = cb * L.q_per_seq + i0

        def length_of(qi):
            t = L.lens[b] if L.q_start is None else max(L.q_start[cb], 0) + qi + 1
            return 0 if t < 0 else min(int(t), L.max_seq_len)
        T = length_of(i0 + nq - 1)
        t_begin = pl[1] if planned else split * L.chunk
        t_end = min(T, pl[2] if planned else t_begin + L.chunk)
        final = (not planned) and L.P == 1
        part = slot if planned else b * L.P + split
        out.append(dict(item=item, b=b, cb=cb, row0=row0, nq=nq, t_begin=t_begin, t_end=t_end, part=part,
                        final=final, rot=(split * 2) & 15, T=T))
    return out


def check_wide(L, max_items=None):
    """Enumerate and check every access of the 128-row kernel; returns counts.
    L.H is the number of heads per query (Hq); with fewer than 128 (grouped
    prefill) a workgroup's 128 rows are q_group queries of Hq heads."""
    _need(not L.fp8, "the 128-row kernel takes a bf16 cache")
    lay = wide_lds_layout()
    Hq = L.H
    counts = dict(copies=0, stores=0, workgroups=0)
    lanes = np.arange(64)
    wgs = wide_items(L)
    if max_items is not None:
        wgs = wgs[:max_items]
    q_rows_total = (len(L.lens) if L.q_start is None else len(L.q_start) * L.q_per_seq) * Hq
    for wg in wgs:
        counts["workgroups"] += 1
        n_rows = wg["nq"] * Hq
        if wg["final"]:
            row_lo = wg["row0"] * Hq
        else:
            row_lo = wg["part"] * Hq
        row_hi = row_lo + n_rows
        tb, te = wg["t_begin"], wg["t_end"]
        if tb >= te:
            # empty: zero rows 32w + r < n_rows, 16 bytes per lane; lse of 32w + h32
            for w in range(4):
                rows = 32 * w + np.arange(32)
                rows = rows[rows < n_rows]
                _need((rows + row_lo >= row_lo) & (rows + row_lo < row_hi), "empty store outside the rows")
                counts["stores"] += rows.size
            continue
        n_tiles = -(-(te - tb) // TILE)
        cb = wg["cb"]
        # ---- query staging (stage_q, two halves per wave) ----
        for w in range(4):
            for hh in range(2):
                qo = min((32 * w + 16 * hh) // Hq, wg["nq"] - 1)
                head0 = (wg["row0"] + qo) * Hq + (32 * w + 16 * hh) % Hq
                for jj in range(16):
                    j = (jj + wg["rot"]) & 15
                    byte = (lanes ^ j) << 4
                    _need((byte >= 0) & (byte + 16 <= 1024), "q_lat read outside its row")
                    _need(head0 + j < q_rows_total, "q_lat row outside the queries")
                    _need((head0 + j) // Hq == wg["row0"] + qo, "q_lat row of another query")
                    dst = lay["kQStage"] + w * lay["kQWave"] + j * 1024 + 16 * lanes
                    _need((dst >= 0) & (dst + 16 <= lay["kSmem"]), "query staging outside LDS")
                for i in range(2):
                    j = 8 * i + (lanes >> 3)
                    byte = (((lanes & 7) ^ ((j >> 1) & 7)) << 4)
                    _need((byte + 16 <= 128) & (head0 + j < q_rows_total), "q_pe read out of bounds")
                    dst = lay["kQStage"] + w * lay["kQWave"] + 16384 + i * 1024 + 16 * lanes
                    _need(dst + 16 <= lay["kSmem"], "q_pe staging outside LDS")
        # ---- tile copies: tiles 0 .. n_tiles + 2 are requested ----
        tiles = np.arange(n_tiles + 3)
        src = np.minimum(tiles, n_tiles - 1)
        t0 = tb + src * TILE
        last = np.minimum(TILE, te - t0) - 1
        if L.block_table is not None:
            _need(t0 % TILE == 0, "tile start not tile-aligned")
            _need((t0 % L.block_size) + last < L.block_size, "tile crosses a block")
        for w in range(4):
            r = 8 * w + (lanes >> 3)                       # [64]
            rc = np.minimum(r[None, :], last[:, None]) if CLAMP_RAGGED_ROWS else np.broadcast_to(r, last.shape + r.shape)
            tok = t0[:, None] + rc
            _need((tok >= tb) & (tok < te), "cache row outside the workgroup's token range")
            for k in range(9):
                if k < 8:
                    byte = (((lanes & 7) ^ lat_swz(r)) << 4) + 128 * k
                    _need((byte >= 0) & (byte + 16 <= 1024), "latent copy outside the row")
                    lat_buf = lay["kLatRing"] + (tiles % lay["NLAT"]) * lay["kLatBytes"]
                    dst = lat_buf[:, None] + w * 8192 + 1024 * k + 16 * lanes[None, :]
                    _need((dst >= lat_buf[:, None]) & (dst + 16 <= lat_buf[:, None] + lay["kLatBytes"]),
                          "latent copy outside its ring buffer")
                else:
                    byte = ((lanes & 7) ^ pe_swizzle(r)) << 4
                    _need(byte + 16 <= 128, "RoPE copy outside the row")
                    pe_buf = lay["kPeRing"] + (tiles % lay["NPE"]) * lay["kPeBytes"]
                    dst = pe_buf[:, None] + w * 1024 + 16 * lanes[None, :]
                    _need(dst + 16 <= pe_buf[:, None] + lay["kPeBytes"], "RoPE copy outside its buffer")
                counts["copies"] += tok.size
            slots = L.slot(cb, tok)
            if L.num_slots is not None:
                _need((slots >= 0) & (slots < L.num_slots), "cache slot outside the allocation")
        # ---- epilogue stores ----
        for w in range(4):
            col0 = 128 * w
            for n in range(4):
                for k in range(8):
                    Lr = 64 * k + lanes
                    row, ch = Lr // 16, Lr % 16
                    keep = (32 * n + row) < n_rows
                    grow = row_lo + 32 * n + row[keep]
                    col = col0 + ch[keep] * 8
                    _need((grow >= row_lo) & (grow < row_hi) & (col + 8 <= 512), "o store outside the rows")
                    counts["stores"] += int(keep.sum())
            hd = 32 * w + np.arange(32)
            _need(row_lo + hd[hd < n_rows] < row_hi, "lse store outside the rows")
    return counts


# ---------------------------------------------------------------------------
# 128-head E4M3 kernel (decode_latent_fp8_kernel<PAGED, STREAM>)
# ---------------------------------------------------------------------------

T8 = 64   # rows per tile


def fp8_lds_layout():
    NW = 4
    kLat8, kPe8, kSc8 = T8 * 512, T8 * 64, 512
    kLatRing = 0
    kPeRing = kLatRing + 4 * kLat8
    kScRing = kPeRing + 3 * kPe8
    kRtsOff = kScRing + 4 * kSc8
    kSmem = kRtsOff + NW * 2 * 256
    return dict(kLat8=kLat8, kPe8=kPe8, kSc8=kSc8, kLatRing=kLatRing, kPeRing=kPeRing, kScRing=kScRing,
                kRtsOff=kRtsOff, kSmem=kSmem)


def fp8_lds_reads():
    """Every LDS byte range the E4M3 kernel reads inside one tile buffer, per
    lane: (name, offsets [n, 64], width, buffer size).  These do not depend on
    the launch."""
    ln = np.arange(64)
    ki, kg = ln & 31, ln >> 5
    out = []
    # K fragments: latent chunks of slices s < 8, token half tb
    kbl = [ki * 512 + (((2 * kg + q) ^ (ki & 15)) << 4) for q in range(2)]
    offs = []
    for tb in range(2):
        for sl in range(8):
            x, m = (sl & 3) << 6, 256 * (sl >> 2) + 16384 * tb
            for q in range(2):
                offs.append((kbl[q] ^ x) + m)
    out.append(("K latent fragment", np.array(offs), 16, T8 * 512))
    pbl = ki * 64 + (((2 * kg) ^ ((ki >> 2) & 3)) << 4)
    out.append(("K RoPE fragment", np.array([pbl + 2048 * tb for tb in range(2)] +
                                            [(pbl ^ 16) + 2048 * tb for tb in range(2)]), 16, T8 * 64))
    # V^T fragments (transposing 8-byte reads)
    vG, vi = ln >> 4, ln & 15
    vr0 = 8 * (vi >> 3) + 4 * (vG >> 1) + ((vi >> 1) & 3)
    vbl = vr0 * 512 + (((vG & 1) ^ vr0) << 4) + 8 * (vi & 1)
    out.append(("V^T fragment", np.array([((vbl ^ ((ct & 7) << 5)) + 256 * (ct >> 3)) + 8192 * q
                                          for ct in range(16) for q in range(4)]), 8, T8 * 512))
    # token scales (first copy of each half) and their reciprocals
    lgo = 16 * kg
    out.append(("token scales", np.array([256 * h + 32 * a4 + lgo for h in range(2) for a4 in range(4)]), 16, 512))
    out.append(("token scale for its reciprocal", np.array([256 * kg + 4 * ki]), 4, 512))
    out.append(("reciprocal scales", np.array([128 * h + 32 * a4 + lgo for h in range(2) for a4 in range(4)]),
                16, 256))
    return out


def check_fp8(L, max_items=None):
    """Enumerate and check every access of the 128-head E4M3 kernel."""
    _need(L.fp8 and L.H == 128 and L.q_group == 1, "the E4M3 128-head kernel")
    lay = fp8_lds_layout()
    _need(lay["kSmem"] <= 160 * 1024, "LDS budget")
    for name, offs, width, size in fp8_lds_reads():
        _need((offs >= 0) & (offs % width == 0) & (offs + width <= size), name + " outside its buffer")
    counts = dict(copies=0, stores=0, workgroups=0)
    lanes = np.arange(64)
    wgs = wide_items(L)
    if max_items is not None:
        wgs = wgs[:max_items]
    q_rows_total = (len(L.lens) if L.q_start is None else len(L.q_start) * L.q_per_seq) * 128
    for wg in wgs:
        counts["workgroups"] += 1
        row_lo = (wg["row0"] if wg["final"] else wg["part"]) * 128
        row_hi = row_lo + 128
        tb, te = wg["t_begin"], wg["t_end"]
        for w in range(4):
            # epilogue (also the empty range): rows 32w + r, 16 bytes per lane; lse of 32w + li
            rows = row_lo + 32 * w + np.arange(32)
            _need((rows >= row_lo) & (rows < row_hi) & (8 * lanes.max() + 8 <= 512), "o store outside the rows")
            counts["stores"] += 32 * 64
        if tb >= te:
            continue
        # query: head 32w + li, 16-byte reads 8s + 4lg + k (latent) and 4lg + k (RoPE)
        for w in range(4):
            head = wg["row0"] * 128 + 32 * w + (lanes & 31)
            _need(head < q_rows_total, "q row outside the queries")
            lat_chunks = np.array([8 * s_ + 4 * (lanes >> 5) + k for s_ in range(8) for k in range(4)])
            _need((lat_chunks >= 0) & (16 * lat_chunks + 16 <= 1024), "q_lat read outside its row")
            pe_chunks = np.array([4 * (lanes >> 5) + k for k in range(4)])
            _need(16 * pe_chunks + 16 <= 128, "q_pe read outside its row")
        n_tiles = -(-(te - tb) // T8)
        cb = wg["cb"]
        tiles = np.arange(n_tiles)[:, None]                  # [n, 1]
        t0 = tb + tiles * T8
        last = np.minimum(T8, te - t0) - 1
        _need(last >= 0, "tile past the range")
        lat = lay["kLatRing"] + (tiles % 4) * lay["kLat8"]
        pe = lay["kPeRing"] + (tiles % 3) * lay["kPe8"]
        sc = lay["kScRing"] + (tiles % 4) * lay["kSc8"]
        if L.block_table is not None:
            for hf in range(2):
                h0 = t0 + 32 * hf
                has = (hf == 0) | (last >= 32)
                rows_h = np.minimum(32, te - h0)
                _need(~has | ((h0 % 32 == 0) & ((h0 % L.block_size) + rows_h <= L.block_size)),
                      "half tile crosses a block")

        def src_row(hf, rc):
            # a copy reads row rc of half hf from that half's first slot
            base_tok = t0 + 32 * hf
            tok = base_tok + rc
            _need((tok >= tb) & (tok < te), "cache row outside the workgroup's token range")
            slot = L.slot(cb, base_tok) + rc
            _need(slot == L.slot(cb, tok), "a half tile's rows are not contiguous slots")
            if L.num_slots is not None:
                _need((slot >= 0) & (slot < L.num_slots), "cache slot outside the allocation")
        for w in range(4):
            for c in range(10):
                if c < 8:
                    r0 = 16 * w + 2 * c
                    hf = np.minimum(r0, last) >> 5
                    r = r0 + (lanes >> 5)
                    rc = np.minimum(r, last) - 32 * hf
                    _need((rc >= 0) & (rc < 32), "latent row outside its half")
                    byte = ((lanes & 31) ^ (r & 15)) << 4
                    _need(byte + 16 <= 512, "latent copy outside the row")
                    dst = lat + r0 * 512 + 16 * lanes
                    _need((dst >= lat) & (dst + 16 <= lat + lay["kLat8"]), "latent copy outside its buffer")
                    # full tiles take the lane-constant form: half w // 2, offset
                    # ((lane chunk ^ lg) << 4 ^ (c << 5)) + (16 (w % 2) + lg + 2c) rows,
                    # LDS lat + 16 w rows + 1024 c (the M0 immediate)
                    full = last == T8 - 1
                    lg = lanes >> 5
                    fast = (((((lanes & 31) ^ lg) << 4) ^ (c << 5)) + (16 * (w & 1) + lg) * L.kv_sb
                            + 2 * c * L.kv_sb)
                    _need(~full | ((hf == w >> 1) & (fast == rc * L.kv_sb + byte)),
                          "full-tile latent copy differs from the clamped form")
                    _need(~full | (lat + 16 * w * 512 + 1024 * c + 16 * lanes == dst),
                          "full-tile latent copy destination differs")
                elif c == 8:
                    r0 = 16 * w
                    hf = np.minimum(r0, last) >> 5
                    r = r0 + (lanes >> 2)
                    rc = np.minimum(r, last) - 32 * hf
                    _need((rc >= 0) & (rc < 32), "RoPE row outside its half")
                    byte = ((lanes & 3) ^ ((r >> 2) & 3)) << 4
                    _need(byte + 16 <= 64, "RoPE copy outside the row")
                    fast = (16 * (w & 1) + (lanes >> 2)) * L.pe_sb + (((lanes & 3) ^ ((lanes >> 4) & 3)) << 4)
                    _need((last != T8 - 1) | ((hf == w >> 1) & (fast == rc * L.pe_sb + byte)),
                          "full-tile RoPE copy differs from the clamped form")
                    dst = pe + r0 * 64 + 16 * lanes
                    _need((dst >= pe) & (dst + 16 <= pe + lay["kPe8"]), "RoPE copy outside its buffer")
                elif w < 2:
                    hf = np.minimum(32 * w, last) >> 5
                    r = 32 * w + (lanes & 31)
                    rc = np.minimum(r, last) - 32 * hf
                    _need((rc >= 0) & (rc < 32), "scale row outside its half")
                    _need((last != T8 - 1) | ((hf == w) & ((lanes & 31) == rc)),
                          "full-tile scale copy differs from the clamped form")
                    dst = sc + 256 * w + 4 * lanes
                    _need((dst >= sc) & (dst + 4 <= sc + lay["kSc8"]), "scale copy outside its buffer")
                else:
                    continue
                src_row(hf, rc)
                counts["copies"] += int(rc.size)
        _need((lat + lay["kLat8"] <= lay["kPeRing"]) & (sc + lay["kSc8"] <= lay["kRtsOff"]), "ring overlap")
        # epilogue staging: wave w's 32 rows of 1 KiB in the latent ring
        for w in range(4):
            stage = w * 32768
            ch = np.arange(64)
            for r in range(32):
                off = stage + r * 1024 + ((ch ^ (r & 15)) << 4)
                _need(off + 16 <= lay["kPeRing"], "output staging outside the latent ring")
    return counts


# ---------------------------------------------------------------------------
# 16-head bf16 kernel (decode_latent16_kernel<NCW, NBUF, PAGED>)
# ---------------------------------------------------------------------------

L16_NCW = 4       # copy waves
L16_NBUF = 3      # ring of tiles
L16_TILE_BYTES = 36864


def latent16_copy_plan(ncw=L16_NCW):
    """Copy i of a tile (0..35: latent row i, then RoPE copies i - 32) goes to
    copy wave i % ncw, which issues j, j + ncw, ..."""
    return [[j + ncw * k for k in range(36 // ncw)] for j in range(ncw)]


def _range_of(L, item, B, H):
    """(b, cache sequence, t_begin, t_end, output row range) of a workgroup,
    as the narrow kernels compute them."""
    max_tiles = -(-L.max_seq_len // 32)
    planned = L.items is not None
    if planned:
        s, f, n, slot = L.items[item]
        if not 0 <= slot < len(L.items):
            return None  # no partial row: the workgroup returns at once
        ok = 0 <= s < len(L.lens) and 0 <= f < max_tiles and n >= 1
        pl = (s, 32 * f, 32 * (f + min(n, max_tiles - f))) if ok else (0, 0, 0)
        qrow, split = pl[0], item
    else:
        qrow, split = item // L.P, item % L.P
    b = qrow if L.q_start is None else B - 1 - qrow
    cb = b // L.q_per_seq
    T = L.lens[b] if L.q_start is None else max(L.q_start[cb], 0) + (b - cb * L.q_per_seq) + 1
    T = 0 if T < 0 else min(int(T), L.max_seq_len)
    tb = pl[1] if planned else split * L.chunk
    te = min(T, pl[2] if planned else tb + L.chunk)
    final = (not planned) and L.P == 1
    part = slot if planned else b * L.P + split
    row_lo = (b * H) if final else part * H
    return b, cb, tb, te, row_lo, row_lo + H


def check_latent16(L, max_items=None):
    """Copies, LDS reads (with the swizzle of the copy undone: each fragment
    must be the token row and 16-byte chunk the MFMA operand needs), the
    merge's LDS regions and the output stores of the 16-head bf16 kernel."""
    H, NBUF = 16, L16_NBUF
    assert H == L.H and not L.fp8
    kRing = NBUF * L16_TILE_BYTES
    kStage, kStat = 2 * 16384, 2 * 16384 + 2 * 8192
    lanes = np.arange(64)
    counts = dict(copies=0, stores=0, workgroups=0, lds_reads=0)
    B = len(L.lens) if L.q_start is None else len(L.q_start) * L.q_per_seq
    n_wg = len(L.items) if L.items is not None else B * L.P
    if max_items is not None:
        n_wg = min(n_wg, max_items)
    plan = latent16_copy_plan()
    _need(sorted(i for p in plan for i in p) == list(range(36)), "copies do not cover the tile once")
    # fragment reads of one tile buffer (the same for every tile)
    r16, g = lanes & 15, lanes >> 4
    for u in range(2):
        kb0 = u * 16 * 1024 + r16 * 1024 + ((g ^ kv_swizzle(r16)) << 4)
        pb0 = TILE * 1024 + u * 16 * 128 + r16 * 128 + ((g ^ pe_swizzle(r16)) << 4)
        for s_ in range(18):
            if s_ < 16:
                ad = (kb0 ^ ((s_ & 3) << 6)) + 256 * (s_ >> 2)
                row, slot = ad // 1024, (ad % 1024) // 16
                _need((row == 16 * u + r16) & ((slot ^ kv_swizzle(row)) == 4 * s_ + g), "K fragment is not its chunk")
            else:
                ad = pb0 ^ ((s_ - 16) << 6)
                off = ad - TILE * 1024
                row, slot = off // 128, (off % 128) // 16
                _need((row == 16 * u + r16) & ((slot ^ pe_swizzle(row)) == 4 * (s_ - 16) + g),
                      "RoPE fragment is not its chunk")
            _need((ad >= 0) & (ad + 16 <= L16_TILE_BYTES), "K read outside the tile")
            counts["lds_reads"] += 64
        rv = 4 * g + ((lanes & 15) >> 2)
        vb0 = u * 16 * 1024 + rv * 1024 + ((((lanes & 3) >> 1) ^ kv_swizzle(rv)) << 4) + ((lanes & 1) << 3)
        for cb_ in range(32):
            ad = vb0 ^ (cb_ << 5)
            row, slot, half = ad // 1024, (ad % 1024) // 16, (ad % 16) // 8
            # transposing read: lane l points at token row 4 (l/16) + (l%16)/4,
            # columns 16 cb + 4 (l%4) .. +3 (chunk 2 cb + (l%4)/2, half (l%4)%2)
            _need((row == 16 * u + rv) & ((slot ^ kv_swizzle(row)) == 2 * cb_ + ((lanes & 3) >> 1))
                  & (half == (lanes & 1)), "V fragment is not its chunk")
            counts["lds_reads"] += 64
    # merge: exchange, staging and statistics inside the ring
    for u in range(2):
        x_other = (1 - u) * 16384 + 16 * lanes
        _need((x_other + 15 * 1024 + 16 <= kStage), "exchange outside its region")
        stage_w = kStage + u * 8192 + r16 * 512 + ((((2 * np.arange(16)[:, None] + (g >> 1)) ^ r16) << 4)
                                                 + ((g & 1) << 3))
        _need((stage_w >= kStage + u * 8192) & (stage_w + 8 <= kStage + (u + 1) * 8192), "staging write outside")
        _need(kStat + ((u * H + r16) * 8) + 8 <= kRing, "statistics outside the ring")
    for item in range(n_wg):
        counts["workgroups"] += 1
        r = _range_of(L, item, B, H)
        if r is None:
            continue
        b, cb, tb, te, row_lo, row_hi = r
        if tb >= te:
            counts["stores"] += H
            continue
        n_tiles = -(-(te - tb) // TILE)
        issued = list(range(min(NBUF - 1, n_tiles)))
        for it in range(n_tiles):
            if it + NBUF - 1 < n_tiles:
                issued.append(it + NBUF - 1)
        _need(sorted(issued) == list(range(n_tiles)), "tiles not copied exactly once")
        for tile in issued:
            t0 = tb + tile * TILE
            last = min(TILE, te - t0) - 1
            _need(last >= 0, "tile past the range")
            if L.block_table is not None:
                _need(t0 % TILE == 0 and (t0 % L.block_size) + last < L.block_size, "tile crosses a block")
            dst0 = (tile % NBUF) * L16_TILE_BYTES
            for copies in plan:
                for i in copies:
                    if i < TILE:
                        tok = t0 + min(i, last)
                        byte = (16 * lanes) ^ (kv_swizzle(i) << 4)
                        _need((byte + 16 <= 1024), "latent copy outside the row")
                        dst = dst0 + i * 1024 + 16 * lanes
                    else:
                        pi = i - TILE
                        r = 8 * pi + (lanes >> 3)
                        c = (lanes & 7) ^ pe_swizzle(r)
                        tok = t0 + np.minimum(r, last)
                        _need((c << 4) + 16 <= 128, "RoPE copy outside the row")
                        dst = dst0 + TILE * 1024 + pi * 1024 + 16 * lanes
                    _need((tok >= tb) & (tok < te), "copy outside the range")
                    if L.num_slots is not None:
                        sl = L.slot(cb, tok)
                        _need((sl >= 0) & (sl < L.num_slots), "cache slot outside the allocation")
                    _need((dst >= dst0) & (dst + 16 <= dst0 + L16_TILE_BYTES) & (dst + 16 <= kRing),
                          "copy outside its tile")
                    counts["copies"] += 64
        # stores: wave u, rows (L >> 5), columns 256 u + 8 (L & 31)
        for u in range(2):
            for k in range(8):
                Lr = 64 * k + lanes
                row, ch = Lr >> 5, Lr & 31
                col = 256 * u + ch * 8
                _need((row_lo + row < row_hi) & (col + 8 <= 512), "o store outside the rows")
                counts["stores"] += 64
    return counts


# ---------------------------------------------------------------------------
# 16/32/64-head kernel (decode_latent_kernel<NW, NBUF, PAGED, FP8>)
# ---------------------------------------------------------------------------

def narrow_config(H, fp8):
    NW = H // 16
    NBUF = 4 if fp8 else {1: 4, 2: 1, 4: 2}[NW]
    return NW, NBUF


COPY_ROWS = 11   # latent rows per copy wave of a 16-head bf16 workgroup


def narrow_copy_plan(NW, NBUF):
    """bf16 tile copies per wave: [(latent rows, RoPE copies)], one entry per
    wave.  A 16-head workgroup's computing wave copies nothing; its three
    copy waves take latent rows from COPY_ROWS * j (the last the rest) and
    RoPE copy j (the last also the fourth)."""
    if NW == 1 and NBUF == 4:
        plan = [([], [])]
        for j in range(3):
            r0 = COPY_ROWS * j
            r1 = r0 + COPY_ROWS if j < 2 else TILE
            plan.append((list(range(r0, r1)), [j] + ([3] if j == 2 else [])))
        return plan
    KV_PW = TILE // NW
    PE_W = NW if NW < 4 else 4
    PE_PW = 4 // PE_W
    return [(list(range(w * KV_PW, (w + 1) * KV_PW)), [w * PE_PW + k for k in range(PE_PW)] if w < PE_W else [])
            for w in range(NW)]


def check_narrow(L, max_items=None):
    H = L.H
    NW, NBUF = narrow_config(H, L.fp8)
    KV8 = 16 // NW
    E8 = (3 + NW - 1) // NW
    kRawTileBytes = 18944
    kTileBytes = 36864
    kBf16Off = ((NBUF * kRawTileBytes + 1023) // 1024) * 1024 if L.fp8 else 0
    kRing = kBf16Off + (kTileBytes if L.fp8 else NBUF * kTileBytes)
    kSmem = kRing + NW * 1024 + H * 4 + 64
    lanes = np.arange(64)
    counts = dict(copies=0, stores=0, workgroups=0)
    B = len(L.lens) if L.q_start is None else len(L.q_start) * L.q_per_seq
    n_wg = len(L.items) if L.items is not None else B * L.P
    if max_items is not None:
        n_wg = min(n_wg, max_items)
    max_tiles = -(-L.max_seq_len // 32)
    for item in range(n_wg):
        counts["workgroups"] += 1
        planned = L.items is not None
        if planned:
            s, f, n, slot = L.items[item]
            if not 0 <= slot < len(L.items):
                continue  # no partial row: the workgroup returns at once
            ok = 0 <= s < len(L.lens) and 0 <= f < max_tiles and n >= 1
            pl = (s, 32 * f, 32 * (f + min(n, max_tiles - f))) if ok else (0, 0, 0)
            qrow, split = pl[0], item
        else:
            qrow, split = item // L.P, item % L.P
        b = qrow if L.q_start is None else B - 1 - qrow
        cb = b // L.q_per_seq
        T = L.lens[b] if L.q_start is None else max(L.q_start[cb], 0) + (b - cb * L.q_per_seq) + 1
        T = 0 if T < 0 else min(int(T), L.max_seq_len)
        tb = pl[1] if planned else split * L.chunk
        te = min(T, pl[2] if planned else tb + L.chunk)
        final = (not planned) and L.P == 1
        part = slot if planned else b * L.P + split
        row_lo = (b * H) if final else part * H
        row_hi = row_lo + H
        if tb >= te:
            counts["stores"] += H
            continue
        # query loads: q[s] = ql[s * 4 + g4] (16 bytes), rows b * H + h
        n_tiles = -(-(te - tb) // TILE)
        issued = list(range(min(NBUF - 1, n_tiles))) if NBUF > 1 else [0]
        for it in range(n_tiles):
            nxt = it + NBUF - 1
            if NBUF > 1 and nxt < n_tiles:
                issued.append(nxt)
            if NBUF == 1 and it + 1 < n_tiles:
                issued.append(it + 1)
        for tile in issued:
            t0 = tb + tile * TILE
            last = min(TILE, te - t0) - 1
            _need(last >= 0, "tile past the range")
            if L.block_table is not None:
                _need(t0 % TILE == 0 and (t0 % L.block_size) + last < L.block_size, "tile crosses a block")
            buf = 0 if NBUF == 1 else tile % NBUF
            dst0 = buf * (kRawTileBytes if L.fp8 else kTileBytes)
            plan = narrow_copy_plan(NW, NBUF)
            if not L.fp8:
                rows_all = sorted(r for rows, _ in plan for r in rows)
                pes_all = sorted(i for _, pes in plan for i in pes)
                _need(rows_all == list(range(TILE)) and pes_all == [0, 1, 2, 3], "copies do not cover the tile once")
            for w in range(len(plan) if not L.fp8 else NW):
                if not L.fp8:
                    for r in plan[w][0]:
                        tok = t0 + min(r, last)
                        byte = (16 * lanes) ^ (kv_swizzle(r) << 4)
                        _need((tok >= tb) & (tok < te) & (byte + 16 <= 1024), "latent copy out of bounds")
                        if L.num_slots is not None:
                            sl = L.slot(cb, tok)
                            _need((sl >= 0) & (sl < L.num_slots), "cache slot outside the allocation")
                        dst = dst0 + r * 1024 + 16 * lanes
                        _need(dst + 16 <= dst0 + kTileBytes, "latent copy outside its tile")
                        counts["copies"] += 64
                    for i in plan[w][1]:
                        r = 8 * i + (lanes >> 3)
                        c = (lanes & 7) ^ pe_swizzle(r)
                        tok = t0 + np.minimum(r, last)
                        _need((tok >= tb) & (tok < te) & ((c << 4) + 16 <= 128), "RoPE copy out of bounds")
                        dst = dst0 + TILE * 1024 + i * 1024 + 16 * lanes
                        _need(dst + 16 <= dst0 + kTileBytes, "RoPE copy outside its tile")
                        counts["copies"] += 64
                else:
                    for k in range(KV8 + E8):
                        if k < KV8:
                            kk = w * KV8 + k
                            r = np.minimum(2 * kk + (lanes >> 5), last)
                            byte = (lanes & 31) << 4
                            _need(byte + 16 <= 512, "E4M3 latent copy outside the row")
                            dst = dst0 + kk * 1024 + 16 * lanes
                            lim = dst0 + 16384
                        else:
                            e = w * E8 + (k - KV8)
                            if e < 2:
                                r = np.minimum(16 * e + (lanes >> 2), last)
                                byte = (lanes & 3) << 4
                                _need(byte + 16 <= 64, "E4M3 RoPE copy outside the row")
                                dst = dst0 + 16384 + e * 1024 + 16 * lanes
                                lim = dst0 + 18432
                            else:
                                r = np.minimum(lanes & 31, last)
                                dst = dst0 + (18432 if e == 2 else 18688) + 4 * lanes
                                lim = dst0 + kRawTileBytes
                        tok = t0 + r
                        _need((tok >= tb) & (tok < te), "E4M3 row outside the range")
                        if L.num_slots is not None:
                            sl = L.slot(cb, tok)
                            _need((sl >= 0) & (sl < L.num_slots), "cache slot outside the allocation")
                        _need((dst >= dst0) & (dst + (16 if k < KV8 or e < 2 else 4) <= lim), "E4M3 copy outside")
                        counts["copies"] += 64
            _need(dst0 + (kRawTileBytes if L.fp8 else kTileBytes) <= kSmem, "tile ring outside LDS")
        # epilogue: 16 rows x C columns per (wave, head block)
        C = 512 // NW
        RC = C // 8
        for w in range(NW):
            for n in range(NW):
                for k in range((16 * RC) // 64):
                    Lr = 64 * k + lanes
                    row, ch = Lr // RC, Lr % RC
                    grow = row_lo + 16 * n + row
                    col = w * C + ch * 8
                    _need((grow < row_hi) & (col + 8 <= 512), "o store outside the rows")
                    counts["stores"] += 64
    return counts


# ---------------------------------------------------------------------------
# Projection kernels (csrc/proj_combine.hip): absorb_q_kernel<NW> and
# expand_v_kernel<NW>, NW = 4 waves per workgroup from 64 heads, else 1.
# Byte offsets are relative to each buffer's start: W [H, 128, 512] bf16,
# q_nope [B, H, 128], q_lat [B, H, 512], o_lat [B, H, 512], out [B, H, 128].
# Besides the bounds, the model checks that every fragment read finds the
# bytes the MFMA operand needs (the copies' swizzle undone).
# ---------------------------------------------------------------------------
PROJ_ROWS = 32


def proj_waves(H):
    return 4 if H >= 64 else 1


def check_absorb_q(B, H):
    """Every copy, LDS access and store of absorb_q_kernel<NW> for B x H."""
    NW = proj_waves(H)
    groups = 8 // NW
    lds_w, lds_q, lds_o = 16384, 8192, 4096
    smem = NW * lds_w + lds_q + NW * lds_o
    ln = np.arange(64)
    nl, g = ln & 15, ln >> 4
    qrow_bytes = H * 128 * 2
    counts = dict(workgroups=0, copies=0, stores=0)
    for item in range(H * groups):
        counts["workgroups"] += 1
        h = item // groups
        full = h == 0  # the fragment contents do not depend on the head: check them for one
        for w in range(NW):
            cb = (item % groups) * NW + w
            wl, ol = w * lds_w, NW * lds_w + lds_q + w * lds_o
            _need(cb < 8, "column block past the head")
            # W block copies: LDS slot (row, slot) <- W[h][row][64 cb + 8 chunk ..]
            lds_src = {}
            for k in range(16):
                src = (ln & 7) ^ (2 * (k & 3))
                row = 8 * k + (ln >> 3)
                off = (h * 128 * 512 + cb * 64) * 2 + 8 * k * 1024 + (ln >> 3) * 1024 + src * 16
                row_start = (h * 128 + row) * 1024
                _need((off >= row_start + cb * 128) & (off + 16 <= row_start + cb * 128 + 128),
                      "W_UK read outside the block's row segment")
                dst = wl + k * 1024 + ln * 16
                _need((dst >= wl) & (dst + 16 <= wl + lds_w), "W block copy outside the wave's LDS region")
                if full:
                    for i in range(64):
                        lds_src[int(dst[i]) - wl] = (int(row[i]), int(src[i]))
                counts["copies"] += 1
            # A fragments: transposing reads of 4 rows x 8 bytes
            for s in range(4 if full else 0):
                for ct in range(4):
                    colb = 32 * ct + (nl & 3) * 8
                    for e in range(2):
                        row = 32 * s + 8 * g + 4 * e + (nl >> 2)
                        chunk = (colb >> 4) ^ (2 * ((row >> 3) & 3))
                        addr = wl + row * 128 + (chunk << 4) + (colb & 15)
                        _need((addr >= wl) & (addr + 8 <= wl + lds_w), "W fragment read outside the region")
                        for i in range(64):
                            slot_start = int(addr[i]) - wl - (int(colb[i]) & 15)
                            r, c = lds_src[slot_start]
                            _need(r == int(row[i]) and c == int(colb[i]) >> 4, "W fragment is not its chunk")
            for b0 in range(0, B, PROJ_ROWS):
                q_src = {}
                for w2 in range(NW):
                    for i2 in range(8 // NW):
                        k = NW * i2 + w2
                        if b0 + 4 * k >= B:
                            continue
                        r0 = b0 + 4 * k
                        row = 4 * k + (ln >> 4)
                        br = np.minimum(b0 + row, B - 1)
                        src = (ln & 15) ^ (row & 15)
                        off = h * 256 + r0 * qrow_bytes + (br - r0) * qrow_bytes + src * 16
                        _need((off >= br * qrow_bytes + h * 256) & (off + 16 <= br * qrow_bytes + h * 256 + 256),
                              "q_nope read outside the head's row")
                        _need(br < B, "q_nope row past the batch")
                        dst = NW * lds_w + k * 1024 + ln * 16
                        _need((dst >= NW * lds_w) & (dst + 16 <= NW * lds_w + lds_q), "query copy outside its LDS")
                        if full:
                            for i in range(64):
                                q_src[int(dst[i]) - NW * lds_w] = (int(row[i]), int(src[i]))
                for mb in range(2):
                    brow = 16 * mb + nl
                    for s in range(4):
                        addr = NW * lds_w + brow * 256 + (((4 * s) + g) ^ (brow & 15)) * 16
                        _need((addr >= NW * lds_w) & (addr + 16 <= NW * lds_w + lds_q), "query read outside")
                        for i in range(64 if full else 0):
                            if b0 + int(brow[i]) < B:  # rows past the batch feed columns that are not stored
                                r, c = q_src[int(addr[i]) - NW * lds_w]
                                _need(r == int(brow[i]) and c == 4 * s + int(g[i]), "query fragment is not its chunk")
                    for ct in range(4):
                        c = 16 * ct + 4 * g
                        chunk = (c >> 3) ^ (brow & 7)
                        addr = ol + brow * 128 + (chunk << 4) + (c & 7) * 2
                        _need((addr >= ol) & (addr + 8 <= ol + lds_o), "output staging write outside")
                for k in range(4):
                    idx = 64 * k + ln
                    row, chunk = idx >> 3, idx & 7
                    addr = ol + row * 128 + ((chunk ^ (row & 7)) << 4)
                    _need((addr >= ol) & (addr + 16 <= ol + lds_o), "output staging read outside")
                    b = b0 + row
                    st = ((b * H + h) * 512 + cb * 64 + chunk * 8) * 2
                    ok = b < B
                    _need(~ok | ((st >= ((b * H + h) * 512 + cb * 64) * 2) & (st + 16 <= ((b * H + h) * 512 + cb * 64 + 64) * 2)),
                          "q_lat store outside the block's row segment")
                    counts["stores"] += int(ok.sum())
        _need(smem <= 160 * 1024, "LDS budget")
    return counts


def check_expand_v(B, H):
    """Every copy, LDS access and store of expand_v_kernel<NW> for B x H."""
    NW = proj_waves(H)
    groups = 8 // NW
    lds_w, lds_o = 16384, 32768
    ln = np.arange(64)
    nl, g = ln & 15, ln >> 4
    orow_bytes = H * 512 * 2
    counts = dict(workgroups=0, copies=0, stores=0)
    for item in range(H * groups):
        counts["workgroups"] += 1
        h = item // groups
        full = h == 0  # the fragment contents do not depend on the head: check them for one
        for w in range(NW):
            jb = (item % groups) * NW + w
            wl = w * lds_w
            _need(jb < 8, "row block past the head")
            w_src = {}
            for k in range(16):
                off = ((h * 128 + 16 * jb) * 512) * 2 + k * 1024 + (ln ^ (k & 15)) * 16
                row_start = (h * 128 + 16 * jb + k) * 1024
                _need((off >= row_start) & (off + 16 <= row_start + 1024), "W_UV read outside its row")
                dst = wl + k * 1024 + ln * 16
                _need((dst >= wl) & (dst + 16 <= wl + lds_w), "W copy outside the wave's LDS region")
                for i in range(64 if full else 0):
                    w_src[int(dst[i]) - wl] = (k, int(ln[i]) ^ (k & 15))
                counts["copies"] += 1
            for b0 in range(0, B, PROJ_ROWS):
                o_src = {}
                for w2 in range(NW):
                    for i2 in range(PROJ_ROWS // NW):
                        k = NW * i2 + w2
                        if b0 + k >= B:
                            continue
                        off = h * 1024 + (b0 + k) * orow_bytes + (ln ^ (k & 15)) * 16
                        rs = (b0 + k) * orow_bytes + h * 1024
                        _need((off >= rs) & (off + 16 <= rs + 1024), "o_lat read outside its row")
                        dst = NW * lds_w + k * 1024 + ln * 16
                        _need((dst >= NW * lds_w) & (dst + 16 <= NW * lds_w + lds_o), "o_lat copy outside its LDS")
                        for i in range(64 if full else 0):
                            o_src[int(dst[i]) - NW * lds_w] = (k, int(ln[i]) ^ (k & 15))
                jrow = nl
                for s in range(16):
                    chunk = 4 * s + g
                    addr = wl + jrow * 1024 + ((chunk ^ (jrow & 15)) << 4)
                    _need((addr >= wl) & (addr + 16 <= wl + lds_w), "W fragment read outside")
                    for i in range(64 if full else 0):
                        r, c = w_src[int(addr[i]) - wl]
                        _need(r == int(jrow[i]) and c == int(chunk[i]), "W fragment is not its chunk")
                    for mb in range(2):
                        brow = 16 * mb + nl
                        addr = NW * lds_w + brow * 1024 + ((chunk ^ (brow & 15)) << 4)
                        _need((addr >= NW * lds_w) & (addr + 16 <= NW * lds_w + lds_o), "o_lat fragment read outside")
                        for i in range(64 if full else 0):
                            if b0 + int(brow[i]) < B:
                                r, c = o_src[int(addr[i]) - NW * lds_w]
                                _need(r == int(brow[i]) and c == int(chunk[i]), "o_lat fragment is not its chunk")
                for mb in range(2):
                    b = b0 + 16 * mb + nl
                    st = ((b * H + h) * 128 + 16 * jb + 4 * g) * 2
                    ok = b < B
                    rs = ((b * H + h) * 128 + 16 * jb) * 2
                    _need(~ok | ((st >= rs) & (st + 8 <= rs + 32)), "out store outside the block's row segment")
                    counts["stores"] += int(ok.sum())
    _need(NW * lds_w + lds_o <= 160 * 1024, "LDS budget")
    return counts
