"""Host-side model of every memory access the two decode kernels make.

For a launch description (the kernel arguments) this module enumerates, per
workgroup, wave and lane, the address arithmetic of the kernels as written in
csrc/decode_latent_wide.hip (128 heads) and csrc/decode_latent.hip (16, 32 and
64 heads):

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
    cache allocation holds; items: planned (seq, first_tile, count) rows or
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

def wide_lds_layout(fp8):
    NW, H = 4, 128
    NLAT, NPE, NRAW = (3, 2, 2) if fp8 else (4, 3, 0)
    kLatBytes, kPeBytes = TILE * 1024, TILE * 128
    kRawWave = 8 * 512 + 8 * 64 + 256
    kPeRing = 0
    kLatRing = kPeRing + NPE * kPeBytes
    kRawRing = kLatRing + NLAT * kLatBytes
    kPOff = kRawRing + NRAW * NW * kRawWave
    kPBuf = NW * 2048
    kAlphaOff = kPOff + 2 * kPBuf
    kFlagOff = kAlphaOff + 2 * H * 4
    kScaleOff = kFlagOff + 64
    kSmem = kScaleOff + (2 * TILE * 4 if fp8 else 0)
    kQStage = kLatRing if fp8 else kLatRing + 2 * kLatBytes
    return dict(NLAT=NLAT, NPE=NPE, kLatBytes=kLatBytes, kPeBytes=kPeBytes, kRawWave=kRawWave, kLatRing=kLatRing,
                kPeRing=kPeRing, kRawRing=kRawRing, kSmem=kSmem, kQStage=kQStage, kQWave=16 * 1024 + 2048,
                kScaleOff=kScaleOff)


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
            s, f, n = L.items[item]
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
        part = item if planned else b * L.P + split
        out.append(dict(item=item, b=b, cb=cb, row0=row0, nq=nq, t_begin=t_begin, t_end=t_end, part=part,
                        final=final, rot=(split * 2) & 15, T=T))
    return out


def check_wide(L, max_items=None):
    """Enumerate and check every access of the 128-row kernel; returns counts.
    L.H is the number of heads per query (Hq); with fewer than 128 (grouped
    prefill) a workgroup's 128 rows are q_group queries of Hq heads."""
    lay = wide_lds_layout(L.fp8)
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
            if not L.fp8:
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
            else:
                rs = np.minimum((8 * w + (lanes & 7))[None, :], last[:, None])
                raw = lay["kRawRing"] + ((tiles & 1) * 4 + w) * lay["kRawWave"]
                for k in range(7):
                    if k < 4:
                        byte = ((lanes & 7) << 4) + 128 * k
                        _need(byte + 16 <= 512, "E4M3 latent copy outside the row")
                        dst = raw[:, None] + 1024 * k + 16 * lanes[None, :]
                        hi = raw[:, None] + 4096
                    elif k < 6:
                        byte = 4 * (lanes & 7) + 32 * (k - 4)
                        _need(byte + 4 <= 64, "E4M3 RoPE copy outside the row")
                        dst = raw[:, None] + 4096 + 256 * (k - 4) + 4 * lanes[None, :]
                        hi = raw[:, None] + 4096 + 512
                    else:
                        stok = t0[:, None] + rs
                        _need((stok >= tb) & (stok < te), "token scale outside the range")
                        dst = raw[:, None] + 4608 + 4 * lanes[None, :]
                        hi = raw[:, None] + lay["kRawWave"]
                    _need((dst >= raw[:, None]) & (dst + (16 if k < 4 else 4) <= hi), "E4M3 copy outside its region")
                    _need(hi <= lay["kSmem"], "raw ring outside LDS")
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
# 16/32/64-head kernel (decode_latent_kernel<NW, NBUF, PAGED, FP8>)
# ---------------------------------------------------------------------------

def narrow_config(H, fp8):
    NW = H // 16
    NBUF = 4 if fp8 else {1: 1, 2: 1, 4: 2}[NW]
    return NW, NBUF


def check_narrow(L, max_items=None):
    H = L.H
    NW, NBUF = narrow_config(H, L.fp8)
    KV_PW = TILE // NW
    PE_W = NW if NW < 4 else 4
    PE_PW = 4 // PE_W
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
            s, f, n = L.items[item]
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
        part = item if planned else b * L.P + split
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
            for w in range(NW):
                if not L.fp8:
                    for k in range(KV_PW):
                        r = w * KV_PW + k
                        tok = t0 + min(r, last)
                        byte = (16 * lanes) ^ (kv_swizzle(r) << 4)
                        _need((tok >= tb) & (tok < te) & (byte + 16 <= 1024), "latent copy out of bounds")
                        if L.num_slots is not None:
                            sl = L.slot(cb, tok)
                            _need((sl >= 0) & (sl < L.num_slots), "cache slot outside the allocation")
                        dst = dst0 + r * 1024 + 16 * lanes
                        _need(dst + 16 <= dst0 + kTileBytes, "latent copy outside its tile")
                        counts["copies"] += 64
                    if w < PE_W:
                        for k in range(PE_PW):
                            i = w * PE_PW + k
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
