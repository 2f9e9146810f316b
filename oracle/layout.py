"""Byte layout of the paged KV pool.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The NInfer guide stores the cache in fixed 64-token pages; TokenSpeed's
``mxfp8`` needs 128-token blocks.  The pages do not give a byte layout, so
this one is this project's design.  It is part of the bit-exact contract
between the GPU encoder and this oracle and is written here from the
formulas below, independently of the HIP sources.

Pool: ``num_pages`` pages, page-major.  A page holds ``H_kv`` head blocks.
A head block is four planes, each padded to 128 bytes:
``K codes | K scales | V codes | V scales``.  Every plane is cut into
token blocks of 16 consecutive slots (P / 16 of them), stored one after
the other.  Inside a token block (local token t = 0..15) the order is:

K codes (bits b = 16, 8 or 4; one row of D values per token)::

    vpc = 128 / b            values per 16-byte chunk
    kk = d // 32, g = (d % 32) // 8, e = d % 8
    i  = kk // (vpc / 8),  j = (kk % (vpc / 8)) * 8 + e
    byte = i * 1024 + (g * 16 + t) * 16 + j * b / 8
    (4-bit: value j sits in the low nibble when j is even)

V codes (t = 4 * g + e, d = 16 * jt + n)::

    8-bit:  byte = (jt // 4) * 1024 + (g * 16 + n) * 16 + (jt % 4) * 4 + e
    16-bit: byte = (jt // 2) * 1024 + (g * 16 + n) * 16 + (jt % 2) * 8 + 2 e
    4-bit:  byte = (jt // 8) * 1024 + (g * 16 + n) * 16 + (jt % 8) * 2 + e // 2,
            high nibble when e is odd: a byte holds column n of the token
            pair (4 g + 2 p, 4 g + 2 p + 1), so writing one token changes
            one nibble of each byte it touches and keeps the other

Scales (G groups per row)::

    f16 scales:            byte = (t * G + grp) * 2   (little endian)
    UE8M0 and K UE4M3:     byte = t * G + grp
    V UE4M3 (t = 4 g + e): byte = g * 4 G + grp * 4 + e

These orders are the lane orders in which the decode kernel consumes a
block, so each of its loads is one contiguous run of memory.
"""

import numpy as np

from . import formats as F

PLANE_ALIGN = 128
TOKEN_BLOCK = 16


def _pad(n):
    return (n + PLANE_ALIGN - 1) // PLANE_ALIGN * PLANE_ALIGN


def code_block_bytes(codec, D):
    return TOKEN_BLOCK * D * F.CODECS[codec][0] // 8


def scale_block_bytes(codec, D):
    return TOKEN_BLOCK * F.n_groups(codec, D) * F.SCALE_BYTES[F.CODECS[codec][2]]


class Geometry:
    """Plane offsets and sizes for one (format, head_dim, page_size, H_kv)."""

    def __init__(self, fmt, D, P, H_kv):
        self.fmt, self.D, self.P, self.H_kv = fmt, D, P, H_kv
        name, self.kc, self.vc, self.k_rot, self.v_rot = F.FORMATS[fmt]
        assert P % TOKEN_BLOCK == 0
        nb = P // TOKEN_BLOCK
        self.kcode_blk = code_block_bytes(self.kc, D)
        self.kscale_blk = scale_block_bytes(self.kc, D)
        self.vcode_blk = code_block_bytes(self.vc, D)
        self.vscale_blk = scale_block_bytes(self.vc, D)
        sizes = [_pad(nb * self.kcode_blk), _pad(nb * self.kscale_blk),
                 _pad(nb * self.vcode_blk), _pad(nb * self.vscale_blk)]
        self.off = np.cumsum([0] + sizes[:-1]).tolist()
        self.head_bytes = int(sum(sizes))
        self.page_bytes = self.head_bytes * H_kv


def page_bytes(fmt, D, P, H_kv):
    return Geometry(fmt, D, P, H_kv).page_bytes


# ------------------------------------------------------ in-block byte offsets

def k_code_pos(bits, t, d):
    """(byte offset in the token block, is-high-nibble) of K element (t, d)."""
    t = np.asarray(t)
    d = np.asarray(d)
    vpc = 128 // bits
    kspc = vpc // 8
    kk, g, e = d // 32, (d % 32) // 8, d % 8
    i = kk // kspc
    j = (kk % kspc) * 8 + e
    byte = i * 1024 + (g * 16 + t) * 16 + (j * bits) // 8
    return byte, (bits == 4) & (j % 2 == 1)


def v_code_pos(bits, t, d):
    """(byte offset in the token block, is-high-nibble) of V element (t, d)."""
    t = np.asarray(t)
    d = np.asarray(d)
    g, e = t // 4, t % 4
    jt, n = d // 16, d % 16
    if bits == 8:
        return (jt // 4) * 1024 + (g * 16 + n) * 16 + (jt % 4) * 4 + e, np.zeros_like(d, bool)
    if bits == 16:
        return (jt // 2) * 1024 + (g * 16 + n) * 16 + (jt % 2) * 8 + 2 * e, np.zeros_like(d, bool)
    if bits == 4:
        return (jt // 8) * 1024 + (g * 16 + n) * 16 + (jt % 8) * 2 + e // 2, e % 2 == 1
    raise ValueError(bits)


def scale_pos(codec, plane, D, t, grp):
    """Byte offset of scale (t, grp) inside the token block of a scale plane."""
    G = F.n_groups(codec, D)
    stype = F.CODECS[codec][2]
    t = np.asarray(t)
    grp = np.asarray(grp)
    if stype == "f16":
        return (t * G + grp) * 2
    if F.CODECS[codec][0] == 4 and plane == "V":  # 4-bit V: a group's 4 tokens together
        return (t // 4) * 4 * G + grp * 4 + (t % 4)
    return t * G + grp


# ------------------------------------------------------ pool writer / reader

def _slot_base(geo, slots, head):
    slots = np.asarray(slots, dtype=np.int64)
    page = slots // geo.P
    off = slots % geo.P
    blk = off // TOKEN_BLOCK
    t = off % TOKEN_BLOCK
    base = page * geo.page_bytes + head * geo.head_bytes
    return base, blk, t


def _write_codes(pool, geo, plane, base, blk, t, codes, bits):
    D = geo.D
    n = codes.shape[0]
    d = np.arange(D)[None, :]
    tt = t[:, None]
    if plane == "K":
        pos, hi = k_code_pos(bits, tt, d)
        start = base[:, None] + geo.off[0] + blk[:, None] * geo.kcode_blk
    else:
        pos, hi = v_code_pos(bits, tt, d)
        start = base[:, None] + geo.off[2] + blk[:, None] * geo.vcode_blk
    addr = start + pos
    if bits == 16:
        c = codes.astype(np.uint16)
        pool[addr] = (c & 0xFF).astype(np.uint8)
        pool[addr + 1] = (c >> 8).astype(np.uint8)
    elif bits == 8:
        pool[addr] = codes.astype(np.uint8)
    else:
        hi = np.broadcast_to(hi, (n, D))
        c = codes.astype(np.uint8) & 0xF
        # a byte holds two values of one K row, or one column of two V
        # tokens: clear this row's nibbles, then set them, so that the other
        # nibble keeps whatever it held (rows of one call use distinct slots)
        val = np.where(hi, c << 4, c).astype(np.uint8)
        own = np.where(hi, 0xF0, 0x0F).astype(np.uint8)
        np.bitwise_and.at(pool, addr.ravel(), ~own.ravel())
        np.bitwise_or.at(pool, addr.ravel(), val.ravel())


def _write_scales(pool, geo, plane, codec, base, blk, t, scales):
    if scales is None:
        return
    D = geo.D
    G = F.n_groups(codec, D)
    grp = np.arange(G)[None, :]
    pos = scale_pos(codec, plane, D, t[:, None], grp)
    if plane == "K":
        start = base[:, None] + geo.off[1] + blk[:, None] * geo.kscale_blk
    else:
        start = base[:, None] + geo.off[3] + blk[:, None] * geo.vscale_blk
    addr = start + pos
    if F.CODECS[codec][2] == "f16":
        s = np.asarray(scales, dtype=np.uint16).reshape(-1, G)
        pool[addr] = (s & 0xFF).astype(np.uint8)
        pool[addr + 1] = (s >> 8).astype(np.uint8)
    else:
        pool[addr] = np.asarray(scales, dtype=np.uint8).reshape(-1, G)


def write_rows(pool, geo, slots, head, kcodes, kscales, vcodes, vscales):
    """Store encoded rows of one kv head at the given slots (page*P + offset)."""
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0  # a negative slot means "do not store this token"
    if not np.any(keep):
        return
    sl = slots[keep]
    base, blk, t = _slot_base(geo, sl, head)
    kb = F.CODECS[geo.kc][0]
    vb = F.CODECS[geo.vc][0]
    _write_codes(pool, geo, "K", base, blk, t, np.asarray(kcodes)[keep], kb)
    _write_codes(pool, geo, "V", base, blk, t, np.asarray(vcodes)[keep], vb)
    _write_scales(pool, geo, "K", geo.kc, base, blk, t,
                  None if kscales is None else np.asarray(kscales)[keep])
    _write_scales(pool, geo, "V", geo.vc, base, blk, t,
                  None if vscales is None else np.asarray(vscales)[keep])


def _read_codes(pool, geo, plane, base, blk, t, bits):
    D = geo.D
    d = np.arange(D)[None, :]
    tt = t[:, None]
    if plane == "K":
        pos, hi = k_code_pos(bits, tt, d)
        start = base[:, None] + geo.off[0] + blk[:, None] * geo.kcode_blk
    else:
        pos, hi = v_code_pos(bits, tt, d)
        start = base[:, None] + geo.off[2] + blk[:, None] * geo.vcode_blk
    addr = start + pos
    if bits == 16:
        return pool[addr].astype(np.uint16) | (pool[addr + 1].astype(np.uint16) << 8)
    if bits == 8:
        return pool[addr]
    b = pool[addr]
    return np.where(hi, b >> 4, b & 0xF).astype(np.uint8)


def _read_scales(pool, geo, plane, codec, base, blk, t):
    G = F.n_groups(codec, geo.D)
    if G == 0:
        return None
    grp = np.arange(G)[None, :]
    pos = scale_pos(codec, plane, geo.D, t[:, None], grp)
    if plane == "K":
        start = base[:, None] + geo.off[1] + blk[:, None] * geo.kscale_blk
    else:
        start = base[:, None] + geo.off[3] + blk[:, None] * geo.vscale_blk
    addr = start + pos
    if F.CODECS[codec][2] == "f16":
        return pool[addr].astype(np.uint16) | (pool[addr + 1].astype(np.uint16) << 8)
    return pool[addr]


def read_rows(pool, geo, slots, head):
    """Codes and scales of one kv head at the given slots."""
    base, blk, t = _slot_base(geo, slots, head)
    kb = F.CODECS[geo.kc][0]
    vb = F.CODECS[geo.vc][0]
    return (_read_codes(pool, geo, "K", base, blk, t, kb),
            _read_scales(pool, geo, "K", geo.kc, base, blk, t),
            _read_codes(pool, geo, "V", base, blk, t, vb),
            _read_scales(pool, geo, "V", geo.vc, base, blk, t))


def written_byte_mask(geo, num_pages, slots):
    """Boolean mask over the pool of every byte that storing ``slots`` (for
    all kv heads) writes; bytes outside it keep whatever the pool held."""
    mask = np.zeros(num_pages * geo.page_bytes, dtype=bool)
    probe = np.zeros_like(mask, dtype=np.uint8)
    slots = np.asarray(slots, dtype=np.int64)
    slots = slots[slots >= 0]
    n = len(slots)
    if n == 0:
        return mask
    D = geo.D
    kc = np.ones((n, D), dtype=np.uint16 if F.CODECS[geo.kc][0] == 16 else np.uint8)
    vc = np.ones((n, D), dtype=np.uint16 if F.CODECS[geo.vc][0] == 16 else np.uint8)
    if F.CODECS[geo.kc][0] == 16:
        kc[:] = 0x0101
    if F.CODECS[geo.vc][0] == 16:
        vc[:] = 0x0101
    if F.CODECS[geo.kc][0] == 4:
        kc[:] = 1
    if F.CODECS[geo.vc][0] == 4:
        vc[:] = 1
    gk = F.n_groups(geo.kc, D)
    gv = F.n_groups(geo.vc, D)
    ks = None if gk == 0 else np.full((n, gk), 0x0101 if F.CODECS[geo.kc][2] == "f16" else 1,
                                      dtype=np.uint16 if F.CODECS[geo.kc][2] == "f16" else np.uint8)
    vs = None if gv == 0 else np.full((n, gv), 0x0101 if F.CODECS[geo.vc][2] == "f16" else 1,
                                      dtype=np.uint16 if F.CODECS[geo.vc][2] == "f16" else np.uint8)
    for h in range(geo.H_kv):
        write_rows(probe, geo, slots, h, kc, ks, vc, vs)
    return probe != 0
