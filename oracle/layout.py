"""Packing of quantized codes into the cache planes -- oracle side.

TEST INFRASTRUCTURE ONLY (see oracle/wushkv_ref.py).  Written from the
layout's text definition; the device kernels implement the same text in their
own code.  The pages fix no storage format: the body holds per-token low-bit
codes plus per-token parameters (digest, method key points; review blog, Key
Terms: per-token QuEST), and the layout below is this implementation's choice.

K code plane -- token-major rows of d*b/8 bytes (body index u = p - sink):
  plane 0: d/16 little-endian u32 words; word w, bits 2f..2f+1 hold the low
           two bits of channel 16w + f.
  plane 1: b = 3: d/32 u32 words; word w, bit 4*((f >> 1) & 7) + (f & 1) + 2*(f >> 4)
           holds bit 2 of channel 32w + f (f in 0..31): nibble k of the word holds
           channels 2k, 2k+1, 16+2k, 17+2k at its bits 0..3.
           b = 4: d/16 u32 words; word w, bits 2f..2f+1 hold bits 2..3 of
           channel 16w + f.

V code plane -- sets of 64 body tokens, 8*d*b bytes per set.  Token
u = 64*sigma + 16*a + 4*c + e (a, c, e in 0..3) and channel j = 16*t + m
(t in 0..d/16-1, m in 0..15) are stored at lane = 16*c + m, field f = 4*a + e.
Even fields fill the low half of a word and odd fields the high half:
  plane 0: u32 words indexed lane*(d/16) + t; the low two bits of the code sit
           at bit 2*(f >> 1) + 16*(f & 1).
  plane 1: b = 3: u16 halfwords indexed lane*(d/16) + t, after plane 0;
           bit 2 of the code sits at bit (f >> 1) + 8*(f & 1).
           b = 4: u32 words indexed as plane 0, after plane 0; bits 2..3 of
           the code sit at bit 2*(f >> 1) + 16*(f & 1).
A set that is only partly filled holds zero codes in its unused fields.
"""
import numpy as np

SET = 64


def k_row_bytes(d, bits):
    return d * bits // 8


def v_set_bytes(d, bits):
    return SET * d * bits // 8


def _words(b):
    return np.frombuffer(np.ascontiguousarray(b, dtype=np.uint8).tobytes(), dtype="<u4")


def _k3_bit(f):
    """Bit of a 3-bit key row's plane-1 word holding channel f (0..31) of its 32."""
    return 4 * ((f >> 1) & 7) + (f & 1) + 2 * (f >> 4)


def pack_k(codes, bits):
    """codes [T, d] ints in [0, 2**bits) -> uint8 [T, d*bits/8]."""
    codes = np.asarray(codes, dtype=np.int64)
    T, d = codes.shape
    lo = codes & 3
    w0 = np.zeros((T, d // 16), dtype=np.uint64)
    for f in range(16):
        w0 |= (lo[:, f::16].astype(np.uint64) << np.uint64(2 * f))
    parts = [w0]
    if bits == 3:
        hi = (codes >> 2) & 1
        w1 = np.zeros((T, d // 32), dtype=np.uint64)
        for f in range(32):
            w1 |= (hi[:, f::32].astype(np.uint64) << np.uint64(_k3_bit(f)))
        parts.append(w1)
    elif bits == 4:
        hi = (codes >> 2) & 3
        w1 = np.zeros((T, d // 16), dtype=np.uint64)
        for f in range(16):
            w1 |= (hi[:, f::16].astype(np.uint64) << np.uint64(2 * f))
        parts.append(w1)
    words = np.concatenate(parts, axis=1).astype("<u4")
    return words.view(np.uint8).reshape(T, -1)


def unpack_k(raw, bits, d, T):
    """uint8 rows [T, d*bits/8] (any buffer of at least that size) -> codes [T, d]."""
    if T == 0:
        return np.zeros((0, d), dtype=np.int64)
    raw = np.ascontiguousarray(np.asarray(raw, dtype=np.uint8).reshape(-1)[: T * k_row_bytes(d, bits)])
    words = _words(raw).reshape(T, -1).astype(np.int64)
    nw0 = d // 16
    codes = np.zeros((T, d), dtype=np.int64)
    for f in range(16):
        codes[:, f::16] = (words[:, :nw0] >> (2 * f)) & 3
    if bits == 3:
        w1 = words[:, nw0:nw0 + d // 32]
        for f in range(32):
            codes[:, f::32] |= ((w1 >> _k3_bit(f)) & 1) << 2
    elif bits == 4:
        w1 = words[:, nw0:2 * nw0]
        for f in range(16):
            codes[:, f::16] |= ((w1 >> (2 * f)) & 3) << 2
    return codes


def _v_index(d):
    """For each (token-in-set, channel): (lane, t, bit of a 2-bit field in a u32,
    bit of a 1-bit field in a u16)."""
    u = np.arange(SET)[:, None]
    j = np.arange(d)[None, :]
    a, c, e = u // 16, (u // 4) % 4, u % 4
    t, m = j // 16, j % 16
    lane = 16 * c + m
    f = 4 * a + e
    b2 = 2 * (f >> 1) + 16 * (f & 1)
    b1 = (f >> 1) + 8 * (f & 1)
    shp = (SET, d)
    return (np.broadcast_to(lane, shp), np.broadcast_to(t, shp), np.broadcast_to(b2, shp),
            np.broadcast_to(b1, shp))


def pack_v(codes, bits):
    """codes [T, d] -> uint8 [ceil(T/64), 8*d*bits] (zero-filled tail)."""
    codes = np.asarray(codes, dtype=np.int64)
    T, d = codes.shape
    nset = -(-T // SET)
    full = np.zeros((nset * SET, d), dtype=np.int64)
    full[:T] = codes
    lane, t, b2, b1 = _v_index(d)
    nt = d // 16
    out = []
    for s in range(nset):
        blk = full[s * SET:(s + 1) * SET]
        w0 = np.zeros(64 * nt, dtype=np.uint64)
        np.bitwise_or.at(w0, (lane * nt + t).ravel(), ((blk & 3).astype(np.uint64) << b2.astype(np.uint64)).ravel())
        parts = [w0.astype("<u4").view(np.uint8)]
        if bits == 3:
            w1 = np.zeros(64 * nt, dtype=np.uint64)
            np.bitwise_or.at(w1, (lane * nt + t).ravel(), (((blk >> 2) & 1).astype(np.uint64) << b1.astype(np.uint64)).ravel())
            parts.append(w1.astype("<u2").view(np.uint8))
        elif bits == 4:
            w1 = np.zeros(64 * nt, dtype=np.uint64)
            np.bitwise_or.at(w1, (lane * nt + t).ravel(), (((blk >> 2) & 3).astype(np.uint64) << b2.astype(np.uint64)).ravel())
            parts.append(w1.astype("<u4").view(np.uint8))
        out.append(np.concatenate(parts))
    if not out:
        return np.zeros((0, v_set_bytes(d, bits)), dtype=np.uint8)
    return np.stack(out)


def unpack_v(raw, bits, d, T):
    """uint8 sets (any buffer holding ceil(T/64) sets) -> codes [T, d]."""
    if T == 0:
        return np.zeros((0, d), dtype=np.int64)
    nset = -(-T // SET)
    sb = v_set_bytes(d, bits)
    raw = np.ascontiguousarray(np.asarray(raw, dtype=np.uint8).reshape(-1)[: nset * sb]).reshape(nset, sb)
    lane, t, b2, b1 = _v_index(d)
    nt = d // 16
    idx = lane * nt + t
    codes = np.zeros((nset * SET, d), dtype=np.int64)
    for s in range(nset):
        w0 = _words(raw[s, :64 * nt * 4]).astype(np.int64)
        c = (w0[idx] >> b2) & 3
        if bits == 3:
            w1 = np.frombuffer(raw[s, 64 * nt * 4:].tobytes(), dtype="<u2").astype(np.int64)
            c |= ((w1[idx] >> b1) & 1) << 2
        elif bits == 4:
            w1 = _words(raw[s, 64 * nt * 4:]).astype(np.int64)
            c |= ((w1[idx] >> b2) & 3) << 2
        codes[s * SET:(s + 1) * SET] = c
    return codes[:T]
