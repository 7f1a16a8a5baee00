"""Independent reader of the packed layout, written from its documentation (the block
comment at the top of weight_only_quant_amd/csrc/qmat_layout.h), in numpy.  Used by the
tests to check qmat_pack by round trip; it shares no code with the packer."""
import numpy as np

NB = {4: 4, 5: 5, 6: 6, 8: 8, 9: 8}  # format id -> 1 KB blocks per unit (9 = Q8)


def dims(fmt, M, K):
    NT = -(-M // 64)
    NU = -(-K // 128)
    code_bytes = NT * NU * NB[fmt] * 1024
    scale_bytes = NT * 256 if fmt == 8 else NT * NU * 256
    return NT, NU, code_bytes, scale_bytes


def _sbyte(v, i):
    return ((v >> np.uint32(8 * i)) & np.uint32(0xFF)).astype(np.uint8).view(np.int8).astype(np.int32)


def _shift(v, s):
    return (v << np.uint32(s)) if s >= 0 else (v >> np.uint32(-s))


def unpack(fmt, M, K, blob):
    """Returns (codes [M,K] int8 or uint8, scales [M,K/64] uint16 or [M] float32)."""
    NT, NU, cb, sbytes = dims(fmt, M, K)
    blob = np.asarray(blob, dtype=np.uint8)
    assert blob.size == cb + sbytes
    nb = NB[fmt]
    seg = blob[:cb].view(np.uint32).reshape(NT, NU, nb, 64, 4)
    W = seg.transpose(0, 1, 3, 2, 4).reshape(NT, NU, 64, 4 * nb)  # W[t,u,L,4j+d]
    Mp, Kp = NT * 64, NU * 128
    out = np.zeros((Mp, Kp), dtype=np.int32)
    L = np.arange(64)
    r16, q = L % 16, L // 16
    t_idx = np.arange(NT)[:, None, None]
    u_idx = np.arange(NU)[None, :, None]
    for ka in range(4):
        for m in range(4):
            rows = (64 * t_idx + 16 * m + r16[None, None, :])  # [NT,1,64]
            for e in range(8):
                if fmt == 4:
                    # byte e % 4, low nibble for e < 4 and high nibble above, two's complement
                    n = W[..., 4 * ka + m]
                    v = ((n >> np.uint32(8 * (e % 4) + 4 * (e // 4))) & np.uint32(0xF)).astype(np.int32)
                    v = np.where(v >= 8, v - 16, v)
                elif fmt == 5:
                    o = 2 * m + e // 4
                    i = e % 4
                    if o < 4:
                        O = W[..., 5 * ka + o] & np.uint32(0xF8F8F8F8)
                    else:
                        d = o - 4
                        O = ((W[..., 5 * ka + d] << np.uint32(5)) & np.uint32(0xE0E0E0E0)) | \
                            (_shift(W[..., 5 * ka + 4], 3 - 2 * d) & np.uint32(0x18181818))
                    v = _sbyte(O, i) >> 3
                elif fmt == 6:
                    p = m // 2
                    A, B, C = (W[..., 6 * ka + 3 * p + z] for z in range(3))
                    i = e % 4
                    if m % 2 == 0:
                        O = (A if e < 4 else B) & np.uint32(0xFCFCFCFC)
                    else:
                        O = (C & np.uint32(0xFCFCFCFC)) if e < 4 else (
                            ((A << np.uint32(6)) & np.uint32(0xC0C0C0C0)) | ((B << np.uint32(4)) & np.uint32(0x30303030)) |
                            ((C << np.uint32(2)) & np.uint32(0x0C0C0C0C)))
                    v = _sbyte(O, i) >> 2
                else:  # FP8 bytes, or Q8 two's complement bytes
                    w = W[..., 8 * ka + 2 * m + e // 4]
                    v = ((w >> np.uint32(8 * (e % 4))) & np.uint32(0xFF)).astype(np.int32)
                    if fmt == 9:
                        v = np.where(v >= 128, v - 256, v)
                cols = (128 * u_idx + 32 * ka + 8 * q[None, None, :] + e)  # [1,NU,64]
                out[np.broadcast_to(rows, v.shape), np.broadcast_to(cols, v.shape)] = v
    if fmt == 8:
        codes = out[:M, :K].astype(np.uint8)
        rs = blob[cb:].view(np.float32).reshape(NT, 16, 4)  # [t, r16, m]
        sc = np.zeros(Mp, np.float32)
        for m in range(4):
            sc[(64 * np.arange(NT)[:, None] + 16 * m + np.arange(16)[None, :]).ravel()] = rs[:, :, m].ravel()
        return codes, sc[:M], out, sc
    codes = out[:M, :K].astype(np.int8)
    s = blob[cb:].view(np.uint16).reshape(NT, NU, 16, 2, 4)  # [t,u,r16,g,m]
    sc = np.zeros((Mp, 2 * NU), np.uint16)
    for m in range(4):
        for g in range(2):
            rr = (64 * np.arange(NT)[:, None, None] + 16 * m + np.arange(16)[None, None, :])
            gg = (2 * np.arange(NU)[None, :, None] + g)
            sc[np.broadcast_to(rr, (NT, NU, 16)), np.broadcast_to(gg, (NT, NU, 16))] = s[:, :, :, g, m]
    return codes, sc[:M, :K // 64], out, sc
