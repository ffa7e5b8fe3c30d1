"""Packed slot-record layout, restated from the ABI header (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages leave the bit layout open (they say only "low-bit", "per-channel",
"asymmetric").  The layout is a documented convention of the C ABI (include/kvq.h,
"Packed cache layout"); this module re-implements it from that text with plain
loops over bit fields, independently of the kernels, so that the GPU's bytes can
be compared with the oracle's.

A slot record holds one 32-token group of one (sequence, kv head):
    Kc    D*kb/32 word columns x 32 tokens: word w of token t at byte
          (w*32 + t)*4; word w holds channels [w*32/kb, (w+1)*32/kb), channel c
          at bits kb*(c mod 32/kb)
    Vc    vb word rows x D channels: word j of channel c at byte (j*D + c)*4;
          token t goes to (word, first bit) given by v_token_position(t, vb)
    Kmeta fp32 scale[D], fp32 zero[D]
    Vmeta per channel group g < D/G_v: fp32 scale[32], fp32 zero[32]
padded with zero bytes to a multiple of 256.

All functions accept any number of leading (batch) dimensions.
"""
from __future__ import annotations

import numpy as np

SLOT = 32
HEADER_BYTES = 16


def record_layout(D: int, kb: int, vb: int, gv: int) -> dict:
    """Byte offsets of the four fields of a slot record and its padded size."""
    kc = SLOT * D * kb // 8
    vc = D * vb * 4
    kmeta = 2 * D * 4
    vmeta = (D // gv) * 2 * SLOT * 4
    raw = kc + vc + kmeta + vmeta
    return {
        "kc_offset": 0,
        "vc_offset": kc,
        "kmeta_offset": kc + vc,
        "vmeta_offset": kc + vc + kmeta,
        "record_bytes": (raw + 255) // 256 * 256,
    }


def record_layout_h16(D: int, kb: int, vb: int, gv: int) -> dict:
    """Integer-code records with fp16 metadata: Kmeta = fp16 scale[D], zero[D];
    Vmeta = per channel group fp16 scale[32 tokens], zero[32 tokens]."""
    kc = SLOT * D * kb // 8
    vc = D * vb * 4
    km = 2 * D * 2
    vm = (D // gv) * 2 * SLOT * 2
    return dict(kc_offset=0, vc_offset=kc, kmeta_offset=kc + vc, vmeta_offset=kc + vc + km,
                record_bytes=(kc + vc + km + vm + 255) // 256 * 256)


def v_token_position(t: int, vb: int):
    """(word, first bit) of token t inside a V channel row of vb u32 words."""
    mm = t // 16
    h = (t // 4) % 2
    e = (t % 4) + 4 * ((t // 8) % 2)
    if vb == 4:
        return 2 * mm + h, 4 * e
    if vb == 2:
        return h, 2 * (8 * mm + e)
    raise ValueError("v bits must be 2 or 4")


def pack_k_words(kcodes: np.ndarray, kb: int) -> np.ndarray:
    """[..., 32, D] codes -> [..., 32, D*kb/32] u32 words."""
    D = kcodes.shape[-1]
    per = 32 // kb
    words = np.zeros(kcodes.shape[:-1] + (D // per,), dtype=np.uint64)
    for c in range(D):
        w, pos = divmod(c, per)
        words[..., w] |= kcodes[..., c].astype(np.uint64) << np.uint64(kb * pos)
    return words.astype(np.uint32)


def pack_v_words(vcodes: np.ndarray, vb: int) -> np.ndarray:
    """[..., D, 32] codes -> [..., D, vb] u32 words."""
    words = np.zeros(vcodes.shape[:-1] + (vb,), dtype=np.uint64)
    for t in range(SLOT):
        w, bit = v_token_position(t, vb)
        words[..., w] |= vcodes[..., t].astype(np.uint64) << np.uint64(bit)
    return words.astype(np.uint32)


def pack_record(kcodes, vcodes, kscale, kzero, vscale, vzero, kb: int, vb: int, gv: int) -> np.ndarray:
    """Bytes of slot records as uint8 [..., record_bytes].

    kcodes [..., 32 tokens, D], vcodes [..., D channels, 32 tokens] (ints < 2^b);
    kscale/kzero [..., D]; vscale/vzero [..., D/gv groups, 32 tokens]."""
    kcodes = np.asarray(kcodes)
    vcodes = np.asarray(vcodes)
    D = kcodes.shape[-1]
    lead = kcodes.shape[:-2]
    lay = record_layout(D, kb, vb, gv)
    assert kcodes.shape[-2] == SLOT and vcodes.shape[-2:] == (D, SLOT)
    assert int(kcodes.max(initial=0)) < 2 ** kb and int(vcodes.max(initial=0)) < 2 ** vb
    n = int(np.prod(lead, dtype=np.int64))
    out = np.zeros((n, lay["record_bytes"]), dtype=np.uint8)

    def put(off, arr):
        b = np.ascontiguousarray(arr).reshape(n, -1).view(np.uint8)
        out[:, off:off + b.shape[1]] = b

    put(lay["kc_offset"], np.swapaxes(pack_k_words(kcodes, kb), -1, -2).astype("<u4"))   # [.., word, token]
    put(lay["vc_offset"], np.swapaxes(pack_v_words(vcodes, vb), -1, -2).astype("<u4"))   # [.., word, channel]
    put(lay["kmeta_offset"], np.concatenate([np.asarray(kscale, "<f4"), np.asarray(kzero, "<f4")], axis=-1))
    vm = np.stack([np.asarray(vscale, "<f4"), np.asarray(vzero, "<f4")], axis=-2)   # [..., G, 2, 32]
    put(lay["vmeta_offset"], vm)
    return out.reshape(lead + (lay["record_bytes"],))


def unpack_record(rec: np.ndarray, D: int, kb: int, vb: int, gv: int) -> dict:
    """Inverse of pack_record: codes, scales and zeros of records uint8 [..., R]."""
    lay = record_layout(D, kb, vb, gv)
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    lead = rec.shape[:-1]
    n = int(np.prod(lead, dtype=np.int64))
    rec = rec.reshape(n, -1)

    def get(off, count, dt):
        return rec[:, off:off + count * 4].copy().view(dt)

    per = 32 // kb
    kw = np.swapaxes(get(lay["kc_offset"], SLOT * D // per, "<u4").reshape(n, D // per, SLOT), 1, 2)
    kcodes = np.zeros((n, SLOT, D), dtype=np.uint16)
    for c in range(D):
        w, pos = divmod(c, per)
        kcodes[:, :, c] = (kw[:, :, w] >> np.uint32(kb * pos)) & np.uint32(2 ** kb - 1)
    vw = np.swapaxes(get(lay["vc_offset"], D * vb, "<u4").reshape(n, vb, D), 1, 2)
    vcodes = np.zeros((n, D, SLOT), dtype=np.uint16)
    for t in range(SLOT):
        w, bit = v_token_position(t, vb)
        vcodes[:, :, t] = (vw[:, :, w] >> np.uint32(bit)) & np.uint32(2 ** vb - 1)
    km = get(lay["kmeta_offset"], 2 * D, "<f4")
    vm = get(lay["vmeta_offset"], (D // gv) * 2 * SLOT, "<f4").reshape(n, D // gv, 2, SLOT)
    G = D // gv
    return {
        "kcodes": kcodes.reshape(lead + (SLOT, D)),
        "vcodes": vcodes.reshape(lead + (D, SLOT)),
        "kscale": km[:, :D].reshape(lead + (D,)),
        "kzero": km[:, D:].reshape(lead + (D,)),
        "vscale": vm[:, :, 0, :].reshape(lead + (G, SLOT)),
        "vzero": vm[:, :, 1, :].reshape(lead + (G, SLOT)),
    }


def pack_header(nvalid: int, mask: int, prot_base: int, token_base: int) -> np.ndarray:
    """The 16-byte slot header as uint8[16]."""
    return np.array([nvalid, mask, prot_base, token_base], dtype=np.int64).astype("<u4").view(np.uint8)
