"""Commit-time quantized KV cache, modelled on the host (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Method (pages): keys and values of a block are quantized once, when the block
is committed, and the block still being denoised stays in full precision
(SoloQ summary page, block-diffusion paragraph).  Keys: KIVI-style per-channel
asymmetric groups along the token axis; values: per-token groups along the
channel axis ("standard low-bit value quantization"); a chosen per-layer set of
key rows stays in high precision (Tai et al., abstract, KProtect).  The cache
reused by the block has a prefix segment and, for the dual cache, a suffix
segment (Tai et al., abstract: prefix and dual cache reuse).

Readings where the pages are silent (each listed in the design notes):
  * group = 32 consecutive tokens starting at the commit's first token; the
    last group of a commit may be partial and is never reopened;
  * protected key tokens cover all kv heads of the layer, are stored in bf16,
    take no part in their group's key statistics and get code 0; their values
    are quantized like any other token;
  * V groups are G_v consecutive channels of one token;
  * a suffix segment is replaced wholesale when it is reset;
  * with a value rotation set (oracle/rotation.py), every committed value row
    is rotated before it is quantized, and the cache holds rotated values;
  * fp16 metadata (an engineering variant of the same quantizer): the fp32
    scale and zero are rounded to fp16 and the codes are taken against the
    rounded pair (oracle/quant.py, asym_quantize_h16);
  * attention-sink protection (SoloQ summary page, paragraph on keeping the
    attention sink in full precision: barely matters at 4-bit KV, matters at
    2-bit), when enabled, protects the first token of every sequence's prefix,
    in addition to the caller's list; the sink is read as that first token.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from .layout import SLOT, pack_record, pack_header, record_layout, record_layout_h16
from .quant import asym_quantize, asym_quantize_h16, dequantize, to_bf16_f32
from .rotation import rotate_f32
from .mxfp4 import mx_quantize, mx_dequantize, record_layout_mx


@dataclasses.dataclass
class _SeqSeg:
    ntok: int = 0
    nslots: int = 0
    chunks: list = dataclasses.field(default_factory=list)   # per commit: dict of arrays
    headers: list = dataclasses.field(default_factory=list)  # per slot: (nvalid, mask, base, tok)
    prot_pos: list = dataclasses.field(default_factory=list)
    prot_rows: list = dataclasses.field(default_factory=list)  # [Hkv, D] fp32 (bf16 values)


class OracleCache:
    """Host model of one layer's cache: B sequences, Hkv kv heads, head dim D."""

    def __init__(self, B: int, Hkv: int, D: int, k_bits: int, v_bits: int, v_group: int, v_rot=None,
                 protect_sink: bool = False, fmt: str = "int"):
        """v_rot: None, or (perm, mix, block) of the K-RPBH value rotation.
        protect_sink: a prefix commit that starts a sequence also protects its
        first token (attention-sink protection).
        fmt: "int" (asymmetric integer codes), "int_h16" (the same with fp16
        scales and zeros) or "mxfp4" (oracle/mxfp4.py; 4-bit, value groups of
        32 channels)."""
        self.protect_sink = protect_sink
        self.fmt = fmt
        assert fmt in ("int", "int_h16", "mxfp4")
        assert fmt != "mxfp4" or (k_bits == 4 and v_bits == 4 and v_group == 32)
        assert D % v_group == 0
        self.v_rot = v_rot
        self.B, self.Hkv, self.D = B, Hkv, D
        self.kb, self.vb, self.gv = k_bits, v_bits, v_group
        if fmt == "mxfp4":
            self.layout = record_layout_mx(D)
        elif fmt == "int_h16":
            self.layout = record_layout_h16(D, k_bits, v_bits, v_group)
        else:
            self.layout = record_layout(D, k_bits, v_bits, v_group) if k_bits <= 4 and v_bits <= 4 else None
        self.seg = {0: [_SeqSeg() for _ in range(B)], 1: [_SeqSeg() for _ in range(B)]}

    # ------------------------------------------------------------------ commit
    def commit(self, segment: int, k: np.ndarray, v: np.ndarray, ntok=None, prot=None,
               reset: bool = False):
        """Quantize and append the first ntok[b] tokens of k, v [B, n_max, Hkv, D].

        prot[b]: sorted positions (relative to this commit) of protected tokens."""
        k = np.asarray(k, dtype=np.float32)
        v = np.asarray(v, dtype=np.float32)
        if self.v_rot is not None:
            v = rotate_f32(v, *self.v_rot)
        B, n_max, Hkv, D = k.shape
        assert (B, Hkv, D) == (self.B, self.Hkv, self.D) and v.shape == k.shape
        if reset:
            self.seg[segment] = [_SeqSeg() for _ in range(self.B)]
        for b in range(B):
            n = n_max if ntok is None else int(ntok[b])
            p = np.zeros(0, np.int64) if prot is None else np.asarray(prot[b], np.int64)
            st = self.seg[segment][b]
            if self.protect_sink and segment == 0 and st.ntok == 0 and n > 0 and (len(p) == 0 or p[0] != 0):
                p = np.concatenate([[0], p]).astype(np.int64)
            self._commit_seq(st, k[b, :n], v[b, :n], p)

    def _commit_seq(self, st: _SeqSeg, kb_: np.ndarray, vb_: np.ndarray, prot: np.ndarray):
        n = kb_.shape[0]
        if n == 0:
            return
        assert np.all(np.diff(prot) > 0) and (len(prot) == 0 or (prot[0] >= 0 and prot[-1] < n))
        ns = -(-n // SLOT)
        Hkv, D, G = self.Hkv, self.D, self.D // self.gv
        kpad = np.zeros((ns * SLOT, Hkv, D), np.float32)
        vpad = np.zeros((ns * SLOT, Hkv, D), np.float32)
        kpad[:n], vpad[:n] = kb_, vb_
        valid = (np.arange(ns * SLOT) < n).reshape(ns, SLOT)
        isprot = np.zeros(ns * SLOT, bool)
        isprot[prot] = True
        isprot = isprot.reshape(ns, SLOT)

        # K: per (slot, head, channel), group = the slot's tokens
        k4 = kpad.reshape(ns, SLOT, Hkv, D).transpose(0, 2, 3, 1)          # [ns, Hkv, D, 32]
        kmem = np.broadcast_to((valid & ~isprot)[:, None, None, :], k4.shape)
        if self.fmt == "mxfp4":
            kc, ks = mx_quantize(np.ascontiguousarray(k4), kmem)            # ks: scale bytes [ns, Hkv, D]
            kz = None
        elif self.fmt == "int_h16":
            kc, ks, kz = asym_quantize_h16(np.ascontiguousarray(k4), self.kb, kmem)
        else:
            kc, ks, kz = asym_quantize(np.ascontiguousarray(k4), self.kb, kmem)
        kcodes = kc.transpose(0, 1, 3, 2)                                   # [ns, Hkv, 32, D]
        # V: per (slot, head, token, channel group), group = G_v channels
        v5 = vpad.reshape(ns, SLOT, Hkv, G, self.gv).transpose(0, 2, 1, 3, 4)  # [ns, Hkv, 32, G, gv]
        vmem = np.broadcast_to(valid[:, None, :, None, None], v5.shape)
        if self.fmt == "mxfp4":
            vc, vs = mx_quantize(np.ascontiguousarray(v5), vmem)            # vs: [ns, Hkv, 32, G]
            vz = None
        elif self.fmt == "int_h16":
            vc, vs, vz = asym_quantize_h16(np.ascontiguousarray(v5), self.vb, vmem)
        else:
            vc, vs, vz = asym_quantize(np.ascontiguousarray(v5), self.vb, vmem)
        vcodes = vc.reshape(ns, Hkv, SLOT, D).transpose(0, 1, 3, 2)          # [ns, Hkv, D, 32]
        vscale = vs.transpose(0, 1, 3, 2)                                    # [ns, Hkv, G, 32]
        vzero = None if vz is None else vz.transpose(0, 1, 3, 2)

        # the packed record exists for the ABI's bit widths; wider codes (used
        # only to study the high-precision limit) are kept unpacked
        records = None
        if self.fmt == "mxfp4":
            records = self._pack_mx(kcodes, vcodes, ks, vscale)
        elif self.fmt == "int_h16":
            records = self._pack_h16(kcodes, vcodes, ks, kz, vscale, vzero)
        elif self.kb in (2, 4) and self.vb in (2, 4):
            records = pack_record(kcodes, vcodes, ks, kz, vscale, vzero, self.kb, self.vb, self.gv)
        headers = []
        base = len(st.prot_pos)
        for j in range(ns):
            mask = 0
            for t in range(SLOT):
                if isprot[j, t]:
                    mask |= 1 << t
            headers.append((int(valid[j].sum()), mask, base, st.ntok + SLOT * j))
            base += int(isprot[j].sum())
        for p in prot:
            st.prot_pos.append(st.ntok + int(p))
            st.prot_rows.append(to_bf16_f32(kb_[p]))                         # [Hkv, D]
        st.chunks.append(dict(kcodes=kcodes, vcodes=vcodes, kscale=ks, kzero=kz,
                              vscale=vscale, vzero=vzero, records=records))
        st.headers.extend(headers)
        st.ntok += n
        st.nslots += ns

    def _pack_mx(self, kcodes, vcodes, kscale, vscale):
        """MX FP4 records: the 4-bit code layout, then the scale bytes."""
        from .layout import pack_k_words, pack_v_words
        lay = self.layout
        lead = kcodes.shape[:-2]
        n = int(np.prod(lead, dtype=np.int64))
        out = np.zeros((n, lay["record_bytes"]), np.uint8)

        def put(off, arr):
            b = np.ascontiguousarray(arr).reshape(n, -1).view(np.uint8)
            out[:, off:off + b.shape[1]] = b
        put(lay["kc_offset"], np.swapaxes(pack_k_words(kcodes, 4), -1, -2).astype("<u4"))
        put(lay["vc_offset"], np.swapaxes(pack_v_words(vcodes, 4), -1, -2).astype("<u4"))
        put(lay["kmeta_offset"], np.asarray(kscale, np.uint8))                  # [.., D]
        put(lay["vmeta_offset"], np.asarray(vscale, np.uint8))                  # [.., G, 32]
        return out.reshape(lead + (lay["record_bytes"],))

    def _pack_h16(self, kcodes, vcodes, kscale, kzero, vscale, vzero):
        """Integer codes in their usual layout; scales and zeros as fp16."""
        from .layout import pack_k_words, pack_v_words
        lay = self.layout
        lead = kcodes.shape[:-2]
        n = int(np.prod(lead, dtype=np.int64))
        out = np.zeros((n, lay["record_bytes"]), np.uint8)

        def put(off, arr):
            b = np.ascontiguousarray(arr).reshape(n, -1).view(np.uint8)
            out[:, off:off + b.shape[1]] = b
        put(lay["kc_offset"], np.swapaxes(pack_k_words(kcodes, self.kb), -1, -2).astype("<u4"))
        put(lay["vc_offset"], np.swapaxes(pack_v_words(vcodes, self.vb), -1, -2).astype("<u4"))
        put(lay["kmeta_offset"], np.concatenate([np.asarray(kscale, "<f2"), np.asarray(kzero, "<f2")], axis=-1))
        put(lay["vmeta_offset"], np.stack([np.asarray(vscale, "<f2"), np.asarray(vzero, "<f2")], axis=-2))
        return out.reshape(lead + (lay["record_bytes"],))

    # ------------------------------------------------------------------ views
    def ntok(self, segment: int, b: int) -> int:
        return self.seg[segment][b].ntok

    def nslots(self, segment: int, b: int) -> int:
        return self.seg[segment][b].nslots

    def _cat(self, segment: int, b: int, key: str):
        ch = self.seg[segment][b].chunks
        if not ch or ch[0][key] is None:
            return None
        return np.concatenate([c[key] for c in ch], axis=0)

    def records(self, segment: int, b: int) -> Optional[np.ndarray]:
        """uint8 [nslots, Hkv, record_bytes] as the ABI lays them out."""
        return self._cat(segment, b, "records")

    def headers(self, segment: int, b: int) -> np.ndarray:
        h = self.seg[segment][b].headers
        if not h:
            return np.zeros((0, 16), np.uint8)
        return np.stack([pack_header(*x) for x in h])

    def codes(self, segment: int, b: int) -> dict:
        keys = ("kcodes", "vcodes", "kscale", "kzero", "vscale", "vzero")
        return {k: self._cat(segment, b, k) for k in keys}

    def protected(self, segment: int, b: int):
        st = self.seg[segment][b]
        rows = np.stack(st.prot_rows) if st.prot_rows else np.zeros((0, self.Hkv, self.D), np.float32)
        return np.asarray(st.prot_pos, np.int32), rows

    def dequantized(self, segment: int, b: int, h: int):
        """(K_hat, V_hat) of the valid tokens of a segment, fp64 [ntok, D] each.

        A protected key token's row is its stored bf16 row."""
        st = self.seg[segment][b]
        if st.ntok == 0:
            return np.zeros((0, self.D)), np.zeros((0, self.D))
        c = self.codes(segment, b)
        ns = st.nslots
        # K: code * scale_c + zero_c, per channel c of the slot
        kc = c["kcodes"][:, h]                                   # [ns, 32, D]
        if self.fmt == "mxfp4":
            khat = mx_dequantize(kc.transpose(0, 2, 1), c["kscale"][:, h]).transpose(0, 2, 1)
        else:
            khat = dequantize(kc.transpose(0, 2, 1), c["kscale"][:, h], c["kzero"][:, h]).transpose(0, 2, 1)
        # V: code * scale_t + zero_t, per token t and channel group
        vc = c["vcodes"][:, h]                                   # [ns, D, 32]
        G = self.D // self.gv
        v5 = vc.reshape(ns, G, self.gv, SLOT).transpose(0, 3, 1, 2)          # [ns, 32, G, gv]
        if self.fmt == "mxfp4":
            vhat = mx_dequantize(v5, c["vscale"][:, h].transpose(0, 2, 1))
        else:
            vhat = dequantize(v5, c["vscale"][:, h].transpose(0, 2, 1), c["vzero"][:, h].transpose(0, 2, 1))
        vhat = vhat.reshape(ns, SLOT, self.D)
        rank_rows = st.prot_rows
        for j, (nvalid, mask, base, _) in enumerate(st.headers):
            r = base
            for t in range(SLOT):
                if mask >> t & 1:
                    khat[j, t] = rank_rows[r][h].astype(np.float64)
                    r += 1
        keep = np.concatenate([np.arange(SLOT) < hd[0] for hd in st.headers])
        return khat.reshape(-1, self.D)[keep], vhat.reshape(-1, self.D)[keep]
