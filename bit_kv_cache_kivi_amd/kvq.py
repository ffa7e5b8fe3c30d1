"""Python binding of the kvq C ABI (include/kvq.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libkvq.so.  PyTorch supplies device memory (the cache buffer, inputs, outputs)
and the current stream.  Importing this module loads libkvq.so and raises if it
has not been built; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import POINTER, byref, c_char_p, c_float, c_int32, c_size_t, c_uint64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

KVQ_OK, KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_ECAPACITY, KVQ_EHIP = range(5)
KVQ_F32, KVQ_BF16 = 0, 1
KVQ_PREFIX, KVQ_SUFFIX = 0, 1
KVQ_FMT_INT, KVQ_FMT_MXFP4, KVQ_FMT_INT_H16 = 0, 1, 2
SLOT = 32


class KvqConfig(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in (
        "batch", "num_kv_heads", "head_dim", "k_bits", "v_bits", "k_group_tokens",
        "v_group_channels", "prefix_slots", "suffix_slots", "prefix_protected",
        "suffix_protected", "max_q_heads", "max_splits", "v_rotation_block", "protect_sink", "kv_format")]


class KvqLayout(ctypes.Structure):
    _fields_ = [
        ("total_bytes", c_uint64), ("record_bytes", c_uint64),
        ("kc_offset", c_uint64), ("vc_offset", c_uint64), ("kmeta_offset", c_uint64),
        ("vmeta_offset", c_uint64),
        ("records_offset", c_uint64 * 2), ("headers_offset", c_uint64 * 2),
        ("prot_rows_offset", c_uint64 * 2), ("prot_pos_offset", c_uint64 * 2),
        ("slot_cap", c_int32 * 2), ("prot_cap", c_int32 * 2),
        ("workspace_offset", c_uint64), ("workspace_bytes", c_uint64),
        ("rotation_offset", c_uint64), ("rotation_bytes", c_uint64),
        ("sel_contrib_offset", c_uint64), ("sel_unit_offset", c_uint64), ("sel_mask_offset", c_uint64),
        ("sel_units_offset", c_uint64),
        ("sel_count_offset", c_uint64),
        ("sel_stats_offset", c_uint64),
    ]


class KvqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"kvq status {status}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                          " (or python bit_kv_cache_kivi_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P = POINTER
    sig = {
        "kvq_required_bytes": (c_size_t, [P(KvqConfig)]),
        "kvq_get_layout": (c_int32, [P(KvqConfig), P(KvqLayout)]),
        "kvq_create": (c_int32, [P(KvqConfig), c_void_p, c_size_t, P(c_void_p)]),
        "kvq_destroy": (c_int32, [c_void_p]),
        "kvq_commit": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_int32, c_int32,
                                 P(c_int32), P(c_int32), P(c_int32), c_void_p]),
        "kvq_block_attn": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                     c_int32, c_int32, c_float, c_void_p, c_int32, c_void_p]),
        "kvq_select": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_int32, c_int32,
                                 c_float, P(ctypes.c_uint32), c_int32, c_int32, c_void_p]),
        "kvq_block_attn_noalloc": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                             c_int32, c_int32, c_float, c_void_p, c_int32, c_void_p]),
        "kvq_block_attn_selected": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                              c_int32, c_int32, c_float, c_void_p, c_int32, c_void_p]),
        "kvq_attend_commit": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                        c_int32, c_int32, c_float, c_void_p, c_int32, P(c_int32), P(c_int32),
                                        P(c_int32), c_void_p]),
        "kvq_attend_select": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                        c_int32, c_int32, c_float, c_void_p, c_int32, P(ctypes.c_uint32), c_int32,
                                        c_int32, c_void_p]),
        "kvq_segment_info": (c_int32, [c_void_p, c_int32, P(c_int32), P(c_int32), P(c_int32)]),
        "kvq_set_split_slots": (c_int32, [c_void_p, c_int32]),
        "kvq_set_v_rotation": (c_int32, [c_void_p, P(c_int32), P(c_float)]),
        "kvq_status_str": (c_char_p, [c_int32]),
        "kvq_last_error": (c_char_p, []),
        "kvq_abi_version": (c_int32, []),
        "kvq_calib_copy": (c_int32, [c_void_p, c_void_p, c_size_t, c_void_p]),
        "kvq_calib_mfma": (c_int32, [c_void_p, c_int32, c_int32, c_void_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def last_error() -> str:
    return lib.kvq_last_error().decode()


def check(status: int):
    if status != KVQ_OK:
        raise KvqError(status, f"{lib.kvq_status_str(status).decode()}: {last_error()}")


def _int_array(vals):
    if vals is None:
        return None
    arr = (c_int32 * len(vals))(*[int(x) for x in vals])
    return arr


def make_config(batch, num_kv_heads, head_dim, k_bits=4, v_bits=4, v_group=128, prefix_slots=1,
                suffix_slots=0, prefix_protected=0, suffix_protected=0, max_q_heads=None, max_splits=0,
                v_rotation_block=0, protect_sink=0, kv_format=0):
    return KvqConfig(batch, num_kv_heads, head_dim, k_bits, v_bits, SLOT, v_group, prefix_slots,
                     suffix_slots, prefix_protected, suffix_protected,
                     max_q_heads if max_q_heads is not None else num_kv_heads, max_splits, v_rotation_block,
                     int(bool(protect_sink)), int(kv_format))


def get_layout(cfg: KvqConfig) -> dict:
    lay = KvqLayout()
    check(lib.kvq_get_layout(byref(cfg), byref(lay)))
    out = {}
    for name, _ in KvqLayout._fields_:
        v = getattr(lay, name)
        out[name] = list(v) if hasattr(v, "__len__") else int(v)
    return out


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return KVQ_F32
    if t.dtype == torch.bfloat16:
        return KVQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return c_void_p(s.cuda_stream)


def _mask_array(query_mask):
    """Per-sequence 32-bit query masks as a host uint32 array (None = all)."""
    if query_mask is None:
        return None
    return (ctypes.c_uint32 * len(query_mask))(*[int(x) & 0xFFFFFFFF for x in query_mask])


def _csr(protected):
    """Per-sequence position lists -> (offsets, indices) C arrays, or (None, None)."""
    if protected is None:
        return None, None
    o = [0]
    flat = []
    for p in protected:
        flat.extend(int(x) for x in p)
        o.append(len(flat))
    return _int_array(o), (_int_array(flat) if flat else (c_int32 * 1)(0))


def _expect(name, t, shape, dtypes=None):
    """Checks one tensor argument before any library call: exact shape,
    contiguity and dtype.  The C ABI receives raw pointers only, so a tensor
    of the wrong shape would be read or written out of bounds by the kernels."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(buffer, **tensors):
    """Every tensor argument must live on the cache buffer's GPU (a host
    pointer handed to a kernel faults the device)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda or t.device != buffer.device:
            raise ValueError(f"{name} is on {t.device}; the cache lives on {buffer.device}")


def _per_sequence(name, vals, B):
    if vals is not None and len(vals) != B:
        raise ValueError(f"{name} has {len(vals)} entries, expected one per sequence ({B})")


class KVCache:
    """One layer's low-bit cache in a torch-owned device buffer."""

    def __init__(self, batch, num_kv_heads, head_dim, k_bits=4, v_bits=4, v_group=128,
                 prefix_tokens=32, suffix_tokens=0, prefix_protected=0, suffix_protected=0,
                 max_q_heads=None, max_splits=0, v_rotation_block=0, protect_sink=False, kv_format=0,
                 device="cuda"):
        import torch
        self.cfg = make_config(batch, num_kv_heads, head_dim, k_bits, v_bits, v_group,
                               -(-prefix_tokens // SLOT), -(-suffix_tokens // SLOT),
                               prefix_protected, suffix_protected, max_q_heads, max_splits,
                               v_rotation_block, protect_sink, kv_format)
        self.layout = get_layout(self.cfg)
        nbytes = self.layout["total_bytes"]
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        h = c_void_p()
        check(lib.kvq_create(byref(self.cfg), c_void_p(self.buffer.data_ptr()), nbytes, byref(h)))
        self._h = h

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h:
            check(lib.kvq_destroy(self._h))
            self._h = c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _q_heads(self, q):
        hq = int(q.shape[2])
        H = self.cfg.num_kv_heads
        if hq < H or hq % H != 0 or hq > self.cfg.max_q_heads:
            raise ValueError(f"q has {hq} heads: a multiple of num_kv_heads {H} up to max_q_heads "
                             f"{self.cfg.max_q_heads} is needed")
        return hq

    def _check_attn(self, q, k_blk, v_blk, out, out_dtype):
        """Shapes [B, 32, Hq, D] (q, out) and [B, 32, Hkv, D] (k_blk, v_blk),
        dtypes, contiguity and device, before any library call; returns out
        (allocated when None)."""
        import torch
        B, H, D = self.cfg.batch, self.cfg.num_kv_heads, self.cfg.head_dim
        fp = (torch.float32, torch.bfloat16)
        if not hasattr(q, "shape") or q.dim() != 4:
            raise ValueError("q must be a [B, 32, Hq, D] tensor")
        hq = self._q_heads(q)
        _expect("q", q, (B, SLOT, hq, D), fp)
        _expect("k_blk", k_blk, (B, SLOT, H, D), fp)
        _expect("v_blk", v_blk, (B, SLOT, H, D), (k_blk.dtype,))
        if out is None:
            _on_device(self.buffer, q=q, k_blk=k_blk, v_blk=v_blk)
            return torch.empty(q.shape, dtype=out_dtype or torch.bfloat16, device=q.device)
        _expect("out", out, (B, SLOT, hq, D), fp)
        _on_device(self.buffer, q=q, k_blk=k_blk, v_blk=v_blk, out=out)
        return out

    def commit(self, k, v, ntok=None, protected=None, segment=KVQ_PREFIX, reset=False, stream=None):
        """k, v: [B, n_max, Hkv, D] (fp32 or bf16, contiguous, on the device).

        ntok: per-sequence token counts (default n_max); protected: per-sequence
        sorted positions, relative to this commit, of key rows kept in bf16."""
        import torch
        B, H, D = self.cfg.batch, self.cfg.num_kv_heads, self.cfg.head_dim
        if not hasattr(k, "shape") or k.dim() != 4:
            raise ValueError("k must be a [B, n_max, Hkv, D] tensor")
        n_max = int(k.shape[1])
        fp = (torch.float32, torch.bfloat16)
        _expect("k", k, (B, n_max, H, D), fp)
        _expect("v", v, (B, n_max, H, D), (k.dtype,))
        _per_sequence("ntok", ntok, B)
        _per_sequence("protected", protected, B)
        _on_device(self.buffer, k=k, v=v)
        nt = _int_array(ntok)
        off, idx = _csr(protected)
        check(lib.kvq_commit(self._h, int(segment), int(bool(reset)), c_void_p(k.data_ptr()),
                             c_void_p(v.data_ptr()), _dtype_code(k), int(k.shape[1]), nt, off, idx,
                             _stream_ptr(stream)))

    def block_attn(self, q, k_blk, v_blk, use_suffix=False, softmax_scale=None, out_dtype=None,
                   out=None, stream=None):
        """q [B, 32, Hq, D]; k_blk, v_blk [B, 32, Hkv, D].  Returns out [B, 32, Hq, D]."""
        import torch
        out = self._check_attn(q, k_blk, v_blk, out, out_dtype)
        D = self.cfg.head_dim
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(D)
        check(lib.kvq_block_attn(self._h, int(bool(use_suffix)), c_void_p(q.data_ptr()), int(q.shape[2]),
                                 _dtype_code(q), c_void_p(k_blk.data_ptr()), c_void_p(v_blk.data_ptr()),
                                 _dtype_code(k_blk), int(q.shape[1]), float(softmax_scale),
                                 c_void_p(out.data_ptr()), _dtype_code(out), _stream_ptr(stream)))
        return out

    def block_attn_noalloc(self, q, k_blk, v_blk, use_suffix=False, softmax_scale=None, out_dtype=None,
                           out=None, stream=None):
        """block_attn with the workspace in the library's per-device scratch
        array (kvq_block_attn_noalloc): no allocation inside the call; out must
        be given to avoid one here as well."""
        out = self._check_attn(q, k_blk, v_blk, out, out_dtype)
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(self.cfg.head_dim)
        check(lib.kvq_block_attn_noalloc(self._h, int(bool(use_suffix)), c_void_p(q.data_ptr()), int(q.shape[2]),
                                         _dtype_code(q), c_void_p(k_blk.data_ptr()), c_void_p(v_blk.data_ptr()),
                                         _dtype_code(k_blk), int(q.shape[1]), float(softmax_scale),
                                         c_void_p(out.data_ptr()), _dtype_code(out), _stream_ptr(stream)))
        return out

    def attend_commit(self, q, k_blk, v_blk, ntok=None, protected=None, use_suffix=False, softmax_scale=None,
                      out_dtype=None, out=None, stream=None):
        """block_attn over the cache as it is, then commit k_blk, v_blk to the
        prefix (ntok, protected as for commit), in one call."""
        out = self._check_attn(q, k_blk, v_blk, out, out_dtype)
        _per_sequence("ntok", ntok, self.cfg.batch)
        _per_sequence("protected", protected, self.cfg.batch)
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(self.cfg.head_dim)
        off, idx = _csr(protected)
        check(lib.kvq_attend_commit(self._h, int(bool(use_suffix)), c_void_p(q.data_ptr()), int(q.shape[2]),
                                    _dtype_code(q), c_void_p(k_blk.data_ptr()), c_void_p(v_blk.data_ptr()),
                                    _dtype_code(k_blk), int(q.shape[1]), float(softmax_scale),
                                    c_void_p(out.data_ptr()), _dtype_code(out), _int_array(ntok), off, idx,
                                    _stream_ptr(stream)))
        return out

    def select(self, q, k_blk, budget, use_suffix=False, query_mask=None, softmax_scale=None, granularity=1,
               stream=None):
        """Rank the cached entries by the mask queries' contributions and keep
        the top `budget` per (sequence, kv head) (granularity 32: the top
        `budget` 32-token units by summed contributions).  query_mask:
        per-sequence 32-bit masks of the mask queries (None = all)."""
        import torch
        B, H, D = self.cfg.batch, self.cfg.num_kv_heads, self.cfg.head_dim
        fp = (torch.float32, torch.bfloat16)
        if not hasattr(q, "shape") or q.dim() != 4:
            raise ValueError("q must be a [B, 32, Hq, D] tensor")
        _expect("q", q, (B, SLOT, self._q_heads(q), D), fp)
        _expect("k_blk", k_blk, (B, SLOT, H, D), fp)
        _per_sequence("query_mask", query_mask, B)
        _on_device(self.buffer, q=q, k_blk=k_blk)
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(self.cfg.head_dim)
        check(lib.kvq_select(self._h, int(bool(use_suffix)), c_void_p(q.data_ptr()), int(q.shape[2]), _dtype_code(q),
                             c_void_p(k_blk.data_ptr()), _dtype_code(k_blk), int(q.shape[1]), float(softmax_scale),
                             _mask_array(query_mask), int(budget), int(granularity), _stream_ptr(stream)))

    def attend_select(self, q, k_blk, v_blk, budget, use_suffix=False, query_mask=None, softmax_scale=None,
                      granularity=1, out_dtype=None, out=None, stream=None):
        """block_attn over the whole cache, then select as select() does,
        with each query row's softmax normaliser taken from that attention.
        Returns out [B, 32, Hq, D]."""
        out = self._check_attn(q, k_blk, v_blk, out, out_dtype)
        _per_sequence("query_mask", query_mask, self.cfg.batch)
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(self.cfg.head_dim)
        check(lib.kvq_attend_select(self._h, int(bool(use_suffix)), c_void_p(q.data_ptr()), int(q.shape[2]),
                                    _dtype_code(q), c_void_p(k_blk.data_ptr()), c_void_p(v_blk.data_ptr()),
                                    _dtype_code(k_blk), int(q.shape[1]), float(softmax_scale),
                                    c_void_p(out.data_ptr()), _dtype_code(out), _mask_array(query_mask),
                                    int(budget), int(granularity), _stream_ptr(stream)))
        return out

    def block_attn_selected(self, q, k_blk, v_blk, use_suffix=False, softmax_scale=None, out_dtype=None,
                            out=None, stream=None):
        """block_attn over the block and the last selection only."""
        out = self._check_attn(q, k_blk, v_blk, out, out_dtype)
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(self.cfg.head_dim)
        check(lib.kvq_block_attn_selected(self._h, int(bool(use_suffix)), c_void_p(q.data_ptr()), int(q.shape[2]),
                                          _dtype_code(q), c_void_p(k_blk.data_ptr()), c_void_p(v_blk.data_ptr()),
                                          _dtype_code(k_blk), int(q.shape[1]), float(softmax_scale),
                                          c_void_p(out.data_ptr()), _dtype_code(out), _stream_ptr(stream)))
        return out

    def selection(self, b, h, nunits):
        """(contributions fp32 [nunits*32], token masks uint32 [nunits], selected
        unit list int32, unit sums fp32 [nunits]) of sequence b, kv head h
        (views of the buffer)."""
        import torch
        L = self.layout
        H = self.cfg.num_kv_heads
        ucap = L["slot_cap"][0] + L["slot_cap"][1]
        pair = b * H + h
        cb = L["sel_contrib_offset"] + pair * ucap * SLOT * 4
        contrib = self.buffer[cb:cb + nunits * SLOT * 4].view(torch.float32)
        mb = L["sel_mask_offset"] + pair * ucap * 4
        masks = self.buffer[mb:mb + nunits * 4].view(torch.int32)
        cnt_off = L["sel_count_offset"] + pair * 4
        n = int(self.buffer[cnt_off:cnt_off + 4].view(torch.int32).item())
        ub = L["sel_units_offset"] + pair * ucap * 4
        units = self.buffer[ub:ub + n * 4].view(torch.int32)
        sb = L["sel_unit_offset"] + pair * ucap * 4
        sums = self.buffer[sb:sb + nunits * 4].view(torch.float32)
        return contrib, masks, units, sums

    def segment_info(self, segment=KVQ_PREFIX):
        B = self.cfg.batch
        a, b_, c = (c_int32 * B)(), (c_int32 * B)(), (c_int32 * B)()
        check(lib.kvq_segment_info(self._h, int(segment), a, b_, c))
        return list(a), list(b_), list(c)

    def set_split_slots(self, n: int):
        check(lib.kvq_set_split_slots(self._h, int(n)))

    def set_v_rotation(self, perm, mix):
        """perm: D channel indices (a permutation); mix: k x k orthogonal matrix,
        k = head_dim / v_rotation_block (any nested sequence or array)."""
        perm = [int(x) for x in perm]
        flat = [float(x) for row in mix for x in row]
        D, blk = self.cfg.head_dim, self.cfg.v_rotation_block
        k = D // blk if blk else 0
        if len(perm) != D or len(flat) != k * k:
            raise ValueError(f"perm needs {D} entries and mix {k}x{k} (v_rotation_block={blk})")
        check(lib.kvq_set_v_rotation(self._h, (c_int32 * len(perm))(*perm), (c_float * len(flat))(*flat)))

    # ---- raw views of the buffer (for inspection and tests)
    def records(self, segment, b):
        """uint8 tensor [nslots, Hkv, record_bytes] of sequence b's slots."""
        L = self.layout
        H, cap, R = self.cfg.num_kv_heads, L["slot_cap"][segment], L["record_bytes"]
        n = self.segment_info(segment)[1][b]
        base = L["records_offset"][segment] + b * H * cap * R
        return self.buffer[base:base + H * cap * R].view(H, cap, R)[:, :n].permute(1, 0, 2)

    def headers(self, segment, b):
        L = self.layout
        cap = L["slot_cap"][segment]
        n = self.segment_info(segment)[1][b]
        base = L["headers_offset"][segment] + b * cap * 16
        return self.buffer[base:base + n * 16].view(n, 16)

    def protected_rows(self, segment, b):
        """(positions int32 [nprot], bf16 bits int16 [nprot, Hkv, D])."""
        import torch
        L = self.layout
        H, D, pcap = self.cfg.num_kv_heads, self.cfg.head_dim, L["prot_cap"][segment]
        n = self.segment_info(segment)[2][b]
        rb = L["prot_rows_offset"][segment] + b * H * pcap * D * 2
        pb = L["prot_pos_offset"][segment] + b * pcap * 4
        rows = self.buffer[rb:rb + H * pcap * D * 2].view(torch.int16).view(H, pcap, D)[:, :n].permute(1, 0, 2)
        pos = self.buffer[pb:pb + n * 4].view(torch.int32)
        return pos, rows
