"""GPU-vs-oracle parity at the full workload sizes, in the launch configuration
the benchmark times (bf16 inputs, the library's default split choice, bf16 and
fp32 outputs).

Every record, header and protected row of every sequence must equal the
oracle's byte for byte, and every attention output must be within the gate
(max |gpu - oracle| <= 2e-3 with fp32 output; plus half a bf16 ulp of the exact
value with bf16 output).  Workloads without a suffix then take one more
per-step commit of a fresh 32-token block, as the benchmark step does, and are
checked again.  The oracle is fast enough at these sizes (vectorised numpy,
about a quarter of a second per 8192-token sequence) to check everything
instead of a sample.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import announce, attention_error, build_case, compare_commit, dev  # noqa: E402


def _check_attention(w, cache, ora, tag):
    c = w.cfg
    use_suffix = bool(c.suffix)
    ref = O.block_attention(ora, w.q, w.k_blk, w.v_blk, use_suffix=use_suffix)
    q, kb, vb = dev(w.q, c.dtype), dev(w.k_blk, c.dtype), dev(w.v_blk, c.dtype)
    out16 = cache.block_attn(q, kb, vb, use_suffix=use_suffix, out_dtype=torch.bfloat16)
    e16, x16 = attention_error(out16, ref, "bf16")
    out32 = cache.block_attn(q, kb, vb, use_suffix=use_suffix, out_dtype=torch.float32)
    e32, x32 = attention_error(out32, ref, "f32")
    print(f"{c.name} {tag}: {ref.size} outputs, fp32-out err={e32:.2e} bf16-out err={e16:.2e}", flush=True)
    assert x32 <= 0, f"{tag}: fp32 output error {e32}"
    assert x16 <= 0, f"{tag}: bf16 output error {e16} exceeds 2e-3 + ulp/2"


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_full_size(name):
    announce("full size", name)
    w, cache, ora = build_case(W.CONFIGS[name], extra_slots=2)
    c = w.cfg
    compare_commit(cache, ora, 0, c.B)
    if c.suffix:
        compare_commit(cache, ora, 1, c.B)
    _check_attention(w, cache, ora, "prefix")
    if not c.suffix:
        k, v, prot = W.step_block(c, 0)
        cache.commit(dev(k, c.dtype), dev(v, c.dtype), protected=prot)
        ora.commit(0, k, v, prot=prot)
        compare_commit(cache, ora, 0, c.B)
        _check_attention(w, cache, ora, "after a per-step commit")
    cache.close()
