"""Large commits, whose task tables go through the pinned host ring (needs an
MI355X): records, headers and protected rows bit-exact against the oracle

  * after six commits of more than 64 slots on one handle;
  * after large commits that alternate between handles of different sizes
    (the device's ring of eight tables is shared by all handles: tables are
    rewritten once their kernels finish, and the ring grows, after waiting for
    every table, when a handle needs larger tables than it holds);
  * for a commit whose workgroups hold more tasks than they keep in LDS (128 kv
    heads leave few workgroups per head, so later tasks come through the
    scalar-load path).
"""
import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from bit_kv_cache_kivi_amd import kvq  # noqa: E402
from gpu_util import announce, compare_commit, dev  # noqa: E402


def test_ring_reuse_six_large_commits():
    announce("staging ring: six commits of 80 slots")
    B, H, D = 2, 2, 64
    g = np.random.default_rng(31)
    cache = kvq.KVCache(B, H, D, 4, 2, 32, prefix_tokens=6 * 40 * 32 + 64, prefix_protected=512, max_q_heads=H)
    ora = O.OracleCache(B, H, D, 4, 2, 32)
    for step in range(6):
        n = 40 * 32 - 5 * step                      # 40 slots per sequence, the last partial after step 0
        k = (g.standard_normal((B, n, H, D)) * g.lognormal(0, 1, (1, 1, H, D))).astype(np.float32)
        v = g.standard_normal((B, n, H, D)).astype(np.float32)
        ntok = [n, n - 7 * step]
        prot = [np.sort(g.choice(ntok[b], size=3 + step, replace=False)) for b in range(B)]
        dt = "bf16" if step % 2 else "f32"
        if dt == "bf16":
            k, v = O.to_bf16_f32(k), O.to_bf16_f32(v)
        cache.commit(dev(k, dt), dev(v, dt), ntok=ntok, protected=prot)
        ora.commit(0, k, v, ntok=ntok, prot=prot)
    compare_commit(cache, ora, 0, B)


def test_tasks_past_the_lds_preload():
    announce("many kv heads: tasks through scalar loads")
    B, H, D, T = 1, 128, 64, 8192 + 40
    g = np.random.default_rng(32)
    k = O.to_bf16_f32(g.standard_normal((B, T, H, D)).astype(np.float32))
    v = O.to_bf16_f32(g.standard_normal((B, T, H, D)).astype(np.float32))
    prot = [np.sort(g.choice(T, size=300, replace=False))]
    cache = kvq.KVCache(B, H, D, 4, 4, 64, prefix_tokens=T + 32, prefix_protected=320, max_q_heads=H)
    ora = O.OracleCache(B, H, D, 4, 4, 64)
    cache.commit(dev(k, "bf16"), dev(v, "bf16"), protected=prot)
    ora.commit(0, k, v, prot=prot)
    compare_commit(cache, ora, 0, B)


def test_ring_shared_by_handles_and_grown():
    announce("staging ring: three handles, alternating, growing")
    H, D = 2, 64
    g = np.random.default_rng(33)
    # (batch, prefix slots): tables of 600, 1200 and 2000 slots
    shapes = [(2, 300), (3, 400), (2, 1000)]
    caches, oras = [], []
    for B, slots in shapes:
        caches.append(kvq.KVCache(B, H, D, 4, 2, 32, prefix_tokens=slots * 32, prefix_protected=2048,
                                  max_q_heads=H))
        oras.append(O.OracleCache(B, H, D, 4, 2, 32))
    # the first commits use only the two smaller handles; the largest joins
    # later, so the ring grows while earlier tables may still be in flight
    order = [0, 1, 0, 1, 0, 1, 0, 1, 0, 2, 1, 2, 0, 1, 2, 1]
    used = [0, 0, 0]
    for step, i in enumerate(order):
        B, slots = shapes[i]
        n = 65 * 32 + 17 * (step % 3)             # 66..67 slots per sequence
        if used[i] + -(-n // 32) > slots:
            continue
        k = O.to_bf16_f32(g.standard_normal((B, n, H, D)).astype(np.float32))
        v = O.to_bf16_f32(g.standard_normal((B, n, H, D)).astype(np.float32))
        prot = [np.sort(g.choice(n, size=5 + step, replace=False)) for _ in range(B)]
        caches[i].commit(dev(k, "bf16"), dev(v, "bf16"), protected=prot)
        oras[i].commit(0, k, v, prot=prot)
        used[i] += -(-n // 32)
    assert min(used) > 64
    for i, (B, _) in enumerate(shapes):
        compare_commit(caches[i], oras[i], 0, B)
