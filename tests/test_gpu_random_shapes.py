"""GPU parity sweep over seeded random shapes, for every attention entry point:
contiguous tree attention, paged prefill (causal, unmasked, sliding window
with sink, tree, K rotated in the kernel or before caching; some cases split
the KV ranges), ragged prefill (causal, unmasked, right and left padding)
and latent attention. Each case is drawn from its own fixed seed, so a failure
names a case that reproduces exactly. Lengths favour the tile edges (0, 1,
15-17, 31-33, 63-65, 127-129); group sizes 1-16 with 1-8 KV heads, both head
dims and dtypes, and the workgroup shape chosen per launch or forced to four
or eight waves. Every row is compared against the oracle, with outputs
NaN-poisoned before the launch.
"""

import numpy as np
import pytest
import torch

from tests.parity import DeviceInputs, compare, run_oracle, say
from workloads import make_custom_mla, make_custom_paged, make_custom_ragged, make_custom_tree

pytestmark = pytest.mark.gpu

EDGES = (0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129)
N_TREE, N_PAGED, N_RAGGED, N_MLA = 24, 40, 20, 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_ragged_gqa_amd as ra
    ra.library()
    yield
    ra.ra_set_workgroup_waves(0)


def _length(rng, hi):
    if rng.random() < 0.5:
        return int(rng.choice([e for e in EDGES if e <= hi]))
    return int(rng.integers(0, hi + 1))


def _heads(rng):
    h_kv = int(rng.choice([1, 2, 4, 8]))
    return h_kv * int(rng.choice([1, 2, 4, 8, 16])), h_kv


def _common(rng):
    return dict(d=int(rng.choice([64, 128])), dtype=str(rng.choice(["f16", "bf16"])),
                sm_scale=None if rng.random() < 0.7 else float(rng.uniform(0.03, 0.3)))


def _run(w, label, waves=0, splits=None):
    import attention_ragged_gqa_amd as ra
    ra.ra_set_workgroup_waves(waves)
    say("[gpu] %s: b=%d total_q=%d h=%d/%d d=%d %s waves=%d splits=%s"
        % (label, w.batch, w.total_q, w.h_q, w.h_kv, w.d, w.dtype, waves, splits))
    try:
        di = DeviceInputs(w)
        di.poison()
        out, lse = di.launch(num_kv_splits=splits) if splits is not None else di.launch()
        torch.cuda.synchronize()
    finally:
        ra.ra_set_workgroup_waves(0)
    ref_out, ref_lse = run_oracle(w)
    d_out, d_lse = compare(out, lse, ref_out, ref_lse, label=label)
    say("[gpu] %s: max|d out| %.2e  max rel|d lse| %.2e" % (label, d_out, d_lse))


def tree_case(i):
    rng = np.random.default_rng(5000 + i)
    sizes = [_length(rng, 200) for _ in range(int(rng.integers(1, 5)))]
    if sum(sizes) == 0:
        sizes[0] = 1
    h_q, h_kv = _heads(rng)
    c = _common(rng)
    rot = int(rng.integers(0, 2))
    w = make_custom_tree(5000 + i, sizes, h_q=h_q, h_kv=h_kv, rotary_mode=rot,
                         max_children=[None, 2, 4][int(rng.integers(0, 3))],
                         rope_theta=float(rng.choice([1e4, 5e5])), rope_scale=float(rng.choice([1.0, 0.5])),
                         position_offset=int(rng.integers(0, 3000)), **c)
    return w, int(rng.choice([0, 4, 8]))


def paged_case(i):
    rng = np.random.default_rng(6000 + i)
    b = int(rng.integers(1, 5))
    kind = str(rng.choice(["causal", "full", "sliding", "tree", "k_rope", "cached_rope"]))
    qo = [_length(rng, 150) for _ in range(b)]
    stored = [q + _length(rng, 300) for q in qo]
    if sum(qo) == 0:
        qo[0], stored[0] = 1, stored[0] + 1
    h_q, h_kv = _heads(rng)
    c = _common(rng)
    kw = dict(causal=0 if kind in ("full", "tree") else 1, extra_pages=int(rng.integers(0, 5)))
    if kind == "sliding":
        offs, sinks = [], []
        for s in stored:
            off = int(rng.integers(0, max(s, 1)))
            offs.append(off)
            sinks.append(min(int(rng.integers(0, off + 1)), 40))
        kw["sliding"] = (offs, sinks)
    elif kind == "tree":
        rot = int(rng.integers(0, 2))
        kw.update(tree=True, tree_max_children=int(rng.choice([2, 4])), tree_max_depth=16, rotary_mode=rot,
                  store_rope="tree" if rot else None, rope_theta=5e5)
    elif kind == "k_rope":
        kw.update(rotary_mode=1, k_rope_pos_offset=[int(x) for x in rng.integers(0, 3000, size=b)],
                  rope_scale=float(rng.choice([1.0, 0.5])))
    elif kind == "cached_rope":
        kw.update(store_rope="linear", rope_theta=1e4)
    w = make_custom_paged(6000 + i, qo, stored, h_q=h_q, h_kv=h_kv, **kw, **c)
    splits = None if rng.random() < 0.6 else int(rng.choice([0, 2, 3, 7]))
    return w, kind, int(rng.choice([0, 4, 8])), splits


def ragged_case(i):
    rng = np.random.default_rng(7000 + i)
    b = int(rng.integers(1, 5))
    kind = str(rng.choice(["causal", "full", "right_pad", "left_pad"]))
    qo = [_length(rng, 200) for _ in range(b)]
    kv = [q + _length(rng, 100) if rng.random() < 0.8 else _length(rng, 200) for q in qo]
    if sum(qo) == 0:
        qo[0], kv[0] = 1, max(kv[0], 1)
    h_q, h_kv = _heads(rng)
    c = _common(rng)
    kw = dict(causal=0 if kind in ("full", "right_pad") else 1)
    if kind in ("right_pad", "left_pad"):
        kw.update(pad_mode=1 if kind == "right_pad" else 2,
                  valid_lens=[int(rng.integers(0, max(qo + kv) + 40)) for _ in range(b)])
    w = make_custom_ragged(7000 + i, qo, kv, h_q=h_q, h_kv=h_kv, **kw, **c)
    return w, kind, int(rng.choice([0, 4, 8]))


def mla_case(i):
    rng = np.random.default_rng(8000 + i)
    b = int(rng.integers(1, 5))
    qo = [_length(rng, 130) for _ in range(b)]
    stored = [q + _length(rng, 200) if rng.random() < 0.85 else _length(rng, 100) for q in qo]
    if sum(qo) == 0:
        qo[0], stored[0] = 1, max(stored[0], 1)
    w = make_custom_mla(8000 + i, qo, stored, h_q=int(rng.choice([1, 2, 8, 16, 32, 64, 128])), d_qk=576,
                        d_latent=512, dtype=str(rng.choice(["f16", "bf16"])), causal=int(rng.integers(0, 2)),
                        extra_pages=int(rng.integers(0, 4)),
                        sm_scale=None if rng.random() < 0.7 else float(rng.uniform(0.02, 0.1)))
    return w


@pytest.mark.parametrize("i", range(N_TREE))
def test_random_tree(i):
    w, waves = tree_case(i)
    _run(w, "random tree[%d] sizes %s rope %d" % (i, np.diff(w.q_indptr).tolist(), w.rotary_mode), waves)


@pytest.mark.parametrize("i", [120])
def test_random_tree_beyond_the_sweep(i):
    """A tree case past the sweep's range whose query rotation once put an
    element exactly on a bf16 rounding tie that a fused multiply-add broke
    the other way (lse 0.1% off on a three-key row); kept as a regression
    case for the rotation's rounding."""
    test_random_tree(i)


@pytest.mark.parametrize("i", range(N_PAGED))
def test_random_paged(i):
    w, kind, waves, splits = paged_case(i)
    _run(w, "random paged[%d] %s qo %s" % (i, kind, np.diff(w.q_indptr).tolist()), waves, splits)


@pytest.mark.parametrize("i", range(N_RAGGED))
def test_random_ragged(i):
    w, kind, waves = ragged_case(i)
    _run(w, "random ragged[%d] %s qo %s" % (i, kind, np.diff(w.q_indptr).tolist()), waves)


@pytest.mark.parametrize("i", range(N_MLA))
def test_random_latent(i):
    w = mla_case(i)
    _run(w, "random latent[%d] h %d qo %s" % (i, w.h_q, np.diff(w.q_indptr).tolist()))
