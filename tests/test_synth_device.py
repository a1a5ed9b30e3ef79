"""The device generator's recipe, checked on the CPU device (torch's CPU generator
stands in for the GPU's Philox: the construction is the same code).

It must reproduce the host recipe's structure: the same token classes and head
types, bf16-representable values, planted directions on the right keys, local
heads clustered around their centre, rotary embedding at the right positions,
and batch entries that do not depend on which other entries are drawn."""
import numpy as np
import torch

from synth import device as dev
from synth import inputs as syn


def _spec(**kw):
    base = dict(seq_len=96, head_dim=64, n_q_heads=8, n_kv_heads=4, batch=3, mix="fixed",
                fixed_types=("special", "punct", "heavy", "local"), decode_steps=10)
    base.update(kw)
    return syn.custom_spec(syn.CONFIGS[1], **base)


def test_classes_types_and_determinism():
    spec = _spec()
    a = dev.make_layer_device(spec, 0, device="cpu")
    b = dev.make_layer_device(spec, 0, device="cpu")
    assert a.types == syn.head_types(spec, 0)
    for i in range(spec.batch):
        assert np.array_equal(a.token_class_host[i], syn.token_classes(spec, i))
    assert torch.equal(a.token_class.cpu(), torch.from_numpy(a.token_class_host))
    for x, y in ((a.Q, b.Q), (a.K, b.K), (a.V, b.V)):
        assert x.dtype == torch.bfloat16 and torch.equal(x, y)
    # another layer draws other values
    c = dev.make_layer_device(spec, 1, device="cpu")
    assert not torch.equal(a.V, c.V)


def test_sub_batch_equals_slice():
    spec = _spec()
    full = dev.make_layer_device(spec, 2, device="cpu")
    one = dev.make_layer_device(spec, 2, device="cpu", batch=[2])
    assert torch.equal(one.Q[0], full.Q[2]) and torch.equal(one.K[0], full.K[2]) and torch.equal(one.V[0], full.V[2])
    ds_full = dev.make_decode_stream_device(spec, 2, device="cpu")
    ds_one = dev.make_decode_stream_device(spec, 2, device="cpu", batch=[1])
    assert torch.equal(ds_one.q[:, 0], ds_full.q[:, 1]) and torch.equal(ds_one.k[:, 0], ds_full.k[:, 1])


def _unrope(x: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Inverse rotation of the rotate-half embedding (rotation by the negative angle)."""
    d = x.shape[-1]
    half = d // 2
    cos, sin = syn._rope_tables(positions, d)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos + b * sin, b * cos - a * sin], axis=-1)


def test_plants_land_on_their_keys():
    spec = _spec(batch=1, seq_len=400)
    li = dev.make_layer_device(spec, 0, device="cpu")
    K = dev.host_f32(li.K[0]).astype(np.float64)
    Q = dev.host_f32(li.Q[0]).astype(np.float64)
    cls = li.token_class_host[0]
    d, G = spec.head_dim, spec.group
    for h, kind in enumerate(li.types):
        if kind not in ("special", "punct", "heavy"):
            continue
        u = syn._direction(syn.canonical_seed(1), spec, 0, h)
        proj = K[h] @ u / np.linalg.norm(u)                          # 6 sqrt(d) on planted keys, N(0,1) elsewhere
        if kind == "special":
            sel = cls == syn.TOKEN_SPECIAL
        elif kind == "punct":
            sel = cls == syn.TOKEN_PUNCT
        else:
            sel = proj > 3.0 * np.sqrt(d)
            assert sel.sum() == spec.seq_len // 20
            assert np.all(cls[sel] == syn.TOKEN_NORMAL)
        assert np.all(proj[sel] > 6 * np.sqrt(d) - 6.0), kind
        assert np.all(np.abs(proj[~sel]) < 6.0), kind
        qp = Q[h * G:(h + 1) * G] @ u / np.linalg.norm(u)            # every query carries u
        assert abs(qp.mean() - np.sqrt(d)) < 0.5, kind


def test_local_head_is_a_rotated_cluster():
    spec = _spec(batch=1, seq_len=300)
    li = dev.make_layer_device(spec, 0, device="cpu")
    h = li.types.index("local")
    c = syn._local_center(syn.canonical_seed(1), spec, 0, h)
    K = dev.host_f32(li.K[0, h]).astype(np.float64)
    base = _unrope(K, np.arange(spec.seq_len))                       # c + 0.3 noise before the rotation
    resid = base - c
    assert abs(resid.std() - 0.3) < 0.03
    assert np.abs(resid.mean(axis=0)).max() < 0.15


def test_unplanted_values_are_standard_normal_and_bf16():
    spec = _spec(batch=2, seq_len=256, fixed_types=("none", "none", "none", "none"))
    li = dev.make_layer_device(spec, 0, device="cpu")
    for t in (li.Q, li.K, li.V):
        x = dev.host_f32(t)
        assert np.array_equal(syn.round_to_bf16(x), x)               # exactly bf16 values
        assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1.0) < 0.02


def test_decode_stream_plants_and_classes():
    spec = _spec(batch=2, seq_len=64, decode_steps=200)
    ds = dev.make_decode_stream_device(spec, 0, device="cpu")
    for b in range(2):
        assert np.array_equal(ds.new_class_host[:, b], syn.new_token_classes(spec, b, 200))
    assert not np.any(ds.new_class_host == syn.TOKEN_SPECIAL)
    h = syn.head_types(spec, 0).index("punct")
    u = syn._direction(syn.canonical_seed(1), spec, 0, h)
    k = dev.host_f32(ds.k[:, 0, h]).astype(np.float64)
    proj = k @ u / np.linalg.norm(u)
    sel = ds.new_class_host[:, 0] == syn.TOKEN_PUNCT
    assert sel.any() and np.all(proj[sel] > 6 * np.sqrt(spec.head_dim) - 6.0)
    assert np.all(np.abs(proj[~sel]) < 6.0)
    # overriding the classes moves the plant with them
    cl = np.zeros((200, 2), np.uint8)
    cl[5, 0] = syn.TOKEN_PUNCT
    ds2 = dev.make_decode_stream_device(spec, 0, device="cpu", classes=cl)
    proj2 = dev.host_f32(ds2.k[:, 0, h]).astype(np.float64) @ u / np.linalg.norm(u)
    assert proj2[5] > 6 * np.sqrt(spec.head_dim) - 6.0 and np.all(np.abs(np.delete(proj2, 5)) < 6.0)
