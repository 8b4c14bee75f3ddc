"""The nn.Module surface (kpnn2 PackedMultiheadAttention page: constructor
parameter table and "Raises", attributes, reset_parameters, forward's
argument rules). CPU only: construction and argument checks do not touch
the GPU."""
import math

import numpy as np
import pytest
import torch

from graph_sparse_head_amd.module import ModuleArgError, PackedMultiheadAttention as PMA


def _ok(**kw):
    base = dict(source_index=[0, 1, 2], target_index=[1, 2, 0], query_features=3,
                key_features=3, embed_dim=8, num_heads=2)
    base.update(kw)
    return PMA(**base)


def test_attributes_and_parameters():
    m = _ok()
    assert (m.query_features, m.key_features, m.embed_dim, m.num_heads, m.head_dim) == (3, 3, 8, 2, 4)
    assert m.nnz == 3 and m.batch_first is True and m.dropout == 0.0
    assert m.source_index.dtype == torch.int64 and m.source_index.tolist() == [0, 1, 2]
    # four E x E projections with bias: 4 E^2 + 4 E parameters, any graph
    assert sum(p.numel() for p in m.parameters()) == 4 * 64 + 4 * 8
    m2 = _ok(bias=False)
    assert sum(p.numel() for p in m2.parameters()) == 4 * 64


def test_self_loops_appended_in_node_order():
    m = _ok(source_index=[2, 1, 0], target_index=[2, 0, 1], add_self_loops=True)
    # (2, 2) exists; (0, 0) and (1, 1) follow the given pairs, ascending
    assert m.source_index.tolist() == [2, 1, 0, 0, 1]
    assert m.target_index.tolist() == [2, 0, 1, 0, 1]


@pytest.mark.parametrize("kw", [
    dict(source_index=[]), dict(source_index=[0, 1]), dict(source_index=[0, 1, 3]),
    dict(target_index=[1, 2, -1]), dict(source_index=[0, 0, 2], target_index=[1, 1, 0]),
    dict(source_index={0, 1, 2}), dict(source_index=[0.0, 1.0, 2.0]),
    dict(source_index=torch.tensor([0.0, 1.0, 2.0])), dict(source_index=[[0, 1, 2]]),
    dict(query_features=0), dict(key_features=True), dict(embed_dim=7), dict(num_heads=3),
    dict(dropout=True), dict(dropout=1.5), dict(dropout=float("nan")), dict(dropout="0.1"),
    dict(bias=1), dict(batch_first=None), dict(add_self_loops=0), dict(kdim=4), dict(vdim=True),
    dict(add_self_loops=True, key_features=4), dict(generator=5),
])
def test_constructor_rejects(kw):
    with pytest.raises(ModuleArgError):
        _ok(**kw)


def test_accepts_numpy_and_tensor_indices():
    a = _ok(source_index=np.array([0, 1, 2], np.int32), target_index=torch.tensor([1, 2, 0]),
            query_features=np.int64(3), kdim=8, vdim=np.int32(8), dropout=0)
    src = np.array([0, 1, 2])
    b = _ok(source_index=src)
    src[0] = 2                      # later writes do not reach the layer
    assert a.source_index.tolist() == b.source_index.tolist() == [0, 1, 2]


def test_reset_parameters_xavier_and_generator():
    g1, g2 = torch.Generator().manual_seed(7), torch.Generator().manual_seed(7)
    a, b = _ok(generator=g1), _ok(generator=g2)
    for x, y in zip(a.parameters(), b.parameters()):
        assert torch.equal(x, y)
    bound = math.sqrt(6.0 / 16)
    for lin in (a.q_proj, a.k_proj, a.v_proj, a.out_proj):
        assert lin.weight.abs().max() <= bound and (lin.bias == 0).all()
    a.reset_parameters(torch.Generator().manual_seed(8))
    assert not torch.equal(a.q_proj.weight, b.q_proj.weight)


def test_from_edgelist_names():
    # the page's feedback-loop example: x feeds a <-> b, which feeds y
    m = PMA.from_edgelist(["x", "a", "b", "a"], ["a", "b", "a", "y"], 8, 2)
    assert m.nodes == ["x", "a", "b", "y"]
    assert (m.query_features, m.key_features, m.nnz) == (4, 4, 4)
    assert m.source_index.tolist() == [0, 1, 2, 1] and m.target_index.tolist() == [1, 2, 1, 3]
    m2 = PMA.from_edgelist(["x", "a"], ["a", "y"], 8, 2, nodes=["y", "a", "x"], add_self_loops=True)
    assert m2.source_index.tolist() == [2, 1, 0, 1, 2]
    with pytest.raises(ModuleArgError):
        PMA.from_edgelist(["x"], ["q"], 8, 2, nodes=["x"])


@pytest.mark.parametrize("call", ["attn_mask", "causal", "nw", "avg", "int", "width", "seq",
                                  "dims", "mask_float", "mask_shape", "train_dropout", "cpu"])
def test_forward_rejects(call):
    m = _ok(dropout=0.1 if call == "train_dropout" else 0.0)
    x = torch.zeros(2, 3, 8)
    kw = {}
    q = k = v = x
    if call == "attn_mask":
        kw["attn_mask"] = torch.zeros(3, 3, dtype=torch.bool)
    elif call == "causal":
        kw["is_causal"] = True
    elif call == "nw":
        kw["need_weights"] = 1
    elif call == "avg":
        kw["average_attn_weights"] = None
    elif call == "int":
        q = k = v = torch.zeros(2, 3, 8, dtype=torch.int32)
    elif call == "width":
        q = k = v = torch.zeros(2, 3, 4)
    elif call == "seq":
        q = torch.zeros(2, 4, 8)
    elif call == "dims":
        q = k = v = torch.zeros(8)
    elif call == "mask_float":
        kw["key_padding_mask"] = torch.zeros(2, 3)
    elif call == "mask_shape":
        kw["key_padding_mask"] = torch.zeros(2, 4, dtype=torch.bool)
    elif call == "train_dropout":
        m.train()
    with pytest.raises(ModuleArgError) as e:
        m(q, k, v, **kw)
    # every case but the last is caught before the device check
    assert ("same GPU" in str(e.value)) == (call == "cpu")


# ---- PackedLinear (CPU: construction and validation only) ----------------
from graph_sparse_head_amd.module import PackedLinear  # noqa: E402


def test_packed_linear_parameters():
    m = PackedLinear([0, 2, 1, 0], [1, 1, 0, 2], 3, 4, generator=torch.Generator().manual_seed(0))
    assert m.weight.shape == (4,) and m.bias.shape == (4,) and m.nnz == 4
    assert m.in_features == 3 and m.out_features == 4
    # weight of an edge into t and bias[t] lie within 1 / sqrt(in-degree of t)
    deg = np.bincount(m.target_index.numpy(), minlength=4)
    bound = 1 / np.sqrt(deg[m.target_index.numpy()])
    assert (np.abs(m.weight.detach().numpy()) <= bound).all()
    assert m.bias[3].item() == 0.0                      # target 3 has no edge
    n = PackedLinear([0, 2, 1, 0], [1, 1, 0, 2], 3, 4, generator=torch.Generator().manual_seed(0))
    assert torch.equal(m.weight, n.weight) and torch.equal(m.bias, n.bias)
    nb = PackedLinear([0], [0], 1, 1, bias=False)
    assert nb.bias is None


def test_packed_linear_self_loops_and_edgelist():
    m = PackedLinear([1], [0], 3, 3, add_self_loops=True)
    assert m.source_index.tolist() == [1, 0, 1, 2] and m.target_index.tolist() == [0, 0, 1, 2]
    e = PackedLinear.from_edgelist(["a", "b"], ["b", "c"])
    assert e.nodes == ["a", "b", "c"] and e.source_index.tolist() == [0, 1]


@pytest.mark.parametrize("kw", [
    dict(source_index=[0, 0], target_index=[1, 1], in_features=2, out_features=2),
    dict(source_index=[2], target_index=[0], in_features=2, out_features=2),
    dict(source_index=[0], target_index=[0], in_features=0, out_features=2),
    dict(source_index=[0], target_index=[0], in_features=2, out_features=3, add_self_loops=True),
    dict(source_index=[0.0], target_index=[0], in_features=2, out_features=2),
    dict(source_index=[0], target_index=[0], in_features=2, out_features=2, bias=1),
])
def test_packed_linear_rejects(kw):
    with pytest.raises(ModuleArgError):
        PackedLinear(**kw)


def test_packed_linear_forward_rejects_cpu_and_width():
    m = PackedLinear([0], [0], 2, 2)
    with pytest.raises(ModuleArgError):
        m(torch.zeros(3, 3))
    with pytest.raises(ModuleArgError):
        m(torch.zeros(3, 2, dtype=torch.int64))
    with pytest.raises(ModuleArgError, match="same GPU"):
        m(torch.zeros(3, 2))
