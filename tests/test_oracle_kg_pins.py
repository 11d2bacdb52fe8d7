"""Pins for the oracle's kernel-generation transformer.

Each block is pinned to torch's own decoder layer (post-norm, ReLU, dropout
off, batch-first, float64) loaded with the same weights, with and without a
key padding mask. Beside that: the softmax and the LayerNorm are checked
against library routines, the mask token against a NaN fill of the rows it
replaces, padding-invariance, and the channels-last layout against the
channels-first one. A slip in the norm order, the head split, the score
scale, a swapped q/k/v slice or a mask applied to the wrong axis fails one
of them.
"""
import numpy as np
import pytest
import scipy.special
import torch

import gkdsynth
from oracle import kg as okg

C, F, NB = 128, 192, 2


def torch_layers(weights, C, F, nb):
    mask_token, blocks = okg.unpack(weights, C, F, nb)
    layers = []
    for b in blocks:
        L = torch.nn.TransformerDecoderLayer(C, C // 64, F, dropout=0.0, activation="relu",
                                             batch_first=True, norm_first=False).double().eval()
        sd = {
            "self_attn.in_proj_weight": b["sa_in_w"], "self_attn.in_proj_bias": b["sa_in_b"],
            "self_attn.out_proj.weight": b["sa_out_w"], "self_attn.out_proj.bias": b["sa_out_b"],
            "multihead_attn.in_proj_weight": b["ca_in_w"],
            "multihead_attn.in_proj_bias": b["ca_in_b"],
            "multihead_attn.out_proj.weight": b["ca_out_w"],
            "multihead_attn.out_proj.bias": b["ca_out_b"],
            "linear1.weight": b["ff1_w"], "linear1.bias": b["ff1_b"],
            "linear2.weight": b["ff2_w"], "linear2.bias": b["ff2_b"],
            "norm1.weight": b["ln1_w"], "norm1.bias": b["ln1_b"],
            "norm2.weight": b["ln2_w"], "norm2.bias": b["ln2_b"],
            "norm3.weight": b["ln3_w"], "norm3.bias": b["ln3_b"],
        }
        L.load_state_dict({k: torch.from_numpy(np.ascontiguousarray(v)) for k, v in sd.items()})
        layers.append(L)
    return mask_token, layers


def inputs(seed, B, R, HW, p_vis=0.7, p_txt=0.6):
    rng = np.random.default_rng(seed)
    vis = rng.standard_normal((B, R, C))
    txt = rng.standard_normal((B, R, C))
    mv = rng.random((B, R)) < p_vis
    mt = rng.random((B, R)) < p_txt
    mv[:, 0] = True
    q = rng.standard_normal((B, C, HW))
    return vis, mv, txt, mt, q


def torch_reference(vis, mv, txt, mt, q, weights):
    mask_token, layers = torch_layers(weights, C, F, NB)
    B, R, _ = vis.shape
    x = np.concatenate([np.where(mv[..., None], vis, mask_token),
                        np.where(mt[..., None], txt, mask_token)], axis=1)
    pad = ~np.concatenate([mv | mt, mv | mt], axis=1)
    xt = torch.from_numpy(x)
    mem = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1)))
    with torch.no_grad():
        for L in layers:
            xt = L(xt, mem, tgt_key_padding_mask=torch.from_numpy(pad))
    return xt.numpy()


def test_kg_matches_torch_decoder_layers_all_rows_prompted():
    w = gkdsynth.kg_weights(C, F, NB, seed=1).astype(np.float64)
    vis, mv, txt, mt, q = inputs(2, B=2, R=6, HW=20, p_vis=1.0, p_txt=1.0)
    got = okg.kg_transformer(vis, mv, txt, mt, q.reshape(2, C, 4, 5), w, NB, F)
    want = torch_reference(vis, mv, txt, mt, q, w)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-10)


def test_kg_matches_torch_with_mask_tokens_and_padding():
    w = gkdsynth.kg_weights(C, F, NB, seed=3).astype(np.float64)
    vis, mv, txt, mt, q = inputs(4, B=3, R=7, HW=12)
    mv[1, 4:] = mt[1, 4:] = False          # padding rows
    got = okg.kg_transformer(vis, mv, txt, mt, q.reshape(3, C, 3, 4), w, NB, F)
    want = torch_reference(vis, mv, txt, mt, q, w)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-10)


def test_kg_masked_prototypes_are_never_read():
    w = gkdsynth.kg_weights(C, F, NB, seed=5).astype(np.float64)
    vis, mv, txt, mt, q = inputs(6, B=2, R=5, HW=9)
    ref = okg.kg_transformer(vis, mv, txt, mt, q.reshape(2, C, 3, 3), w, NB, F)
    vis2, txt2 = vis.copy(), txt.copy()
    vis2[~mv] = np.nan
    txt2[~mt] = np.nan
    got = okg.kg_transformer(vis2, mv, txt2, mt, q.reshape(2, C, 3, 3), w, NB, F)
    np.testing.assert_array_equal(got, ref)


def test_kg_padding_rows_do_not_change_prompted_rows():
    w = gkdsynth.kg_weights(C, F, NB, seed=7).astype(np.float64)
    vis, mv, txt, mt, q = inputs(8, B=1, R=4, HW=6)
    base = okg.kg_transformer(vis, mv, txt, mt, q.reshape(1, C, 2, 3), w, NB, F)
    R2 = 9
    vis2 = np.concatenate([vis, np.ones((1, R2 - 4, C))], axis=1)
    txt2 = np.concatenate([txt, np.ones((1, R2 - 4, C))], axis=1)
    mv2 = np.concatenate([mv, np.zeros((1, R2 - 4), bool)], axis=1)
    mt2 = np.concatenate([mt, np.zeros((1, R2 - 4), bool)], axis=1)
    got = okg.kg_transformer(vis2, mv2, txt2, mt2, q.reshape(1, C, 2, 3), w, NB, F)
    ok = mv[0] | mt[0]
    np.testing.assert_allclose(got[0, :4][ok], base[0, :4][ok], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[0, R2:R2 + 4][ok], base[0, 4:8][ok], rtol=0, atol=1e-12)


def test_kg_crop_without_prompts_is_finite_and_token_layout_agrees():
    w = gkdsynth.kg_weights(C, F, NB, seed=9).astype(np.float64)
    vis, mv, txt, mt, q = inputs(10, B=2, R=3, HW=8)
    mv[1] = mt[1] = False
    a = okg.kg_transformer(vis, mv, txt, mt, q.reshape(2, C, 2, 4), w, NB, F)
    b = okg.kg_transformer(vis, mv, txt, mt, q.transpose(0, 2, 1), w, NB, F, tokens=True)
    assert np.all(np.isfinite(a))
    np.testing.assert_array_equal(a, b)
    # every slot of the unprompted crop starts as the mask token and sees the
    # same (empty) SA keys, so all its rows agree
    np.testing.assert_allclose(a[1], np.broadcast_to(a[1, 0], a[1].shape), rtol=0, atol=1e-12)


def test_kg_softmax_and_layer_norm_match_library_routines():
    rng = np.random.default_rng(11)
    s = rng.standard_normal((5, 17)) * 4
    ok = rng.random(17) < 0.6
    ok[3] = True
    want = np.zeros_like(s)
    want[:, ok] = scipy.special.softmax(s[:, ok], axis=1)
    np.testing.assert_allclose(okg.softmax_rows(s, ok[None]), want, rtol=0, atol=1e-15)
    assert np.all(okg.softmax_rows(s, np.zeros((1, 17), bool)) == 0)
    x = rng.standard_normal((6, 40)) * 3 + 1
    g, b = rng.standard_normal(40), rng.standard_normal(40)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (40,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5).numpy()
    np.testing.assert_allclose(okg.layer_norm(x, g, b), ref, rtol=0, atol=1e-12)


def test_kg_weight_layout_size_and_rejects():
    w = gkdsynth.kg_weights(C, F, NB, seed=0)
    assert w.size == C + NB * okg.block_size(C, F)
    with pytest.raises(ValueError):
        okg.unpack(w[:-1], C, F, NB)
