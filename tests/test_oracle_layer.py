"""Pin for the decode-layer oracle: the same chain written with torch CPU fp64
library routines (rms_norm, linear, scaled_dot_product_attention, silu) and an
unpaged per-request K/V list, rounded to bf16 at the same storage points.  A
wiring mistake (swapped gate/up, a missing residual, a wrong q/k/v slice, a
cache written after attention) moves the logits by O(1) and fails here.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
import synth
from oracle.layer import DenseLayerOracle, LayerDims


def _bf(x: torch.Tensor) -> torch.Tensor:
    """fp64 -> bf16 value (as fp64) through the pinned single-step rounding."""
    return torch.from_numpy(oracle.bf16_to_f64(oracle.round_bf16(x.numpy())))


class TorchLayer:
    def __init__(self, d: LayerDims, w: dict):
        self.d = d
        self.w = {k: v.double() for k, v in w.items()}
        self.cache = {}

    def step(self, tokens, reqs, positions):
        d, w = self.d, self.w
        x = w["embed"][torch.tensor(tokens)]
        a = _bf(F.rms_norm(x, (d.hidden,), w["ln1"], eps=d.eps))
        qkv = _bf(F.linear(a, w["wqkv"]))
        hq, hkv, hd = d.num_q_heads, d.num_kv_heads, d.head_dim
        outs = []
        for b, (r, p) in enumerate(zip(reqs, positions)):
            q = qkv[b, : hq * hd].reshape(hq, hd)
            k = qkv[b, hq * hd:(hq + hkv) * hd].reshape(hkv, hd)
            v = qkv[b, (hq + hkv) * hd:].reshape(hkv, hd)
            ks, vs = self.cache.setdefault(r, ([], []))
            assert len(ks) == p
            ks.append(k)
            vs.append(v)
            K = torch.stack(ks, 1).repeat_interleave(hq // hkv, 0)   # [Hq, L, D]
            V = torch.stack(vs, 1).repeat_interleave(hq // hkv, 0)
            o = F.scaled_dot_product_attention(q[:, None, :], K, V, scale=hd ** -0.5)
            outs.append(o[:, 0, :].reshape(-1))
        o = _bf(torch.stack(outs))
        h = _bf(x + _bf(F.linear(o, w["wo"])))
        a2 = _bf(F.rms_norm(h, (d.hidden,), w["ln2"], eps=d.eps))
        gu = _bf(F.linear(a2, w["wgu"]))
        s = _bf(F.silu(gu[:, : d.intermediate]) * gu[:, d.intermediate:])
        o2 = _bf(h + _bf(F.linear(s, w["wd"])))
        return F.linear(o2, w["lm_head"]).float()


def test_layer_oracle_matches_torch_composition():
    d = LayerDims(hidden=64, num_q_heads=4, num_kv_heads=2, head_dim=16, intermediate=96,
                  vocab=300, page_size=4)
    w = synth.dense_layer_weights(64, 4, 2, 16, 96, 300, seed=1)
    ref = TorchLayer(d, w)
    orc = DenseLayerOracle(d, {k: synth.bf16_bits(v) for k, v in w.items()}, num_pages=64)
    # three requests, pages handed out from a seeded permutation
    perm = synth.page_ids(64, seed=3).numpy()
    tables = {r: perm[r * 16:(r + 1) * 16] for r in range(3)}
    toks = {0: 5, 1: 17, 2: 250}
    pos = {0: 0, 1: 0, 2: 0}
    rng = np.random.default_rng(0)
    for step in range(9):
        reqs = sorted(rng.choice(3, size=rng.integers(1, 4), replace=False).tolist())
        tokens = [toks[r] for r in reqs]
        positions = [pos[r] for r in reqs]
        bt = np.stack([tables[r] for r in reqs]).astype(np.int32)
        lo, to = orc.step(tokens, bt, positions)
        lr = ref.step(tokens, reqs, positions).numpy()
        rms = np.sqrt(np.mean(lr.astype(np.float64) ** 2))
        assert np.abs(lo - lr).max() <= 1e-4 * rms, step
        for i, r in enumerate(reqs):
            toks[r] = int(to[i])
            pos[r] += 1
