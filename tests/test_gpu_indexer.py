"""GPU lightning-indexer backward with KL loss vs the fp64 oracle on the same seeded inputs.

Every gradient tensor must satisfy the parity bar of tests.common.compare (rel-L2 <= 5e-3, and
the per-element bound), the loss a relative error of 1e-3.  Cases cover the causal offset with
S1 < S2, no mask with padded batches, varlen TND with an empty sequence, every index-head tile
shape (G = 16, 24, 64) and main-head count up to 128, rope-less calls, fp16, and reproducibility.
"""

import numpy as np
import pytest

from oracle import indexer as ix
from sparse_mla_flash_amd import inputs
from tests.common import compare, from_dev, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "bsnd_n16_g16_causal": (dict(layout="BSND", B=1, S1=100, S2=100, N1=16, G=16, sparse_mode=3), 1),
    "bsnd_n64_g64_s1_lt_s2": (dict(layout="BSND", B=1, S1=40, S2=150, N1=64, G=64, sparse_mode=3), 2),
    "bsnd_n128_g64_nomask_padded": (dict(layout="BSND", B=2, S1=30, S2=70, N1=128, G=64, sparse_mode=0,
                                         seq_q=[30, 17], seq_kv=[70, 33]), 3),
    "tnd_n8_g24_varlen_empty": (dict(layout="TND", B=3, seq_q=[20, 0, 45], seq_kv=[33, 5, 45], N1=8, G=24,
                                     sparse_mode=3), 4),
}


class IxCase:
    def __init__(self, p, rope=True):
        self.p, self.rope = p, rope
        dt = p.dtype
        self.geo = ix.IndexerGeometry(p.layout, p.B, p.S1, p.S2, p.N1, p.G, p.Di, p.D, p.Dr, p.seq_q, p.seq_kv,
                                      p.sparse_mode, p.scale)
        f = lambda x: inputs.bits_to_f64(x, dt)
        self.q, self.k, self.qi, self.ki, self.w = f(p.q), f(p.k), f(p.qi), f(p.ki), f(p.w)
        self.qr = f(p.qr) if rope else np.zeros(p.shape(p.N1, p.Dr))
        self.kr = f(p.kr) if rope else np.zeros(p.shape(1, p.Dr, "k"))
        sm, ss = ix.main_stats(self.geo, self.q, self.k, self.qr, self.kr)
        mi, si = ix.index_stats(self.geo, self.qi, self.ki, self.w)
        # the operator's inputs: fp32 statistics
        self.sm, self.ss = sm.astype(np.float32), ss.astype(np.float32)
        self.mi, self.si = mi.astype(np.float32), si.astype(np.float32)

    def ref(self):
        d = np.float64
        return ix.indexer_grad(self.geo, self.q, self.k, self.qr, self.kr, self.sm.astype(d), self.ss.astype(d),
                               self.qi, self.ki, self.w, self.mi.astype(d), self.si.astype(d))

    def run_gpu(self):
        import sparse_mla_flash_amd as sf
        p, dt = self.p, self.p.dtype
        stat = (p.B, p.N1, p.S1) if p.layout == "BSND" else (p.N1, p.S1)
        istat = (p.B, p.S1) if p.layout == "BSND" else (p.S1,)
        return sf.lightning_indexer_grad_kl_loss(
            to_dev(p.q, dt), to_dev(p.k, dt), to_dev(p.qi, dt), to_dev(p.ki, dt), to_dev(p.w, dt),
            to_dev(self.sm.reshape(stat), "raw"), to_dev(self.ss.reshape(stat), "raw"),
            to_dev(self.mi.reshape(istat), "raw"), to_dev(self.si.reshape(istat), "raw"), p.seq_q, p.seq_kv,
            to_dev(p.qr, dt) if self.rope else None, to_dev(p.kr, dt) if self.rope else None,
            scale_value=p.scale, layout=p.layout, sparse_mode=p.sparse_mode)


def make(name, dtype="bf16"):
    kw, seed = CASES[name]
    p = inputs.indexer_problem(**kw, dtype=dtype, name=name)
    return inputs.indexer_generate(p, seed)


def check(case, outs, label, u=2.0 ** -8, rel_l2=5e-3):
    dqi, dki, dw, loss = outs
    rloss, _, rdqi, rdki, rdw = case.ref()
    p = case.p
    res = {
        "dqi": compare(label + "/dqi", from_dev(dqi), rdqi.reshape(p.shape(p.G, p.Di)), u=u, rel_l2=rel_l2),
        "dki": compare(label + "/dki", from_dev(dki), rdki.reshape(p.shape(1, p.Di, "k")), u=u, rel_l2=rel_l2),
        "dw": compare(label + "/dw", from_dev(dw), rdw.reshape(p.shape(p.G, 1)[:-1]), u=u, rel_l2=rel_l2),
    }
    got = float(from_dev(loss)[0])
    assert abs(got - rloss) <= 1e-3 * abs(rloss) + 1e-4, (label, got, rloss)
    return res, got, rloss


@pytest.mark.parametrize("name", sorted(CASES))
def test_indexer_backward_matches_oracle(name):
    case = IxCase(make(name))
    res, got, rl = check(case, case.run_gpu(), name)
    print(name, {k: f"{v[0]:.2e}/{v[1]:.2e}" for k, v in res.items()}, f"loss {got:.6f} / {rl:.6f}")


def test_indexer_ropeless_matches_oracle():
    case = IxCase(make("bsnd_n16_g16_causal"), rope=False)
    check(case, case.run_gpu(), "ropeless")


def test_indexer_fp16_matches_oracle():
    import torch
    case = IxCase(make("bsnd_n64_g64_s1_lt_s2", dtype="fp16"))
    outs = case.run_gpu()
    assert outs[0].dtype == torch.float16 and outs[2].dtype == torch.float16
    check(case, outs, "fp16", u=2.0 ** -11, rel_l2=1e-3)


def test_indexer_is_bit_reproducible():
    import torch
    case = IxCase(make("tnd_n8_g24_varlen_empty"))
    first = [t.clone() for t in case.run_gpu()]
    for _ in range(3):
        again = case.run_gpu()
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a,
                               b.view(torch.int16) if b.dtype != torch.float32 else b)
