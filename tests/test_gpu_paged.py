"""The PagedAttention-style comparison baseline vs the fp64 oracle (needs an
MI355X): same attention, computed per beam from a 16-token block-paged cache
(prompt blocks shared by reference, re-read by every beam)."""
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from generative_recommendation_beam_amd import device as dv
from generative_recommendation_beam_amd import xattn
from generative_recommendation_beam_amd.inputs import make_workload
from oracle import attention as oa
from parity import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    xattn.lib()


CASES = {
    "ragged": dict(R=3, B=5, Hq=8, Hkv=2, D=128, prefix_len=[150, 0, 67], unshared_len=[3, 1, 2], T_max=4),
    "aligned": dict(R=2, B=8, Hq=8, Hkv=2, D=128, prefix_len=[256, 64], unshared_len=[2, 3]),
    "d64": dict(R=2, B=6, Hq=4, Hkv=1, D=64, prefix_len=[257, 30], unshared_len=[2, 3]),
    "g8": dict(R=2, B=4, Hq=16, Hkv=2, D=128, prefix_len=[520, 64], unshared_len=[5, 1]),
    "g6": dict(R=1, B=9, Hq=12, Hkv=2, D=128, prefix_len=[131], unshared_len=[2]),
    "long": dict(R=2, B=3, Hq=8, Hkv=2, D=128, prefix_len=[1300, 700], unshared_len=[4, 2]),
    "no_gen": dict(R=2, B=4, Hq=8, Hkv=2, D=128, prefix_len=[200, 90], unshared_len=[0, 0], T_max=2),
    "no_prefix": dict(R=2, B=4, Hq=8, Hkv=2, D=128, prefix_len=[0, 0], unshared_len=[3, 2]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_paged_baseline_matches_oracle(name):
    w = make_workload(name, seed_key=(330, zlib.crc32(name.encode()) % 1000), **CASES[name])
    d = dv.upload(w)
    dv.build_cache(d)
    pc = dv.build_paged(d)
    o = torch.full((d.rows, w.D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((d.rows,), float("nan"), dtype=torch.float32, device="cuda")
    nb = xattn.paged_workspace_size(d.dims, pc.max_seq_len)
    ws = torch.zeros(max(nb, 1), dtype=torch.uint8, device="cuda")
    dv.paged_decode(d, pc, o, lse, ws, nb)
    torch.cuda.synchronize()
    O, L = oa.attention(w)
    compare(o.cpu().numpy().reshape(O.shape), O, lse.cpu().numpy().reshape(L.shape), L, w.dtype,
            f"paged {name}")


def test_paged_copy_blocks_bit_exact():
    w = make_workload("cp", seed_key=(331, 0), **CASES["aligned"])
    d = dv.upload(w)
    dv.build_cache(d)
    pc = dv.build_paged(d)
    before_k = pc.k_cache.clone()
    before_v = pc.v_cache.clone()
    xattn.paged_copy_blocks(d.dims, pc.k_cache, pc.v_cache, pc.parent_tail, pc.spare)
    torch.cuda.synchronize()
    src = pc.parent_tail.long()
    dst = pc.spare.long()
    assert torch.equal(pc.k_cache[dst].view(torch.int16), before_k[src].view(torch.int16))
    assert torch.equal(pc.v_cache[dst].view(torch.int16), before_v[src].view(torch.int16))
    keep = torch.ones(pc.k_cache.shape[0], dtype=torch.bool, device="cuda")
    keep[dst] = False
    assert torch.equal(pc.k_cache[keep].view(torch.int16), before_k[keep].view(torch.int16))
