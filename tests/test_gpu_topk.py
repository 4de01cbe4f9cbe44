"""Beam-search survivor selection on the GPU vs the oracle, bit-exact
(needs an MI355X). Pools of 128x128 to 512x512 candidates per request, plus
ragged shapes, exact ties, masked (-inf) tails, more survivors than beams,
and all-equal pools (which take the kernel's block-merge path)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from generative_recommendation_beam_amd import xattn
from generative_recommendation_beam_amd.inputs import make_topk
from oracle import beam_topk as bt

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    xattn.lib()


def run(x):
    dev = "cuda"
    bs = torch.from_numpy(x.beam_score).to(dev)
    lp = torch.from_numpy(x.logprob).to(dev)
    tk = torch.from_numpy(x.token).to(dev)
    parent = torch.full((x.R, x.n_out), -7, dtype=torch.int32, device=dev)
    tok = torch.full((x.R, x.n_out), -7, dtype=torch.int32, device=dev)
    score = torch.full((x.R, x.n_out), float("nan"), dtype=torch.float32, device=dev)
    xattn.beam_topk(bs, lp, tk, x.n_out, parent, tok, score)
    torch.cuda.synchronize()
    return parent.cpu().numpy(), tok.cpu().numpy(), score.cpu().numpy()


def check(x):
    p, t, s = run(x)
    P, T, S = bt.select(x.beam_score, x.logprob, x.token, x.n_out)
    assert np.array_equal(p, P), f"{x.name}: parents differ at {np.argwhere(p != P)[:5].tolist()}"
    assert np.array_equal(t, T)
    assert np.array_equal(s.view(np.uint32), S.view(np.uint32))


@pytest.mark.parametrize("dist", ["softmax", "ties", "masked"])
@pytest.mark.parametrize("R,BW,K", [(8, 128, 128), (4, 256, 256), (2, 512, 512)])
def test_topk_pools(dist, R, BW, K):
    check(make_topk(f"pool{BW}", R=R, BW=BW, K=K, seed_key=(400, BW, K), dist=dist))


@pytest.mark.parametrize("R,BW,K,n_out", [(3, 100, 37, 100), (2, 64, 64, 200), (5, 33, 1, 33),
                                          (1, 7, 5, 35), (2, 300, 9, 150), (1, 1, 64, 16),
                                          # n_out <= 128: seed samples and survivors in 1 to 8 runs of 128
                                          (2, 300, 40, 100), (1, 1024, 4, 128), (3, 64, 128, 128),
                                          (2, 50, 50, 1), (2, 200, 16, 127)])
def test_topk_ragged(R, BW, K, n_out):
    check(make_topk("ragged", R=R, BW=BW, K=K, n_out=n_out, seed_key=(401, BW, K, n_out), vocab=256))


@pytest.mark.parametrize("BW,K", [(128, 128), (512, 512)])
def test_topk_all_equal_takes_exact_merge_path(BW, K):
    check(make_topk("equal", R=2, BW=BW, K=K, seed_key=(402, BW), dist="equal"))


def test_topk_more_survivors_than_fit():
    """n_out above the beam count: no seed bound, the whole pool survives the
    walk (16384 candidates > the 8192 LDS keys), so the block merge runs."""
    check(make_topk("big", R=2, BW=128, K=128, n_out=1000, seed_key=(403, 0), dist="masked"))


def test_topk_deterministic():
    x = make_topk("det", R=4, BW=256, K=256, seed_key=(404, 0), dist="ties")
    a = run(x)
    b = run(x)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32))
