"""GPU parity of qlora_linear_ce (output head + cross-entropy, chunked over
tokens) against the oracle's float64 definition.

Seeded inputs: hidden states X ~ N(0, 1) bf16 [T, D] (a normalised hidden
state), head W ~ N(0, (2/sqrt(D))^2) bf16 [V, D] (logits of standard deviation
about 2, so the softmax is neither flat nor one-hot), targets uniform over the
V classes, with every 7th token set to the ignore value in some cases.

Cases: every small case is compared in full (per-token losses, the mean loss
and dX): ragged chunks and token tiles, V that is not a multiple of the
256-column tile, a vocabulary-split dX product (few tokens, V = 32000), the
loss alone without dX, every target ignored, and no tokens.  The full-size
case (T = 4096 tokens, D = 4096, V = 128256, the page's vocabulary) is checked
on 24 sampled tokens (their per-token losses and dX rows against the oracle
run on those tokens alone, its dX rescaled from their count to the count of
all tokens with a target), and its mean loss against the oracle's loss over
all 4096 tokens (computed in token chunks, loss only).  The confident regime
of late training is covered by logits of standard deviation about 10 with
every target the largest logit (mean loss well below 0.5), where the loss is
the small difference of two large numbers.

Bars: the logits are fp32 (fp32 accumulation of exact bf16 products) and
(softmax - onehot)/n is rounded to bf16 before the dX product, so the
per-token losses and the loss are held to 1e-3 (relative), dX to the 1e-2
relative Frobenius bar of every floating-point output.  Two calls give
identical bits.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import linear_ce as olc

from gpu_util import bf16_dev, f64_host, rel_fro

pytestmark = pytest.mark.gpu

q = pytest.importorskip("qlora_fine_tuning_linear_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.load_library()


def _inputs(T, D, V, seed, every, logit_std=2.0):
    X = synth.normal_bf16(seed, 50, T * D).reshape(T, D)
    W = synth.normal_bf16(seed, 51, V * D, 0.0, logit_std / np.sqrt(D)).reshape(V, D)
    t = synth.targets(seed, 52, T, V, ignore_every=every)
    return X, W, t


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# (name, T, D, V, chunk, ignore_every, want_dx)
CASES = [
    ("t5_d64_v128", 5, 64, 128, 4, 0, True),
    ("t300_d128_v960_ign", 300, 128, 960, 128, 7, True),
    ("t257_d256_v2048_ign", 257, 256, 2048, 100, 7, True),
    ("t1024_d512_v4096", 1024, 512, 4096, 512, 0, True),
    ("t64_d4096_v32000_split", 64, 4096, 32000, 64, 0, True),
    ("t600_d256_v3072_loss_only", 600, 256, 3072, 256, 5, False),
]


@pytest.mark.parametrize("name,T,D,V,chunk,every,want_dx", CASES, ids=[c[0] for c in CASES])
def test_linear_ce_matches_oracle(name, T, D, V, chunk, every, want_dx):
    print("case", name, flush=True)
    X, W, t = _inputs(T, D, V, 4000 + T + V, every)
    Xd, Wd = bf16_dev(X), bf16_dev(W)
    td = torch.from_numpy(t).cuda()
    loss, tl, dX = q.qlora_linear_ce(Xd, Wd, td, chunk=chunk, want_dx=want_dx, want_token_loss=True)
    torch.cuda.synchronize()
    lr, tlr, dXr = olc.linear_ce(X, W, t, want_grad=want_dx)
    assert _rel(tl.cpu().numpy(), tlr) <= 1e-3
    assert abs(loss.item() - lr) <= 1e-3 * abs(lr)
    if want_dx:
        assert rel_fro(dX, dXr) <= 1e-2
        ign = t == olc.IGNORE_INDEX
        if ign.any():
            assert torch.count_nonzero(dX[torch.from_numpy(ign).cuda()]).item() == 0
    else:
        assert dX is None
    # reproducible to the bit
    loss2, tl2, dX2 = q.qlora_linear_ce(Xd, Wd, td, chunk=chunk, want_dx=want_dx, want_token_loss=True)
    assert torch.equal(loss.view(torch.int32), loss2.view(torch.int32))
    assert torch.equal(tl.view(torch.int32), tl2.view(torch.int32))
    if want_dx:
        assert torch.equal(dX.view(torch.int16), dX2.view(torch.int16))


@pytest.mark.parametrize("T,D,V,chunk", [(300, 256, 2048, 128), (96, 1024, 32000, 64)])
def test_linear_ce_confident_regime(T, D, V, chunk):
    """Large logits (standard deviation about 10) with every target the
    largest logit: the per-token losses are small differences of large
    numbers, log-sum-exp minus the target logit."""
    print("case confident T=%d D=%d V=%d" % (T, D, V), flush=True)
    X, W, _ = _inputs(T, D, V, 4300 + V, 0, logit_std=10.0)
    from oracle.qlora import as_f64
    Z = as_f64(X) @ as_f64(W).T
    t = Z.argmax(axis=1).astype(np.int32)
    lr, tlr, dXr = olc.linear_ce(X, W, t)
    assert lr < 0.5, lr  # the regime this case is for
    Xd, Wd = bf16_dev(X), bf16_dev(W)
    loss, tl, dX = q.qlora_linear_ce(Xd, Wd, torch.from_numpy(t).cuda(), chunk=chunk, want_token_loss=True)
    torch.cuda.synchronize()
    assert _rel(tl.cpu().numpy(), tlr) <= 1e-3, _rel(tl.cpu().numpy(), tlr)
    assert abs(loss.item() - lr) <= 1e-3 * abs(lr), (loss.item(), lr)
    assert rel_fro(dX, dXr) <= 1e-2, rel_fro(dX, dXr)


def test_linear_ce_all_ignored_and_empty():
    T, D, V = 40, 64, 192
    X, W, _ = _inputs(T, D, V, 4100, 0)
    Xd, Wd = bf16_dev(X), bf16_dev(W)
    td = torch.full((T,), olc.IGNORE_INDEX, dtype=torch.int32, device="cuda")
    loss, tl, dX = q.qlora_linear_ce(Xd, Wd, td, chunk=16, want_token_loss=True)
    assert loss.item() == 0.0
    assert torch.count_nonzero(tl).item() == 0 and torch.count_nonzero(dX).item() == 0
    e = torch.empty(0, D, dtype=torch.bfloat16, device="cuda")
    loss0, _, dX0 = q.qlora_linear_ce(e, Wd, torch.empty(0, dtype=torch.int32, device="cuda"))
    assert loss0.item() == 0.0 and dX0.shape == (0, D)


def test_linear_ce_full_size_sampled():
    T, D, V, chunk = 4096, 4096, 128256, 1024
    print("case full size", flush=True)
    X, W, t = _inputs(T, D, V, 4200, 11)
    Xd, Wd = bf16_dev(X), bf16_dev(W)
    td = torch.from_numpy(t).cuda()
    loss, tl, dX = q.qlora_linear_ce(Xd, Wd, td, chunk=chunk, want_token_loss=True)
    torch.cuda.synchronize()
    tl_h = tl.cpu().numpy().astype(np.float64)
    valid = t != olc.IGNORE_INDEX
    n = int(valid.sum())
    # the loss against the oracle's over every token (loss only, in chunks of
    # tokens: the per-token terms do not depend on the other tokens)
    tl_ref = np.concatenate([olc.linear_ce(X[c:c + 256], W, t[c:c + 256], want_grad=False)[1]
                             for c in range(0, T, 256)])
    loss_ref = tl_ref.sum() / n
    assert abs(loss.item() - loss_ref) <= 1e-3 * abs(loss_ref), (loss.item(), loss_ref)
    rng = np.random.default_rng(7)
    idx = np.sort(rng.choice(T, 24, replace=False))
    lr, tlr, dXr = olc.linear_ce(X[idx], W, t[idx])
    ns = int((t[idx] != olc.IGNORE_INDEX).sum())
    assert _rel(tl_h[idx], tlr) <= 1e-3
    dX_s = f64_host(dX)[idx]
    ref = dXr * (ns / n)
    assert np.linalg.norm(dX_s - ref) <= 1e-2 * np.linalg.norm(ref)
