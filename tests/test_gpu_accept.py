"""GPU parity of spec_accept_resample (HIP) against the oracle's accept /
resample rule on the same seeded logits and Philox streams."""
import numpy as np
import pytest
import torch

from oracle.sampling import accept_resample
from gpu_common import MARGIN, i32, say, ws

pytestmark = pytest.mark.gpu


def _case(B, k, V, inv_temp, seed, spread=0.3):
    rng = np.random.default_rng(seed)
    zp = rng.normal(size=(B, k + 1, V)).astype(np.float32) * 2.0
    zq = (zp[:, :k] + spread * rng.normal(size=(B, k, V))).astype(np.float32)
    # drafts: mostly the draft's argmax, sometimes random
    d = np.argmax(zq, axis=-1).astype(np.int32)
    flip = rng.random(size=d.shape) < 0.3
    d[flip] = rng.integers(0, V, size=int(flip.sum()))
    t = rng.integers(0, 5000, size=B).astype(np.int32)
    return zp, zq, d, t


@pytest.mark.parametrize("B,k,V", [(16, 4, 1000), (8, 5, 20000), (4, 0, 3000), (6, 1, 128256), (3, 8, 152064)])
@pytest.mark.parametrize("inv_temp", [0.0, 1.0, 1.0 / 0.7])
def test_accept_resample_matches_oracle(B, k, V, inv_temp):
    from layer_speculative_decoding_amd import api
    say(f"accept B={B} k={k} V={V} invT={inv_temp}")
    invt = float(np.float32(inv_temp))
    seed = 1234 + B * 7 + k
    zp, zq, d, t = _case(B, k, V, invt, seed)
    vt = np.concatenate([np.zeros((B, 1), np.int32), d], axis=1)        # [x_t, d_1..d_k]
    P = torch.tensor(zp, device="cuda")
    Q = torch.tensor(zq, device="cuda") if k > 0 else None
    VT = i32(vt)
    n_acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
    com = torch.zeros(B, k + 1, dtype=torch.int32, device="cuda")
    w = ws(api.spec_accept_workspace_bytes(B, k, V))
    api.spec_accept_resample(B, k, V, P, Q, VT[:, 1:] if k else None, k + 1, i32(t), invt, seed, n_acc, nxt, 1,
                             com, w)
    torch.cuda.synchronize()
    a_g, y_g, c_g = n_acc.cpu().numpy(), nxt.cpu().numpy(), com.cpu().numpy()
    checked = excluded = 0
    for b in range(B):
        a, y, info = accept_resample(zp[b].astype(np.float64), zq[b].astype(np.float64) if k else np.zeros((0, V)),
                                     list(d[b]), int(t[b]), invt, seed, b)
        if min(m for _, _, m in info["margins"]) < MARGIN:
            excluded += 1
            continue
        checked += 1
        assert a_g[b] == a, (b, a_g[b], a)
        assert y_g[b] == y, (b, y_g[b], y)
        assert list(c_g[b, :a + 1]) == list(d[b, :a]) + [y]
    say(f"  checked {checked} excluded {excluded}; accepted {a_g.tolist()}")
    assert checked >= B // 2


@pytest.mark.parametrize("V", [4, 16, 256])
def test_accept_chi2_on_gpu(V):
    """The GPU rule keeps p: the first emitted token of 10^6 independent
    sequences (one launch, one row each) follows p (chi-square), at small
    vocabularies with Dirichlet p and q."""
    from scipy import stats
    from layer_speculative_decoding_amd import api
    B = 1_000_000
    rng = np.random.default_rng(9 + V)
    p = rng.dirichlet(np.full(V, 0.7)) + 1e-3
    q = rng.dirichlet(np.full(V, 0.7)) + 1e-3
    p, q = p / p.sum(), q / q.sum()
    lp = torch.tensor(np.log(p), dtype=torch.float32, device="cuda")
    lq = torch.tensor(np.log(q), dtype=torch.float32, device="cuda")
    # drafts ~ q drawn on the host with an independent generator
    d = rng.choice(V, size=B, p=q).astype(np.int32)
    P = lp.expand(B, 2, V).contiguous()
    Q = lq.expand(B, 1, V).contiguous()
    VT = i32(np.stack([np.zeros(B, np.int32), d], 1))
    n_acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    nxt = torch.zeros(B, dtype=torch.int32, device="cuda")
    w = ws(api.spec_accept_workspace_bytes(B, 1, V))
    api.spec_accept_resample(B, 1, V, P, Q, VT[:, 1:], 2, i32(np.full(B, 40)), 1.0, 77, n_acc, nxt, 1, None, w)
    a = n_acc.cpu().numpy()
    y = nxt.cpu().numpy()
    first = np.where(a == 1, d, y)
    counts = np.bincount(first, minlength=V)
    pv = stats.chisquare(counts, p * B).pvalue
    # the acceptance rate is sum_v min(p, q)
    alpha = float(np.minimum(p, q).sum())
    say(f"  V={V}: chi-square p-value {pv:.3g}, acceptance {a.mean():.4f} (sum min(p, q) = {alpha:.4f})")
    assert pv > 1e-4
    assert abs(a.mean() - alpha) < 5 * np.sqrt(alpha * (1 - alpha) / B)
