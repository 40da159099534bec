"""GPU parity of pose retrieval with full SO(3) rotations (WorldKV Sec. 5.1:
squared-L2 translation + geodesic rotation, each min-max normalised) against
the oracle.

Both sides evaluate the same float64 operation sequence except atan2, whose
last bit may differ between the device and host libraries: distances agree
to 1e-12 and retrieved sets are equal outside a 1e-12 band around the k-th
distance (band sizes printed); planted exact ties resolve to the lower index.
"""
import numpy as np
import pytest
import torch

import wkv_synth as S
from oracle import wkv_oracle as O
from tests.parity import gpu_ready, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


def bank(seed, M):
    g = torch.Generator().manual_seed(seed)
    P = torch.zeros((M, 8), dtype=torch.float32)
    P[:, :3] = torch.cumsum(0.5 * torch.randn((M, 3), generator=g), 0)
    P[:, 3:7] = torch.randn((M, 4), generator=g)
    return P


def check(w, P, q, k, label):
    say("pose_so3", label, P.shape[0], k)
    idx, dist = w.wkv_pose_topk_so3(P.to("cuda:0"), q, k)
    torch.cuda.synchronize()
    o_idx, o_d = O.pose_topk_so3(P.numpy(), np.asarray(q, np.float32), k)
    M = P.shape[0]
    k_eff = min(k, M)
    srt = np.sort(o_d)
    band = set()
    if k_eff < M:
        thr = 0.5 * (srt[k_eff - 1] + srt[k_eff])
        band = set(np.nonzero(np.abs(o_d - thr) <= 1e-12)[0].tolist())
    g = idx.cpu().numpy()
    assert len(g) == k_eff and np.all(np.diff(g) > 0)
    assert (set(g.tolist()) - band) == (set(o_idx.tolist()) - band), label
    assert np.max(np.abs(dist.cpu().numpy() - o_d[g])) <= 1e-12
    print(f"  {label}: band {len(band)}", flush=True)


@pytest.mark.parametrize("M,k", [(8, 2), (20, 3), (120, 6), (1000, 4), (8192, 17), (5, 9)])
def test_random_banks(w, M, k):
    P = bank(M, M)
    q = bank(M + 1, 1)[0].tolist()
    check(w, P, q, k, f"random M={M}")


def test_ties_identity_query_and_degenerate_rotation(w):
    P = bank(3, 64)
    P[40] = P[12]                                       # exact tie: 12 wins
    P[41] = P[12]
    check(w, P, P[12].tolist(), 1, "tie")
    idx, _ = w.wkv_pose_topk_so3(P.to("cuda:0"), P[12].tolist(), 1)
    assert idx.cpu().tolist() == [12]
    R = P.clone()
    R[:, 3:7] = torch.tensor([0.3, -0.1, 0.2, 0.9])    # every rotation equal: the term is 0
    check(w, R, R[5].tolist(), 4, "equal rotations")
    Z = P.clone()
    Z[:, 4:6] = 0.0                                     # rotations about z only
    check(w, Z, Z[7].tolist(), 5, "z rotations")


def test_yaw_walk_as_quaternions(w):
    """The 1.3B-class pose walk, its yaw turned into z-axis quaternions."""
    walk = S.pose_walk(2, 23)
    P = torch.zeros((20, 8), dtype=torch.float32)
    P[:, :3] = walk[1:21, :3]
    P[:, 3] = torch.cos(walk[1:21, 3].double() / 2).float()
    P[:, 6] = torch.sin(walk[1:21, 3].double() / 2).float()
    qy = walk[22]
    q = [float(qy[0]), float(qy[1]), float(qy[2]), float(np.cos(float(qy[3]) / 2)), 0.0, 0.0,
         float(np.sin(float(qy[3]) / 2))]
    check(w, P, q, 3, "yaw walk")
