"""The library's probe bits against rocRAND's open-source Philox4x32-10 engine, an
implementation independent of both the library and the oracle.  Three routes to the bits
are checked: the packed planes of zo_gen_probes, the signs zo_perturb regenerates inline
(theta = 0, alpha = 1 gives theta = z), and the signs zo_update regenerates inline (theta =
0, weights one-hot at probe k, eta = -1 gives theta = z_k).  Offsets put the Philox block
index above 2^32, where the high counter word is in play."""
import numpy as np
import pytest
import torch

import forward_only_amd as zo
import rocrand_ref

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not rocrand_ref.available(), reason="rocRAND header not installed")]

CASES = [(0, 0, 0, 0, 4096 + 77),
         (0x243F6A8885A308D3, 9, 3, 128 * 4099, 50_000),
         (2**64 - 1, 2**32 - 1, 200, 128 * ((1 << 32) + 11), 9_000)]


def _signs(plane, n):
    bits = np.unpackbits(plane, bitorder="little")[:n]
    return np.where(bits == 1, 1.0, -1.0).astype(np.float32)


@pytest.mark.parametrize("seed,step,probe,offset,n", CASES)
def test_planes_match_rocrand(seed, step, probe, offset, n):
    print(f"[rocrand] planes seed={seed} step={step} probe={probe} offset={offset} n={n}",
          flush=True)
    ctx = zo.zo_init(seed)
    got = zo.zo_gen_probes(ctx, step, probe, 4, offset, n).cpu().numpy()
    ctx.close()
    for p in range(4):
        assert np.array_equal(got[p], rocrand_ref.plane(seed, step, probe + p, offset, n)), p


@pytest.mark.parametrize("seed,step,probe,offset,n", CASES)
def test_inline_perturb_signs_match_rocrand(seed, step, probe, offset, n):
    print(f"[rocrand] perturb seed={seed} offset={offset} n={n}", flush=True)
    ctx = zo.zo_init(seed)
    t = torch.zeros(n, dtype=torch.float32, device="cuda")
    zo.zo_perturb(ctx, t, offset, step, probe, 1.0)
    got = t.cpu().numpy()
    ctx.close()
    assert np.array_equal(got, _signs(rocrand_ref.plane(seed, step, probe, offset, n), n))


@pytest.mark.parametrize("seed,step,probe,offset,n", CASES)
def test_inline_update_signs_match_rocrand(seed, step, probe, offset, n):
    print(f"[rocrand] update seed={seed} offset={offset} n={n}", flush=True)
    npert = 16
    k = probe % npert
    ctx = zo.zo_init(seed)
    t = torch.zeros(n, dtype=torch.float32, device="cuda")
    c = torch.zeros(npert, dtype=torch.float32, device="cuda")
    c[k] = 1.0
    zo.zo_update(ctx, t, offset, step, c, -1.0)
    got = t.cpu().numpy()
    ctx.close()
    assert np.array_equal(got, _signs(rocrand_ref.plane(seed, step, k, offset, n), n))
