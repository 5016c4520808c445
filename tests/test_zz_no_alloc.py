"""leyline_splice_noalloc (through the C ABI) against leyline_splice: the same
splices from identical images give identical results, bit for bit, on two
calls in a row, the second with a smaller input."""

import numpy as np
import pytest

from tests import relocation_cases as rc

pytestmark = pytest.mark.gpu


def _image(lay, layers, B, bps, seqs, keys):
    import torch
    n_blocks = len(seqs) * bps + 2
    import kvsynth
    r = kvsynth.rng(*keys, 99)
    perm = r.permutation(n_blocks).astype(np.int32)
    bt = torch.from_numpy(perm[: len(seqs) * bps].reshape(len(seqs), bps)).cuda()
    pf, rp = rc.random_image(lay, layers, n_blocks * B, keys)
    return pf, rp, n_blocks, bt


def _both(lay, layers, B, bps, seqs, keys):
    """Run leyline_splice and leyline_splice_noalloc on copies of one image."""
    import torch
    import rope_rotation_splice_amd as rrs
    pf, rp, n_blocks, bt = _image(lay, layers, B, bps, seqs, keys)
    lens, dirs = [s[0] for s in seqs], [s[1:] for s in seqs]
    stubs_d = []
    for i, (n, s0, s1, rl, m) in enumerate(seqs):
        spf, srp = rc.random_image(lay, layers, rl, keys + (500 + i,))
        tp, tr = rc.rows_to_device(lay, spf, srp)
        stubs_d.append(rrs.Rows(tp, tr))
    results = []
    for fn in (rrs.leyline_splice, rrs.leyline_splice_noalloc):
        cache, keep = rc.to_device(lay, pf, rp, n_blocks, B)
        new_lens, st = fn(cache, bt, lens, dirs, stubs_d)
        torch.cuda.synchronize()
        assert rrs.device_errors() == 0
        results.append((list(new_lens), st, rc.from_device(lay, cache)))
    (la, sa, (pa, ra)), (lb, sb, (pb, rb)) = results
    assert la == lb and sa == sb
    assert np.array_equal(pa.view(np.uint16), pb.view(np.uint16))
    assert np.array_equal(rc.bits(ra), rc.bits(rb))
    # and both match the oracle
    want = rc.check_splice(lay, (pf, rp), (pb, rb), bt.cpu().numpy(), B, lens, dirs,
                           [rc.random_image(lay, layers, s[3], keys + (500 + i,)) for i, s in enumerate(seqs)])
    assert lb == want


def test_noalloc_matches_leyline_splice_twice_second_smaller():
    import rope_rotation_splice_amd as rrs
    from rope_rotation_splice_amd import _abi
    assert _abi.load().kvr_noalloc_scratch_bytes() == 8 << 20
    # first: twelve layers, shifts of -1 and +2 (chains far longer than 64
    # bands): the ticketed mover, whose counters and flags live in the scratch
    seqs = [(3000, 100, 102, 1, 0), (2800, 40, 41, 3, 0), (2500, 7, 600, 12, 0)]
    _both(rc.MLA, 12, 64, 48, seqs, (91,))
    # second, smaller: two layers, one sequence, on the same scratch
    _both(rc.MLA, 2, 16, 64, [(1000, 10, 12, 1, 0)], (92,))


def test_noalloc_rejects_calls_beyond_its_scratch():
    """A call whose ticket flags would not fit the scratch is refused before
    anything is enqueued (KVR_E_SCRATCH), and leaves the image untouched."""
    import torch
    import rope_rotation_splice_amd as rrs
    # Delta = -1 over 65,535 rows: 2,048 ticketed tiles per layer; 1,200
    # layers need 2,457,600 flags (9.4 MiB) in one launch
    n = 1 << 16
    layers = 1200
    c = _abi_cache(layers, n)
    with pytest.raises(rrs.KVRError) as err:
        rrs.leyline_splice_noalloc(c, torch.zeros((1, 1), dtype=torch.int32, device="cuda"), [n], [(1, 2, 0, 0)])
    assert err.value.status == -8


def _abi_cache(layers, n):
    """A cache whose parts are narrow views of one small tensor (never read:
    the call is refused during planning)."""
    import torch
    import rope_rotation_splice_amd as rrs
    pool = torch.zeros((1, 1, n, 576), dtype=torch.bfloat16, device="cuda")
    v = pool.expand(layers, 1, n, 576)
    return rrs.KVCache.mla(v)
