"""GPU check of the QK same-traffic copy probe (qrw_probe_copy_qk_traffic,
include/qrw_probe.h) that the benchmark times beside the per-head QK RMSNorm +
RoPE operators: on arbitrary 16-bit patterns it must read and write exactly
the bytes its header states (the operators' loads and stores, with byte
selection in place of arithmetic), compared here bit for bit with the same
selection written out in numpy.  A probe that skipped a load or a store
would report a ceiling for less traffic than the operator moves."""
import ctypes

import numpy as np
import pytest
import torch

import quant_row_workgroup_amd as qrw

pytestmark = pytest.mark.gpu

ROW = 6144            # 32 + 8 + 8 heads of 128 channels
QG, KG = 512, 128     # granules of the q heads, of the k heads (and of the v heads)


def _u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _expected(x, wq, wk, c, s, slots, num_slots, kv):
    """x: [T, 6144] uint16 before the call; returns (x after, k cache, v cache,
    k scales, v scales) as the header defines them (caches start as 0xA5 bytes,
    scales as 0xFFFFFFFF words, and keep them where nothing is written)."""
    T = x.shape[0]
    xo = x.copy()
    kc = np.full((num_slots, 1024), 0xA5, np.uint8)
    vc = kc.copy()
    ks = np.full((num_slots, 8), 0xFFFFFFFF, np.uint32)
    vs = ks.copy()
    gr = x.reshape(T, 768, 8)
    for t in range(T):
        for gi in range(QG + KG + (KG if kv else 0)):
            j = gi % 16
            cs = c[t, 8 * (j % 8):8 * (j % 8) + 8] ^ s[t, 8 * (j % 8):8 * (j % 8) + 8]
            if gi < QG or (not kv and gi < QG + KG):
                w = wq if gi < QG else wk
                xo[t, 8 * gi:8 * gi + 8] = gr[t, gi] ^ w[8 * j:8 * j + 8] ^ cs
                continue
            slot = slots[t]
            if not 0 <= slot < num_slots:
                continue
            is_v = gi >= QG + KG
            hg = gi - (QG + KG if is_v else QG)
            m = cs if is_v else (wk[8 * j:8 * j + 8] ^ cs)
            (vc if is_v else kc)[slot, 8 * hg:8 * hg + 8] = ((gr[t, gi] ^ m) >> 8).astype(np.uint8)
            if j == 0:
                word = int(gr[t, gi, 0]) | (int(gr[t, gi, 1]) << 16)
                (vs if is_v else ks)[slot, hg // 16] = word & 0x3FFFFFFF
    return xo, kc, vc, ks, vs


@pytest.mark.parametrize("kv", [0, 1])
@pytest.mark.parametrize("tokens", [1, 37])
def test_qk_probe_moves_the_stated_bytes(kv, tokens):
    P = qrw.load_probe()
    g = torch.Generator().manual_seed(1000 + 10 * tokens + kv)
    rnd = lambda *shape: torch.randint(-32768, 32768, shape, generator=g, dtype=torch.int32).to(
        torch.int16)
    x = rnd(tokens, ROW)
    wq, wk = rnd(128), rnd(128)
    c, s = rnd(tokens, 64), rnd(tokens, 64)
    num_slots = 2 * tokens + 3
    slots = torch.randperm(num_slots, generator=g)[:tokens].to(torch.int64)
    if tokens > 4:
        slots[1] = -1               # skipped, as in the operator
        slots[3] = num_slots        # out of range: skipped
    dev = [t.cuda() for t in (x, wq, wk, c, s, slots)]
    kc = torch.full((num_slots, 1024), 0xA5, dtype=torch.uint8, device="cuda")
    vc = kc.clone()
    ks = torch.full((num_slots, 8), -1, dtype=torch.int32, device="cuda")
    vs = ks.clone()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    print(f"qrw_probe_copy_qk_traffic kv={kv} tokens={tokens}", flush=True)
    rc = P.qrw_probe_copy_qk_traffic(p(dev[0]), p(dev[1]), p(dev[2]), p(dev[3]), p(dev[4]),
                                     p(kc), p(vc), p(ks), p(vs), p(dev[5]), num_slots, tokens, kv,
                                     None)
    assert rc == 0
    torch.cuda.synchronize()
    exp = _expected(_u16(x), _u16(wq), _u16(wk), _u16(c), _u16(s), slots.numpy(), num_slots, kv)
    np.testing.assert_array_equal(_u16(dev[0]), exp[0])
    if kv:
        np.testing.assert_array_equal(kc.cpu().numpy(), exp[1])
        np.testing.assert_array_equal(vc.cpu().numpy(), exp[2])
        np.testing.assert_array_equal(ks.cpu().numpy().view(np.uint32), exp[3])
        np.testing.assert_array_equal(vs.cpu().numpy().view(np.uint32), exp[4])
    else:  # the caches are not touched
        assert bool((kc == 0xA5).all()) and bool((ks == -1).all())
