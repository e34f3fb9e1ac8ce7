"""GPU pins of the binary32 identities the quantising kernels form without a
division instruction (quant_row_workgroup_amd/csrc/qrw_device.h), swept over
every input in their ranges on the GPU that runs them:

- recip_rn(s): the hardware reciprocal refined by one Newton step must equal
  the correctly rounded 1/s for every binary32 s in [2^-23, 2^120).  Every
  per-token and per-group scale of a finite amax lies there
  (max(amax, 1e-4)/448 >= 2^-22).  Markstein's correction in div_rn gives the
  correctly rounded quotient x/s only when its reciprocal is correctly
  rounded, so the bit-exact codes of the per-token cast ("TileLang tutorial,
  ch. 13", s3.1.5), the KV-cache write and the staged fused form rest on it;
- scale_e4m3(a): the scale RN(a/448) by the same correction must equal the
  correctly rounded quotient for every binary32 a in [2^-14, 2^128);
- the device's own binary32 division 1.0f/s, checked the same way, as a
  control of the sweep's reference.

The reference is the binary32 value nearest to the binary64 quotient, tested
in binary64 (qrw_probe_sweep, include/qrw_probe.h).  A second check draws
random and edge-case inputs, forms both functions on the GPU and compares
them with numpy's IEEE binary32 arithmetic on the host."""
import numpy as np
import pytest
import torch

import quant_row_workgroup_amd as qrw

pytestmark = pytest.mark.gpu

PER_THREAD = 1024
BLOCK = 256


def _bits(x):
    return int(np.float32(x).view(np.uint32))


def _sweep(kind, lo, hi):
    P = qrw.load_probe()
    per_block = BLOCK * PER_THREAD
    blocks = (hi - lo + per_block - 1) // per_block
    counts = torch.full((blocks,), -1, dtype=torch.int32, device="cuda")
    rc = P.qrw_probe_sweep(kind, lo, hi, PER_THREAD, counts.data_ptr(), blocks,
                           torch.cuda.current_stream().cuda_stream)
    assert rc == 0, rc
    torch.cuda.synchronize()
    c = counts.cpu().numpy().astype(np.int64)
    assert (c >= 0).all(), "a workgroup wrote no count"
    return int(c.sum()), hi - lo


@pytest.mark.parametrize("kind,lo,hi,what", [
    (0, _bits(2.0 ** -23), _bits(2.0 ** 120), "recip_rn == RN(1/s), s in [2^-23, 2^120)"),
    (1, _bits(2.0 ** -14), 0x7F800000, "scale_e4m3 == RN(a/448), a in [2^-14, 2^128)"),
    (2, _bits(2.0 ** -23), _bits(2.0 ** 120), "control: 1.0f/s == RN(1/s)"),
])
def test_identity_holds_for_every_input(kind, lo, hi, what):
    print(f"sweep: {what}", flush=True)
    bad, n = _sweep(kind, lo, hi)
    print(f"{what}: {n} inputs, {bad} mismatches", flush=True)
    assert n > 10 ** 9 and bad == 0


def test_against_host_ieee_arithmetic():
    rng = np.random.default_rng(11)
    lo, hi = _bits(2.0 ** -23), _bits(2.0 ** 120)
    bits = rng.integers(lo, hi, size=1 << 22, dtype=np.int64).astype(np.uint32)
    edge = []
    for e in range(-23, 120):
        m = _bits(2.0 ** e)
        edge += [m, m + 1, m + 2, m + 0x7FFFFF - 1, m + 0x7FFFFF, m + 0x400000, m + 0x3FFFFF]
    s = np.concatenate([bits, np.array(edge, dtype=np.uint32)]).view(np.float32)
    st = torch.from_numpy(s).cuda()
    r = torch.empty_like(st)
    sc = torch.empty_like(st)
    P = qrw.load_probe()
    assert P.qrw_probe_recip_values(st.data_ptr(), r.data_ptr(), sc.data_ptr(), st.numel(),
                                    torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    with np.errstate(all="raise"):
        want_r = np.float32(1.0) / s                    # IEEE binary32 division
        want_s = s / np.float32(448.0)
    got_r, got_s = r.cpu().numpy(), sc.cpu().numpy()
    assert np.array_equal(got_r.view(np.uint32), want_r.view(np.uint32))
    big = s >= np.float32(2.0 ** -14)
    assert np.array_equal(got_s[big].view(np.uint32), want_s[big].view(np.uint32))
