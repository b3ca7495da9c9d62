"""GPU regression test of the direct global -> LDS loads' base address.

Those loads take a wave-uniform 64-bit base that the kernels rebuild from two
32-bit halves.  Widening the low half as a signed value once sign-extended a
low half with bit 31 set over the high half and faulted the GPU.  Here every
buffer of a forward and a backward (Q, K, V, O, LSE, dO, dQ, dK, dV and the
backward workspace) lies at an address whose low 32 bits have bit 31 set,
and the results must equal those of ordinarily allocated buffers bit for
bit.  All addresses stay inside one allocation, so every access is in
bounds."""

import pytest
import torch

from exact_io_aware_55_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LOW = 0x80001000          # low 32 bits of the first placed buffer: bit 31 set


def placed(pool, cursor, shape, dtype):
    """A contiguous tensor carved from ``pool`` at byte offset cursor[0]
    (256-byte aligned); advances the cursor."""
    nbytes = 1
    for s in shape:
        nbytes *= s
    nbytes *= torch.empty((), dtype=dtype).element_size()
    off = cursor[0]
    cursor[0] = (off + nbytes + 255) // 256 * 256
    return pool[off:off + nbytes].view(dtype).view(shape)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_buffers_with_address_bit31_set(gpu_lib, d, causal):
    B, N, H = 1, 700, 2
    print(f"\n[addresses] d={d} causal={causal}", flush=True)
    x = inputs.make_qkv(B, N, H, d, torch.bfloat16, seed=90 + d, with_do=True)
    ws_bytes = gpu_lib.bwd_workspace_size(B, H, N, d)
    elem = B * N * H * d * 2
    total = 9 * (elem + 256) + 2 * (B * H * N * 4 + 256) + ws_bytes + 256
    # room to reach the next address whose low 32 bits equal LOW, plus the buffers
    pool = torch.empty((1 << 32) + total, dtype=torch.uint8, device=DEV)
    base = pool.data_ptr()
    start = (LOW - (base & 0xFFFFFFFF)) % (1 << 32)
    assert start + total <= pool.numel()
    cur = [start]
    shape = (B, N, H, d)
    q, k, v, do = (placed(pool, cur, shape, torch.bfloat16) for _ in range(4))
    for t, n in zip((q, k, v, do), ("q", "k", "v", "do")):
        t.copy_(x[n].to(DEV))
    o = placed(pool, cur, shape, torch.bfloat16)
    lse = placed(pool, cur, (B, H, N), torch.float32)
    dq, dk, dv = (placed(pool, cur, shape, torch.bfloat16) for _ in range(3))
    ws = placed(pool, cur, (ws_bytes,), torch.uint8)
    for t in (q, k, v, do, o, lse, dq, dk, dv, ws):
        a = t.data_ptr()
        assert a & 0x80000000 and a % 256 == 0 and pool.data_ptr() <= a < pool.data_ptr() + pool.numel()
    gpu_lib.forward(q, k, v, causal=causal, out=o, lse=lse)
    gpu_lib.backward(q, k, v, o, do, lse, causal=causal, workspace=ws, out=(dq, dk, dv))
    steps, _ = gpu_lib.backward_steps(q, k, v, o, do, lse, causal=causal, workspace=ws,
                                      preprocess=True)
    # the same computation on ordinarily allocated buffers
    qr, kr, vr, dor = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    o2, lse2 = gpu_lib.forward(qr, kr, vr, causal=causal)
    g2 = gpu_lib.backward(qr, kr, vr, o2, dor, lse2, causal=causal)
    steps2, _ = gpu_lib.backward_steps(qr, kr, vr, o2, dor, lse2, causal=causal, preprocess=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b in zip((dq, dk, dv) + tuple(steps), tuple(g2) + tuple(steps2)):
        assert torch.equal(a, b)
