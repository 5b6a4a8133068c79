"""The measurement kernels behind the bench's measured ceilings: the stream copy moves every
byte (also in place, and for a size that leaves a partial last workgroup), and the bf16
matrix-core loop returns the same finite result on every call."""
import pytest

pytestmark = pytest.mark.gpu


def test_stream_copy_moves_every_byte(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    print("\n[gpu-case] gdn_mb_stream: 3 MiB + 48 bytes, copy and in place", flush=True)
    n = (3 << 20) + 48
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    gdn.gdn_mb_stream(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    keep = src.clone()
    gdn.gdn_mb_stream(src, src)
    torch.cuda.synchronize()
    assert torch.equal(src, keep)


def test_mfma_loop_is_deterministic(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    print("\n[gpu-case] gdn_mb_mfma_bf16: 64 workgroups x 32 iterations, twice", flush=True)
    a = torch.empty(64, dtype=torch.float32, device="cuda")
    b = torch.empty(64, dtype=torch.float32, device="cuda")
    flops = gdn.gdn_mb_mfma_bf16(a, 32)
    gdn.gdn_mb_mfma_bf16(b, 32)
    torch.cuda.synchronize()
    assert flops == 64 * 4 * 32 * 4 * 32768
    assert torch.isfinite(a).all() and torch.equal(a, b)
    assert (a != 0).any()
