"""The measurement probes (libkvq_probe.so) read and copy what they claim."""

import pytest
import torch

from _gpu_common import note

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


def test_copy_is_exact():
    from decode_attention_quant_amd import probe
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    for n in (16, 1024, 4096 + 48, (1 << 20) + 16 * 5):
        note("probe copy", n)
        src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=g)
        dst = torch.zeros(n + 256, dtype=torch.uint8, device="cuda")
        probe.copy(dst, src)
        torch.cuda.synchronize()
        assert torch.equal(dst[:n], src) and int(dst[n:].sum()) == 0


@pytest.mark.parametrize("nontemporal", [False, True])
@pytest.mark.parametrize("chunks,where", [(1, 0), (5, 4), (64, 37), (4096 + 3, 4096 + 2)])
def test_read_reaches_every_chunk(chunks, where, nontemporal):
    """A lane whose 16 bytes fold to the marker writes the sink, so placing
    the marker in one chunk shows that chunk was read (the last chunks of a
    size that is not a multiple of four take the kernel's remainder path)."""
    from decode_attention_quant_amd import probe
    note("probe read", chunks, where, "nt" if nontemporal else "plain")
    buf = torch.zeros(chunks * 256, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    probe.read(buf, sink, nontemporal=nontemporal)
    torch.cuda.synchronize()
    assert int(sink[0]) == 0
    buf[where * 256 + 4 * 9] = torch.tensor(MAGIC, dtype=torch.int64).to(torch.int32)  # lane 9's first word
    probe.read(buf, sink, nontemporal=nontemporal)
    torch.cuda.synchronize()
    assert int(sink[0]) & 0xFFFFFFFF == MAGIC
