"""The memory-ceiling probes (measurement only) compute what include/engram_probe.h says.

Every byte of the test buffer is 0x38: as an FP8 E4M3 code that is exactly
1.0, as an E8M0 byte in the records probe it becomes 2^-7, and four of them
read as an fp32 scale give the value below.  So each probe output has a
closed form.
"""
import numpy as np
import pytest
import torch

from gpu_support import lib

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def test_copy_reproduces_the_source_and_read_leaves_the_sink():
    _say("probe copy and read, 8 MiB")
    hg = lib()
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    src = torch.randint(0, 256, (8 << 20,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    hg.probe_copy(src, dst)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    hg.probe_read(torch.zeros(8 << 20, dtype=torch.uint8, device="cuda"), sink)
    hg.probe_random(torch.zeros(8 << 20, dtype=torch.uint8, device="cuda"), 512, 1 << 20, sink)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    assert int(sink.item()) == 0  # the xor of zeros never matches the sink's trigger value


@pytest.mark.parametrize("layout", ["rows_only", "separate_f32", "inline_f32_260", "inline_e8m0_264"])
def test_records_sum_has_its_closed_form(layout):
    _say(f"probe records, {layout}")
    hg = lib()
    buf = torch.full((4 << 20,), 0x38, dtype=torch.uint8, device="cuda")
    out = torch.full((1000, 2, 256), float("nan"), dtype=torch.float32, device="cuda")
    hg.probe_records(buf, layout, out, seed=11)
    torch.cuda.synchronize()
    if layout == "rows_only":
        expect = np.float32(24.0)
    elif layout == "inline_e8m0_264":
        expect = np.float32(24 * 2.0 ** -7)
    else:
        s = np.frombuffer(bytes([0x38] * 4), dtype=np.float32)[0]
        acc = np.float32(0)
        for _ in range(24):
            acc = np.float32(acc + s)  # 1.0 * s is exact, so each fused multiply-add is one rounded add
        expect = acc
    got = out.cpu().numpy()
    assert np.all(got == expect), (layout, float(expect), np.unique(got)[:5])
