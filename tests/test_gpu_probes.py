"""The measurement kernels bench.py times: the plain streaming read reads every
16-byte granule of the buffer once in each variant and grid (checked through
its per-workgroup sums), and the empty kernel launches."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant", ["contig4", "contig8", "interleave4", "interleave8",
                                     "interleave16", "contig4-nt", "contig8-nt", "interleave4-nt",
                                     "interleave8-nt", "interleave16-nt"])
def test_read_probe_reads_every_granule_once(gpu, variant):
    import torch
    import context_lookup_drafting_amd as lcd
    dev = torch.device("cuda:0")
    rng = np.random.Generator(np.random.PCG64(91))
    words = rng.integers(-2**31, 2**31, 300_004, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(words).to(dev)
    for nbytes in (16, 16 * 1001, words.nbytes):
        g = words[: nbytes // 4].reshape(-1, 4).astype(np.int64)
        want = int((((g[:, 0] ^ g[:, 1]) + (g[:, 2] ^ g[:, 3])).sum()) % 2**32)
        for blocks in (1, 7, 1024, 8192):
            out = torch.zeros(blocks, dtype=torch.int32, device=dev)
            lcd.read_probe(buf, nbytes, blocks, out, variant=variant)
            got = int(out.cpu().numpy().astype(np.int64).sum()) % 2**32
            assert got == want, (variant, nbytes, blocks)


def test_empty_probe_and_probe_argument_checks(gpu):
    import torch
    import context_lookup_drafting_amd as lcd
    dev = torch.device("cuda:0")
    lcd.empty_probe(256, dev)
    torch.cuda.synchronize()
    buf = torch.zeros(64, dtype=torch.int32, device=dev)
    out = torch.zeros(4, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        lcd.read_probe(buf, 512, 4, out)          # past the buffer
    with pytest.raises(lcd.LCDError):
        lcd.read_probe(buf, 24, 4, out)           # not a whole number of granules
