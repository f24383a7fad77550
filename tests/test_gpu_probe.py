"""The read probe (a measurement kernel, not a step of the path) reads every byte of its
buffer: the XOR of its per-workgroup words equals the XOR of the buffer's 32-bit words, for
sizes that leave some waves a partial batch of 1 KB blocks and some none."""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kib", [1, 4095, 4096 * 8 + 5, 131072 + 3])
def test_read_probe_reads_every_word(kib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sparse_06_amd as dsa
    print(f"[case] read probe {kib} KiB", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(kib)
    host = rng.integers(0, 2**32, kib * 256, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((dsa.dsa_read_probe_sink_words(),), -1, dtype=torch.int32, device="cuda")
    dsa.dsa_read_probe(buf, sink)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))
