"""The measurement probes behind the achievable-peak figures: the streaming
read touches every byte exactly once (the XOR of its per-thread words equals
the XOR of the whole buffer), and the MFMA probe is deterministic with the
operation count it reports."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_bytes,n_wg", [(16, 1), (4096 * 16 + 48, 3), (1 << 24, 64), ((1 << 22) + 16 * 7, 4096)])
def test_read_probe_reads_every_word_once(gpu_lib, n_bytes, n_wg):
    import torch
    from head_latent_attention_cache_amd import api
    print(f"[case] read probe {n_bytes} B over {n_wg} work-groups", flush=True)
    g = torch.Generator(device="cpu").manual_seed(n_bytes)
    host = torch.randint(-2**31, 2**31 - 1, (n_bytes // 4,), generator=g, dtype=torch.int64).to(torch.int32)
    src = host.cuda()
    out = torch.empty(n_wg * 256, dtype=torch.int32, device="cuda")
    assert api.probe_hbm_read(src, n_wg, out) == n_bytes
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("toggle", [False, True])
def test_mfma_probe_count_and_determinism(gpu_lib, toggle):
    import torch
    from head_latent_attention_cache_amd import api
    print("[case] MFMA probe", flush=True)
    n_wg, iters = 8, 10
    a = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    flops = api.probe_mfma(n_wg, iters, a, toggle)
    assert flops == n_wg * 4 * iters * 16 * 2 * 32 * 32 * 16
    api.probe_mfma(n_wg, iters, b, toggle)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all() and torch.equal(a, b) and a.abs().sum() > 0
