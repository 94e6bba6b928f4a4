"""qd_sample_noalloc (no handle, scratch in the library's static device array)
against qd_sample on a handle, through the C ABI: the same sampled ids, bit
for bit (the same kernels run the same arithmetic), on consecutive calls
that share the static scratch, the second with a smaller batch and
vocabulary than the first, then the largest batch; sizes beyond the array's
limits are rejected before any launch."""
import numpy as np
import pytest

from paged_kv_gqa_qwen3_amd import binding, synth
from paged_kv_gqa_qwen3_amd.decoder import Decoder
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on a CPU host)")
    return _t


# temperature, top_k, top_p: greedy, the fast top-k lists, a top-k beyond
# them (alone and with top-p) and top-p beyond the first 64 tokens (the
# multi-workgroup selection), top-p inside the first 64 tokens, no limit
SETTINGS = [(0.0, 0, 1.0), (0.7, 20, 0.95), (1.0, 200, 1.0), (0.3, 0, 0.9),
            (1.0, 0, 0.999), (1.0, 0, 1.0), (0.8, 64, 0.5), (1.3, 1, 1.0),
            (1.1, 500, 0.9)]


def _inputs(torch, B, V, seed):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((B, V)).astype(np.float32) * np.float32(2.0)
    lg[1::4] = np.round(lg[1::4])  # many ties
    st = [SETTINGS[(seed + b) % len(SETTINGS)] for b in range(B)]
    dev = "cuda"
    return (torch.from_numpy(lg).to(dev),
            torch.tensor([s[0] for s in st], dtype=torch.float32, device=dev),
            torch.tensor([s[1] for s in st], dtype=torch.int32, device=dev),
            torch.tensor([s[2] for s in st], dtype=torch.float32, device=dev),
            torch.from_numpy(rng.random(B).astype(np.float32)).to(dev))


def test_noalloc_sample_matches_handle_sample(torch):
    stream = torch.cuda.current_stream().cuda_stream
    for call, (B, V) in enumerate([(16, 151936), (5, 4096), (64, 151936)]):
        say(f"no-alloc sampling call {call}: batch {B}, vocab {V}")
        shape = synth.ModelShape(f"v{V}", 1, 256, 4, 2, 64, 704, V, True)
        dec = Decoder(shape, 64, 4, 8)
        lg, T, k, p, u = _inputs(torch, B, V, 900 + call)
        want = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        got = torch.full((B,), -2, dtype=torch.int32, device="cuda")
        dec.sample(lg, T, k, p, u, want)
        binding.qd_sample_noalloc(B, V, lg, T, k, p, u, got, stream)
        torch.cuda.synchronize()
        w, g = want.cpu().numpy(), got.cpu().numpy()
        assert (w >= 0).all() and (w < V).all()
        np.testing.assert_array_equal(g, w)
        dec.close()


def test_noalloc_sample_rejects_sizes_beyond_its_scratch(torch):
    B, V = 4, 4096
    lg, T, k, p, u = _inputs(torch, B, V, 7)
    out = torch.full((B,), -3, dtype=torch.int32, device="cuda")
    for bad_b, bad_v in ((0, V), (65, V), (B, 262144 + 64), (B, 32)):
        with pytest.raises(binding.QdError):
            binding.qd_sample_noalloc(bad_b, bad_v, lg, T, k, p, u, out)
    with pytest.raises(binding.QdError):
        binding.qd_sample_noalloc(B, V, lg, T, k, p, u, None)
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == -3).all()  # nothing was launched
