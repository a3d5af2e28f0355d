"""gqa_decode_noalloc (the decode entry point whose workspace is the
library's static per-GPU scratch array) against gqa_decode with a caller
workspace: two calls in a row, the second smaller, must give bitwise the
same outputs and lse; sizes beyond the scratch are refused before any
launch.  Collected last so that a failure here hides no other test."""
import sys

import numpy as np
import pytest

import synth
from tests.gpu_cases import bf16_to_torch, cache_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gha_lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import grouped_head_latent_amd as gha
    gha.load_library()
    return gha


def run_both(gha, B, h_q, h_kv, s_q, L_cap, seqlens, d, seed):
    seqlens = np.array(seqlens, dtype=np.int32)
    q = bf16_to_torch(synth.normal_bf16((B, h_q, s_q, d), seed, 1))
    k = bf16_to_torch(cache_bits(B, h_kv, L_cap, d, seqlens, seed, 2))
    v = bf16_to_torch(cache_bits(B, h_kv, L_cap, d, seqlens, seed, 3))
    sl = torch.from_numpy(seqlens).cuda()
    ref, ref_lse = gha.gqa_decode(q, k, v, sl, out_dtype=torch.float32, return_lse=True)
    out = torch.full((B, h_q, s_q, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, h_q, s_q), float("nan"), dtype=torch.float32, device="cuda")
    gha.gqa_decode_noalloc(q, k, v, sl, out=out, lse=lse)
    torch.cuda.synchronize()
    return ref, ref_lse, out, lse


@pytest.mark.parametrize("first,second", [
    # streaming kernel (8 rows per KV head), then a smaller batch
    ((8, 32, 8, 1, 4096, [4096, 1, 3000, 77, 2048, 4000, 129, 1000], 128), (3, 32, 8, 1, 1100, [1, 700, 1100], 128)),
    # register-fed kernel (64 rows per KV head), then a smaller one
    ((3, 32, 1, 2, 2000, [2, 1999, 600], 128), (2, 32, 1, 2, 300, [4, 299], 128)),
    # head dim 64 and s_q = 2, then head dim 128 at batch 1
    ((4, 16, 4, 2, 3000, [2999, 5, 1500, 2000], 64), (1, 8, 2, 1, 200, [150], 128)),
])
def test_noalloc_matches_gqa_decode_twice(gha_lib, first, second):
    for i, case in enumerate((first, second)):
        say(f"noalloc call {i}: B,h_q,h_kv,s_q,L_cap,L,d = {case}")
        ref, ref_lse, out, lse = run_both(gha_lib, *case, seed=41 + i)
        assert torch.equal(out, ref), "outputs differ from gqa_decode"
        assert torch.equal(lse, ref_lse), "lse differs from gqa_decode"


def test_noalloc_refuses_sizes_beyond_its_scratch(gha_lib):
    """The scratch limit is checked on the host: nothing is launched."""
    limit = gha_lib.gqa_decode_noalloc_scratch_bytes()
    say(f"noalloc scratch {limit} bytes")
    assert limit == 16 << 20
    B, h_q, h_kv, s_q, L_cap, d = 64, 64, 64, 1, 256, 128   # 4096 (sequence, KV head) units: 36 MB of partials
    q = torch.zeros((B, h_q, s_q, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, h_kv, L_cap, d), dtype=torch.bfloat16, device="cuda")
    sl = torch.full((B,), L_cap, dtype=torch.int32, device="cuda")
    out = torch.empty((B, h_q, s_q, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gha_lib.GhaError, match="GHA_ERR_WORKSPACE"):
        gha_lib.gqa_decode_noalloc(q, k, k, sl, out=out)
