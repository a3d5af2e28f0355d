"""Host-only checks of the Python binding: every wrapper rejects tensors of
the wrong dtype or on the wrong device before the library is called (so no
kernel ever receives a host pointer or reinterprets fp32 as bf16)."""
import pytest

torch = pytest.importorskip("torch")

import grouped_head_latent_amd as gha  # noqa: E402

bf, f32 = torch.bfloat16, torch.float32


def t(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def sl(B, dtype=torch.int32):
    return torch.ones(B, dtype=dtype)


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not __import__("os").path.exists(gha.library_path()):
        from grouped_head_latent_amd import build
        build.build()
    return gha.load_library()


def test_fp8_decode_requires_bf16_query():
    q = t(1, 8, 1, 128, dtype=f32)
    k = torch.zeros((1, 2, 64, 128), dtype=torch.uint8)
    with pytest.raises(TypeError, match="q has dtype"):
        gha.gqa_decode_fp8(q, k, k, sl(1), k_scale=1.0, v_scale=1.0)


def test_fp8_decode_requires_uint8_codes():
    q = t(1, 8, 1, 128)
    with pytest.raises(TypeError, match="E4M3"):
        gha.gqa_decode_fp8(q, t(1, 2, 64, 128), t(1, 2, 64, 128), sl(1), k_scale=1.0, v_scale=1.0)


@pytest.mark.parametrize("call", [
    lambda: gha.gqa_prefill(t(1, 8, 16, 64), t(1, 2, 16, 64, dtype=f32), t(1, 2, 16, 64)),
    lambda: gha.gqa_decode(t(1, 8, 1, 128), t(1, 2, 64, 128), t(1, 2, 64, 128, dtype=torch.float16), sl(1)),
    lambda: gha.gqa_decode_paged(t(1, 8, 1, 128), t(1, 2, 64, 128, dtype=f32), t(1, 2, 64, 128), sl(1)),
    lambda: gha.gta_shared_score_prefill(t(1, 4, 16, 64), t(1, 4, 16, 64), t(1, 16, 16, 64, dtype=f32)),
    lambda: gha.gta_shared_score_decode(t(1, 4, 1, 64), t(1, 4, 64, 64, dtype=f32), t(1, 16, 64, 64), sl(1)),
    lambda: gha.gqla_gqa_decode(t(1, 16, 1, 128), t(1, 16, 1, 64), t(1, 2, 64, 128), t(1, 64, 64, dtype=f32),
                                t(1, 2, 64, 128), sl(1), scale=0.07),
    lambda: gha.gqla_gqa_prefill(t(1, 16, 8, 128), t(1, 16, 8, 64), t(1, 2, 8, 128), t(1, 8, 64),
                                 t(1, 2, 8, 128, dtype=f32), scale=0.07),
    lambda: gha.latent_absorb_decode(t(1, 1, 16, 512), t(1, 1, 16, 64), t(1, 64, 512, dtype=f32), t(1, 64, 64),
                                     sl(1), scale=0.07),
    lambda: gha.gqla_absorb_decode(t(1, 1, 16, 128), t(1, 1, 16, 64), t(256, 512, dtype=f32), t(256, 512),
                                   t(1, 64, 512), t(1, 64, 64), sl(1), g=2, scale=0.07),
])
def test_inputs_must_share_the_query_dtype(call):
    with pytest.raises(TypeError, match="has dtype"):
        call()


@pytest.mark.parametrize("call", [
    lambda: gha.gqa_decode(t(1, 8, 1, 128), t(1, 2, 64, 128), t(1, 2, 64, 128), sl(1, torch.int64)),
    lambda: gha.gta_shared_score_decode(t(1, 4, 1, 64), t(1, 4, 64, 64), t(1, 16, 64, 64), sl(1, torch.int64)),
    lambda: gha.latent_absorb_decode(t(1, 1, 16, 512), t(1, 1, 16, 64), t(1, 64, 512), t(1, 64, 64),
                                     sl(1, torch.int64), scale=0.07),
])
def test_lengths_must_be_int32(call):
    with pytest.raises(TypeError, match="int32"):
        call()


def test_block_table_must_be_int32():
    with pytest.raises(TypeError, match="block_table"):
        gha.gqa_decode_paged(t(1, 8, 1, 128), t(4, 2, 32, 128), t(4, 2, 32, 128), sl(1),
                             block_table=torch.zeros((1, 4), dtype=torch.int64), page_size=32)


@pytest.mark.parametrize("bad", [torch.float16, torch.float64])
def test_output_must_be_bf16_or_fp32(bad):
    with pytest.raises(TypeError):
        gha.gqa_prefill(t(1, 8, 16, 64), t(1, 2, 16, 64), t(1, 2, 16, 64), out_dtype=bad)
    with pytest.raises(TypeError):
        gha.gqa_decode(t(1, 8, 1, 128), t(1, 2, 64, 128), t(1, 2, 64, 128), sl(1), out=t(1, 8, 1, 128, dtype=bad))


@pytest.mark.parametrize("call", [
    lambda: gha.gqa_prefill(t(1, 8, 16, 64), t(1, 2, 16, 64), t(1, 2, 16, 64)),
    lambda: gha.gqa_decode(t(1, 8, 1, 128), t(1, 2, 64, 128), t(1, 2, 64, 128), sl(1)),
    lambda: gha.gqa_decode_fp8(t(1, 8, 1, 128), torch.zeros((1, 2, 64, 128), dtype=torch.uint8),
                               torch.zeros((1, 2, 64, 128), dtype=torch.uint8), sl(1), k_scale=1.0, v_scale=1.0),
    lambda: gha.gta_shared_score_prefill(t(1, 4, 16, 64), t(1, 4, 16, 64), t(1, 16, 16, 64)),
    lambda: gha.latent_absorb_decode(t(1, 1, 16, 512), t(1, 1, 16, 64), t(1, 64, 512), t(1, 64, 64), sl(1),
                                     scale=0.07),
])
def test_host_tensors_are_rejected(call):
    """CPU tensors never reach the library (their pointers are host memory)."""
    with pytest.raises(ValueError, match="GPU"):
        call()
