"""GPU tests of dit_attn_mfma_ceiling, the matrix-core reference the benchmark
sets the attention kernels against: its products issue back to back (32
shader cycles per 32x32x16 bf16 product, 64 per 32x32x64 e4m3 product, one
wave per SIMD), its rate and clock stay within the card's published peak,
and an undersized record is refused before any launch."""
import pytest
import torch

from parity import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

PEAK = {0: 2516.6, 1: 5033.2}          # dense bf16 / e4m3 TFLOP/s at the 2.4 GHz peak engine clock
CYCLES = {0: 32.0, 1: 64.0}


@pytest.mark.parametrize("dtype", [0, 1])
def test_ceiling_products_issue_back_to_back(dtype):
    import diffusion_transformer_attention_non_amd as dit
    r = dit.mfma_ceiling(dtype, rounds=4000, reps=2)
    say(f"[gpu] mfma ceiling dtype {dtype}: {r}")
    assert CYCLES[dtype] <= r["cycles_per_product"] <= CYCLES[dtype] * 1.02, r
    assert 100.0 < r["clock_mhz"] <= 2450.0, r
    assert 0.05 * PEAK[dtype] < r["tflops"] <= PEAK[dtype] * 1.02, r


def test_ceiling_record_too_small_is_refused():
    import diffusion_transformer_attention_non_amd as dit
    n_wg = torch.cuda.get_device_properties(DEV).multi_processor_count
    rec = torch.full((n_wg * 8,), -7, dtype=torch.int64, device=DEV)
    st, khz = dit.dit_attn_mfma_ceiling(0, 10, n_wg, rec, rec.numel() * 8 - 8,
                                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == dit.DIT_ATTN_EWORKSPACE
    assert (rec == -7).all()
    st, khz = dit.dit_attn_mfma_ceiling(0, 10, 0, rec, rec.numel() * 8, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == dit.DIT_ATTN_OK and khz > 0
    assert (rec.view(-1, 2) > 0).all()
