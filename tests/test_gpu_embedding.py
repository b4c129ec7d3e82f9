"""GPU parity of nf4_embedding_rows (selected-row decode of a packed table)
against the oracle: the decoded rows must equal the oracle's rows bit for bit
(Aner docs "Native model adaptation and NF4": embeddings decode only the
selected rows, on the device)."""
import numpy as np
import pytest
import torch

import workloads
from tests.parity import bits

pytestmark = pytest.mark.gpu


def _ids(V: int, T: int, seed: int) -> np.ndarray:
    """Seeded token ids with the first and last row and a repeat included."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, V, size=T, dtype=np.int64)
    if T >= 3:
        ids[0], ids[1], ids[2] = V - 1, 0, ids[T // 2]
    return ids


def _case(gpu, orc, V, D, T, dq, seed):
    W = workloads.weight_with_outliers((V, D), seed=seed)
    ref = orc.quantize(W.numpy(), dq)
    E = gpu.quantize(W.cuda(), dq)
    ids = _ids(V, T, seed)
    idt = torch.from_numpy(ids).cuda()
    status = torch.full((1,), 777, dtype=torch.int32, device="cuda")
    out_f = gpu.embedding_rows(E, idt, torch.float32, status=status)
    out_b = gpu.embedding_rows(E, idt, torch.bfloat16)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    np.testing.assert_array_equal(bits(out_f), orc.embedding_rows(ref, D, ids, "f32").view(np.uint32))
    np.testing.assert_array_equal(bits(out_b), orc.embedding_rows(ref, D, ids, "bf16"))


@pytest.mark.parametrize("dq", [True, False])
def test_smollm2_tied_table(gpu, orc, dq):
    """The tied 49152 x 576 embedding of the SmolLM2 stack, 512 tokens."""
    print(f"[embed] 49152x576 dq={dq}", flush=True)
    _case(gpu, orc, 49152, 576, 512, dq, seed=49152)


@pytest.mark.parametrize("V,D,T", [(300, 77, 100), (1000, 8, 3000), (17, 64, 5), (1, 24, 4), (40, 1, 9),
                                   (3, 5, 7)])
@pytest.mark.parametrize("dq", [True, False])
def test_ragged_tables(gpu, orc, V, D, T, dq):
    """Row widths that are not multiples of 8 (element-wise form), blocks that
    straddle rows, one-row and one-column tables."""
    print(f"[embed] V={V} D={D} T={T} dq={dq}", flush=True)
    _case(gpu, orc, V, D, T, dq, seed=V * 131 + D)


def test_out_of_range_ids_give_zero_rows_and_status(gpu, orc):
    V, D = 50, 128
    W = workloads.weight_with_outliers((V, D), seed=5)
    ref = orc.quantize(W.numpy(), True)
    E = gpu.quantize(W.cuda(), True)
    ids = torch.tensor([-1, V, 3, 2 ** 40, V - 1], dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = gpu.embedding_rows(E, ids, torch.float32, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == -1  # NF4_EINVAL
    o = out.cpu().numpy()
    assert not o[[0, 1, 3]].any()
    np.testing.assert_array_equal(o[[2, 4]], orc.embedding_rows(ref, D, [3, V - 1], "f32"))
    # a later valid call resets the status word
    gpu.embedding_rows(E, ids[2:3], torch.float32, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0


def test_no_tokens(gpu):
    E = gpu.quantize(workloads.normal_f32((10, 64), 0.02, 1, "cuda"), True)
    status = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    out = gpu.embedding_rows(E, torch.zeros(0, dtype=torch.int64, device="cuda"), status=status)
    torch.cuda.synchronize()
    assert out.shape == (0, 64) and int(status.item()) == 0


def test_rows_match_full_dequantize_at_llama_vocab_width(gpu):
    """A 32000 x 4096 table (the Llama vocabulary width), 4096 tokens: the rows
    equal the same rows of nf4_dequantize bit for bit (the oracle covers the
    arithmetic on the smaller tables above)."""
    V, D = 32000, 4096
    W = workloads.normal_f32((V, D), 0.02, 777, "cuda")
    E = gpu.quantize(W, True)
    del W
    ids = torch.from_numpy(_ids(V, 4096, 3)).cuda()
    rows = gpu.embedding_rows(E, ids, torch.bfloat16)
    full = gpu.dequantize(E, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(rows.view(torch.int16), full[ids].view(torch.int16))
