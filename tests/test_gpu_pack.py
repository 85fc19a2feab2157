"""GPU: the tiled expert-weight layout written by dg_pack_experts.

The expected layout is built here with plain tensor reshapes from its
definition in include/dg.h (16-row by TK-column tiles, slice l holding row
l % 16 and columns (l // 16) * TK/4 ..), independently of the kernel's index
arithmetic, and compared byte for byte; the error paths are checked too."""
import pytest
import torch

from diffusion_decoding_amd import _lib

pytestmark = pytest.mark.gpu


def expected_tiled(w: torch.Tensor, tk: int) -> torch.Tensor:
    n, rows, cols = w.shape
    v = w.reshape(n, rows // 16, 16, cols // tk, 4, tk // 4)    # [n][rb][r][kt][q][j]
    return v.permute(0, 1, 3, 4, 2, 5).contiguous().reshape(n, rows, cols)  # [n][rb][kt][q][r][j]


@pytest.fixture(scope="module")
def rt():
    from diffusion_decoding_amd import runtime
    _lib.load()
    return runtime


@pytest.mark.parametrize("dtype,n,rows,cols,tk", [
    ("bf16", 3, 48, 96, 32),
    ("bf16", 2, 1408, 2048, 32),
    ("fp8", 3, 32, 128, 64),
    ("fp8", 2, 64, 96, 32),      # cols % 64 == 32: 32-column fp8 tiles
    ("fp8", 2, 2048, 704, 64),
])
def test_pack_layout(rt, dtype, n, rows, cols, tk):
    print(f"pack {dtype} n={n} rows={rows} cols={cols}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(rows * 7 + cols)
    if dtype == "bf16":
        w = torch.randn(n, rows, cols, generator=g).to(torch.bfloat16).cuda()
        wbits = w.view(torch.int16)
    else:
        w = torch.randint(0, 256, (n, rows, cols), generator=g, dtype=torch.uint8).cuda()
        wbits = w
    out = rt.pack_experts(w, dtype)
    torch.cuda.synchronize()
    obits = out.view(torch.int16) if dtype == "bf16" else out
    assert torch.equal(obits.cpu(), expected_tiled(wbits.cpu(), tk))


def test_pack_rejects_bad_shapes(rt):
    w = torch.zeros(1, 24, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.DGError):
        rt.pack_experts(w, "bf16")                       # rows % 16 != 0
    w = torch.zeros(1, 32, 48, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.DGError):
        rt.pack_experts(w, "bf16")                       # cols % 32 != 0
    w = torch.zeros(1, 32, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.DGError):                    # in place: src and dst overlap
        _lib.dg_pack_experts(w.data_ptr(), w.data_ptr(), 1, 32, 64, _lib.DG_DTYPE_BF16, None)
