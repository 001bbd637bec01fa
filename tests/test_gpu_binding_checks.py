"""The binding refuses bad tensor arguments before any kernel is launched:
a host tensor beside device data, and buffers shorter than the call needs
(the C ABI receives bare pointers and cannot check either)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_entry_points_refuse_host_and_short_tensors(device):
    import fp4_rollout_guided_amd as tr
    rows, cols = 8, 64
    n = rows * cols
    x = torch.randn(rows, cols, device=device).to(torch.bfloat16)
    ts = tr.tensor_scale(x)
    sc, bt, cd = tr.capture(x, ts, want_codes=True)
    host_ts = ts.cpu()
    short = lambda t: t[:-1]
    with pytest.raises(ValueError, match="must be on"):
        tr.capture(x, host_ts)
    with pytest.raises(ValueError, match="must be on"):
        tr.guided_fakequant_fwd(x, sc, host_ts, bt)
    with pytest.raises(ValueError, match="at least"):
        tr.guided_fakequant_fwd(x, short(sc), ts, bt)
    with pytest.raises(ValueError, match="at least"):
        tr.guided_fakequant_fwd(x, sc, ts, short(bt))
    with pytest.raises(ValueError, match="at least"):
        tr.full_info_fakequant_fwd(x, sc, ts, short(cd))
    with pytest.raises(ValueError, match="at least"):
        tr.rne_fakequant_fwd(x, sc, ts, y=torch.empty(n - 8, dtype=torch.bfloat16, device=device))
    with pytest.raises(ValueError, match="at least"):
        tr.rne_fakequant_fwd(x, sc, ts, mask=torch.empty(n // 8 - 1, dtype=torch.uint8, device=device))
    _, m, _ = tr.guided_fakequant_fwd(x, sc, ts, bt)
    with pytest.raises(ValueError, match="at least"):
        tr.ste_bwd(x, short(m))
    with pytest.raises(ValueError, match="must be on"):
        tr.ste_bwd(x, m.cpu())
    with pytest.raises(ValueError, match="at least"):
        tr.ste_bwd(x, m, grad_in=torch.empty(n - 8, dtype=torch.bfloat16, device=device))
    with pytest.raises(ValueError, match="must be on"):
        tr.tensor_scale(x, out=torch.empty(1))
    offsets = torch.tensor([0, 3, rows], dtype=torch.int64, device=device)
    gts = tr.grouped_tensor_scale(x, offsets)
    with pytest.raises(ValueError, match="at least"):
        tr.grouped_capture(x, offsets, short(gts))
    with pytest.raises(ValueError, match="must be on"):
        tr.grouped_capture(x, offsets.cpu(), gts)
    with pytest.raises(ValueError, match="at least"):
        tr.lowbits_fakequant_fwd(x, sc, ts, 3, bt)          # one plane where three are needed
    with pytest.raises(ValueError, match="at least"):
        tr.mx_guided_fakequant_fwd(x, torch.zeros(n // 32 - 1, dtype=torch.uint8, device=device), bt)
    with pytest.raises(ValueError, match="at least"):
        tr.mx8_full_info_fakequant_fwd(x, torch.zeros(n // 32, dtype=torch.uint8, device=device), cd)
    with pytest.raises(ValueError, match="at least"):
        tr.gather_records(short(bt), sc, None, cols, torch.zeros(2, dtype=torch.int64, device=device))
    with pytest.raises(ValueError, match="must be on"):
        tr.capture_batch([x], [host_ts])
    with pytest.raises(ValueError, match="at least"):
        tr.mismatch_stats(x, sc, ts, bt, short(cd))
    # forwards on records read back in place: the source's row count comes
    # from the scale bytes, and every other record plane must cover it
    idx = torch.arange(rows, dtype=torch.int64, device=device)
    with pytest.raises(ValueError, match="at least"):
        tr.gathered_guided_fakequant_fwd(x, idx, sc, ts, short(bt))
    with pytest.raises(ValueError, match="at least"):
        tr.gathered_full_info_fakequant_fwd(x, idx, sc, ts, short(cd))
    with pytest.raises(ValueError, match="one entry per row"):
        tr.gathered_guided_fakequant_fwd(x, torch.cat([idx, idx[:1]]), sc, ts, bt)
    with pytest.raises(ValueError, match="at least"):
        tr.gathered_guided_fakequant_fwd(x, idx[:-1], sc, ts, bt)
    with pytest.raises(ValueError, match="must be on"):
        tr.gathered_guided_fakequant_fwd(x, idx.cpu(), sc, ts, bt)
    with pytest.raises(ValueError, match="must be on"):
        tr.gathered_guided_fakequant_fwd(x, idx, sc, host_ts, bt)
    with pytest.raises(ValueError, match="at least"):
        tr.gathered_guided_fakequant_fwd(x, idx, sc, short(gts), bt, offsets=offsets)
    with pytest.raises(ValueError, match="must be on"):
        tr.gathered_guided_fakequant_fwd(x, idx, sc, gts, bt, offsets=offsets.cpu())
    with pytest.raises(ValueError, match="at least"):
        tr.gathered_guided_fakequant_fwd(x, idx, sc, ts, bt, mask=torch.empty(n // 8 - 1, dtype=torch.uint8,
                                                                              device=device))
    with pytest.raises(ValueError, match="must be on"):
        tr.gathered_rne_fakequant_fwd(x, idx, sc, host_ts)
    with pytest.raises(ValueError, match="at least"):
        tr.gathered_rne_fakequant_fwd(x, idx, sc, short(gts), offsets=offsets)
    torch.cuda.synchronize()
