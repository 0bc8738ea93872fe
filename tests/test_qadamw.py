"""GPU parity of the AdamW state codec ("Full-Stack FP4 ...", section 2.2,
Q-AdamW) with the oracle: nvfp4_qadamw_encode's two views (codes, block
scales, tensor scales) and BF16 block means, and nvfp4_qadamw_decode's FP32
moments, all bit-exact, from tiny to the full 20480 x 5120 state."""
import numpy as np
import pytest
import torch

import bit_block_scaled_nvfp4_amd as nv
from bit_block_scaled_nvfp4_amd import workloads as W
from oracle import oracle as O

from .parity import DEV, assert_quant_equal, to_oracle_view

pytestmark = pytest.mark.gpu


def _moments(rows, cols, seed):
    d = W.adamw_state(seed=seed, rows=rows, cols=cols)
    return d["m"], d["v"]


def _gpu_state_host(st: nv.QAdamWState) -> O.QAdamWState:
    return O.QAdamWState(to_oracle_view(st.m), to_oracle_view(st.v),
                         st.v_means.cpu().numpy().view(np.uint16).reshape(st.m.rows, st.m.cols // 16))


def _check(m, v, rht_seed, sr_seed, sr_stream, got: nv.QAdamWState, m_out, v_out, what):
    want = O.qadamw_encode(m.numpy(), v.numpy(), rht_seed, sr_seed, sr_stream)
    host = _gpu_state_host(got)
    assert_quant_equal(host.m, want.m, f"{what}: m")
    assert_quant_equal(host.v, want.v, f"{what}: v")
    np.testing.assert_array_equal(host.v_means, want.v_means, err_msg=f"{what}: means")
    wm, wv = O.qadamw_decode(want, rht_seed)
    gm, gv = m_out.cpu().numpy(), v_out.cpu().numpy()
    for g, w, name in ((gm, wm, "m"), (gv, wv, "v")):
        bad = np.flatnonzero(g.view(np.uint32) != w.view(np.uint32))
        assert bad.size == 0, f"{what}: decoded {name} differs at {bad.size} elements, first {bad[:5]}"


@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (17, 80), (64, 1024), (130, 4112)])
def test_qadamw_encode_decode_match_oracle(rows, cols):
    m, v = _moments(rows, cols, rows + cols)
    st = nv.qadamw_encode(m.to(DEV), v.to(DEV), 0x1234, 0x5678, 3)
    gm, gv = nv.qadamw_decode(st, 0x1234)
    torch.cuda.synchronize()
    _check(m, v, 0x1234, 0x5678, 3, st, gm, gv, f"{rows}x{cols}")


def test_qadamw_strided_rows_and_reuse():
    rows, cols = 40, 96
    m, v = _moments(rows, cols, 9)
    bm = torch.zeros(rows, 128)
    bv = torch.zeros(rows, 128)
    bm[:, :cols], bv[:, :cols] = m, v
    dm, dv = bm.to(DEV), bv.to(DEV)
    ws = nv.new_workspace(nv.nvfp4_qadamw_workspace_size(), DEV)
    st = nv.QAdamWState.empty(rows, cols, DEV)
    om = torch.full((rows, 128), 7.0, device=DEV)
    ov = torch.full((rows, 128), 7.0, device=DEV)
    for k in range(2):  # the same workspace and state twice
        nv.qadamw_encode(dm[:, :cols], dv[:, :cols], 77, 78 + k, state=st, workspace=ws)
        nv.qadamw_decode(st, 77, om[:, :cols], ov[:, :cols])
        torch.cuda.synchronize()
        _check(m, v, 77, 78 + k, 0, st, om[:, :cols], ov[:, :cols], f"strided, call {k}")
    assert (om[:, cols:] == 7.0).all() and (ov[:, cols:] == 7.0).all()


def test_qadamw_zero_and_empty():
    z = torch.zeros(8, 32, device=DEV)
    st = nv.qadamw_encode(z, z, 1, 2)
    gm, gv = nv.qadamw_decode(st, 1)
    torch.cuda.synchronize()
    assert st.m.tensor_scale.item() == 0 and st.v.tensor_scale.item() == 0
    assert (gm == 0).all() and (gv == 0).all()
    _check(z.cpu(), z.cpu(), 1, 2, 0, st, gm, gv, "zeros")
    e = torch.zeros(0, 32, device=DEV)
    st = nv.qadamw_encode(e, e, 1, 2)
    gm, gv = nv.qadamw_decode(st, 1)
    torch.cuda.synchronize()
    assert gm.shape == (0, 32) and st.m.tensor_scale.item() == 0


def test_qadamw_full_size():
    """The 20480 x 5120 state, compared in full."""
    d = W.adamw_state()
    m, v = d["m"], d["v"]
    st = nv.qadamw_encode(m.to(DEV), v.to(DEV), d["rht_seed"], d["sr_seed"])
    gm, gv = nv.qadamw_decode(st, d["rht_seed"])
    torch.cuda.synchronize()
    _check(m, v, d["rht_seed"], d["sr_seed"], 0, st, gm, gv, "adamw_state")
    # reconstruction error of sqrt(v), against plain NVFP4 of v (RNE, no transform)
    sv = np.sqrt(v.numpy().astype(np.float64))
    e_codec = np.abs(np.sqrt(gv.cpu().numpy().astype(np.float64)) - sv)
    plain = nv.quantize(v.to(DEV))
    torch.cuda.synchronize()
    pv = O.dequantize(to_oracle_view(plain))[0]
    e_plain = np.abs(np.sqrt(np.maximum(pv, 0.0)) - sv)
    print(f"\nparity adamw_state: bit-exact; sqrt(v) RMS error codec {np.sqrt((e_codec ** 2).mean()):.3e}"
          f" vs plain NVFP4 of v {np.sqrt((e_plain ** 2).mean()):.3e}", flush=True)
