"""Labelling of profiled dispatches with the library's kernel slots (CPU)."""
from chunked_prefill_hybrid_rmsnorm_amd.profiling import SLOTS, SlotLabeler

GEMM = "void hl::gemm_dma_kernel<288, 128, 2, 4, {e}, 3, 64>(unsigned short const*, int)"
SPLIT_CALL = [
    "void hl::rmsnorm_kernel<8>(unsigned short const*)",
    GEMM.format(e=0),
    "void hl::rope_append_wide_kernel<4>(unsigned short*, float const*)",
    "void hl::attention_kernel<128>(hl::AttnArgs)",
    "void hl::attention_merge_kernel<128>(hl::AttnArgs)",
    GEMM.format(e=1),
    "void hl::gemm_splitk_reduce_norm<2, 8>(float const*, unsigned short*)",
    GEMM.format(e=2),
    "void hl::gemm_splitk_reduce_swiglu<4>(float const*, unsigned short*, int, int)",
    GEMM.format(e=1),
    "void hl::gemm_splitk_reduce<1, 8>(float const*, unsigned short*)",
]
# no split anywhere: no reduces, no merge, the second RMSNorm is a plain kernel
PLAIN_CALL = [SPLIT_CALL[i] for i in (0, 1, 2, 3, 5)] + [
    "void hl::rmsnorm_kernel<8>(unsigned short const*)"] + [SPLIT_CALL[i] for i in (7, 9)]


def test_split_call_fills_every_slot_in_order():
    lab = SlotLabeler()
    assert [lab.label(k) for k in SPLIT_CALL * 2] == list(SLOTS) * 2


def test_unsplit_call_labels():
    lab = SlotLabeler()
    got = [lab.label(k) for k in PLAIN_CALL + SPLIT_CALL[:2]]
    assert got == ["rmsnorm1", "gemm_qkv", "rope_kv_append", "attention", "gemm_o",
                   "gemm_o_reduce_rmsnorm2", "gemm_gate_up", "gemm_down", "rmsnorm1", "gemm_qkv"]


def test_reduce_of_a_plain_gemm_is_not_the_down_reduce():
    lab = SlotLabeler()
    lab.label(GEMM.format(e=0))
    assert lab.label("void hl::gemm_splitk_reduce<0, 4>(float const*, unsigned short*)") is None


def test_foreign_kernels_are_skipped():
    lab = SlotLabeler()
    assert lab.label("__amd_rocclr_copyBuffer") is None
    assert lab.label("void at::native::vectorized_elementwise_kernel<16>(int)") is None


def test_mfma_summary_from_counter_rows(tmp_path):
    """Four counters of one gate/up dispatch: flops are MOPS x 512, the
    utilisation is busy cycles over SIMDs x per-XCD active cycles."""
    import csv
    from chunked_prefill_hybrid_rmsnorm_amd.profiling import MFMA_COUNTERS, SIMDS, XCDS, mfma_summary
    path = tmp_path / "m_counter_collection.csv"
    vals = {"SQ_INSTS_VALU_MFMA_MOPS_BF16": 1000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 500.0,
            "SQ_BUSY_CU_CYCLES": 7.0, "GRBM_GUI_ACTIVE": 8.0 * 2.0}
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, k in enumerate(SPLIT_CALL[:8]):
            for c in MFMA_COUNTERS:
                v = vals[c] if "gemm_dma_kernel<288, 128, 2, 4, 2" in k else 0.0
                w.writerow([i + 1, k, c, v])
    res = mfma_summary(str(path))
    assert list(res) == ["gemm_gate_up"]
    e = res["gemm_gate_up"]
    assert e["flops"] == 1000.0 * 512
    assert e["active_cycles_per_xcd"] == 2.0 and XCDS == 8
    assert abs(e["mfma_util"] - 500.0 / (SIMDS * 2.0)) < 1e-12


def test_chained_call_labels():
    """Cross-layer fusion: no first RMSNorm, the down reduce also normalises;
    unsplit, the next layer's RMSNorm follows the down projection."""
    lab = SlotLabeler()
    chained = SPLIT_CALL[1:10] + ["void hl::gemm_splitk_reduce_norm<4, 4>(float const*)"]
    assert [lab.label(k) for k in chained] == list(SLOTS[1:])
    lab = SlotLabeler(chained=True)
    got = [lab.label(k) for k in PLAIN_CALL[1:] + ["void hl::rmsnorm_kernel<8>(unsigned short const*)"]]
    assert got[-2:] == ["gemm_down", "gemm_down_reduce"]


def test_agpr_swiglu_kernel_is_the_gate_up_slot():
    lab = SlotLabeler()
    lab.label(GEMM.format(e=1))
    assert lab.label("void hl::gemm_swiglu_agpr_kernel<288>(unsigned short const*)") == "gemm_gate_up"
    assert lab.label(GEMM.format(e=1)) == "gemm_down"


def test_agpr_plain_and_residual_kernels_label_by_epilogue():
    lab = SlotLabeler()
    qkv = "void hl::gemm_agpr_kernel<288, 5, 0>(unsigned short const*, int)"
    res = "void hl::gemm_agpr_kernel<288, 4, 1>(unsigned short const*, int)"
    assert lab.label(qkv) == "gemm_qkv"
    assert lab.label(res) == "gemm_o"
    lab.label("void hl::gemm_swiglu_agpr_kernel<288>(unsigned short const*)")
    assert lab.label(res) == "gemm_down"
