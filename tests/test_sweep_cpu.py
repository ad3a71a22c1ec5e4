"""Host side of the token-budget sweep: the tables it writes (no GPU)."""
from chunked_prefill_hybrid_rmsnorm_amd import sweep as S


def _fake_result():
    res = {"grid": {}, "pad_step": {}, "n_chunks": {}, "scan": {}, "decode_only": {}}
    for lp in S.LPS:
        for bd in S.BDS:
            # ms: the chunk alone costs lp/1000, each decode adds 0.5 us
            res["grid"][f"{lp},{bd}"] = lp / 1000 + bd * 0.0005
    for bd in S.BDS[1:]:
        res["decode_only"][str(bd)] = 0.1 + bd * 0.001
    for lp in (256, 257):
        for pad in S.PADS:
            res["pad_step"][f"{lp},{pad}"] = 0.2 if lp == 256 else 0.21
    for nc in S.NS:
        res["n_chunks"][str(nc)] = {"ms": 0.9 * nc, "attention_ms": 0.1 * nc, "reread_bytes": 0}
    for lp in S.SCAN:
        res["scan"][str(lp)] = 0.1 + (lp // 256) * 0.05
    res["plateau_ends"] = S.plateau_ends(res["scan"])
    return res


def test_piggyback_table(tmp_path):
    """Added cost of the decodes = hybrid minus chunk alone, and its ratio to
    the separate decode call."""
    path = tmp_path / "sweep.md"
    S.write_md(str(path), _fake_result(), "python -m chunked_prefill_hybrid_rmsnorm_amd.sweep")
    text = path.read_text()
    assert "## Piggybacked decodes against a separate decode call" in text
    lines = text.splitlines()
    i = lines.index("| alone (Lp = 0) | 116.0 | 164.0 | 228.0 |")
    # Lp = 128: +8 us for 16 decodes against 116 us alone (0.07), +32 / 164, +64 / 228
    assert lines[i + 1] == "| 128 | +8.0 (0.07) | +32.0 (0.20) | +64.0 (0.28) |"


def test_plateau_ends_mark_steps():
    scan = {"16": 1.0, "32": 1.05, "48": 1.3, "64": 1.31}
    assert S.plateau_ends(scan) == [32, 64]
