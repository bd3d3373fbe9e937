"""Host-side checks of the rocprof harness: its counter passes stay within the
per-block limits of one rocprofv3 run, and its operand sizes match the half-step
kernels the traces name (k_lse<0, NCH, 0> for fp32 inputs: NCH 32-slot chunks)."""

from log_domain_sinkhorn_half_amd import rocprof_harness as h


def test_counter_passes_fit_one_run():
    for p in (h.SQ_PASS, h.LDS_PASS):
        assert sum(c.startswith("SQ_") for c in p) <= 8
        assert sum(c.startswith("GRBM_") for c in p) <= 2
        assert len(set(p)) == len(p)


def test_operand_slots_match_kernel_instances():
    # d = 3 -> k_lse<0, 1>, d = 32 -> k_lse<0, 10>, d = 64 -> k_lse<0, 18>, d = 88 (the fp32 limit) -> 23 chunks
    assert h.operand_slots(3, False) == 32
    assert h.operand_slots(32, False) == 320
    assert h.operand_slots(64, False) == 576
    assert h.operand_slots(88, False) == 23 * 32
    assert h.operand_slots(128, True) == 128
    assert h.operand_slots(300, True) == 320


def test_algorithmic_bytes_of_the_headline_workload():
    # half of an iteration's 2 (n+m) d s + 20 (n+m) bytes: fp32 coordinates, d = 3
    assert h.algorithmic_bytes(3) == (2 * 140000 * 3 * 4 + 20 * 140000) / 2
    # bf16 inputs at d = 128: 2-byte coordinates
    assert h.algorithmic_bytes(4) == (2 * 98304 * 128 * 2 + 20 * 98304) / 2
    assert h.operand_bytes(3) == 2 * 70000 * 32 * 2 + 70000 * 4


def test_code_hash_ignores_comments_and_spacing():
    a = "int f(int x) {\n  return x + 1;  // add one\n}\n"
    b = "/* doc */ int f(int x) { return x + 1; }"
    assert h.code_hash(a) == h.code_hash(b)
    assert h.code_hash(a) != h.code_hash(a.replace("+ 1", "+ 2"))
    assert len(h.kernel_source_hash()) == 16
