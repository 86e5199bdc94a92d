"""Host checks of the launch-form choice (no GPU).

Every launch form runs the same items in the same order (the GPU tests pin
each form to the oracle); here the choice itself: AUTO picks the form of
least modelled time among the eligible ones -- the LDS-resident column
kernel for small and mid sizes, the single-workgroup kernel where a column
would hold too many chunks, one launch per step once the working set
outgrows the column limit -- forced forms fall back to one launch per step
where not eligible, and the limits gate eligibility.  Without a GPU the
library assumes 64 KiB of LDS per workgroup; sizes whose choice depends on
the device's LDS are not asserted.
"""
import pytest

import allreduce_reduction_amd as hc


def test_auto_regimes_ring_p8_fp16():
    with hc.Comm(8, "ring") as c:
        assert c.exec_choice("allreduce", 512, "fp16") == "lds"            # 1 KiB per rank
        assert c.exec_choice("allreduce", 32 << 10, "fp16") == "lds"       # 64 KiB per rank
        assert c.exec_choice("allreduce", 2 << 20, "fp16") in ("lds", "columns")  # 4 MiB per rank (32 MiB total)
        assert c.exec_choice("allreduce", 8 << 20, "fp16") == "steps"      # 16 MiB per rank: over the limit
        assert c.exec_choice("allreduce", 64 << 20, "fp32") == "steps"     # the 256 MiB per rank workload


def test_auto_small_rhd_many_ranks_prefers_the_single_workgroup():
    # 1 KiB per rank over 64 ranks: 16-byte segments, so every LDS column
    # holds chunks of many segments' steps; one workgroup is cheaper
    with hc.Comm(64, "rhd") as c:
        assert c.exec_choice("allreduce", 512, "fp16") == "fused"
        assert c.exec_choice("allreduce", 8 << 10, "fp16") == "lds"
    # over 16 ranks (64-byte segments) the LDS form's columns fit within a
    # segment and its halving passes alone count (on MI355X: 12.3-12.5 us
    # against 14.9-15.1 us for the single workgroup)
    with hc.Comm(16, "rhd") as c:
        assert c.exec_choice("allreduce", 512, "fp16") == "lds"


def test_auto_prefers_steps_where_launches_are_few_and_bytes_many():
    # Flat has two steps: at 4 MiB per rank (64 MiB in all, within the column
    # limit) two launches beat streaming every rank buffer through LDS and
    # folding 16 sources per chunk there
    with hc.Comm(16, "flat") as c:
        assert c.exec_choice("allreduce", 2 << 20, "fp16") == "steps"
        assert c.exec_choice("allreduce", 32 << 10, "fp16") == "lds"


def test_forced_forms_and_fallbacks():
    with hc.Comm(8, "ring") as c:
        c.set_exec_mode("steps")
        assert c.exec_choice("allreduce", 512, "fp16") == "steps"
        c.set_exec_mode("fused")
        assert c.exec_choice("allreduce", 32 << 10, "fp16") == "fused"
        c.set_fused_limit(1000)
        assert c.exec_choice("allreduce", 32 << 10, "fp16") == "steps"      # over the fused limit
        c.set_exec_mode("columns")
        assert c.exec_choice("allreduce", 512, "fp16") == "columns"
        assert c.exec_choice("allreduce", 8 << 20, "fp16") == "steps"      # over the column limit
        # a single busy step is never worth a column launch
        assert c.exec_choice("allreduce", 512, "fp16", first=0, last=1) == "steps"
        c.set_columns(0)
        assert c.exec_choice("allreduce", 512, "fp16") == "steps"
        c.set_exec_mode("lds")
        assert c.exec_choice("allreduce", 512, "fp16") == "steps"          # over the column limit
        c.set_exec_mode("auto")
        assert c.exec_choice("allreduce", 512, "fp16") == "steps"          # no one-launch form eligible
        c.set_fused_limit(64 << 20)
        c.set_columns(64 << 20)
        assert c.exec_choice("allreduce", 512, "fp16") == "lds"
        c.set_exec_mode("lds")
        assert c.exec_choice("allreduce", 512, "fp16") == "lds"
        assert c.exec_choice("allreduce", 512, "fp16", first=0, last=1) == "steps"
        # 8 ranks x 1 MiB columns cannot fit one workgroup's LDS
        c.set_columns(64 << 20, 1 << 20)
        assert c.exec_choice("allreduce", 1 << 20, "fp16") == "steps"
        c.set_columns(64 << 20, 1024)
        assert c.exec_choice("allreduce", 1 << 20, "fp16") == "lds"


def test_fused_needs_at_most_256_items_per_step():
    # a 2 x 2 pipeline with 1 KiB loops over 256 KiB has 256 loops of 4 blocks: > 256 items per step
    with hc.Comm(4, "pipeline", 2, 2, 1024) as c:
        L = 64 << 10
        assert max(c.step_info("allreduce", L, "fp32", s)["nitems"]
                   for s in range(c.plan_info("allreduce", L, "fp32")["nsteps"])) > 256
        c.set_exec_mode("fused")
        assert c.exec_choice("allreduce", L, "fp32") == "steps"


def test_exec_choice_edges_and_validation():
    with hc.Comm(8, "ring") as c:
        assert c.exec_choice("allreduce", 0, "fp32") == "steps"
        with pytest.raises(hc.HbmcError):
            c.exec_choice("allreduce", 100, "fp32", first=3, last=99)
        with pytest.raises(KeyError):
            c.set_exec_mode("bogus")
        lib = hc.load_library()
        assert lib.hbmc_comm_set_exec_mode(c._h, 5) == 1
    with hc.Comm(1, "ring") as c:
        assert c.exec_choice("allreduce", 100, "fp32") == "steps"
