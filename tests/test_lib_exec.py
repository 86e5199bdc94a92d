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
        assert c.exec_choice("allreduce", 512, "fp16") == "regs"           # 1 KiB per rank
        assert c.exec_choice("allreduce", 32 << 10, "fp16") == "regs"      # 64 KiB per rank
        assert c.exec_choice("allreduce", 2 << 20, "fp16") == "regs"       # 4 MiB per rank (32 MiB total)
        assert c.exec_choice("allreduce", 8 << 20, "fp16") == "steps"      # 16 MiB per rank: over the limit
        assert c.exec_choice("allreduce", 64 << 20, "fp32") == "steps"     # the 256 MiB per rank workload
        # the ring's reduce-scatter (prefixes of one fold) and all-gather
        # (copies) run in registers too
        assert c.exec_choice("reduce_scatter", 512, "fp16") == "regs"
        assert c.exec_choice("all_gather", 32 << 10, "fp16") == "regs"


def test_auto_small_rhd_many_ranks_prefers_the_single_workgroup():
    # 1 KiB per rank over 64 ranks (a tree of 64 leaves: no register form):
    # 16-byte segments, so every LDS column holds chunks of many segments'
    # steps; one workgroup is cheaper
    with hc.Comm(64, "rhd") as c:
        assert c.exec_choice("allreduce", 512, "fp16") == "fused"
        assert c.exec_choice("allreduce", 8 << 10, "fp16") == "lds"
    # over 16 ranks the register form takes the whole tree (on MI355X, graphs
    # of ten: 7.0-7.1 us against 14.2 us in the LDS form and 15.4 us in the
    # single workgroup), and its reduce-scatter as the tree's nodes
    with hc.Comm(16, "rhd") as c:
        assert c.exec_choice("allreduce", 512, "fp16") == "regs"
        assert c.exec_choice("reduce_scatter", 512, "fp16") == "regs"


def test_auto_prefers_steps_where_launches_are_few_and_bytes_many():
    # Flat has two steps: at 4 MiB per rank (64 MiB in all, within the column
    # limit) two launches beat streaming every rank buffer through LDS and
    # folding 17 sources per chunk there; a fold over 16 ranks fits the
    # register form instead
    with hc.Comm(16, "flat") as c:
        assert c.exec_choice("allreduce", 32 << 10, "fp16") == "regs"
    # over 17 ranks the fold is too long for registers
    with hc.Comm(17, "flat") as c:
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
        assert c.exec_choice("allreduce", 512, "fp16") == "regs"
        c.set_exec_mode("regs")
        assert c.exec_choice("allreduce", 512, "fp16") == "regs"
        c.set_columns(0)
        assert c.exec_choice("allreduce", 512, "fp16") == "steps"          # over the column limit
        c.set_columns(64 << 20)
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
        assert lib.hbmc_comm_set_exec_mode(c._h, 7) == 1
        assert lib.hbmc_comm_set_exec_mode(c._h, 6) == 0
    with hc.Comm(1, "ring") as c:
        assert c.exec_choice("allreduce", 100, "fp32") == "steps"


def _footprint(items, P, L, e):
    """Each rank's elements read by some item once, plus those written once
    (boolean masks per rank; independent of the library's interval union)."""
    import numpy as np
    rd = np.zeros((P, L), bool)
    wr = np.zeros((P, L), bool)
    for it in items:
        for r in it["src"]:
            rd[r, it["begin"]:it["begin"] + it["count"]] = True
        for r in it["dst"]:
            wr[r, it["begin"]:it["begin"] + it["count"]] = True
    return int(rd.sum() + wr.sum()) * e


@pytest.mark.parametrize("algo,P", [("ring", 8), ("rhd", 8), ("rhd", 5), ("ring", 16)])
@pytest.mark.parametrize("coll", ["allreduce", "reduce_scatter", "all_gather"])
def test_exec_bytes_per_form(algo, P, coll):
    """hbmc_exec_bytes: steps = the plan's algorithmic bytes; fused / columns =
    the compulsory footprint; LDS = what its kernel loads and stores, which
    for a whole AllReduce is every rank loaded and stored once (2 P D) and
    never more than 2 P D; AUTO reports its pick's figure."""
    e, L = 2, 40_000 + 7
    D = L * e
    with hc.Comm(P, algo) as c:
        info = c.plan_info(coll, L, "fp16")
        assert c.exec_bytes(coll, L, "fp16", "steps") == info["hbm_bytes"]
        items = c.plan_items(coll, L, "fp16")
        fp = _footprint(items, P, L, e)
        assert c.exec_bytes(coll, L, "fp16", "fused") == fp
        assert c.exec_bytes(coll, L, "fp16", "columns") == fp
        lds = c.exec_bytes(coll, L, "fp16", "lds")
        assert lds <= 2 * P * D
        if coll == "allreduce":
            assert fp == 2 * P * D
            assert lds == 2 * P * D
        if coll == "all_gather":
            # columns composed into stores load only the owners' copies
            assert (P - 1) * D <= lds <= (P + 2) * D
        form = c.exec_choice(coll, L, "fp16")
        assert c.exec_bytes(coll, L, "fp16", "auto") == c.exec_bytes(coll, L, "fp16", form)
        # a step range: every rank loaded, only the ranks its steps write stored
        n = info["nsteps"]
        if n >= 2:
            first, last = 0, n // 2
            part = [it for it in items if first <= it["step"] < last]
            assert c.exec_bytes(coll, L, "fp16", "steps", first=first, last=last) == \
                sum(c.step_info(coll, L, "fp16", s)["hbm_bytes"] for s in range(first, last))
            assert c.exec_bytes(coll, L, "fp16", "columns", first=first, last=last) == _footprint(part, P, L, e)
            r = c.exec_bytes(coll, L, "fp16", "lds", first=first, last=last)
            written = len({d for it in part for d in it["dst"]})
            assert P * D <= r <= P * D + written * D


def test_exec_bytes_rejects_bad_ranges():
    lib = hc.load_library()
    import ctypes
    with hc.Comm(8, "ring") as c:
        b = ctypes.c_uint64()
        assert lib.hbmc_exec_bytes(c._h, 0, 0, 1000, 1, 3, 2, 1, ctypes.byref(b)) == 1   # first > last
        assert lib.hbmc_exec_bytes(c._h, 0, 0, 1000, 1, 0, 15, 1, ctypes.byref(b)) == 1  # past the end
        assert lib.hbmc_exec_bytes(c._h, 0, 0, 1000, 1, 0, 0, 9, ctypes.byref(b)) == 1   # bad mode
        assert lib.hbmc_exec_bytes(c._h, 0, 0, 1000, 1, 0, 0, 1, None) == 1
        assert lib.hbmc_exec_bytes(c._h, 0, 0, 0, 1, 0, 0, 4, ctypes.byref(b)) == 0 and b.value == 0


def test_regs_only_where_the_expression_is_a_fold_tree_copy_or_prefix():
    """Calls whose elements end with other expressions keep another form; a
    forced REGS falls back to one launch per step."""
    with hc.Comm(8, "pipeline", 2, 4) as c:
        c.set_exec_mode("regs")
        assert c.exec_choice("allreduce", 10_000, "fp32") == "steps"      # folds of folds
        assert c.exec_choice("reduce_scatter", 10_000, "fp32") == "steps"
        assert c.exec_choice("all_gather", 10_000, "fp32") == "regs"      # copies
    with hc.Comm(8, "hier", 2, 4) as c:
        c.set_exec_mode("regs")
        assert c.exec_choice("allreduce", 10_000, "fp32") == "steps"
    with hc.Comm(8, "tree", 0, 2) as c:  # a binary heap of 8: neither fold nor complete tree
        c.set_exec_mode("regs")
        assert c.exec_choice("allreduce", 10_000, "fp32") == "steps"
    with hc.Comm(8, "rhd") as c:
        c.set_exec_mode("regs")
        # partial trees: every rank holds its input or a node of the tree above its own leaf
        assert c.exec_choice("reduce_scatter", 10_000, "fp32") == "regs"
        assert c.exec_choice("reduce", 10_000, "fp32", root=3) == "regs"
        assert c.exec_choice("all_gather", 10_000, "fp32") == "regs"
        assert c.exec_choice("broadcast", 10_000, "fp32", root=3) == "regs"
    with hc.Comm(6, "rhd") as c:  # not a power of two: merged pairs under partial trees
        c.set_exec_mode("regs")
        assert c.exec_choice("reduce_scatter", 10_000, "fp32") == "steps"
        assert c.exec_choice("reduce", 10_000, "fp32", root=3) == "steps"
    with hc.Comm(8, "ring") as c:
        c.set_exec_mode("regs")
        assert c.exec_choice("reduce_scatter", 10_000, "fp32") == "regs"
        assert c.exec_choice("allreduce", 10_000, "fp32") == "regs"
        assert c.exec_choice("allreduce", 10_000, "fp32", first=0, last=3) == "steps"
        # one-step calls are one launch anyway
    with hc.Comm(2, "ring") as c:
        c.set_exec_mode("regs")
        assert c.exec_choice("reduce_scatter", 10_000, "fp32") == "steps"
    for P in (17, 64):  # folds and copies of more than 16 ranks
        with hc.Comm(P, "ring") as c:
            c.set_exec_mode("regs")
            for coll in ("allreduce", "reduce_scatter", "all_gather"):
                assert c.exec_choice(coll, 10_000, "fp32") == "steps"


@pytest.mark.parametrize("algo,P", [("ring", 2), ("ring", 3), ("ring", 8), ("ring", 16), ("rhd", 5), ("rhd", 6),
                                    ("rhd", 8), ("rhd", 16), ("rhd", 24), ("flat", 7), ("flat", 16)])
def test_regs_offered_for_folds_and_trees(algo, P):
    with hc.Comm(P, algo) as c:
        c.set_exec_mode("regs")
        for L in (1, 5, 1001, 100_003):
            assert c.exec_choice("allreduce", L, "bf16") == "regs", L
            assert c.exec_bytes("allreduce", L, "bf16", "regs") == 2 * P * L * 2
    with hc.Comm(P, algo) as c:
        c.set_exec_mode("regs")
        if algo == "ring" and P > 2:
            assert c.exec_bytes("reduce_scatter", 1001, "bf16", "regs") == (2 * P - 1) * 1001 * 2
            assert c.exec_bytes("all_gather", 1001, "bf16", "regs") == P * 1001 * 2
        if algo == "rhd" and P & (P - 1) == 0 and P > 2:
            # every rank loaded; per element, P/2 ranks receive a node (the owner
            # the root, the others the subtrees they kept)
            assert c.exec_bytes("reduce_scatter", 1001, "bf16", "regs") == (P + P // 2) * 1001 * 2
