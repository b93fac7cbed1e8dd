"""Runs a golden block-manager script against any manager object.

The manager must offer allocate/append_slot/free/fork/slot/num_free_blocks/
num_cached_tokens/get_table/swap_out/swap_in/dump with the oracle's
semantics; sequence names from the pages ("x", "a", ...) are mapped to small
integers.
"""


def run_steps(bm, spec, oob_exc):
    names = {}

    def sid(name):
        return names.setdefault(name, len(names) + 1)

    for i, st in enumerate(spec["steps"]):
        op, exp = st["op"], st.get("expect")
        where = f"step {i} {st}"
        if op == "allocate":
            if exp == "OutOfBlocks":
                before = bm.dump()
                try:
                    bm.allocate(sid(st["seq"]), st["tokens"])
                except oob_exc:
                    pass
                else:
                    raise AssertionError(f"{where}: no OutOfBlocks")
                if st.get("state_unchanged"):
                    assert bm.dump() == before, f"{where}: state changed"
            else:
                got = bm.allocate(sid(st["seq"]), st["tokens"])
                assert list(got) == exp, f"{where}: got {got}"
        elif op == "swap_out":
            got = bm.swap_out(sid(st["seq"]))
            assert list(got) == exp, f"{where}: got {got}"
        elif op == "swap_in":
            if exp == "OutOfBlocks":
                before = bm.dump()
                try:
                    bm.swap_in(sid(st["seq"]))
                except oob_exc:
                    pass
                else:
                    raise AssertionError(f"{where}: no OutOfBlocks")
                if st.get("state_unchanged"):
                    assert bm.dump() == before, f"{where}: state changed"
            else:
                table, first = bm.swap_in(sid(st["seq"]))
                assert (list(table), first) == (exp["table"], exp["first_restore"]), \
                    f"{where}: got {table}, {first}"
        elif op == "swapped":
            want = {sid(k): v for k, v in exp.items()}
            assert bm.dump()["swapped"] == want, f"{where}: got {bm.dump()['swapped']}"
        elif op == "append_slot":
            slot, _cow = bm.append_slot(sid(st["seq"]), st["token"])
            assert slot == exp, f"{where}: got {slot}"
        elif op == "free":
            bm.free(sid(st["seq"]))
        elif op == "slot":
            assert bm.slot(sid(st["seq"]), st["pos"]) == exp, where
        elif op == "num_free_blocks":
            assert bm.num_free_blocks == exp, f"{where}: got {bm.num_free_blocks}"
        elif op == "free_list":
            assert bm.dump()["free"] == exp, f"{where}: got {bm.dump()['free']}"
        elif op == "evictable":
            assert bm.dump()["evictable"] == exp, f"{where}: got {bm.dump()['evictable']}"
        elif op == "refs":
            got = "".join(str(r) for r in bm.dump()["ref"])
            assert got == exp, f"{where}: got {got}"
        elif op == "cached":
            assert bm.num_cached_tokens(sid(st["seq"])) == exp, where
        elif op == "table":
            assert list(bm.get_table(sid(st["seq"]))) == exp, where
        else:
            raise ValueError(op)
        bm.check_invariants()
