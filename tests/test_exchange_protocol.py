"""The split-row protocol of the one-launch step, checked on the CPU.

A row of the step split over S workgroups meets twice in the workspace: at
the score exchange each split stores its pages' keys into the row's slots,
then reads the other splits' slots (a bounded number of times) until none
reads 0, which no key is; at the finish each split counts itself in, and the
last one (`row_finish`) resets the counter, clears the row's slots and
merges.  `poll_row_keys`, `row_finish` and their call sites in `k_step` are
the whole protocol, and the model below is a transcription of them:

* every store is relaxed: it is issued into a per-split set of stores in
  flight, each of which may land in memory at any later point, in any order;
* `stores_done()` (s_waitcnt vmcnt(0)) is a step that is enabled only once all
  of the split's stores in flight have landed;
* a fetch-add, a load or a landed store acts on one coherent copy of each
  word (device-scope atomics are performed at the chip's shared cache level);
* each split's operations are issued in program order;
* a split's slots are one word in the model (each real slot goes through the
  same values: 0, then this call's key, then 0 once every split finished),
  and one poll reads the other splits' words together.

Every interleaving of S <= 4 splits, with every poll budget from 0 (every
split times out at once) to 3, is explored over two consecutive calls (the
second call starts from the memory the first one left).  In every reachable
state: a split that leaves the exchange with every slot written reads every
other split's keys of the current call, the merging split reads every
split's partial state of the current call, and the counter and every slot
are zero once a call has ended, which is what the next call starts from.
The structure of the model is tied to the source: the test reads the two
functions and the step kernel from the device header and checks that they
perform the same operations in the same order.
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEVICE_H = os.path.join(ROOT, "query_aware_sparse_bbox_amd", "csrc", "tsv_device.h")

# program counters of one split
(KEY_STORE, POLL, PART_STORE, PART_WAIT, FINISH, CLEAR_DONE, CLEAR_KEYS, MERGE,
 END) = range(9)

# memory: done, key[0..S-1] (a split's slots), part[0..S-1]
DONE_W = 0
NWORDS = 1


def explore(S, polls, calls=2, mistake=None):
    """Depth-first search of every interleaving; returns (states, calls ended).

    `mistake` plants one error in the protocol, to show that the checks
    catch it: "no_validate" (a split takes the other splits' slots after one
    read, written or not), "no_part_wait" (a split counts itself finished
    before its partial state lands), "keys_unwaited" (likewise before its key
    stores land), "no_key_clear" (the last split to finish leaves the slots
    set) or "done_left_set" (it leaves the counter set)."""
    key = lambda s: NWORDS + s
    part = lambda s: NWORDS + S + s
    mem0 = (0,) * (NWORDS + 2 * S)
    # split state: (pc, polls left, stores in flight)
    split0 = tuple((KEY_STORE, 0, frozenset()) for _ in range(S))
    start = (1, mem0, split0)
    seen = {start}
    stack = [start]
    ended = 0

    def succ(state):
        call, mem, sp = state
        out = []
        for s, (pc, left, pend) in enumerate(sp):
            # a store in flight lands
            for loc, val in pend:
                m = list(mem)
                m[loc] = val
                ns = list(sp)
                ns[s] = (pc, left, pend - {(loc, val)})
                out.append((call, tuple(m), tuple(ns)))

            def go(pc2, left2=left, pend2=pend, mem2=mem):
                ns = list(sp)
                ns[s] = (pc2, left2, pend2)
                out.append((call, mem2, tuple(ns)))

            if pc == KEY_STORE:
                # nothing waits for these stores before the poll
                go(POLL, left2=polls, pend2=pend | {(key(s), call)})
            elif pc == POLL:
                others = [k for k in range(S) if k != s]
                if left == 0:
                    go(PART_STORE)  # timed out: this split scores every page itself
                elif mistake == "no_validate" or all(mem[key(k)] != 0 for k in others):
                    for k in others:
                        assert mem[key(k)] == call, (
                            f"S={S} polls={polls}: split {s} read split {k}'s keys of call "
                            f"{mem[key(k)]} in call {call}")
                    go(PART_STORE)
                else:
                    go(POLL, left2=left - 1)
            elif pc == PART_STORE:
                go(FINISH if mistake == "no_part_wait" else PART_WAIT,
                   pend2=pend | {(part(s), call)})
            elif pc == PART_WAIT:
                waited = {x for x in pend if x[0] == part(s)} if mistake == "keys_unwaited" else pend
                if not waited:
                    go(FINISH)
            elif pc == FINISH:
                got = mem[DONE_W]
                m = list(mem)
                m[DONE_W] = got + 1
                go(CLEAR_DONE if got == S - 1 else END, mem2=tuple(m))
            elif pc == CLEAR_DONE:
                go(CLEAR_KEYS,
                   pend2=pend if mistake == "done_left_set" else pend | {(DONE_W, 0)})
            elif pc == CLEAR_KEYS:
                clears = set() if mistake == "no_key_clear" else {(key(k), 0) for k in range(S)}
                go(MERGE, pend2=pend | clears)
            elif pc == MERGE:
                for k in range(S):
                    assert mem[part(k)] == call, (
                        f"S={S} polls={polls}: the merge read split {k}'s partial state of call "
                        f"{mem[part(k)]} in call {call}")
                go(END)
        return out

    while stack:
        state = stack.pop()
        call, mem, sp = state
        nxt = succ(state)
        if not nxt:
            # every split ended and every store landed: the launch is over
            assert all(x[0] == END and not x[2] for x in sp), f"stuck state {state}"
            assert not any(mem[:NWORDS + S]), (
                f"S={S} polls={polls}: counter and slots {mem[:NWORDS + S]} left after "
                f"call {call}")
            ended += 1
            if call < calls:
                nxt = [(call + 1, mem, split0)]
        for n in nxt:
            if n not in seen:
                seen.add(n)
                stack.append(n)
    return len(seen), ended


@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("polls", [0, 1, 2, 3])
def test_every_interleaving(S, polls):
    states, ended = explore(S, polls)
    assert ended >= 1 and states > S


@pytest.mark.parametrize("mistake,pattern", [
    ("no_validate", "keys of call"),
    ("no_part_wait", "partial state of call"),
    ("keys_unwaited", "left after call|keys of call"),
    ("no_key_clear", "left after call|keys of call"),
    ("done_left_set", "left after call"),
])
def test_model_catches_planted_mistakes(mistake, pattern):
    with pytest.raises(AssertionError, match=pattern):
        explore(2, 2, mistake=mistake)


# --- the model's operations, read from the source -------------------------

def function_body(text, signature):
    i = text.index(signature)
    i = text.index("{", i)
    depth = 0
    for k in range(i, len(text)):
        if text[k] == "{":
            depth += 1
        elif text[k] == "}":
            depth -= 1
            if depth == 0:
                return text[i:k + 1]
    raise AssertionError("unbalanced braces")


def ops(body):
    """The counter operations of a function body, in source order."""
    pat = re.compile(r"__hip_atomic_fetch_add\(c \+ (\w+)|st_dev\(c \+ (\w+), (\w+)\)|"
                     r"ld_dev\(c \+ (\w+)\)")
    out = []
    for m in pat.finditer(body):
        if m.group(1):
            out.append(("fetch_add", m.group(1)))
        elif m.group(2):
            out.append(("store", m.group(2), m.group(3)))
        else:
            out.append(("load", m.group(4)))
    return out


def test_model_matches_the_source():
    text = open(DEVICE_H).read()
    step = function_body(text, "void k_step(")
    # a published key is never 0, the value of a slot not yet written, and the
    # split's own copy holds the same value
    assert re.search(r"const uint32_t k = max\(s_key\[p\], 1u\);\s*s_key\[p\] = k;\s*"
                     r"st_dev\(xrow \+ p, k\);", step)
    poll = function_body(text, "int poll_row_keys(")
    # up to `polls` rounds, each reading every other split's slots, until
    # none reads 0
    assert re.search(r"for \(int it = 0; it < polls; \+\+it\) \{", poll)
    assert re.search(r"v\[j\] = p < n && \(p / PB\) % S != split \? ld_dev\(xrow \+ p\) : 1u;", poll)
    assert re.search(r"if \(p < n && \(p / PB\) % S != split\) \{\s*s_key\[p\] = v\[j\];"
                     r"\s*missing \|= v\[j\] == 0u;", poll)
    assert re.search(r"if \(!__syncthreads_or\(missing\)\) return 1;", poll)
    assert "st_dev" not in poll
    fin = function_body(text, "int row_finish(uint32_t* c, int S)")
    assert ops(fin) == [("fetch_add", "kSyncDone"), ("store", "kSyncDone", "0u")]
    assert re.search(r"if \(o != \(uint32_t\)S - 1\) return 0;", fin)
    # the slots are written twice: this split's keys before the poll, zeros
    # by the last split to finish
    assert re.findall(r"st_dev\(xrow \+ p, ([^)]*)\)", step) == ["k", "0u"]
    i_pub = step.index("st_dev(xrow + p, k);")
    i_poll = step.index("poll_row_keys<NT, PB>(xrow, s_key, n, S, split, polls)")
    i_fin = step.index("row_finish(rsync, S)")
    assert i_pub < i_poll < i_fin
    # a split that timed out scores every batch itself
    assert re.search(r"if \(poll_row_keys<NT, PB>\(xrow, s_key, n, S, split, polls\)\) break;"
                     r"\s*__syncthreads\(\);[^\n]*\n\s*share = false;", step)
    # every split's stores (keys and partial state) are waited for before it
    # counts itself finished
    before_fin = step[:i_fin]
    assert before_fin.rindex("stores_done();") > before_fin.rindex("finish_split<")
    assert before_fin.rindex("stores_done();") > i_pub
    # only the last split clears the slots, then merges
    assert re.search(r"if \(!s_flag\) \{[^}]*return;\s*\}\s*if \(xchg\)\s*"
                     r"for \(int p = tid; p < n; p \+= NT\) st_dev\(xrow \+ p, 0u\);\s*merge_row<",
                     step[i_fin:])
