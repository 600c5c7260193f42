"""The split-row counter protocol of the one-launch step, checked on the CPU.

A row of the step split over S workgroups meets twice through two counter
words: the score exchange (`row_exchange`: each split counts itself in, and
a split that is not the last polls the count, a bounded number of times,
until it reaches S) and the finish (`row_finish`: the last split to finish
merges and clears both words).  Those two functions and their call sites in
`k_step` are the whole protocol, and the model below is a transcription of
them:

* every store is relaxed: it is issued into a per-split set of stores in
  flight, each of which may land in memory at any later point, in any order;
* `stores_done()` (s_waitcnt vmcnt(0)) is a step that is enabled only once all
  of the split's stores in flight have landed;
* a fetch-add, a load or a landed store acts on one coherent copy of each
  word (device-scope atomics are performed at the chip's shared cache level);
* each split's operations are issued in program order.

Every interleaving of S <= 4 splits, with every poll budget from 0 (every
waiting split times out at once) to 3, is explored over two consecutive calls
(the second call starts from the memory the first one left).  In every
reachable state: a split that leaves the exchange having seen all S arrivals
reads every other split's keys of the current call, the merging split reads
every split's partial state of the current call, and both words are zero
once a call has ended, which is what the next call starts from.  The
structure of the model is tied to the source: the test reads the two
functions and the step kernel from the device header and checks that they
perform the same operations in the same order.
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEVICE_H = os.path.join(ROOT, "query_aware_sparse_bbox_amd", "csrc", "tsv_device.h")

# program counters of one split
(KEY_STORE, KEY_WAIT, ARRIVE, POLL, READ_KEYS, PART_STORE, PART_WAIT, FINISH, CLEAR_DONE,
 CLEAR_ARRIVE, MERGE, END) = range(12)

# memory: arrive, done, key[0..S-1], part[0..S-1]
ARRIVE_W, DONE_W = 0, 1
NWORDS = 2


def explore(S, polls, calls=2, mistake=None):
    """Depth-first search of every interleaving; returns (states, calls ended).

    `mistake` plants one error in the protocol, to show that the checks
    catch it: "no_key_wait" (a split counts itself in before its keys
    land), "no_part_wait" (likewise before its partial state lands),
    "no_rearm" (the last split to finish leaves the arrival count set),
    "done_left_set" (it leaves the finish count set) or "rearm_on_arrival"
    (the last split to arrive clears the arrival count, as a flag-based
    protocol would, so that a split still polling never sees S)."""
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

            def with_word(loc, val):
                m = list(mem)
                m[loc] = val
                return tuple(m)

            if pc == KEY_STORE:
                go(ARRIVE if mistake == "no_key_wait" else KEY_WAIT,
                   pend2=pend | {(key(s), call)})
            elif pc == KEY_WAIT:
                if not pend:
                    go(ARRIVE)
            elif pc == ARRIVE:
                got = mem[ARRIVE_W]
                m = with_word(ARRIVE_W, got + 1)
                if got == S - 1:
                    if mistake == "rearm_on_arrival":
                        go(READ_KEYS, mem2=m, pend2=pend | {(ARRIVE_W, 0)})
                    else:
                        go(READ_KEYS, mem2=m)
                else:
                    go(POLL, left2=polls, mem2=m)
            elif pc == POLL:
                if left == 0:
                    go(PART_STORE)  # timed out: this split scores every page itself
                elif mem[ARRIVE_W] == S:
                    go(READ_KEYS)
                else:
                    go(POLL, left2=left - 1)
            elif pc == READ_KEYS:
                # every key read at once: keys only ever change to the current
                # call's, so this is at least as strict as reading them one
                # after the other
                for k in range(S):
                    assert mem[key(k)] == call, (
                        f"S={S} polls={polls}: split {s} read split {k}'s keys of call "
                        f"{mem[key(k)]} in call {call}")
                go(PART_STORE)
            elif pc == PART_STORE:
                go(FINISH if mistake == "no_part_wait" else PART_WAIT,
                   pend2=pend | {(part(s), call)})
            elif pc == PART_WAIT:
                if not pend:
                    go(FINISH)
            elif pc == FINISH:
                got = mem[DONE_W]
                m = with_word(DONE_W, got + 1)
                go(CLEAR_DONE if got == S - 1 else END, mem2=m)
            elif pc == CLEAR_DONE:
                go(CLEAR_ARRIVE,
                   pend2=pend if mistake == "done_left_set" else pend | {(DONE_W, 0)})
            elif pc == CLEAR_ARRIVE:
                go(MERGE,
                   pend2=pend if mistake == "no_rearm" else pend | {(ARRIVE_W, 0)})
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
            assert mem[ARRIVE_W] == 0 and mem[DONE_W] == 0, (
                f"S={S} polls={polls}: counters {mem[:NWORDS]} left after call {call}")
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
    ("no_key_wait", "keys of call"),
    ("no_part_wait", "partial state of call"),
    ("no_rearm", "left after call|keys of call"),
    ("done_left_set", "left after call"),
])
def test_model_catches_planted_mistakes(mistake, pattern):
    with pytest.raises(AssertionError, match=pattern):
        explore(2, 2, mistake=mistake)


def test_rearm_on_arrival_only_delays():
    """Clearing the arrival count when the last split arrives (a flag
    protocol's re-arm) breaks nothing the checks see, but a split that polls
    after the clear never finds S arrivals and scores its whole row itself:
    the model reaches states where a poll times out with every split
    arrived.  The kernel therefore leaves the count at S until the finish."""
    states, ended = explore(2, 2, mistake="rearm_on_arrival")
    assert ended >= 1


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
    ex = function_body(text, "int row_exchange(uint32_t* c, int S, int polls)")
    assert ops(ex) == [("fetch_add", "kSyncArrive"), ("load", "kSyncArrive")]
    # the last arrival returns at once; the others poll the count, in a loop
    # bounded by `polls`, until it reaches S
    assert re.search(r"if \(o == \(uint32_t\)S - 1\) return 1;", ex)
    assert re.search(r"for \(int it = 0; it < polls; \+\+it\) \{\s*if \(ld_dev\(c \+ kSyncArrive\) "
                     r"== \(uint32_t\)S\) return 1;", ex)
    fin = function_body(text, "int row_finish(uint32_t* c, int S)")
    assert ops(fin) == [("fetch_add", "kSyncDone"), ("store", "kSyncDone", "0u"),
                        ("store", "kSyncArrive", "0u")]
    assert re.search(r"if \(o != \(uint32_t\)S - 1\) return 0;", fin)
    # call sites: each split's stores are waited for before it counts itself in
    step = function_body(text, "void k_step(")
    i_ex = step.index("row_exchange(rsync, S, polls)")
    i_fin = step.index("row_finish(rsync, S)")
    before_ex = step[:i_ex]
    assert before_ex.rindex("stores_done();") > before_ex.rindex("st_dev(krow + p, s_key[p]);")
    before_fin = step[:i_fin]
    assert before_fin.rindex("stores_done();") > before_fin.rindex("finish_split<")
    # keys are read only when the exchange succeeded; the merge only by the last
    after_ex = step[i_ex:]
    assert re.search(r"if \(s_flag\) \{\s*for \(int p = tid; p < n; p \+= NT\)\s*"
                     r"if \(\(p / PB\) % S != split\) s_key\[p\] = ld_dev\(krow \+ p\);", after_ex)
    assert re.search(r"if \(!s_flag\) \{[^}]*return;\s*\}\s*merge_row<", step[i_fin:])
