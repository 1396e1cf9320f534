"""Static check of the built kernels: no workgroup barrier can be reached
while an LDS write of the same wave may still be in flight.

`__syncthreads()` is `s_barrier` plus the compiler's waits, and the compiler
has been seen to drop the LDS wait of a barrier at a loop head: the barrier
then lets other waves read LDS before the last writes land (a race that
shows up only now and then on the GPU). This test compiles every kernel
source for gfx950 to assembly with the library's own flags, splits each
kernel into basic blocks, and runs a forward dataflow over the control-flow
graph: the state is the number of LDS operations issued since the oldest
LDS write not yet proven complete (LDS operations of a wave complete in
order, so `s_waitcnt lgkmcnt(n)` with n at most that number proves the
write complete). Any `s_barrier` reached with an unproven write fails.
LDS-DMA tile copies (`global_load_lds_*`) are waited with vmcnt by the
kernels' own explicit waits and are not covered here.
"""
import os
import re
import subprocess
import tempfile

import pytest

from decode_attention_paged_amd import build as B

INF = 10 ** 9


def kernel_bodies(asm: str):
    """{kernel symbol: [instruction or label lines]} of an assembly file."""
    bodies, cur = {}, None
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\S*|[A-Za-z_]\w*):", line)
        if m and not line.startswith(".") and cur is None:
            cur = m.group(1)
            bodies[cur] = []
            continue
        if cur is not None and line.startswith(".Lfunc_end"):
            cur = None
            continue
        if cur is not None:
            t = line.split(";")[0].strip()
            if t and (not t.startswith(".") or re.match(r"^\.LBB\S*:$", t)):
                bodies[cur].append(t)
    return bodies


def unwaited_barriers(body):
    """Barriers reachable with an LDS write not proven complete."""
    blocks, cur = [], {"label": "__entry", "ins": []}
    for t in body:
        if re.match(r"^\.LBB\S*:$", t):
            blocks.append(cur)
            cur = {"label": t[:-1], "ins": []}
            continue
        cur["ins"].append(t)
        if t.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append(cur)
            cur = {"label": None, "ins": []}
    blocks.append(cur)
    blocks = [b for b in blocks if b["ins"] or b["label"]]
    index = {b["label"]: i for i, b in enumerate(blocks) if b["label"]}
    succ = []
    for i, b in enumerate(blocks):
        last = b["ins"][-1] if b["ins"] else ""
        s = []
        if last.startswith("s_branch"):
            s.append(index[last.split()[1]])
        elif last.startswith("s_cbranch"):
            s.append(index[last.split()[1]])
            s.append(i + 1)
        elif not last.startswith(("s_endpgm", "s_setpc")):
            s.append(i + 1)
        succ.append([j for j in s if j < len(blocks)])
    state_in = [INF] * len(blocks)
    state_in[0] = INF
    bad = set()
    changed = True
    while changed:
        changed = False
        for i, b in enumerate(blocks):
            d = state_in[i]
            for k, t in enumerate(b["ins"]):
                if t.startswith("s_barrier") and d < INF:
                    bad.add((i, k))
                if t.startswith("ds_"):
                    if d < INF:
                        d += 1
                    if t.startswith(("ds_write", "ds_store")):
                        d = min(d, 0)
                if t.startswith("s_waitcnt"):
                    m = re.search(r"lgkmcnt\((\d+)\)", t)
                    if m and d < INF and int(m.group(1)) <= d:
                        d = INF
            for j in succ[i]:
                if d < state_in[j]:
                    state_in[j] = d
                    changed = True
    nbar = sum(t.startswith("s_barrier") for b in blocks for t in b["ins"])
    return nbar, sorted(bad)


# ---------------------------------------------------------------- the checker
def _one(body):
    return unwaited_barriers(body)


def test_checker_flags_a_write_before_a_barrier():
    assert _one(["ds_write_b32 v0, v1", "s_barrier", "s_endpgm"])[1]


def test_checker_accepts_a_wait_between():
    assert not _one(["ds_write_b32 v0, v1", "s_waitcnt lgkmcnt(0)", "s_barrier", "s_endpgm"])[1]


def test_checker_counts_later_lds_operations():
    # two LDS reads after the write: lgkmcnt(2) proves it complete, (3) does not
    ok = ["ds_write_b32 v0, v1", "ds_read_b32 v2, v3", "ds_read_b32 v4, v3",
          "s_waitcnt lgkmcnt(2)", "s_barrier", "s_endpgm"]
    no = ok[:3] + ["s_waitcnt lgkmcnt(3)"] + ok[4:]
    assert not _one(ok)[1] and _one(no)[1]


def test_checker_follows_branches_and_loops():
    # the wait sits on one branch only: the other path reaches the barrier
    branchy = ["ds_write_b32 v0, v1", "s_cbranch_scc1 .LBB0_2",
               ".LBB0_1:", "s_waitcnt lgkmcnt(0)",
               ".LBB0_2:", "s_barrier", "s_endpgm"]
    assert _one(branchy)[1]
    # a write at the end of a loop body reaches the barrier at its head
    loop = [".LBB0_1:", "s_barrier", "ds_write_b32 v0, v1", "s_cbranch_scc1 .LBB0_1", "s_endpgm"]
    assert _one(loop)[1]
    fixed = [".LBB0_1:", "s_barrier", "ds_write_b32 v0, v1", "s_waitcnt lgkmcnt(0)",
             "s_cbranch_scc1 .LBB0_1", "s_endpgm"]
    assert not _one(fixed)[1]


# ---------------------------------------------------------------- the kernels
@pytest.fixture(scope="module")
def kernels():
    srcs = sorted(os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC) if f.endswith(".hip"))
    out = {}
    with tempfile.TemporaryDirectory() as tmp:
        for src in srcs:
            asm = os.path.join(tmp, os.path.basename(src) + ".s")
            cmd = [B.HIPCC] + B.COMMON + ["--offload-device-only", "-S", src, "-o", asm]
            res = subprocess.run(cmd, capture_output=True, text=True)
            assert res.returncode == 0, res.stderr[-2000:]
            for name, body in kernel_bodies(open(asm).read()).items():
                out[(os.path.basename(src), name)] = body
    return out


def test_every_kernel_waits_for_its_lds_writes_before_each_barrier(kernels):
    attn = [k for k in kernels if "attn_ws_kernel" in k[1]]
    assert len(attn) >= 9, "the attention kernel's instantiations were not found in the assembly"
    failures = []
    for (src, name), body in kernels.items():
        nbar, bad = unwaited_barriers(body)
        if "attn_ws_kernel" in name:
            assert nbar >= 10, (name, nbar)
        if bad:
            failures.append(f"{src}: {name}: {len(bad)} of {nbar} barriers")
    assert not failures, "barriers reachable with an LDS write in flight:\n" + "\n".join(failures)
