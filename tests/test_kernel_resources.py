"""Register, scratch and LDS use of every kernel, from hipcc's resource-usage
remarks for gfx950 (a device-only compile on the CPU; no GPU needed).

Why this matters for correctness, not only speed: the LDS-staged and
row-in-LDS backward kernels wait for their direct buffer-to-LDS loads with
hand-counted `s_waitcnt vmcnt(N)` immediates, N being the number of vector
memory operations the kernel itself issued after the loads it waits for.
Scratch accesses (register spills) are vector memory operations too and
count in vmcnt, so a spill inserted by the compiler would make such a wait
return before the staged row has landed: the kernel would read stale LDS and
write a wrong dx, silently.  The kernels with counted waits must compile with
no scratch and no spill of any kind (they are named explicitly, so that the
test also fails if they ever disappear from the report); the others may not
use scratch either, except a few known builds for rows wider than every
configured workload."""
import pytest

from bwd_rmsnorm_fwd_amd import _build

SOURCES = list(_build.SOURCES)
COUNTED_WAIT_KERNELS = ("bwd_rows_staged_kernel", "bwd_rows_ldsrow_kernel")


@pytest.fixture(scope="module")
def usage():
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=4) as ex:
        parts = list(ex.map(_build.resource_usage, SOURCES))
    return dict(zip(SOURCES, parts))


def test_every_source_reports_kernels(usage):
    total = sum(len(u) for u in usage.values())
    assert total > 50, {s: len(u) for s, u in usage.items()}


# Builds that do use scratch today, all for rows wider than every configured
# workload: the fp32 forward of rows past 16384 (residual) or 32768 elements
# (1024-lane workgroups cap a lane at 128 VGPRs), and the streaming backward
# recomputing r for fp32 rows past 32768 and bf16 rows past 32768 elements.
# None of them counts its waits by hand.  The list may only shrink: a build
# not named here that starts to use scratch fails the test.
KNOWN_SCRATCH = {
    "_ZN3rms10fwd_kernelIfLi4ELi1024ELi8ELi1024ELb1EEEvPKT_S3_S3_PS1_S4_Pflif",
    "_ZN3rms10fwd_kernelIfLi4ELi1024ELi16ELi1024ELb1EEEvPKT_S3_S3_PS1_S4_Pflif",
    "_ZN3rms10fwd_kernelIfLi4ELi1024ELi16ELi1024ELb0EEEvPKT_S3_S3_PS1_S4_Pflif",
    "_ZN3rms20bwd_rows_wide_kernelIfLi4ELi512ELi32ELb1ELb0EEEvPKT_S3_S3_PKfS3_PS1_Pfliif",
    "_ZN3rms20bwd_rows_wide_kernelIfLi4ELi512ELi32ELb0ELb0EEEvPKT_S3_S3_PKfS3_PS1_Pfliif",
    "_ZN3rms20bwd_rows_wide_kernelItLi8ELi512ELi16ELb1ELb0EEEvPKT_S3_S3_PKfS3_PS1_Pfliif",
    "_ZN3rms20bwd_rows_wide_kernelItLi8ELi512ELi16ELb0ELb0EEEvPKT_S3_S3_PKfS3_PS1_Pfliif",
}


@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch_outside_the_known_wide_builds(usage, src):
    """No kernel touches scratch memory except the known wide-row builds.
    (SGPR spills alone go to VGPR lanes, not to memory, and are allowed.)"""
    bad = {k: v for k, v in usage[src].items()
           if (v.get("ScratchSize", 0) or v.get("VGPRsSpill", 0)) and k not in KNOWN_SCRATCH}
    assert not bad, f"{src}: kernels with scratch or VGPR spills: {bad}"


def test_known_scratch_list_is_current(usage):
    every = {k for u in usage.values() for k in u}
    assert KNOWN_SCRATCH <= every, KNOWN_SCRATCH - every


def test_counted_wait_kernels_present_and_spill_free(usage):
    for name in COUNTED_WAIT_KERNELS:
        found = {k: v for u in usage.values() for k, v in u.items() if name in k}
        assert found, f"{name} missing from the resource report"
        for k, v in found.items():
            assert v["ScratchSize"] == 0 and v["VGPRsSpill"] == 0 and v["SGPRsSpill"] == 0, (k, v)
