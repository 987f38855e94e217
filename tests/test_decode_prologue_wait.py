"""The decode kernels' first read of their LDS scale bytes comes after a
wait that covers the direct-to-LDS copies of those bytes, in the compiled
gfx950 code of every instantiation.

The copies (`buffer_load ... lds`) are issued before the code loads of the
ring; vector memory operations complete in order, so a wait `vmcnt(X)` with
at most X loads issued after the last copy has seen the copies land.  The
kernels wait for a count of the ring's loads where every wave has enough
tiles (the count is right only while the compiler issues all of the ring's
loads before the wait, which it did not when the loop's first pass sat
behind a branch), else for vmcnt(0).  The compiler does not track the LDS
writes of these copies itself.  Checked on the assembly in program text
order from the last copy to the first `ds_read`."""
import re


def _copies_landed_before_first_lds_read(insts):
    copies = [i for i, s in enumerate(insts) if s.startswith("buffer_load") and s.endswith(" lds")]
    assert copies, "no direct-to-LDS copy found"
    issued, landed = 0, False
    for s in insts[copies[-1] + 1:]:
        if s.startswith("s_waitcnt") and "vmcnt" in s:
            if int(re.search(r"vmcnt\((\d+)\)", s).group(1)) <= issued:
                landed = True
        elif s.startswith(("buffer_load", "global_load")) and not s.endswith(" lds"):
            issued += 1
        elif s.startswith("ds_read"):
            return landed
    raise AssertionError("no LDS read after the copies")


def test_decode_scale_copies_land_before_their_first_read(gemm_kernels_asm):
    decode = {k: v for k, v in gemm_kernels_asm.items() if k.startswith("_ZN") and "gemm_decode_kernel" in k}
    assert len(decode) >= 16, f"only {len(decode)} decode kernels found: the listing format changed"
    counted = [k for k in decode if "ELb1E" in k]
    assert counted, "no instantiation with the counted wait"
    bad = [k for k, ins in decode.items() if not _copies_landed_before_first_lds_read(ins)]
    assert not bad, f"{len(bad)} decode kernels may read scale bytes before their copies land: {bad[:3]}"
