"""Device-code hashes of the build (host logic, no GPU): the per-kernel hash
that decides whether a committed counter profile still describes the built
kernel ignores what another kernel of the same source shifts (the function
index in local labels, the compiler's comments, the compile-unit id) and
changes with any instruction of the kernel itself."""

from decode_attention_03_amd.build import assembly_sha256


def _asm(first_index, second_index, comment, extra_instr=""):
    return f"""\t.text
__hip_cuid_{first_index:x}abc:
_Z1av:                                  ; @_Z1av
\ts_mov_b32 s0, 1                    ; {comment}
.LBB{first_index}_1:                  ; =>This Loop Header: Depth=1
\ts_cbranch_scc1 .LBB{first_index}_1
\ts_endpgm
.Lfunc_end{first_index}:
_Z1bv:
\tv_mov_b32 v0, 0
{extra_instr}.LBB{second_index}_2:
\ts_cbranch_scc0 .LBB{second_index}_2   ;   in Loop: Header=BB{second_index}_2 Depth=1
\ts_endpgm
.Lfunc_end{second_index}:
"""


def test_label_indices_and_comments_do_not_change_kernel_hashes():
    w0, k0 = assembly_sha256(_asm(0, 1, "first"))
    w1, k1 = assembly_sha256(_asm(2, 5, "other words"))
    assert set(k0) == {"_Z1av", "_Z1bv"}
    assert k0 == k1 and w0 == w1


def test_an_instruction_changes_only_its_kernel_hash():
    _, k0 = assembly_sha256(_asm(0, 1, "x"))
    _, k1 = assembly_sha256(_asm(0, 1, "x", extra_instr="\tv_add_f32 v0, v0, v0\n"))
    assert k0["_Z1av"] == k1["_Z1av"]
    assert k0["_Z1bv"] != k1["_Z1bv"]
