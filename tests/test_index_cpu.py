"""The kernels' integer index arithmetic on the CPU: every lane -> LDS offset
of the tile copies and fragment reads (16-bit forward, backward, fp8
forward, paged decode) lies inside its tile and delivers the element the
MFMA operand layout needs, the swizzles are bijections, the key-tile ranges
and skip/full/edge classes are right for every launch shape, mask and a set
of ragged lengths, the merge slots fit, and the paged decode's even split of
its tile list visits every tile once and merges exactly the waves that
wrote (tests/index_check.hip, built with hipcc as a host program from the
kernels' own header).  Planted
mistakes in a copy of the header must make it fail."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_25_amd", "csrc")
SOURCE = os.path.join(ROOT, "tests", "index_check.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build_and_run(tmp, header_dir=CSRC):
    exe = os.path.join(tmp, "index_check")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", header_dir,
                    "-I", os.path.join(ROOT, "include"), "-o", exe, SOURCE], check=True,
                   stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return subprocess.run([exe], capture_output=True, text=True, timeout=120)


def test_index_arithmetic(tmp_path):
    r = build_and_run(str(tmp_path))
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "all index checks passed" in r.stdout


MUTANTS = {
    "k_row_bits_not_swapped": ("return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);", "return m;"),
    "k_swizzle_bit_dropped": ("return (b0 ^ b2) | (b1 << 1) | (b3 << 2) | (D == 128 ? (b2 << 3) : 0);",
                              "return (b0 ^ b2) | (b1 << 1) | (D == 128 ? (b2 << 3) : 0);"),
    "v_swizzle_wrong_bits": ("return (c << 1) | (D == 128 ? ((c & 1) << 3) : 0);",
                             "return (c << 2) | (D == 128 ? ((c & 1) << 3) : 0);"),
    "v_read_unit_order": ("const int unit = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);",
                          "const int unit = 4 * db + ((lane >> 4) & 1) + 2 * ((lane & 3) >> 1);"),
    "k_frag_half_ignored": ("return swizzled_offset(row, 2 * ds + lane / 32, swizzle_of<D, KIND>(row), 2 * D);",
                            "return swizzled_offset(row, 2 * ds, swizzle_of<D, KIND>(row), 2 * D);"),
    "copy_wrong_units_per_row": ("const int row = lds_unit / (D / 8), phys = lds_unit % (D / 8);",
                                 "const int row = lds_unit / (D / 16), phys = lds_unit % (D / 16);"),
    "split_share_rounds_down": ("const int chunk = (t_last - t_first + SPLIT - 1) / SPLIT;",
                                "const int chunk = (t_last - t_first) / SPLIT;"),
    "causal_range_one_short": ("if (CAUSAL) kv_end = q_last + 1;", "if (CAUSAL) kv_end = q_last;"),
    "full_tile_ignores_tail": ("bool full = j_last < L;", "bool full = true;"),
    "window_skip_off_by_one": ("skip = skip || j_last < qa - window;", "skip = skip || j_last <= qa - window;"),
    "f8_v_row_half": ("const int row = 8 * (grp / 2) + li / 2;", "const int row = 8 * (grp % 2) + li / 2;"),
    "merge_slot_stride": ("return (i % kPerBuffer) * 64 * kPart; }", "return (i % kPerBuffer) * 32 * kPart; }"),
    "decode_tiles_end_rounds_down": ("st.t_hi = (n + kDecTile - 1) / kDecTile;", "st.t_hi = n / kDecTile;"),
    "decode_first_key_without_lq": ("return window >= 0 && n - Lq - window > 0 ? n - Lq - window : 0;",
                                    "return window >= 0 && n - window > 0 ? n - window : 0;"),
    "decode_row_block_wrap": ("if (++c.rb < n_rowblk) return c;", "if (++c.rb <= n_rowblk) return c;"),
    "decode_cursor_head_from_wrong_digit": ("c.g = seg / n_rowblk;", "c.g = seg % n_rowblk;"),
    "decode_merge_one_wave_too_many": ("w.hi = (f_seg + tiles - 1) / P;", "w.hi = (f_seg + tiles) / P;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_index_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(os.path.join(CSRC, "attn_common.h")).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    hdr = tmp_path / "hdr"
    hdr.mkdir()
    (hdr / "attn_common.h").write_text(src.replace(old, new))
    r = build_and_run(str(tmp_path), str(hdr))
    assert r.returncode != 0, f"planted mistake {name} not caught:\n{r.stdout}"
