// index_check.hip -- the kernels' integer index arithmetic, checked on the
// CPU (no GPU call is made).  Built with hipcc as a host program from the
// same header the kernels use (attn_common.h) and run by
// tests/test_index_cpu.py.
//
// For the 16-bit forward, the backward, the fp8 forward and the paged
// decode it enumerates every lane, step and launch shape and checks:
//   * each XOR swizzle maps a row's 16-byte units onto themselves (a
//     bijection within the row);
//   * the tile copies: the units the waves of a workgroup fill cover the
//     tile exactly once, every source offset lies inside the tile, and the
//     unit placed at each LDS position is the logical unit the swizzle puts
//     there;
//   * the fragment reads: every LDS offset lies inside its tile, and each
//     lane's 16-byte K fragment is the row and d-range the MFMA operand
//     layout needs; the transposing V reads are simulated lane by lane
//     (lane 4a + b of each 16-lane group receives element b of the chunks of
//     lanes a, a+4, a+8, a+12) and every element a lane receives must be the
//     V^T element its operand slot needs;
//   * the key tiles of each workgroup for every launch shape, mask and a set
//     of ragged lengths: the groups' shares partition the workgroup's tiles,
//     every tile holding a visible (query, key) pair of a wave is processed
//     and not skipped, tiles marked full hold only visible pairs, skipped
//     tiles none;
//   * the merge slots of the split shapes fit their LDS buffers;
//   * the paged decode's even split of its tile list over W waves, for
//     seeded random batches (empty, short and clamped sequences, windows,
//     several row blocks, more than 64 sequences): each sequence's tiles hold
//     every key its query rows see; every wave's run, walked with the
//     kernel's own cursor steps from the kernel's own starting cursor, visits
//     list positions f_begin .. f_end - 1 in order (so the runs cover the
//     list exactly once), inside the sequences, heads and row blocks; every
//     result slot a wave writes lies below the slot count the workspace
//     holds; and the merge's wave range of each segment is exactly the set
//     of waves that wrote a result for it.
// Exit status 0 when every check holds; the first failures are printed.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "attn_common.h"

static int g_failures = 0;
#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        if (!(cond)) {                                                    \
            if (g_failures < 20) {                                        \
                std::printf("FAIL %s:%d: ", __FILE__, __LINE__);          \
                std::printf(__VA_ARGS__);                                 \
                std::printf("\n");                                        \
            }                                                             \
            ++g_failures;                                                 \
        }                                                                 \
    } while (0)

// ---------------------------------------------------------------- 16-bit tiles
// A tile of 64 rows x D 16-bit values in LDS: `lds_src[u]` = index of the
// source (global, row-major) 16-byte unit stored at LDS unit u.
template <int D, int KIND>
static std::vector<int> copy_tile_16(int rows, int nw, int chunks)
{
    const int units = rows * (D / 8);
    std::vector<int> lds_src(units, -1), seen(units, 0);
    for (int c = 0; c < chunks; ++c)
        for (int w = 0; w < nw; ++w)
            for (int lane = 0; lane < 64; ++lane) {
                const int unit_idx = (c * nw + w) * 64 + lane;  // LDS unit this lane fills
                CHECK(unit_idx < units, "copy unit %d outside the tile (%d units)", unit_idx, units);
                if (unit_idx >= units) continue;
                const int src = copy_src_offset<D, KIND>(unit_idx);
                CHECK(src >= 0 && src + 16 <= rows * 2 * D && src % 16 == 0, "copy source offset %d out of tile", src);
                lds_src[unit_idx] = src / 16;
                ++seen[src / 16 < units ? src / 16 : 0];
            }
    for (int u = 0; u < units; ++u) {
        CHECK(lds_src[u] >= 0, "LDS unit %d never filled (D=%d kind=%d)", u, D, KIND);
        CHECK(seen[u] == 1, "source unit %d copied %d times (D=%d kind=%d)", u, seen[u], D, KIND);
    }
    return lds_src;
}

// Which source unit a read at LDS byte offset `off` (16-byte aligned part)
// returns, and the byte within that unit.
static void lds_lookup(const std::vector<int> &lds_src, int off, int *src_unit, int *byte_in_unit)
{
    *src_unit = lds_src[off / 16];
    *byte_in_unit = off % 16;
}

template <int D>
static void check_swizzles()
{
    for (int kind = 0; kind < 3; ++kind)
        for (int row = 0; row < 64; ++row) {
            const int f = kind == 0 ? k_swizzle<D>(row) : (kind == 1 ? v_swizzle<D>(row) : dual_swizzle<D>(row));
            CHECK(f >= 0 && f < D / 8, "swizzle %d of row %d out of range (D=%d)", f, row, D);
            std::vector<int> hit(D / 8, 0);
            for (int u = 0; u < D / 8; ++u) ++hit[(u ^ f) % (D / 8)];
            for (int u = 0; u < D / 8; ++u) CHECK(hit[u] == 1, "swizzle kind %d row %d not a bijection", kind, row);
        }
    for (int row = 0; row < 64; ++row) {
        const int f = f8_swizzle<D>(row);
        CHECK(f >= 0 && f < D / 16, "fp8 swizzle %d of row %d out of range (D=%d)", f, row, D);
    }
}

// K fragments (A operand of S^T = K Q^T): lane l needs row 32 kb +
// k_row_for_lane(l % 32), d = 16 ds + 8 (l / 32) .. + 7, i.e. source unit
// row * D/8 + 2 ds + l / 32.
template <int D, int KIND>
static void check_k_reads(const std::vector<int> &lds_src, const char *what)
{
    for (int kb = 0; kb < 2; ++kb)
        for (int ds = 0; ds < D / 16; ++ds)
            for (int lane = 0; lane < 64; ++lane) {
                const int off = 32 * kb * 2 * D + k_frag_offset<D, KIND>(lane, ds);
                CHECK(off >= 0 && off + 16 <= 64 * 2 * D && off % 16 == 0, "%s: K read offset %d out of tile", what, off);
                int su, b;
                lds_lookup(lds_src, off, &su, &b);
                const int want = (32 * kb + k_row_for_lane(lane % 32)) * (D / 8) + 2 * ds + lane / 32;
                CHECK(su == want && b == 0, "%s: D=%d kb=%d ds=%d lane=%d reads unit %d, needs %d", what, D, kb, ds,
                      lane, su, want);
            }
}

// Transposing V reads for the A operand V^T of O^T += V^T P^T: after the
// reads at r4 = 0 and 1 of slice ks, lane l holds elements j = 4 r4 + c
// (c = 0..3) of V[16 ks + 8 (l / 32) + j][32 db + l % 32].  `row_step` > 0:
// the r4 = 1 read is the r4 = 0 address plus row_step bytes (the forward and
// the decode); else it uses v_tr_offset(..., 1) (the backward's dual swizzle).
template <int D, int KIND>
static void check_v_reads(const std::vector<int> &lds_src, int rows, int slices, int row_step, const char *what)
{
    for (int ks = 0; ks < slices; ++ks)
        for (int db = 0; db < D / 32; ++db)
            for (int r4 = 0; r4 < 2; ++r4) {
                int addr[64];
                for (int lane = 0; lane < 64; ++lane) {
                    int off = 16 * ks * 2 * D + v_tr_offset<D, KIND>(lane, db, row_step > 0 ? 0 : r4);
                    if (row_step > 0) {
                        off += r4 * row_step;
                        const int own = 16 * ks * 2 * D + v_tr_offset<D, KIND>(lane, db, r4);
                        CHECK(off == own, "%s: r4 = 1 by address step differs from its own offset", what);
                    }
                    CHECK(off >= 0 && off + 8 <= rows * 2 * D && off % 8 == 0, "%s: V read offset %d out of tile", what,
                          off);
                    addr[lane] = off;
                }
                for (int lane = 0; lane < 64; ++lane) {
                    const int g = lane / 16, a = (lane % 16) / 4, b = lane % 4;
                    for (int c = 0; c < 4; ++c) {
                        const int src_lane = 16 * g + a + 4 * c;
                        int su, byte;
                        lds_lookup(lds_src, addr[src_lane], &su, &byte);
                        // element b (16 bits) of the 8-byte chunk at that address
                        const int elem = su * 8 + byte / 2 + b;  // flat index row * D + d in the source tile
                        const int row = elem / D, d = elem % D;
                        const int want_row = 16 * ks + 8 * (lane / 32) + 4 * r4 + c;
                        const int want_d = 32 * db + lane % 32;
                        CHECK(row == want_row && d == want_d,
                              "%s: D=%d ks=%d db=%d r4=%d lane=%d slot %d gets V[%d][%d], needs V[%d][%d]", what, D, ks,
                              db, r4, lane, c, row, d, want_row, want_d);
                    }
                }
            }
}

template <int D>
static void check_16bit()
{
    check_swizzles<D>();
    // forward: K tile (K swizzle) and V tile (V swizzle), every workgroup size
    for (int nw : {2, 4, 8}) {
        const int chunks = 64 * (D / 8) / (64 * nw);
        const std::vector<int> k = copy_tile_16<D, kSwzK>(64, nw, chunks);
        const std::vector<int> v = copy_tile_16<D, kSwzV>(64, nw, chunks);
        check_k_reads<D, kSwzK>(k, "forward");
        check_v_reads<D, kSwzV>(v, 64, 4, 4 * 2 * D, "forward");
    }
    // backward: tiles read both ways (dual swizzle), V of dQ (K swizzle)
    {
        const std::vector<int> t = copy_tile_16<D, kSwzDual>(64, 4, 64 * (D / 8) / 256);
        check_k_reads<D, kSwzDual>(t, "backward");
        check_v_reads<D, kSwzDual>(t, 64, 4, 0, "backward");
        const std::vector<int> v = copy_tile_16<D, kSwzK>(64, 4, 64 * (D / 8) / 256);
        check_k_reads<D, kSwzK>(v, "backward V rows");
    }
    // paged decode: V tiles of 32 keys copied as two 16-row halves by one wave
    {
        const int half_copies = 16 * (D / 8) / 64;
        const std::vector<int> h = copy_tile_16<D, kSwzV>(16, 1, half_copies);
        // the second half is the same placement 16 rows further
        std::vector<int> v(32 * (D / 8));
        for (int u = 0; u < 16 * (D / 8); ++u) {
            v[u] = h[u];
            v[u + 16 * (D / 8)] = h[u] + 16 * (D / 8);
        }
        check_v_reads<D, kSwzV>(v, 32, 2, 4 * 2 * D, "decode");
    }
}

// ---------------------------------------------------------------- operand layouts
// The 32x32 accumulator of v_mfma_f32_32x32x16: register r of lane l holds
// row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.  With K rows fed in the
// order k_row_for_lane, S^T register r of lane half hi holds key 16 (r / 8) +
// 8 hi + r % 8 of its 32-key block (the mask and the weights use that), and
// the B operand of the second product (lane l: keys 8 (l / 32) + 0..7 of a
// 16-key slice, for query l % 32) is exactly registers 8 (ks % 2) + 0..7 of
// block ks / 2: the weights need no exchange between lanes.
static void check_operand_layout()
{
    for (int hi = 0; hi < 2; ++hi)
        for (int r = 0; r < 16; ++r) {
            const int acc_row = 8 * (r / 4) + 4 * hi + r % 4;  // A-operand row = S^T row
            CHECK(k_row_for_lane(acc_row) == 16 * (r / 8) + 8 * hi + r % 8,
                  "S^T register %d of half %d holds key %d", r, hi, k_row_for_lane(acc_row));
        }
    for (int ks = 0; ks < 4; ++ks)
        for (int hi = 0; hi < 2; ++hi)
            for (int e = 0; e < 8; ++e) {
                const int kb = ks / 2, r = 8 * (ks % 2) + e;
                const int key_held = 32 * kb + k_row_for_lane(8 * (r / 4) + 4 * hi + r % 4);
                CHECK(key_held == 16 * ks + 8 * hi + e, "P^T slice %d element %d of half %d is key %d", ks, e, hi,
                      key_held);
            }
    // k_row_for_lane is a permutation of 0..31
    int hit[32] = {};
    for (int m = 0; m < 32; ++m) ++hit[k_row_for_lane(m) & 31];
    for (int m = 0; m < 32; ++m) CHECK(hit[m] == 1, "k_row_for_lane is not a permutation");
}

// LDS bank conflicts of one read instruction under the two bank models the
// swizzles were chosen for: 32 banks x 4 bytes serving 128 bytes per cycle,
// or 64 banks serving 256 bytes; lanes are served in consecutive groups of
// (bytes per cycle / bytes per lane).  Two lanes of a group conflict when
// they touch the same bank at different addresses.
static int conflicts(const int *addr, int bytes_per_lane, int banks)
{
    const int group = banks * 4 / bytes_per_lane;
    int n = 0;
    for (int g0 = 0; g0 < 64; g0 += group) {
        int owner[64];
        for (int b = 0; b < banks; ++b) owner[b] = -1;
        for (int lane = g0; lane < g0 + group; ++lane)
            for (int w = 0; w < bytes_per_lane / 4; ++w) {
                const int word = addr[lane] / 4 + w;
                const int bank = word % banks;
                if (owner[bank] >= 0 && owner[bank] != word) ++n;
                owner[bank] = word;
            }
    }
    return n;
}

template <int D, int KIND>
static void check_bank_conflicts(bool v_reads, const char *what)
{
    for (int banks : {32, 64}) {
        int n = 0, addr[64];
        for (int kb = 0; kb < 2; ++kb)
            for (int ds = 0; ds < D / 16; ++ds) {
                for (int lane = 0; lane < 64; ++lane) addr[lane] = 32 * kb * 2 * D + k_frag_offset<D, KIND>(lane, ds);
                n += conflicts(addr, 16, banks);
            }
        CHECK(n == 0, "%s: %d bank conflicts of the K fragment reads (D=%d, %d banks)", what, n, D, banks);
        if (!v_reads) continue;
        n = 0;
        for (int ks = 0; ks < 4; ++ks)
            for (int db = 0; db < D / 32; ++db)
                for (int r4 = 0; r4 < 2; ++r4) {
                    for (int lane = 0; lane < 64; ++lane)
                        addr[lane] = 16 * ks * 2 * D + v_tr_offset<D, KIND>(lane, db, r4);
                    n += conflicts(addr, 8, banks);
                }
        CHECK(n == 0, "%s: %d bank conflicts of the transposing reads (D=%d, %d banks)", what, n, D, banks);
    }
}

template <int D, int KIND>
static void check_v_bank_conflicts(const char *what)
{
    for (int banks : {32, 64}) {
        int n = 0, addr[64];
        for (int ks = 0; ks < 4; ++ks)
            for (int db = 0; db < D / 32; ++db)
                for (int r4 = 0; r4 < 2; ++r4) {
                    for (int lane = 0; lane < 64; ++lane)
                        addr[lane] = 16 * ks * 2 * D + v_tr_offset<D, KIND>(lane, db, r4);
                    n += conflicts(addr, 8, banks);
                }
        CHECK(n == 0, "%s: %d bank conflicts of the transposing reads (D=%d, %d banks)", what, n, D, banks);
    }
}

// ---------------------------------------------------------------- fp8 tiles
template <int D>
static void check_fp8()
{
    const int units = 2 * 64 * D / 16;  // K tile then V tile, 16-byte units
    for (int nw : {4, 8}) {
        const int chunks = units / (64 * nw);
        std::vector<int> lds_src(units, -1), seen(units, 0);
        for (int c = 0; c < chunks; ++c)
            for (int w = 0; w < nw; ++w)
                for (int lane = 0; lane < 64; ++lane) {
                    const int unit = (c * nw + w) * 64 + lane;
                    const int src = f8_copy_src_offset<D>(unit);
                    CHECK(src >= 0 && src + 16 <= 64 * D && src % 16 == 0, "fp8 copy source %d out of tile", src);
                    const int tile = unit / (units / 2);
                    const int su = tile * (units / 2) + src / 16;
                    lds_src[unit] = su;
                    ++seen[su];
                }
        for (int u = 0; u < units; ++u) CHECK(seen[u] == 1 && lds_src[u] >= 0, "fp8 unit %d copied %d times", u, seen[u]);
        // K fragments: lane l needs row 32 kb + k_row_for_lane(l % 32), bytes
        // 64 ds + 32 (l / 32) + 16 sp .. + 15, i.e. unit 4 ds + 2 (l / 32) + sp
        for (int kb = 0; kb < 2; ++kb)
            for (int ds = 0; ds < D / 64; ++ds)
                for (int sp = 0; sp < 2; ++sp)
                    for (int lane = 0; lane < 64; ++lane) {
                        const int off = 32 * kb * D + f8_k_frag_offset<D>(lane, ds, sp);
                        CHECK(off >= 0 && off + 16 <= 64 * D && off % 16 == 0, "fp8 K read %d out of tile", off);
                        const int want = (32 * kb + k_row_for_lane(lane % 32)) * (D / 16) + 4 * ds + 2 * (lane / 32) + sp;
                        CHECK(lds_src[off / 16] == want, "fp8 K: D=%d lane=%d kb=%d ds=%d sp=%d", D, lane, kb, ds, sp);
                    }
        // V transposing reads: read rho = 2 kb + t at the base + (32 kb + 16 t)
        // rows addresses key row 32 kb + 16 t + 8 (grp / 2) + li / 2, d bytes
        // 32 db + 16 (grp % 2) + 8 (li % 2) .. + 7
        for (int rho = 0; rho < 4; ++rho)
            for (int db = 0; db < D / 32; ++db)
                for (int lane = 0; lane < 64; ++lane) {
                    const int kb = rho / 2, t = rho % 2, grp = lane / 16, li = lane % 16;
                    const int off = (32 * kb + 16 * t) * D + f8_v_tr_offset<D>(lane, db);
                    CHECK(off >= 0 && off + 8 <= 64 * D && off % 8 == 0, "fp8 V read %d out of tile", off);
                    const int su = lds_src[units / 2 + off / 16] - units / 2;
                    const int byte = su * 16 + off % 16;
                    const int row = byte / D, d = byte % D;
                    CHECK(row == 32 * kb + 16 * t + 8 * (grp / 2) + li / 2 && d == 32 * db + 16 * (grp % 2) + 8 * (li % 2),
                          "fp8 V: D=%d lane=%d rho=%d db=%d reads row %d byte %d", D, lane, rho, db, row, d);
                }
    }
}

// ---------------------------------------------------------------- key tiles
template <bool CAUSAL, bool WINDOW, int SPLIT>
static void check_tiles_for(int nw, int L, int window)
{
    const int block_q = 32 * nw, block_k = 64;
    const int n_qblk = (L + block_q - 1) / block_q, n_tiles = (L + block_k - 1) / block_k;
    for (int qblk = 0; qblk < n_qblk; ++qblk) {
        const int q_first = qblk * block_q, q_last = (q_first + block_q < L ? q_first + block_q : L) - 1;
        std::vector<int> owner(n_tiles + SPLIT * n_tiles + 8, -1);
        int steps = -1;
        for (int grp = 0; grp < SPLIT; ++grp) {
            const TileRange r = key_tiles<CAUSAL, WINDOW, SPLIT>(q_first, q_last, L, window, block_k, grp);
            CHECK(r.t_begin >= 0 && r.t_stop >= r.t_end, "tile range [%d, %d) stop %d", r.t_begin, r.t_end, r.t_stop);
            if (steps < 0) steps = r.t_stop - r.t_begin;
            CHECK(r.t_stop - r.t_begin == steps, "groups run different step counts");
            for (int t = r.t_begin; t < r.t_end; ++t) {
                CHECK(t < n_tiles, "tile %d past the keys (L=%d)", t, L);
                if (t < n_tiles) {
                    CHECK(owner[t] == -1, "tile %d in two groups", t);
                    owner[t] = grp;
                }
            }
        }
        for (int w = 0; w < nw; ++w) {
            const int qa = q_first + 32 * w;
            if (qa >= L) continue;
            const int qb = (qa + 32 < L ? qa + 32 : L) - 1;
            for (int t = 0; t < n_tiles; ++t) {
                const int j0 = t * block_k;
                int visible_pairs = 0, pairs = 0;
                for (int i = qa; i <= qb; ++i)
                    for (int j = j0; j < j0 + block_k; ++j) {
                        ++pairs;
                        visible_pairs += visible<CAUSAL, WINDOW>(i, j, L, window) ? 1 : 0;
                    }
                const int cls = tile_class<CAUSAL, WINDOW>(j0, qa, qb, L, window, block_k);
                if (visible_pairs > 0) {
                    CHECK(owner[t] >= 0, "L=%d w=%d qblk=%d wave=%d: tile %d has visible keys but no group", L, window,
                          qblk, w, t);
                    CHECK(cls != 0, "L=%d window=%d wave rows %d..%d: tile %d skipped with visible keys", L, window, qa,
                          qb, t);
                }
                if (cls == 0) CHECK(visible_pairs == 0, "skipped tile %d has %d visible pairs", t, visible_pairs);
                if (cls == 1) CHECK(visible_pairs == pairs, "full tile %d has masked pairs (L=%d)", t, L);
            }
        }
    }
}

template <bool CAUSAL, bool WINDOW>
static void check_tiles_mask()
{
    const int lengths[] = {1, 2, 31, 63, 64, 65, 127, 128, 129, 255, 256, 300, 513, 777};
    const int windows[] = {0, 1, 37, 63, 64, 100, 200};
    for (int L : lengths)
        for (int wi = 0; wi < (WINDOW ? 7 : 1); ++wi) {
            const int window = WINDOW ? windows[wi] : -1;
            for (int nw : {2, 4, 8}) {
                check_tiles_for<CAUSAL, WINDOW, 1>(nw, L, window);
                check_tiles_for<CAUSAL, WINDOW, 2>(nw, L, window);
                check_tiles_for<CAUSAL, WINDOW, 4>(nw, L, window);
            }
        }
}

// ---------------------------------------------------------------- merge slots
template <int D, int NW, int SPLIT>
static void check_merge()
{
    typedef MergeLayout<D, NW, SPLIT> ML;
    CHECK(ML::kPerBuffer >= 1, "merge: no slot fits (D=%d NW=%d SPLIT=%d)", D, NW, SPLIT);
    for (int i = 0; i < ML::kBatch; ++i) {
        const int end = ML::slot_float_offset(i) * 4 + ML::kSlotBytes;
        CHECK(ML::slot_float_offset(i) >= 0 && end <= ML::kBufferBytes, "merge slot %d ends at byte %d of %d", i, end,
              ML::kBufferBytes);
        for (int j = 0; j < i; ++j)
            if ((i < ML::kPerBuffer) == (j < ML::kPerBuffer)) {
                const int a = ML::slot_float_offset(i), b = ML::slot_float_offset(j), n = 64 * ML::kPart;
                CHECK(a + n <= b || b + n <= a, "merge slots %d and %d overlap", i, j);
            }
    }
    CHECK(ML::kBatch <= 2 * ML::kPerBuffer, "merge batch larger than the slots");
}

// ---------------------------------------------------------------- paged decode partition
static uint64_t g_lcg = 12345;
static int rnd(int n)  // uniform in [0, n)
{
    g_lcg = g_lcg * 6364136223846793005ULL + 1442695040888963407ULL;
    return (int)((g_lcg >> 33) % (uint64_t)n);
}

static void check_decode_case(int B, int H_kv, int group, int Lq, int window, int max_len, int W_req,
                              const std::vector<int> &lens_raw)
{
    const DecodeShape sh = decode_shape(B, (int64_t)H_kv * group, H_kv, Lq, max_len);
    const int n_rowblk = (int)sh.n_rowblk, nseg = (int)sh.nseg;
    const int W = W_req < sh.waves_cap ? W_req : (int)sh.waves_cap;  // the launch takes min(resident, cap)
    auto len = [&](int b) {
        const int n = lens_raw[b] < 0 ? 0 : lens_raw[b];
        return n < max_len ? n : max_len;
    };
    std::vector<int64_t> first(B + 1, 0);
    std::vector<DecSeqTiles> st(B);
    for (int b = 0; b < B; ++b) {
        const int n = len(b);
        st[b] = decode_seq_tiles(n, Lq, window);
        CHECK(st[b].t_lo >= 0 && st[b].t_hi >= st[b].t_lo, "decode: sequence %d tiles [%d, %d)", b, st[b].t_lo, st[b].t_hi);
        // every key a query row of the sequence sees lies in its tiles
        for (int i = 0; i < Lq; ++i) {
            const int pos = n - Lq + i;
            if (pos < 0) continue;
            const int lo = window >= 0 && pos - window > 0 ? pos - window : 0;
            CHECK(lo >= kDecTile * st[b].t_lo && pos < kDecTile * st[b].t_hi,
                  "decode: n=%d Lq=%d window=%d row %d sees keys %d..%d outside tiles [%d, %d)", n, Lq, window, i, lo,
                  pos, st[b].t_lo, st[b].t_hi);
        }
        first[b + 1] = first[b] + (int64_t)(st[b].t_hi - st[b].t_lo) * nseg;
    }
    const int64_t total = first[B];
    int64_t P = (total + W - 1) / W;
    if (P < kMinTiles) P = kMinTiles;
    // segment index (b, g, rb) -> the waves that wrote a result for it
    std::vector<int64_t> seg_lo((size_t)B * nseg, -1), seg_hi((size_t)B * nseg, -1);
    for (int w = 0; w < W; ++w) {
        const int64_t f0 = (int64_t)w * P, f1 = f0 + P < total ? f0 + P : total;
        if (f0 >= f1) continue;
        int b = 0;
        while (first[b + 1] <= f0) ++b;  // the sequence whose tiles hold f0
        DecCursor c = decode_cursor_at(b, len(b), st[b], f0 - first[b], n_rowblk);
        int last_seg = -1;
        for (int64_t f = f0; f < f1; ++f) {
            const bool inside = c.b >= 0 && c.b < B && c.g >= 0 && c.g < H_kv && c.rb >= 0 && c.rb < n_rowblk &&
                                c.t >= c.t_lo && c.t < c.t_hi;
            CHECK(inside, "decode: wave %d at f=%lld: cursor b=%d g=%d rb=%d t=%d [%d, %d) out of range", w,
                  (long long)f, c.b, c.g, c.rb, c.t, c.t_lo, c.t_hi);
            if (!inside) return;
            const int64_t pos = first[c.b] + (int64_t)(c.g * n_rowblk + c.rb) * (c.t_hi - c.t_lo) + (c.t - c.t_lo);
            CHECK(pos == f, "decode: wave %d step f=%lld is at list position %lld", w, (long long)f, (long long)pos);
            CHECK(c.t_lo == st[c.b].t_lo && c.t_hi == st[c.b].t_hi && c.n == len(c.b), "decode: cursor tiles stale");
            const int seg = (c.b * H_kv + c.g) * n_rowblk + c.rb;
            if (seg != last_seg) {
                const int64_t slot = (int64_t)w + seg;
                CHECK(slot < sh.n_slots, "decode: slot %lld of %lld", (long long)slot, (long long)sh.n_slots);
                if (seg_lo[seg] < 0) seg_lo[seg] = w;
                CHECK(seg_hi[seg] < w, "decode: wave %d writes segment %d twice or out of order", w, seg);
                seg_hi[seg] = w;
                last_seg = seg;
            }
            c = decode_next_tile(c, B, H_kv, n_rowblk, Lq, window, len);
        }
        // past the end of the run the cursor stays inside the batch (its tile is
        // loaded but not used)
        CHECK(c.b >= 0 && c.b < B && c.t >= 0, "decode: cursor past the run leaves the batch");
    }
    for (int b = 0; b < B; ++b)
        for (int sg = 0; sg < nseg; ++sg) {
            const int seg = b * nseg + sg;
            const int64_t tiles = st[b].t_hi - st[b].t_lo;
            if (tiles == 0) {
                CHECK(seg_lo[seg] < 0, "decode: empty segment %d has results", seg);
                continue;
            }
            const DecWaves ws = decode_segment_waves(first[b] + (int64_t)sg * tiles, tiles, P);
            CHECK(ws.lo == seg_lo[seg] && ws.hi == seg_hi[seg] && ws.hi < W,
                  "decode: segment %d: merge reads waves %lld..%lld, written by %lld..%lld (W=%d)", seg,
                  (long long)ws.lo, (long long)ws.hi, (long long)seg_lo[seg], (long long)seg_hi[seg], W);
        }
}

static void check_decode_partition()
{
    const int windows[] = {-1, -1, 0, 5, 100, 4096};
    const int waves[] = {1, 3, 64, 2048, 3072, 4096};
    for (int trial = 0; trial < 400; ++trial) {
        const int B = 1 + rnd(trial % 4 == 0 ? 150 : 12);
        const int H_kv = 1 + rnd(4), group = 1 + rnd(12), Lq = 1 + rnd(5);
        const int window = windows[rnd(6)];
        const int max_len = 1 + rnd(trial % 3 == 0 ? 20000 : 3000);
        std::vector<int> lens(B);
        for (int b = 0; b < B; ++b) {
            const int kind = rnd(6);
            lens[b] = kind == 0 ? 0 : kind == 1 ? -5 : kind == 2 ? max_len + 100 : kind == 3 ? 1 : rnd(max_len + 1);
        }
        check_decode_case(B, H_kv, group, Lq, window, max_len, waves[rnd(6)], lens);
    }
}

int main()
{
    check_operand_layout();
    check_bank_conflicts<64, kSwzK>(false, "forward K");
    check_bank_conflicts<128, kSwzK>(false, "forward K");
    check_v_bank_conflicts<64, kSwzV>("forward V");
    check_v_bank_conflicts<128, kSwzV>("forward V");
    check_bank_conflicts<64, kSwzDual>(true, "backward dual");
    check_bank_conflicts<128, kSwzDual>(true, "backward dual");
    check_16bit<64>();
    check_16bit<128>();
    check_fp8<64>();
    check_fp8<128>();
    check_tiles_mask<false, false>();
    check_tiles_mask<true, false>();
    check_tiles_mask<true, true>();
    check_tiles_mask<false, true>();
    // the split shapes the forward launches: 8x2 (d=64), 4x2, 4x4 (d=64), 2x4 (d=64)
    check_merge<64, 8, 2>();
    check_merge<64, 4, 2>();
    check_merge<128, 4, 2>();
    check_merge<64, 4, 4>();
    check_merge<64, 2, 4>();
    check_decode_partition();
    std::printf("%s (%d failures)\n", g_failures ? "INDEX CHECKS FAILED" : "all index checks passed", g_failures);
    return g_failures ? 1 : 0;
}
