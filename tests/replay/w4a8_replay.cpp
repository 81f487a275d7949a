// Host replay of the index arithmetic of the W4A8 GEMMs (one tile per workgroup, persistent, and
// the single-launch forward's item walk) and of the two front ends (the 1024-thread
// frontend_small_kernel and the single-launch forward's 256-thread one).
//
// The GEMM offsets come from the kernels' own functions (w4a8_index.h, compiled here for the
// host); the front ends' few index expressions are replayed loop by loop.  For every tile, chunk,
// wave and lane it checks that each buffer load lies inside its descriptor (or starts beyond it,
// so that it reads zero), that no 32-bit offset wraps, that every LDS access stays inside its
// array and every global store inside its buffer, and that the tiles of each list cover every
// row once (the multi-launch GEMMs' list, whose last tiles take up to 96 rows and three token
// blocks, and the single-launch forward's 64-row one).  Problem sizes: the W4A8 decode layer at every
// token count of its sweep, the small test cases, and random ones up to E = 256, k = 32 and 2048
// slots, with uniform, skewed, one-expert and dropped-slot routings.  Exit status 0: all in range.
#include <cstdio>
#include <cstdlib>
#include <cstdint>
#include <vector>
#include <string>

#include "../../token_permute_grouped_amd/csrc/w4a8_index.h"

using namespace tpg::w4;

static long g_checks = 0, g_fail = 0;
static std::string g_case;

static void fail(const char *what, long long a, long long b) {
    if (g_fail < 20) std::printf("OUT OF RANGE [%s] %s: %lld vs %lld\n", g_case.c_str(), what, a, b);
    ++g_fail;
}
// a load of `bytes` at voffset v + soffset so from a descriptor of n bytes: inside, or dead.  The
// loads that end exactly at their descriptor's end are counted (the checks are tight: the last
// bytes of every weight array and activation array are addressed).
static long g_exact_end = 0;
static void check_load(const char *what, uint32_t v, uint32_t so, int bytes, long long n) {
    ++g_checks;
    if ((unsigned long long)v + so >= (1ull << 32)) return fail(what, (long long)v + so, 1ll << 32);
    if ((long long)v >= n) return;  // past the descriptor: reads zero
    if ((long long)v + so + bytes > n) fail(what, (long long)v + so + bytes, n);
    if ((long long)v + so + bytes == n) ++g_exact_end;
}
static void check_range(const char *what, long long first, long long bytes, long long n) {
    ++g_checks;
    if (first < 0 || first + bytes > n) fail(what, first + bytes, n);
}

struct Rng {
    uint64_t s;
    uint32_t next() {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return (uint32_t)(s >> 33);
    }
    int below(int n) { return (int)(next() % (uint32_t)n); }
};

struct Problem {
    int T, H, I, E, k;
    bool mx, tiled;
};

// expert-major rows: counts per expert (dropped slots have none), offsets, row_src
struct Routing {
    std::vector<int> idx;  // [T*k]: expert or -1
    std::vector<int> offsets, row_src, slot_row;
    std::vector<int> tiles[2];  // tile lists: [0] 64-row m-tiles, [1] with merged last tiles
    int n_mt[2] = {0, 0};
};

static Routing make_routing(const Problem &p, int mode, Rng &rng) {
    Routing r;
    const int S = p.T * p.k;
    r.idx.assign(S, -1);
    for (int t = 0; t < p.T; ++t) {
        // k distinct experts per token
        std::vector<int> taken;
        for (int j = 0; j < p.k; ++j) {
            int e;
            for (;;) {
                if (mode == 1) e = (int)((double)p.E * (rng.next() / 4294967296.0) * (rng.next() / 4294967296.0));
                else if (mode == 2 && (int)taken.size() < p.k) e = (j == 0 ? 0 : rng.below(p.E));
                else e = rng.below(p.E);
                bool dup = false;
                for (int x : taken) dup |= x == e;
                if (!dup) break;
                if (mode == 1) mode = 0;  // fall back to uniform for the remaining draws
            }
            taken.push_back(e);
            r.idx[t * p.k + j] = e;
        }
        if (mode == 3)
            for (int j = 0; j < p.k; ++j)
                if (rng.below(10) == 0) r.idx[t * p.k + j] = -1;
    }
    r.offsets.assign(p.E + 1, 0);
    for (int s = 0; s < S; ++s)
        if (r.idx[s] >= 0) r.offsets[r.idx[s] + 1]++;
    for (int e = 0; e < p.E; ++e) r.offsets[e + 1] += r.offsets[e];
    r.row_src.assign(S, -1);
    r.slot_row.assign(S, -1);
    std::vector<int> fill(r.offsets.begin(), r.offsets.end() - 1);
    for (int s = 0; s < S; ++s)
        if (r.idx[s] >= 0) {
            const int row = fill[r.idx[s]]++;
            r.row_src[row] = s;
            r.slot_row[s] = row;
        }
    // the tile lists of the W4A8 GEMMs: each expert's 64-row m-tiles together ([0], the
    // single-launch forward's), and the same with a last remainder of 1..32 rows (after at least
    // one full tile) left to the tile before it ([1], the multi-launch GEMMs')
    // (the merged list puts the experts whose last tile is a merged one first)
    for (int merge = 0; merge < 2; ++merge) {
        for (int section = 0; section < 2; ++section)
            for (int e = 0; e < p.E; ++e) {
                const int cnt = r.offsets[e + 1] - r.offsets[e];
                int n = (cnt + kBM - 1) / kBM;
                const bool merged_last = merge && cnt > kBM && cnt % kBM >= 1 && cnt % kBM <= kBM / 2;
                if (merged_last) --n;
                if (section == 0 && n != m_tiles(cnt, merge == 1)) fail("m-tiles of an expert", n, m_tiles(cnt, merge == 1));
                if ((section == 0) != merged_last) continue;
                for (int m = 0; m < n; ++m) {
                    r.tiles[merge].push_back(e);
                    r.tiles[merge].push_back(m * kBM);
                }
            }
        r.n_mt[merge] = (int)r.tiles[merge].size() / 2;
    }
    return r;
}

// index of expert e's first m-tile in tile list m
static int first_mt_of(const Routing &r, int m, int e) {
    for (int i = 0; i < r.n_mt[m]; ++i)
        if (r.tiles[m][2 * i] == e) return i;
    return -1;
}

static long long max_m_tiles(const Problem &p) { return ((long long)p.T * p.k + kBM - 1) / kBM + p.E; }

// one GEMM (swiglu: the first) over every tile of the list; kloop: whole-array descriptors (the
// persistent and single-launch forms), else per-tile ones; gather: activations from the token rows;
// merge: the multi-launch GEMMs' tile list (token blocks staged: exactly the tile's, up to three),
// else the single-launch forward's (at most two token blocks staged for every tile)
static void replay_gemm(const Problem &p, const Routing &r, bool swiglu, bool kloop, bool gather, bool rows_too,
                        bool merge) {
    const int ml = merge ? 1 : 0;
    const int n_mt = r.n_mt[ml];
    const int *tiles = r.tiles[ml].data();
    const int S = p.T * p.k, K = swiglu ? p.H : p.I, N = swiglu ? 2 * p.I : p.H;
    const int sb = p.mx ? 32 : 16, nc = K / kKC, nb_n = N / kBN;
    const int w_pitch = p.tiled ? kKC / 2 : K / 2, w_step = p.tiled ? 32 * (kKC / 2) : kKC / 2;
    const int s_pitch = p.tiled ? kKC / sb : K / sb, s_step = p.tiled ? 32 * (kKC / sb) : kKC / sb;
    const int a_rows = gather ? p.T : S;
    const long long max_tiles = max_m_tiles(p);
    if (n_mt > max_tiles) fail("tile count", n_mt, max_tiles);
    // every row of every expert in exactly one tile of each n-tile
    std::vector<int> cover((size_t)S * nb_n, 0);
    for (int v = 0; v < n_mt * nb_n; ++v) {
        const Tile t = tile_of(v, nb_n, r.offsets.data(), tiles, n_mt, merge);
        if (!t.valid || t.nt < 0 || t.nt >= nb_n || t.rows < 1) continue;
        for (int i = 0; i < t.rows && t.row_begin + i < S; ++i) cover[(size_t)(t.row_begin + i) * nb_n + t.nt]++;
    }
    for (int row = 0; row < r.offsets[p.E]; ++row)
        for (int nt = 0; nt < nb_n; ++nt)
            if (cover[(size_t)row * nb_n + nt] != 1) fail("row covered by tiles", cover[(size_t)row * nb_n + nt], 1);
    if (!swiglu) {
        // scatter epilogue (MOE_FLAG_SCATTER_Y): row r of the expert-major order goes to y row
        // row_src[r]; over the live rows these are the live slots, each exactly once
        std::vector<int> hit(S, 0);
        for (int row = 0; row < r.offsets[p.E]; ++row) {
            const int s = r.row_src[row];
            check_range("scatter destination row", s, 1, S);
            if (s >= 0 && s < S) hit[s]++;
        }
        for (int s = 0; s < S; ++s)
            if (hit[s] != (r.slot_row[s] >= 0 ? 1 : 0)) fail("scatter rows per slot", hit[s], r.slot_row[s] >= 0);
    }
    for (int v = 0; v < n_mt * nb_n; ++v) {
        const Tile t = tile_of(v, nb_n, r.offsets.data(), tiles, n_mt, merge);
        if (!t.valid) fail("tile of a live block", v, n_mt * nb_n);
        check_range("tile rows", t.row_begin, t.rows, (long long)r.offsets[t.e + 1]);
        if (t.rows < 1 || t.row_begin < r.offsets[t.e]) fail("tile rows", t.rows, t.row_begin);
        if (t.rows > (merge ? kMaxRows : kBM)) fail("tile rows", t.rows, merge ? kMaxRows : kBM);
        if (t.nt < 0 || t.nt >= nb_n) fail("n-tile", t.nt, nb_n);
        if (t.mt < 0 || t.mt >= n_mt) fail("m-tile", t.mt, n_mt);
        const int need = (t.rows + 31) / 32;
        for (int NTB = need; NTB <= (merge ? need : 2); ++NTB) {  // token blocks the kernel stages
        // descriptors
        const long long w_rows = kloop ? (long long)p.E * N : N;
        const long long nW = w_rows * (K / 2), nWs = w_rows * (K / sb);
        const long long nA = (long long)(gather || kloop ? a_rows : t.rows) * K;
        const long long nS = (long long)(gather || kloop ? a_rows : t.rows) * (K / 128) * 4;
        const int er = kloop ? t.e * N : 0;
        const int rb = kloop ? t.row_begin : 0;
        for (int wave = 0; wave < 4; ++wave) {
            const int blk = er + weight_row(swiglu, t.nt, wave, 0, p.I, 0);
            // every interleaved row of the block must be the block's own (weight_row(r) = row(0) + r)
            for (int il : {0, 32})
                for (int rl = 0; rl < 32; ++rl)
                    if (weight_row(swiglu, t.nt, wave, rl, p.I, il) != weight_row(swiglu, t.nt, wave, 0, p.I, il) + rl)
                        fail("weight block rows", rl, il);
            // weight offsets depend only on (expert, n-tile): once per pair; offsets grow linearly with
            // the chunk, so its first and last chunk bound every other
            if (t.mt != first_mt_of(r, ml, t.e) || NTB != need) continue;
            for (int lane = 0; lane < 64; ++lane)
                for (int c : {0, nc - 1}) {
                    for (int i = 0; i < 4; ++i)
                        check_load("weight codes",
                                   p.tiled ? w_code_off_tiled(blk, K, lane, i) : w_code_off(blk, K, lane, i, w_pitch),
                                   (uint32_t)(c * w_step), 16, nW);
                    check_load("weight scales",
                               p.tiled ? w_scale_off_tiled(blk, K, sb, lane) : w_scale_off(blk, K, sb, lane, s_pitch),
                               (uint32_t)(c * s_step), w_scale_bytes(sb), nWs);
                }
        }
        if (!rows_too) continue;  // the row addressing does not depend on the weight format or layout
        for (int tid = 0; tid < kThreads; ++tid) {
            const int g = act_gran(tid);
            for (int i = 0; i < NTB * 2; ++i) {
                const int row = act_row(tid, i);
                int rr;
                if (gather) {
                    const int s = r.row_src[t.row_begin + imin(row, t.rows - 1)];
                    if (s < 0 || s >= S) fail("row_src of a live row", s, S);
                    rr = s / p.k;
                } else {
                    rr = rb + row;
                }
                const uint32_t off = row >= t.rows ? kDeadOff : a_off(rr, K, g);
                for (int c : {0, nc - 1}) check_load("activations", off, (uint32_t)(c * kKC), 16, nA);
            }
            const int srow = act_scale_row(tid);
            int rs = gather ? r.row_src[t.row_begin + imin(srow, t.rows - 1)] / p.k : rb + srow;
            const uint32_t so = srow >= t.rows ? kDeadOff : s_off(rs, K);
            for (int c : {0, nc - 1}) check_load("activation scales", so, (uint32_t)(c * 8), 8, nS);
        }
        // the epilogue's stores (the LDS accesses, the same for every tile, are checked by replay_lds)
        for (int lane = 0; lane < 64; ++lane) {
            const int h = lane >> 5;
            (void)h;
            if (false) {
            for (int i = 0; i < 4; ++i) check_range("LDS weight write", lds_wcode(lane, i), 16, kWScales);
            check_range("LDS weight scale write", lds_wscale(lane, p.mx), p.mx ? 4 : 8, kWSlot);
            const int h = lane >> 5;
            for (int q = 0; q < 2; ++q) {
                for (int tt = 0; tt < 2; ++tt) {
                    check_range("LDS weight read", lds_wread(lane) + 64 * q + 16 * tt, 16, kWScales);
                    for (int tb = 0; tb < NTB; ++tb) {
                        const int rr = tb * 32 + (lane & 31);
                        check_range("LDS activation read", lds_act(rr, gran_lo(p.mx, q, tt, h)), 16, kActBuf);
                        check_range("LDS activation read", lds_act(rr, gran_hi(p.mx, q, tt, h)), 16, kActBuf);
                    }
                }
                check_range("LDS scale read", p.mx ? lds_wsread(lane) - 4 * h + 4 * q : lds_wsread(lane) + 8 * q, 4,
                            kWSlot);
                for (int tb = 0; tb < NTB; ++tb)
                    for (int buf = 0; buf < 2; ++buf)
                        check_range("LDS scale read", 4 * lds_xs(buf, tb * 32 + (lane & 31), q), 4, 4 * 2 * kMaxRows * 2);
            }
            }
            for (int wave = 0; wave < 4; ++wave)
                for (int tb = 0; tb < NTB; ++tb) {
                    const int tok = tb * 32 + (lane & 31);
                    if (tok >= t.rows) continue;
                    for (int g4 = 0; g4 < 4; ++g4) {
                        if (swiglu && wave < 2) {
                            const int col = h_col(t.nt, wave, g4, lane);
                            if (col + 4 > p.I) fail("h column", col + 4, p.I);
                            check_range("h store", ((long long)(t.row_begin + tok) * p.I + col) * 4, 16, (long long)S * p.I * 4);
                        }
                        if (!swiglu) {
                            const int col = y_col(t.nt, wave, g4, lane);
                            if (col + 4 > N) fail("y column", col + 4, N);
                            check_range("y store", ((long long)(t.row_begin + tok) * p.H + col) * 2, 8, (long long)S * p.H * 2);
                            check_range("y scatter store", ((long long)r.row_src[t.row_begin + tok] * p.H + col) * 2, 8,
                                        (long long)S * p.H * 2);
                        }
                    }
                }
        }
        }
    }
}

// GEMM1 split in two K halves (NVFP4 at decode sizes, one tile per workgroup): each half's chunk
// range, its partial-sum stores [2 halves][gate, up][S][I] and the re-quantisation's reads of them
static bool split_gemm1(const Problem &p) {
    const long long experts = p.E < (long long)p.T * p.k ? p.E : (long long)p.T * p.k;
    return experts * (2LL * p.I / 128) <= 256 && p.H % 512 == 0 && p.T <= 32;
}
static void replay_split(const Problem &p, const Routing &r) {
    const int S = p.T * p.k, nb_n = 2 * p.I / kBN, nc = p.H / kKC;
    const long long stride = (long long)S * p.I, n_part = 4 * stride;
    if (nc % 2 != 0) fail("K chunks of a split GEMM1", nc, 2);
    for (int v = 0; v < r.n_mt[1] * nb_n * 2; ++v) {
        const Tile t = tile_of(v >> 1, nb_n, r.offsets.data(), r.tiles[1].data(), r.n_mt[1], true);
        if (!t.valid) continue;
        if (t.rows > 32) fail("rows of a split tile", t.rows, 32);
        const int h = v & 1, c_first = h * (nc / 2), c_last = c_first + nc / 2 - 1;
        if (c_first < 0 || c_last >= nc) fail("chunk of a K half", c_last, nc);
        for (int wave = 0; wave < 4; ++wave)
            for (int lane = 0; lane < 64; ++lane) {
                const int tok = lane & 31;
                if (tok >= t.rows) continue;
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int col = h_col(t.nt, wave & 1, g4, lane);
                    if (col + 4 > p.I) fail("partial column", col + 4, p.I);
                    check_range("partial store",
                                ((2LL * h + (wave >> 1)) * stride + (long long)(t.row_begin + tok) * p.I + col) * 4, 16,
                                n_part * 4);
                }
            }
    }
    // the re-quantisation: row < offsets[E], lane's two columns of block b, in all four planes
    for (int row = 0; row < r.offsets[p.E]; ++row)
        for (int b = 0; b < p.I / 128; ++b)
            for (int pl = 0; pl < 4; ++pl)
                check_range("partial read", (pl * stride + (long long)row * p.I + b * 128 + 2 * 63) * 4, 8, n_part * 4);
}

// every LDS access of the tile pipeline (the same for every tile): activation and scale staging,
// weight staging, operand reads, the SwiGLU hand-over
static void replay_lds() {
    for (bool mx : {false, true})
        for (int NTB = 1; NTB <= 3; ++NTB) {
            for (int tid = 0; tid < kThreads; ++tid) {
                for (int i = 0; i < NTB * 2; ++i) check_range("LDS activation write", lds_act(act_row(tid, i), act_gran(tid)), 16, kActBuf);
                if (tid < NTB * 32) {
                    if (act_scale_row(tid) != tid) fail("activation scale row", act_scale_row(tid), tid);
                    for (int buf = 0; buf < 2; ++buf) check_range("LDS scale write", 4 * lds_xs(buf, tid, 0), 8, 4 * 2 * kMaxRows * 2);
                }
            }
            for (int lane = 0; lane < 64; ++lane) {
                const int h = lane >> 5;
                for (int i = 0; i < 4; ++i) check_range("LDS weight write", lds_wcode(lane, i), 16, kWScales);
                check_range("LDS weight scale write", lds_wscale(lane, mx), mx ? 4 : 8, kWSlot);
                for (int q = 0; q < 2; ++q) {
                    for (int tt = 0; tt < 2; ++tt) {
                        check_range("LDS weight read", lds_wread(lane) + 64 * q + 16 * tt, 16, kWScales);
                        for (int tb = 0; tb < NTB; ++tb) {
                            const int rr = tb * 32 + (lane & 31);
                            check_range("LDS activation read", lds_act(rr, gran_lo(mx, q, tt, h)), 16, kActBuf);
                            check_range("LDS activation read", lds_act(rr, gran_hi(mx, q, tt, h)), 16, kActBuf);
                        }
                    }
                    check_range("LDS scale read", mx ? lds_wsread(lane) - 4 * h + 4 * q : lds_wsread(lane) + 8 * q, 4,
                                kWSlot);
                    for (int tb = 0; tb < NTB; ++tb)
                        for (int buf = 0; buf < 2; ++buf)
                            check_range("LDS scale read", 4 * lds_xs(buf, tb * 32 + (lane & 31), q), 4, 4 * 2 * kMaxRows * 2);
                }
                for (int wu = 0; wu < 2; ++wu)
                    for (int tb = 0; tb < NTB; ++tb)
                        for (int v16 = 0; v16 < 16; ++v16)
                            check_range("LDS hand-over", 4 * lds_xch(wu, NTB, tb, v16, lane), 4, kActBuf);
            }
        }
}

// the tiled layout: its code granules and scale bytes fill each piece exactly once, and a lane's
// loads of a chunk (codes of step i = 2 q + t, its scale bytes) are the bytes its operands take:
// row l % 32, code granule 4 q + 2 h + t (h = l / 32), scale bytes 8 q + 4 h + 2 t, +1 (NVFP4) or
// 4 q + 2 h + t (MXFP4)
static void replay_tiled_layout() {
    std::vector<int> seen(256, 0);
    for (int r = 0; r < 32; ++r)
        for (int g = 0; g < 8; ++g) {
            const int pos = tiled_code_pos(r, g);
            check_range("tiled code granule", pos, 16, 4096);
            if (pos % 16 != 0) fail("tiled code granule alignment", pos, 16);
            else if (pos >= 0 && pos < 4096) seen[pos / 16]++;
        }
    for (int u = 0; u < 256; ++u)
        if (seen[u] != 1) fail("tiled code granule use", seen[u], 1);
    for (int lane = 0; lane < 64; ++lane)
        for (int i = 0; i < 4; ++i) {
            const int q = i >> 1, t = i & 1, h = lane >> 5;
            if ((int)w_code_off_tiled(0, kKC, lane, i) != tiled_code_pos(lane & 31, 4 * q + 2 * h + t))
                fail("tiled code load", lane, i);
        }
    for (bool mx : {false, true}) {
        const int sb = mx ? 32 : 16, per = kKC / sb;
        std::vector<int> used(32 * per, 0);
        for (int r = 0; r < 32; ++r)
            for (int j = 0; j < per; ++j) {
                const int pos = tiled_scale_pos(r, j, mx);
                check_range("tiled scale byte", pos, 1, 32 * per);
                if (pos >= 0 && pos < 32 * per) used[pos]++;
            }
        for (int u = 0; u < 32 * per; ++u)
            if (used[u] != 1) fail("tiled scale byte use", used[u], 1);
        for (int lane = 0; lane < 64; ++lane) {
            const int r = lane & 31, h = lane >> 5, base = (int)w_scale_off_tiled(0, kKC, sb, lane);
            check_range("tiled scale load", base, w_scale_bytes(sb), 32 * per);
            for (int q = 0; q < 2; ++q)
                for (int t = 0; t < 2; ++t) {
                    if (mx) {
                        if (base + 2 * q + t != tiled_scale_pos(r, 4 * q + 2 * h + t, true)) fail("tiled MX scale", lane, q);
                    } else {
                        for (int u = 0; u < 2; ++u)
                            if (base + 4 * q + 2 * t + u != tiled_scale_pos(r, 8 * q + 4 * h + 2 * t + u, false))
                                fail("tiled NV scale", lane, q);
                    }
                }
        }
    }
}

// the single-launch forward's counters, re-quantisation and combine
static void replay_fused_tails(const Problem &p, const Routing &r) {
    const int S = p.T * p.k, n_cb = p.I / 128, nb1 = 2 * p.I / kBN;
    const long long max_tiles = max_m_tiles(p);
    constexpr int kLine = 32;  // counters one 128-byte line apart
    const long long n_counters = (max_tiles * n_cb + max_tiles) * kLine;
    const int n_mt = r.n_mt[0];
    const int *tiles = r.tiles[0].data();
    for (int v = 0; v < n_mt * nb1; ++v) {
        const Tile t = tile_of(v, nb1, r.offsets.data(), tiles, n_mt, false);
        const int cb = t.nt >> 1;
        check_range("re-quantisation counter", ((long long)t.mt * n_cb + cb) * kLine, 1, max_tiles * n_cb * kLine);
        check_range("ready counter", (max_tiles * n_cb + t.mt) * kLine, 1, n_counters);
        for (int wave = 0; wave < 4; ++wave)
            for (int i = 0; i < kBM / 4; ++i) {
                const int rr = wave + 4 * i;
                if (rr >= t.rows) continue;
                const long long row = t.row_begin + rr;
                for (int lane = 0; lane < 64; ++lane) {
                    check_range("h32 read", (row * p.I + cb * 128 + 2 * lane) * 4, 8, (long long)S * p.I * 4);
                    check_range("h8 store", row * p.I + cb * 128 + 2 * lane, 2, (long long)S * p.I);
                }
                check_range("hs store", row * n_cb + cb, 1, (long long)S * n_cb);
            }
    }
    // each 128-column block of h: exactly two GEMM1 tiles per m-tile
    std::vector<int> pairs((size_t)n_mt * n_cb, 0);
    for (int v = 0; v < n_mt * nb1; ++v) {
        const Tile t = tile_of(v, nb1, r.offsets.data(), tiles, n_mt, false);
        pairs[(size_t)t.mt * n_cb + (t.nt >> 1)]++;
    }
    for (int c : pairs)
        if (c != 2) fail("GEMM1 tiles per 128-column block", c, 2);
    // the combine: token tok, 16-byte chunk c of its row, slots j (rows and weights staged in LDS)
    for (int tok = 0; tok < p.T; ++tok)
        for (int j = 0; j < p.k; ++j) {
            check_range("slot_row read", (long long)tok * p.k + j, 1, S);
            check_range("LDS slot row", j * 4, 4, 4096);
            const int row = r.slot_row[tok * p.k + j];
            if (row < 0) continue;
            check_range("y read", ((long long)row * p.H + (p.H / 8 - 1) * 8) * 2, 16, (long long)S * p.H * 2);
            check_range("y read", (long long)row * p.H * 2, 16, (long long)S * p.H * 2);
        }
    check_range("out store", ((long long)(p.T - 1) * p.H + (p.H / 8 - 1) * 8) * 2, 16, (long long)p.T * p.H * 2);
}

// the front ends: routing rows, LDS ids and counts, tables and tile list
// the single-workgroup tables kernel after the router (up to 2048 slots): slot s is thread
// s % 1024 of pass s / 1024, its counter group pass * 16 + wave, counters [2 * 16][256]
static void replay_tables_small(const Problem &p, const Routing &r) {
    const int S = p.T * p.k;
    if (S > 2048) fail("slots of the tables kernel", S, 2048);
    for (int s = 0; s < S; ++s) {
        const int x = r.idx[s];
        const int g = (s / 1024) * 16 + (s % 1024) / 64;
        if (x >= 0) {
            check_range("LDS count", (long long)g * 256 + x, 1, 2LL * 16 * 256);
            check_range("row_src store", r.slot_row[s], 1, S);
        }
        check_range("slot_row store", s, 1, S);
    }
    check_range("offsets store", p.E, 1, p.E + 1);
}

static void replay_front_end(const Problem &p, const Routing &r, int threads) {
    const int S = p.T * p.k, waves = threads / 64;
    const int sid_n = threads == 1024 ? 1024 : 2048;
    if (S > sid_n) fail("slots of the front end", S, sid_n);
    // routing: four 16-lane rows per wave, tokens t0 + lane / 16, t0 = 4 w + 4 waves i
    for (int w = 0; w < waves; ++w)
        for (int t0 = w * 4; t0 < p.T; t0 += waves * 4)
            for (int lane = 0; lane < 64; ++lane) {
                const int t = t0 + (lane >> 4);
                if (t >= p.T) continue;  // loads use token T - 1, nothing is stored
                const int i = lane & 15;
                for (int h = 0; h < 16; ++h) {
                    const int j = i + 16 * h;
                    if (j >= p.k) continue;
                    check_range("LDS expert id", (long long)t * p.k + j, 1, sid_n);
                    check_range("topk store", (long long)t * p.k + j, 1, S);
                }
                for (int q = 0; q < 16; ++q)
                    if (i + 16 * q < p.E) check_range("logit read", (long long)t * p.E + i + 16 * q, 1, (long long)p.T * p.E);
            }
    // counts, ranks: per-wave counters [waves][256], rows < S
    for (int s = 0; s < S; ++s) {
        const int x = r.idx[s];
        const int w = (s % threads) / 64;
        if (x >= 0) {
            check_range("LDS count", (long long)w * 256 + x, 1, (long long)waves * 256);
            check_range("row_src store", r.slot_row[s], 1, S);
        }
        check_range("slot_row store", s, 1, S);
    }
    check_range("offsets store", p.E, 1, p.E + 1);
    check_range("tile list", (long long)r.n_mt[0] * 2 - 1, 1, 2 * max_m_tiles(p));
    check_range("tile list", (long long)r.n_mt[1] * 2 - 1, 1, 2 * max_m_tiles(p));
}

// argv[1], if given: a file of further problems, one "T H I E k" line each (both weight formats,
// both layouts)
int main(int argc, char **argv) {
    g_case = "LDS";
    replay_lds();
    g_case = "tiled layout";
    replay_tiled_layout();
    Rng rng{12345};
    std::vector<Problem> probs;
    for (int T : {1, 2, 4, 8, 16, 32, 64, 128, 256})
        for (bool mx : {false, true})
            for (bool tiled : {false, true}) probs.push_back({T, 7168, 2048, 32, 8, mx, tiled});
    // the small W4A8 GPU cases (K multiples of 256)
    const int small[][5] = {{64, 256, 256, 8, 2}, {1, 256, 256, 4, 4}, {100, 512, 512, 6, 3}, {300, 768, 768, 5, 2},
                            {90, 512, 256, 4, 2}, {32, 1024, 1024, 64, 8}, {30, 512, 512, 6, 3}, {16, 1024, 1024, 32, 8},
                            {1, 1024, 512, 8, 4}, {2, 1024, 1024, 4, 2}, {200, 512, 512, 5, 2}, {96, 512, 256, 4, 4},
                            {97, 512, 256, 4, 4}, {16, 65536, 1024, 4, 2}, {65536, 32768, 256, 2, 1}};
    for (auto &c : small)
        for (bool mx : {false, true}) probs.push_back({c[0], c[1], c[2], c[3], c[4], mx, false});
    // random shapes: E up to 256, k up to 32, up to 2048 slots, H, I multiples of 1024
    for (int n = 0; n < 8; ++n) {
        const int E = 1 + rng.below(n < 4 ? 256 : 64), k = 1 + rng.below(E < 32 ? E : 32);
        const int T = 1 + rng.below(2048 / k < 256 ? 2048 / k : 256) / (n < 4 ? 4 : 1);
        probs.push_back({T, 1024 * (1 + rng.below(4)), 1024 * (1 + rng.below(3)), E, k, rng.below(2) == 1,
                         rng.below(2) == 1});
    }
    if (argc > 1) {
        FILE *f = std::fopen(argv[1], "r");
        if (!f) {
            std::printf("cannot open %s\n", argv[1]);
            return 2;
        }
        int T, H, I, E, k;
        while (std::fscanf(f, "%d %d %d %d %d", &T, &H, &I, &E, &k) == 5)
            for (bool mx : {false, true})
                for (bool tiled : {false, true}) probs.push_back({T, H, I, E, k, mx, tiled});
        std::fclose(f);
    }
    for (const Problem &p : probs)
        for (int mode = 0; mode < 4; ++mode) {
            char buf[160];
            std::snprintf(buf, sizeof buf, "T=%d H=%d I=%d E=%d k=%d %s %s routing %d", p.T, p.H, p.I, p.E, p.k,
                          p.mx ? "mxfp4" : "nvfp4", p.tiled ? "tiled" : "rows", mode);
            g_case = buf;
            const Routing r = make_routing(p, mode, rng);
            const bool fits = (long long)p.E * 2 * p.I * (p.H / 2) < (1ll << 31);
            const bool kloop_ok = p.H % 1024 == 0 && p.I % 1024 == 0 && fits;
            const bool rows_too = p.mx == p.tiled;  // once per shape and routing (two of the four formats)
            // multi-launch GEMMs (merged tile list): one tile per workgroup, and the persistent form
            // (T <= 32); the single-launch forward's GEMM phases (64-row tile list, two token blocks)
            for (int form = 0; form < 3; ++form) {
                const bool kloop = form > 0, merge = form < 2;
                if (kloop && !kloop_ok) continue;
                if (form == 1 && p.T > 32) continue;
                replay_gemm(p, r, true, kloop, true, rows_too, merge);   // the forward: GEMM1 gathers through row_src
                if (form < 2) replay_gemm(p, r, true, kloop, false, rows_too, merge);  // moe_grouped_ffn: GEMM1 on x_perm
                replay_gemm(p, r, false, kloop, false, rows_too, merge);
            }
            if (split_gemm1(p)) replay_split(p, r);
            const int S = p.T * p.k;
            if (kloop_ok && p.T <= 256 && S <= 2048 && rows_too) {
                replay_fused_tails(p, r);
                replay_front_end(p, r, 256);
            }
            if (S <= 1024 && p.T <= 256) replay_front_end(p, r, 1024);
            if (S <= 2048) replay_tables_small(p, r);
        }
    std::printf("%zu problems x 4 routings: %ld index checks, %ld out of range, %ld loads ending exactly at their "
                "buffer's end\n", probs.size(), g_checks, g_fail, g_exact_end);
    return g_fail == 0 && g_exact_end > 0 ? 0 : 1;
}
