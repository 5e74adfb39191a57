// Launch-geometry choice and dispatch: for M <= 8 the 16-byte-piece streaming
// kernels (piece_b*.hip: dense, SwiGLU, affine b = 2, 4, 8), else the group
// streaming or tiled VALU kernels (proj_b*.hip); dense matrix-core kernels
// (mfma_*.hip) for dense and SwiGLU calls with M = 9..32, for large-N and
// wide small-N ones from M = 3 on and for short ones with K <= 2048 from
// M = 5 on; affine
// matrix-core kernels for 2-, 4- and 8-bit codes (affine_mfma*.hip; on small
// matrices from M = 5 on, affine_split.hip), at K = 4096 the multi-tile
// kernel where it measured fastest (affine_burst*.hip) and, where a K fits
// their LDS ring, for every width from M = 5 on (affine_tile_b*.hip); plus
// the code-unpack kernel.
#include "affine_mfma.h"
#include "affine_burst.h"
#include "affine_split.h"
#include "affine_tile.h"
#include "mfma_split.h"
#include "mfma_tile.h"
#include "piece_kernel.h"
#include "stream_kernel.h"

namespace aqg {
namespace {

int ctz_u(unsigned v) { int n = 0; while (v && !(v & 1u)) { v >>= 1; ++n; } return n; }

constexpr size_t kLdsBudget = detail::kLdsBudget;
constexpr int kValuThreads = detail::kMaxThreads;

LaunchCfg choose_valu(int bits, bool swiglu, int M, int N, int K)
{
    LaunchCfg c{};
    c.path = PATH_VALU;
    c.MT = 1;
    while (c.MT < M) c.MT <<= 1;
    const int UK = bits ? 64 : 8;
    int per_unit = 16;  // LDS bytes per (m, unit)
    if (bits) per_unit = (bits == 8 ? 16 * 16 : 16 * 8) + 8;
    const int U = K / UK;                                   // units per row
    // Lanes per row, 2^L.  Upper bound: a power of two dividing U (each lane
    // gets the same number of units), at most 64, and small enough that a
    // K-tile of 2^L units fits in LDS at the largest M.  Lower bound: 2^L
    // consecutive units span >= 128 contiguous bytes of a row.  Between the
    // two, the smallest L that still gives ~2048 wavefronts.  The choice
    // depends on (bits, N, K) only, so every M sums each output in the same
    // order.
    const int unit_bytes = bits ? 8 * bits : 16;
    int Lcap = ctz_u((unsigned)U);
    if (Lcap > 6) Lcap = 6;
    const int64_t fit_max = (int64_t)kLdsBudget / ((int64_t)32 * per_unit);
    while (Lcap > 0 && fit_max < (1 << Lcap)) --Lcap;
    int L = 0;
    while ((unit_bytes << L) < 128) ++L;
    if (L > Lcap) L = Lcap;
    while (L < Lcap && (((int64_t)N << L) >> 6) < 2048) ++L;
    const int64_t fit = (int64_t)kLdsBudget / ((int64_t)c.MT * per_unit);  // units per tile
    const int LPR = 1 << L;
    int64_t kt_units = (fit / LPR) * LPR;
    if (kt_units > U) kt_units = U;
    if (kt_units < LPR) kt_units = LPR;
    c.lpr_log2 = L;
    c.KT = (int)(kt_units * UK);
    c.lds = (size_t)c.MT * kt_units * per_unit;
    const int G = 64 >> L;
    const int64_t tiles1 = ((int64_t)N + G - 1) / G;        // wave tiles at R = 1
    c.R = (!swiglu && tiles1 >= 8192) ? 2 : 1;
    const int64_t wave_tiles = ((int64_t)N + G * c.R - 1) / (G * c.R);
    int64_t nw = kValuThreads / 64;
    if (nw > wave_tiles) nw = wave_tiles;
    c.nwaves = (int)nw;
    c.blocks = (int)((wave_tiles + nw - 1) / nw);
    return c;
}

// Matrix-core geometry: workgroups of 8 wavefronts = NR row groups x NK
// k-splits.  NK grows (up to 8) until there are ~2048 wavefronts; large N
// uses NK = 1 and two 16-row tiles per row group.  Depends on (N, K) only.
LaunchCfg choose_mfma(bool swiglu, int M, int N, int K)
{
    LaunchCfg c{};
    c.path = PATH_MFMA;
    c.MT = M <= 16 ? 16 : 32;
    const int64_t tiles16 = ((int64_t)N + 15) / 16;
    int nk = 1;
    while (nk < 8 && tiles16 * nk < 2048) nk <<= 1;
    const int nr = 8 / nk;
    c.R = (nk == 1 && tiles16 >= 4096) ? 2 : 1;
    c.ksplit_log2 = ctz_u((unsigned)nk);
    c.nwaves = 8;
    c.blocks = (int)((tiles16 + (int64_t)nr * c.R - 1) / ((int64_t)nr * c.R));
    int kt = (int)(kLdsBudget / ((size_t)c.MT * 2)) / 32 * 32;
    if (kt > K) kt = K;
    c.KT = kt;
    size_t lds = (size_t)c.MT * kt * 2;
    const size_t red = nk > 1 ? (size_t)c.nwaves * (swiglu ? 2 : 1) * c.R * (c.MT / 16) * 4 * 64 * 4 : 0;
    c.lds = lds > red ? lds : red;
    return c;
}

// Persistent matrix-core geometry for large N (M = 9..32, dense / SwiGLU):
// K a multiple of 64, at least 2048 row tiles of 16 rows, and x^T for the
// whole K plus the output staging fit in LDS at M = 32 with one 8-wavefront
// workgroup per CU.  The choice depends on (N, K) only, so every M = 9..32 of
// a shape takes it.
bool choose_mfma_stream(bool swiglu, int M, int N, int K, LaunchCfg& c)
{
    c = LaunchCfg{};
    if (K % 64 != 0) return false;
    const int64_t T = ((int64_t)N + 15) / 16;
    if (T < 2048) return false;
    const int64_t tmax = (T + 2047) / 2048;
    if (detail::mfma_stream_lds_bytes(32, K, tmax) > detail::kMfmaStreamLdsMax) return false;
    c.path = PATH_MFMA_STREAM;
    c.MT = M <= 16 ? 16 : 32;
    c.KT = K;
    c.nwaves = detail::kMfmaStreamThreads / 64;
    c.R = 1;
    (void)swiglu;
    return true;
}

// Large-N dense matrix-core geometry with whole tiles copied into LDS
// (mfma_tile.h): M = 5..32 padded to 16 or 32 columns, K = 512 .. 2048 in
// steps of 512, at least 2048 row tiles.  Depends on (N, K) only.
bool choose_mfma_tile(bool swiglu, int M, int N, int K, LaunchCfg& c)
{
    c = LaunchCfg{};
    if (!detail::mfma_tile_supported(N, K, swiglu)) return false;
    c.path = PATH_MFMA_TILE;
    c.MT = M <= 16 ? 16 : 32;
    c.KT = K;
    c.nwaves = detail::kMfmaTileWaves;
    c.R = 1;
    return true;
}

// Small-N matrix-core geometry (dense / SwiGLU; used from M = 9, or from
// M = 5 on matrices with N >= 4096 and K <= 2048): fewer than 2048
// row tiles of 16 and K/32 k-steps that split evenly into pairs over at most
// 16 wavefronts.  Depends on (N, K) only.
bool choose_mfma_split(bool swiglu, int M, int N, int K, LaunchCfg& c)
{
    c = LaunchCfg{};
    const int64_t T = ((int64_t)N + 15) / 16;
    const int spw = detail::mfma_split_spw(K, swiglu);
    if (T >= 2048 || spw == 0) return false;
    c.path = PATH_MFMA_SPLIT;
    c.MT = M <= 16 ? 16 : 32;
    c.KT = K;
    c.nwaves = (K / 32) / spw;
    c.blocks = (int)T;
    c.R = 1;
    return true;
}

// Small-N affine matrix-core geometry (2-, 4- and 8-bit codes; affine_split.h):
// whole 128-byte k-blocks per row split over at most 16 wavefronts; at most
// 256 row tiles of 16 for M = 5..16 and 128 for M = 17..32, which run in
// two 16-column workgroups per tile (4096 x 4096 at M = 32: 14.5-25 us that
// way, twice as many workgroups each staging x^T of K = 4096).  Depends on
// (bits, N, K) and the column bucket, and every M of a bucket computes each
// output the same way (both buckets alike with at most 128 tiles).
bool choose_affine_split(int bits, bool swiglu, int M, int N, int K, LaunchCfg& c)
{
    c = LaunchCfg{};
    const int64_t tiles = ((int64_t)N + 15) / 16;
    const int maxw = swiglu ? detail::affine_split_max_waves<2>() : detail::affine_split_max_waves<1>();
    // 3, 5, 6, 7 bits (per-lane code windows): from M = 1, and up to 256
    // row tiles at any M: the dot-product kernels these replace spend most
    // of their time unpacking (3584 x 1024 at M = 16: 14.2 -> 4.5 us, at
    // M = 2: 5.7 -> 4.0 us; fused SwiGLU 2 x 4096 x 1536 at M = 32: 58 ->
    // 12 us, at M = 2: 11.7 -> 7.3 us)
    const bool nat = !(bits == 2 || bits == 4 || bits == 8);
    const int min_m = (nat || swiglu) ? 1 : 5;   // SwiGLU: the caller picks below M = 5
    // (M = 17..32 up to 256 tiles where no 32-column tile ring serves:
    // 8-bit 4096 x 4096 at M = 32: 25.7 us against 290 on the VALU kernel)
    const int64_t max_tiles =
        (M > 16 && !swiglu && !nat && detail::affine_tile_supported(bits, N, K, 32)) ? 128 : 256;
    if (M < min_m || M > 32 || tiles > max_tiles || detail::affine_split_kpw(bits, K, maxw) == 0)
        return false;
    c.path = PATH_AFFINE_SPLIT;
    c.MT = M <= 16 ? 16 : 32;
    c.KT = K;
    c.R = 1;
    return true;
}

// Multi-tile affine geometry (affine_burst.h): K = 4096, at most 4 row tiles
// per workgroup on one CU each (up to 1024 tiles on 256 CUs), where it was
// measured fastest (us, against the kernel the shape ran on before; 4096 x
// 4096 = 256 tiles, 14336 x 4096 = 896):
//   2 bits from M = 3 (14336 x 4096 at M = 4: 11.5 against 16.2, M = 8:
//     11.8 against 14.2, M = 16: 13.1 against 15.3), at M = 2 on up to 256
//     tiles (4096 x 4096: 5.9 against 6.6);
//   4 bits from M = 3 (4096 x 4096 at M = 4: 7.2 against 9.0, M = 16: 8.8
//     against 9.5; 14336 x 4096 at M = 8: 14.5 against 15.0);
//   5 bits at M <= 2 on up to 256 tiles (M = 1: 9.9 against 10.5);
//   6, 7 bits at M = 3, 4 (14336 x 4096: 23.9 against 26.4, 25.8 against
//     29.3) and on up to 256 tiles at M <= 4 (6 bits) or M <= 2 (7 bits:
//     10.6 against 12.6 at M = 1);
//   8 bits at M = 3, 4 (14336 x 4096 at M = 4: 24.1 against 27.2) and on
//     more than 256 tiles from M = 5 (24.5 against 25.9 at M = 8), also at
//     M = 17..32 as two 16-column launches (no tile ring holds 32 columns
//     of 8-bit K = 4096 rows);
//   never at 3 bits (the per-lane windows load slower than the tile and
//     streaming kernels read them).
// Depends on (bits, N, K) and M: every M it serves computes each output
// the same way (16 columns per launch).
bool affine_burst_measured(int bits, int M, int64_t tiles)
{
    const bool small = tiles <= 256;
    switch (bits) {
        case 2: return M >= 3 || (M == 2 && small);
        case 4: return M >= 3;
        case 5: return small && M <= 2;
        case 6: return (M >= 3 && M <= 4) || (small && M <= 4);
        case 7: return (M >= 3 && M <= 4) || (small && M <= 2);
        case 8: return (M >= 3 && M <= 4) || (M >= 5 && !small);
        default: return false;
    }
}

bool choose_affine_burst(int bits, int M, int N, int K, LaunchCfg& c)
{
    c = LaunchCfg{};
    const int64_t tiles = ((int64_t)N + 15) / 16;
    int cus = 256;
    if (detail::device_cus(cus) != hipSuccess) cus = 256;
    if (!detail::affine_burst_supported(bits, N, K) || tiles > (int64_t)detail::kAffineBurstMaxTiles * cus) return false;
    // (fewer than 192 tiles: not measured here, the one-tile-per-workgroup
    // kernels keep them)
    if (tiles < 192) return false;
    if (M > 16 && !(bits == 8 && tiles > 256)) return false;
    if (M <= 16 && !affine_burst_measured(bits, M, tiles)) return false;
    c.path = PATH_AFFINE_BURST;
    c.MT = 16;
    c.KT = K;
    c.nwaves = 8;
    c.R = 1;
    return true;
}

// Affine matrix-core geometry with whole tiles copied into LDS (2- to 8-bit
// codes; affine_tile.h): M = 5..32 padded to 16 or 32 columns, the
// (bits, K) pairs with a tile ring.  Depends on (bits, N, K) and the column
// bucket.
bool choose_affine_tile(int bits, int M, int N, int K, LaunchCfg& c)
{
    c = LaunchCfg{};
    const int MT = M <= 16 ? 16 : 32;
    if (bits < 2 || bits > 8 || !detail::affine_tile_supported(bits, N, K, MT)) return false;
    c.path = PATH_AFFINE_TILE;
    c.MT = MT;
    c.KT = K;
    c.nwaves = detail::kMfmaTileWaves;
    c.R = 1;
    return true;
}

// Affine matrix-core geometry (2-, 4- and 8-bit codes): whole 128-byte
// k-blocks per row (K a multiple of 1024/bits) and K at most 4096.  With fewer
// than 2048 row tiles of 16 the workgroup's wavefronts split K (2, 4 or 8
// chunks, each at least one k-block) so that small matrices still spread over
// the chip; the workgroup's LDS (x^T, the X fragments, the wavefronts' tables
// and, with a split, the partial tiles) must fit a CU's.  Depends on (N, K,
// bits) and on whether M fits 16 columns.
bool choose_affine_mfma(int bits, int M, int N, int K, LaunchCfg& c)
{
    c = LaunchCfg{};
    if ((bits != 2 && bits != 4 && bits != 8) || (K * bits) % 1024 != 0 || K > 4096) return false;
    const int64_t T = ((int64_t)N + 15) / 16;
    const int MT = M <= 16 ? 16 : 32;
    const int kbl = detail::affine_mfma_kbl(K, bits);
    int cus = 256;
    if (detail::device_cus(cus) != hipSuccess) cus = 256;
    // smallest split that gives ~2048 work items, then more chunks while the
    // LDS does not fit (smaller chunks need smaller bias tables)
    auto fits = [&](int n) {
        if (detail::affine_mfma_gps(K, bits, n) == 0) return false;
        int blocks = 0;
        int64_t tmax = 0;
        detail::affine_mfma_geometry(T, n, cus, 1, blocks, tmax);   // most tiles per slot (one workgroup per CU)
        return detail::affine_mfma_lds_bytes(MT, K, bits, n, tmax) <= detail::kMfmaStreamLdsMax;
    };
    int nkc = 1;
    while (nkc < 8 && 2 * nkc <= kbl && T * nkc < 2048) nkc *= 2;
    while (!fits(nkc) && nkc > 1 && nkc < 8 && 2 * nkc <= kbl) nkc *= 2;
    if (!fits(nkc)) return false;
    c.path = PATH_AFFINE_MFMA;
    c.MT = MT;
    c.KT = K;
    c.ksplit_log2 = nkc == 1 ? 0 : nkc == 2 ? 1 : nkc == 4 ? 2 : 3;
    c.nwaves = detail::kAffineMfmaThreads / 64;
    c.R = 1;
    return true;
}

int ceil_log2(int v) { int l = 0; while ((1 << l) < v) ++l; return l; }

// Persistent streaming geometry (M <= 8, large N).  Lanes per row: dense up
// to 64 (one row per tile, 1 KB per load); affine: the smallest power of two
// >= the groups per row (<= 64), so each lane owns at most one group per row
// and, for M <= 2, keeps that group's x in registers.  Returns false when the
// shape is better served by the tiled kernel (too few row tiles to stream, or
// x does not fit in LDS).
bool choose_stream(int bits, bool swiglu, int M, int N, int K, LaunchCfg& c)
{
    c = LaunchCfg{};
    c.path = PATH_STREAM;
    c.MT = 1;
    while (c.MT < M) c.MT <<= 1;
    if (c.MT > 8) return false;
    const int UK = bits ? 64 : 8;
    const int U = K / UK;
    int L;
    if (bits == 0) {
        // one row per tile: a load instruction reads 1 KB of one row
        L = ctz_u((unsigned)U);
        if (L > 6) L = 6;
    } else {
        L = ceil_log2(U);
        if (L > 6) L = 6;
    }
    c.lpr_log2 = L;
    const int G = 64 >> L;
    const int64_t T = ((int64_t)N + G - 1) / G;
    if (T < 2048) return false;
    c.xreg = (bits != 0 && U <= 64 && (c.MT == 1 || (c.MT == 2 && bits != 8 && !swiglu))) ? 1 : 0;
    const size_t per_unit = bits ? (bits == 8 ? 16 * 16 : 16 * 8) + 8 : 16;
    c.lds = (size_t)c.MT * U * per_unit;   // staged x (also the source of register-resident x)
    // output staging, bounded with the fewest wavefronts the launch can get
    // (one 4-wave workgroup per CU)
    const int64_t row_bytes = bits ? (int64_t)K * bits / 8 : (int64_t)K * 2;
    int64_t ct = 4096 / (G * row_bytes);
    if (ct < 1) ct = 1;
    const int64_t st = (T + ct - 1) / ct;
    const int64_t tmax = ((st + 1023) / 1024) * ct;
    const int vpl = (c.MT + (1 << L) - 1) >> L;
    if (c.lds + (size_t)4 * tmax * 64 * vpl * 4 > detail::kStreamLdsMax) return false;
    c.KT = K;
    c.nwaves = 4;
    c.R = 1;
    // tiles per wavefront and the grid are set at launch from the kernel's
    // occupancy (every resident wavefront gets an equal range of tiles)
    return true;
}

// 16-byte-piece streaming geometry (M <= 8; dense, SwiGLU, b = 2, 4, 8).
// Rows of >= 64 pieces: 64 lanes per row (one instruction reads 1 KB of a
// row), J = ceil(pieces / 64) pieces per lane, rounded up to 8 when 5..7.
// Shorter rows: 16 lanes per row and J = 2..4 (measured faster than 32 lanes
// with J = 1 on the 4-bit LM head), or, for rows of <= 16 pieces, the
// smallest 2^L >= pieces with J = 1.  Lane slots past the row's end compute
// with zero x.  x stays in registers when its operands need at most 128
// (dense) or 64 (affine) registers per lane.  The path is feasible or not for
// all M <= 8 of a shape alike (checked at M = 8), so every M <= 8 computes
// each output the same way.
bool choose_piece(int bits, bool swiglu, int M, int N, int K, LaunchCfg& c)
{
    c = LaunchCfg{};
    if (!(bits == 0 || bits == 2 || bits == 4 || bits == 8)) return false;
    c.path = PATH_PIECE;
    c.MT = 1;
    while (c.MT < M) c.MT <<= 1;
    if (c.MT > 8) return false;
    const int KPP = bits ? 128 / bits : 8;
    if (K % KPP != 0) return false;
    const int PR = K / KPP;
    int L, J;
    if (PR >= 64) {
        L = 6;
        J = (PR + 63) / 64;
        if (J > 4 && J <= 8) J = 8;
        if (J > 8) return false;
    } else if (PR > 16) {
        L = 4;
        J = (PR + 15) / 16;
    } else {
        L = PR > 8 ? 4 : (PR > 4 ? 3 : 2);
        J = 1;
    }
    // a tile's scales and biases come in with one bf16 per lane each
    if (bits != 0 && (int64_t)(64 >> L) * (K / 64) > 64) return false;
    const int NPP = bits == 0 ? 4 : (bits == 2 ? 32 : 16);
    const int budget = bits == 0 ? detail::piece_xreg_budget<0>() : detail::piece_xreg_budget<4>();
    auto xreg_at = [&](int mt) { return NPP * J * mt <= budget; };
    // LDS at M = 8: staged x (unless in registers) plus the output staging
    // with the fewest wavefronts a launch can get (one 4-wave workgroup per CU)
    const int G = 64 >> L;
    const int PRP = J << L;
    const int64_t T = ((int64_t)N + G - 1) / G;
    const int64_t row_bytes = (int64_t)PR * 16;
    int64_t ct = (bits == 0 ? 8192 : 4096) / (G * row_bytes);
    if (ct < 1) ct = 1;
    // tiles per wavefront with any super-tile size up to ct and at least one
    // 4-wavefront workgroup per CU
    const int64_t tmax = (T + 1023) / 1024 + ct;
    const size_t x8 = (bits == 0 && xreg_at(8)) ? 0 : (size_t)8 * PRP * (4 * NPP + (bits ? 8 : 0));
    if (x8 + (size_t)4 * tmax * G * 8 * 4 > detail::kPieceLdsMax) return false;
    c.lpr_log2 = L;
    c.pieces_per_lane = J;
    c.xreg = xreg_at(c.MT) ? 1 : 0;
    c.lds = (bits == 0 && c.xreg) ? 0 : (size_t)c.MT * PRP * (4 * NPP + (bits ? 8 : 0));
    c.KT = K;
    c.nwaves = 4;
    c.R = 1;
    return true;
}

}  // namespace

LaunchCfg choose_config(int bits, bool swiglu, int M, int N, int K)
{
    LaunchCfg c;
    if (swiglu && bits != 0) {
        // fused SwiGLU over affine gate and up matrices: both weight streams
        // through the same x operands, on the small-matrix matrix-core kernel
        // (at most 256 row tiles), else on the dot-product kernels
        // 2, 4, 8 bits below M = 5: the matrix core where the piece kernel
        // does not serve (2 x 4096 x 1536 on the streaming kernel at M = 1..4:
        // 7.8-20.6 us, on the matrix core 6.4-6.7 us) and at M = 3, 4 for
        // 4 and 8 bits (2 x 3584 x 1024 4-bit: 5.2 -> 5.0 us, 8-bit 7.5 ->
        // 6.3 us); the piece kernel at M = 1, 2 (3.7 against 4.9 us) and for
        // 2 bits (4.9 against 6.0 us at M = 4)
        LaunchCfg cp;
        const bool nat = !(bits == 2 || bits == 4 || bits == 8);
        const bool piece = choose_piece(bits, true, M, N, K, cp);
        if ((nat || M >= 5 || !piece || (M >= 3 && bits != 2)) && choose_affine_split(bits, true, M, N, K, c))
            return c;
        if (piece) return cp;
        if (choose_stream(bits, true, M, N, K, c)) return c;
        return choose_valu(bits, true, M, N, K);
    }
    // Large-N dense from M = 3 on: the tile kernel streams the 100000 x 1536
    // LM head at ~48-49 us for any M <= 16 (against ~50 us for the
    // dot-product kernel at M = 3, 4 and ~64 us at M = 5..8, which pads M to
    // 4 or 8); M <= 2 stays on the latter (~45 us).
    if (bits == 0 && M >= 3 && choose_mfma_tile(swiglu, M, N, K, c)) return c;
    if (bits == 0 && M > 8 && choose_mfma_stream(swiglu, M, N, K, c)) return c;
    // Small-N matrix core from M = 3 on for N >= 4096, K <= 2048 (SwiGLU
    // 2 x 4096 x 1536: 8.1 us at M = 16 against 10.6 us for the dot-product
    // kernel at M = 8, 7.0 us at M = 8 against 7.8 us for the latter at M =
    // 4; up/gate 4096 x 1536: 5.7 against 6.4 us) and from M = 5 on for at
    // most 128 row tiles with K <= 2048 (two 4-column workgroups per tile);
    // longer matrices keep the dot-product kernel up to M = 8 (down 1536 x
    // 4096: 7.4 against 10.0 us).
    if (bits == 0 &&
        (M > 8 || (M >= 3 && N >= 4096 && K <= 2048) || (M >= 5 && K <= 2048 && ((int64_t)N + 15) / 16 <= 128)) &&
        choose_mfma_split(swiglu, M, N, K, c))
        return c;
    // Affine matrix core: its cost does not grow with M (up to 16), the
    // dot-product kernels' does.  4-bit from M = 3 on (measured on the 151936
    // x 1024 LM head: 27.5 us at any M <= 16 against 32 us for the piece
    // kernel at M = 4), 2- and 8-bit from M = 9 on; with a K split (few row
    // tiles) from M = 9 on, below which the piece kernel's shorter prologue
    // wins.
    // Affine tiles through LDS from M = 5 on where they serve (K = 2048 / 4096
    // and 8-bit K = 1024: 14336 x 4096 at M = 16 54.7 -> 18.4 us at 4 bits).
    // Small matrices from M = 5 on: one workgroup per tile with every load
    // issued at once (4-bit 1024 x 3584 at M = 16: 11.8 -> 7.3 us; 1024 x
    // 1024: 7.4 -> 4.0 us; 8-bit 4096 x 4096: 15.1 -> 14.2 us; 2- and 4-bit
    // 4096 x 4096 level with the tile kernel).
    // (3, 5, 6, 7 bits: the tile kernel first where it serves, 0.5-1 us
    // faster on 4096 x 4096 at M = 5..16)
    // (and at M = 1 the streaming kernel where it serves: 3-bit 4096 x 4096
    // 8.4 us against 9.3 us)
    const bool nat = bits == 3 || bits == 5 || bits == 6 || bits == 7;
    if (!swiglu && choose_affine_burst(bits, M, N, K, c)) return c;
    if (!swiglu && nat && M >= 5 && choose_affine_tile(bits, M, N, K, c)) return c;
    if (!swiglu && nat && M == 1 && choose_stream(bits, false, M, N, K, c)) return c;
    if (!swiglu && choose_affine_split(bits, false, M, N, K, c)) return c;
    if (!swiglu && M >= 5 && choose_affine_tile(bits, M, N, K, c)) return c;
    if (!swiglu && M >= 3 && choose_affine_mfma(bits, M, N, K, c) &&
        (M > 8 || (bits == 4 && c.ksplit_log2 == 0))) return c;
    if (bits == 0 && M > 8 && K % 32 == 0) return choose_mfma(swiglu, M, N, K);
    if (choose_piece(bits, swiglu, M, N, K, c)) return c;
    if (choose_stream(bits, swiglu, M, N, K, c)) return c;
    return choose_valu(bits, swiglu, M, N, K);
}

bool argmax_fused(const LaunchCfg& c)
{
    return c.path == PATH_PIECE || c.path == PATH_MFMA_TILE || (c.path == PATH_AFFINE_MFMA && c.ksplit_log2 == 0);
}

hipError_t launch_proj_table(int bits, bool swiglu, const ProjArgs& a, const LaunchCfg& c, hipStream_t s);

hipError_t launch_proj(int bits, bool swiglu, const ProjArgs& a0, const LaunchCfg& c, hipStream_t s)
{
    if (a0.nseg > 0) return launch_proj_table(bits, swiglu, a0, c, s);
    // one projection: a one-segment table
    ProjArgs a = a0;
    a.nseg = 1;
    a.seg_row0[0] = 0;
    for (int i = 1; i <= kMaxSegments; ++i) a.seg_row0[i] = a.N;
    for (int i = 0; i < kMaxSegments; ++i) {
        a.seg_w[i] = a.w0;
        a.seg_scales[i] = a.scales;
        a.seg_biases[i] = a.biases;
        a.seg_y[i] = a.y;
    }
    return launch_proj_table(bits, swiglu, a, c, s);
}

hipError_t launch_proj_table(int bits, bool swiglu, const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    if (c.path == PATH_AFFINE_TILE) {
        if (swiglu) return hipErrorInvalidValue;
        switch (bits) {
            case 2: return launch_affine_tile<2>(a, c, s);
            case 3: return launch_affine_tile<3>(a, c, s);
            case 4: return launch_affine_tile<4>(a, c, s);
            case 5: return launch_affine_tile<5>(a, c, s);
            case 6: return launch_affine_tile<6>(a, c, s);
            case 7: return launch_affine_tile<7>(a, c, s);
            case 8: return launch_affine_tile<8>(a, c, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (c.path == PATH_AFFINE_BURST) {
        if (swiglu) return hipErrorInvalidValue;
        switch (bits) {
            case 2: return launch_affine_burst<2>(a, c, s);
            case 3: return launch_affine_burst<3>(a, c, s);
            case 4: return launch_affine_burst<4>(a, c, s);
            case 5: return launch_affine_burst<5>(a, c, s);
            case 6: return launch_affine_burst<6>(a, c, s);
            case 7: return launch_affine_burst<7>(a, c, s);
            case 8: return launch_affine_burst<8>(a, c, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (c.path == PATH_AFFINE_SPLIT) {
        switch (bits) {
            case 2: return swiglu ? launch_affine_split<2, true>(a, c, s) : launch_affine_split<2, false>(a, c, s);
            case 3: return swiglu ? launch_affine_split<3, true>(a, c, s) : launch_affine_split<3, false>(a, c, s);
            case 4: return swiglu ? launch_affine_split<4, true>(a, c, s) : launch_affine_split<4, false>(a, c, s);
            case 5: return swiglu ? launch_affine_split<5, true>(a, c, s) : launch_affine_split<5, false>(a, c, s);
            case 6: return swiglu ? launch_affine_split<6, true>(a, c, s) : launch_affine_split<6, false>(a, c, s);
            case 7: return swiglu ? launch_affine_split<7, true>(a, c, s) : launch_affine_split<7, false>(a, c, s);
            case 8: return swiglu ? launch_affine_split<8, true>(a, c, s) : launch_affine_split<8, false>(a, c, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (c.path == PATH_AFFINE_MFMA) {
        if (swiglu) return hipErrorInvalidValue;
        switch (bits) {
            case 2: return launch_affine_mfma<2>(a, c, s);
            case 4: return launch_affine_mfma<4>(a, c, s);
            case 8: return launch_affine_mfma<8>(a, c, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (c.path == PATH_MFMA_TILE) {
        if (bits != 0 || swiglu) return hipErrorInvalidValue;
        return launch_mfma_tile(a, c, s);
    }
    if (c.path == PATH_MFMA_SPLIT) {
        if (bits != 0) return hipErrorInvalidValue;
        return swiglu ? launch_mfma_split<true>(a, c, s) : launch_mfma_split<false>(a, c, s);
    }
    if (c.path == PATH_MFMA_STREAM) {
        if (bits != 0) return hipErrorInvalidValue;
        return swiglu ? launch_mfma_stream<true>(a, c, s) : launch_mfma_stream<false>(a, c, s);
    }
    if (c.path == PATH_MFMA) {
        if (bits != 0) return hipErrorInvalidValue;
        return swiglu ? launch_mfma<true>(a, c, s) : launch_mfma<false>(a, c, s);
    }
    if (c.path == PATH_PIECE) {
        if (swiglu) {
            switch (bits) {
                case 0: return launch_piece<0, true>(a, c, s);
                case 2: return launch_piece<2, true>(a, c, s);
                case 4: return launch_piece<4, true>(a, c, s);
                case 8: return launch_piece<8, true>(a, c, s);
                default: return hipErrorInvalidValue;
            }
        }
        switch (bits) {
            case 0: return launch_piece<0, false>(a, c, s);
            case 2: return launch_piece<2, false>(a, c, s);
            case 4: return launch_piece<4, false>(a, c, s);
            case 8: return launch_piece<8, false>(a, c, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (c.path == PATH_STREAM) {
        if (swiglu) {
            switch (bits) {
                case 0: return launch_stream<0, true>(a, c, s);
                case 2: return launch_stream<2, true>(a, c, s);
                case 3: return launch_stream<3, true>(a, c, s);
                case 4: return launch_stream<4, true>(a, c, s);
                case 5: return launch_stream<5, true>(a, c, s);
                case 6: return launch_stream<6, true>(a, c, s);
                case 7: return launch_stream<7, true>(a, c, s);
                case 8: return launch_stream<8, true>(a, c, s);
                default: return hipErrorInvalidValue;
            }
        }
        switch (bits) {
            case 0: return launch_stream<0, false>(a, c, s);
            case 2: return launch_stream<2, false>(a, c, s);
            case 3: return launch_stream<3, false>(a, c, s);
            case 4: return launch_stream<4, false>(a, c, s);
            case 5: return launch_stream<5, false>(a, c, s);
            case 6: return launch_stream<6, false>(a, c, s);
            case 7: return launch_stream<7, false>(a, c, s);
            case 8: return launch_stream<8, false>(a, c, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (swiglu) {
        switch (bits) {
            case 0: return launch_bits<0, true>(a, c, s);
            case 2: return launch_bits<2, true>(a, c, s);
            case 3: return launch_bits<3, true>(a, c, s);
            case 4: return launch_bits<4, true>(a, c, s);
            case 5: return launch_bits<5, true>(a, c, s);
            case 6: return launch_bits<6, true>(a, c, s);
            case 7: return launch_bits<7, true>(a, c, s);
            case 8: return launch_bits<8, true>(a, c, s);
            default: return hipErrorInvalidValue;
        }
    }
    switch (bits) {
        case 0: return launch_bits<0, false>(a, c, s);
        case 2: return launch_bits<2, false>(a, c, s);
        case 3: return launch_bits<3, false>(a, c, s);
        case 4: return launch_bits<4, false>(a, c, s);
        case 5: return launch_bits<5, false>(a, c, s);
        case 6: return launch_bits<6, false>(a, c, s);
        case 7: return launch_bits<7, false>(a, c, s);
        case 8: return launch_bits<8, false>(a, c, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_unpack(int bits, const uint32_t* Wq, uint8_t* codes, int N, int K, hipStream_t s)
{
    const int64_t ng = (int64_t)N * (K / 64);
    const dim3 grid((unsigned)((ng + 255) / 256)), block(256);
    switch (bits) {
#define AQG_UNPACK(B) case B: hipLaunchKernelGGL(detail::unpack_kernel<B>, grid, block, 0, s, Wq, codes, ng); break;
        AQG_UNPACK(2) AQG_UNPACK(3) AQG_UNPACK(4) AQG_UNPACK(5) AQG_UNPACK(6) AQG_UNPACK(7) AQG_UNPACK(8)
#undef AQG_UNPACK
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace aqg
