// Launch-geometry choice and dispatch to the per-width kernel instantiations
// (proj_b*.hip), plus the code-unpack kernel.
#include "proj_kernel.h"

namespace aqg {
namespace detail {

int ctz_u(unsigned v) { int n = 0; while (v && !(v & 1u)) { v >>= 1; ++n; } return n; }

}  // namespace detail
using detail::ctz_u;
using detail::kLdsBudget;
using detail::kMaxThreads;

LaunchCfg choose_valu(int bits, bool swiglu, int M, int N, int K)
{
    LaunchCfg c{};
    c.MT = 1;
    while (c.MT < M) c.MT <<= 1;
    const int UK = bits ? 64 : 8;
    int per_unit = 16;  // LDS bytes per (m, unit)
    if (bits) per_unit = (bits == 8 ? 16 * 16 : 16 * 8) + 8;
    const int U = K / UK;                                   // units per row
    // Lanes per row: the largest power of two (<= 16) dividing U that still
    // lets a K-tile of 2^L units fit at the largest M.  It depends on (bits, K)
    // only, so every M sums each output in the same order.
    int L = ctz_u((unsigned)U);
    if (L > 4) L = 4;
    const int64_t fit_max = (int64_t)kLdsBudget / ((int64_t)32 * per_unit);
    while (L > 0 && fit_max < (1 << L)) --L;
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
    c.R = (!swiglu && c.MT <= 16 && tiles1 >= 4096) ? 2 : 1;
    const int64_t wave_tiles = ((int64_t)N + G * c.R - 1) / (G * c.R);
    int64_t nw = wave_tiles / 512;
    if (nw < 1) nw = 1;
    if (nw > kMaxThreads / 64) nw = kMaxThreads / 64;
    c.nwaves = (int)nw;
    c.blocks = (int)((wave_tiles + nw - 1) / nw);
    return c;
}

hipError_t launch_valu(int bits, bool swiglu, const ProjArgs& a, const LaunchCfg& c, hipStream_t s)
{
    if (swiglu) {
        if (bits != 0) return hipErrorInvalidValue;
        return launch_bits<0, true>(a, c, s);
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
