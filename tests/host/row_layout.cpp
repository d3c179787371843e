// Host check of the padded tile layouts: for every row length, the layout
// code row_lay(L) must place the L x row_np(L) elements of a tile at distinct
// indices below lay_elems(L, row_np(L), row_lay(L)) (the same for the 2-D
// out-axis tiles of out_lay(L, 1) with their out_tw(L, 1) lines and the
// register-flow row tiles of lngp_lay(L) with lngp_nl(L) lines), and the split
// index used by the LDS passes (lane part + loop constant) must equal the
// plain index for every access of every pass of the length's radix plan and
// of the reversed plan
// (loads at j + r L/R, stores at (j / NS) NS R + j % NS + r NS).  Prints one
// line per length; exits non-zero on the first failure.
#include <cstdio>
#include <vector>

#include "../../dimensional_fft_long_amd/csrc/fft_core.h"
#include "../../dimensional_fft_long_amd/csrc/plan.h"

using namespace hyenand;

template <int L, int NP = row_np(L), int LP = row_lay(L)>
static bool check()
{
    constexpr int E = lay_elems(L, NP, LP);
    std::vector<unsigned char> seen(E, 0);
    for (int pos = 0; pos < L; ++pos)
        for (int l = 0; l < NP; ++l) {
            const int e = tile_idx<LP>(pos, l);
            if (e < 0 || e >= E || seen[e]++) {
                std::printf("FAIL L=%d: element (%d, %d) at %d of %d\n", L, pos, l, e, E);
                return false;
            }
        }
    // the forward plan, then the reversed plan (the inverse transforms of
    // the out-axis and register-flow row kernels)
    for (int q = 0, ns = 1; q < 2 * plan_passes(L); ++q) {
        const int p = q < plan_passes(L) ? q : 2 * plan_passes(L) - 1 - q;
        if (q == plan_passes(L)) ns = 1;
        const int R = plan_radix(L, p);
        for (int j = 0; j < L / R; ++j)
            for (int r = 0; r < R; ++r)
                for (int l = 0; l < NP; ++l) {
                    const int base = (j / ns) * ns * R + j % ns;
                    if (tile_idx_split<LP>(j, r * (L / R), l) != tile_idx<LP>(j + r * (L / R), l) ||
                        tile_idx_split<LP>(base, r * ns, l) != tile_idx<LP>(base + r * ns, l)) {
                        std::printf("FAIL L=%d: split index of pass %d, j %d, r %d\n", L, p, j, r);
                        return false;
                    }
                }
        ns *= R;
    }
    std::printf("ok L=%d NP=%d layout %d: %d elements (%d bytes)\n", L, NP, LP, E, 8 * E);
    return true;
}

int main()
{
    const bool ok = check<4>() && check<8>() && check<16>() && check<32>() && check<64>() && check<128>() &&
                    check<256>() && check<512>() && check<1024>() && check<2048>() && check<4096>() &&
                    check<256, out_tw(256, 1), out_lay(256, 1)>() && check<512, out_tw(512, 1), out_lay(512, 1)>() &&
                    check<1024, out_tw(1024, 1), out_lay(1024, 1)>() &&
                    check<1024, lngp_nl(1024), lngp_lay(1024)>() && check<2048, lngp_nl(2048), lngp_lay(2048)>() &&
                    check<4096, lngp_nl(4096), lngp_lay(4096)>() && check<8192, lngp_nl(8192), lngp_lay(8192)>();
    std::printf(ok ? "all ok\n" : "failed\n");
    return ok ? 0 : 1;
}
