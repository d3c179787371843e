// Host check of the out-axis work-item order: for every 3-D and 2-D geometry
// the library supports (up to a size cap), out_tile must visit each (channel,
// slot tile, row pair, batch entry) exactly once, and the kernel-spectrum and
// backward tile widths must give the same property.  Prints one line per
// geometry; exits non-zero on the first failure.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../dimensional_fft_long_amd/csrc/conv_bodies.h"

using namespace hyenand;

template <int NR, int TW>
static bool check(const Geom& g, int B, int nch, const char* what)
{
    const int ct = (g.S + TW - 1) / TW;
    const int nrp = NR == 1 ? 1 : g.N_mid / 2;
    const long long W = (long long)nch * nrp * ct * B;
    std::vector<unsigned char> seen((size_t)W, 0);
    for (int bid = 0; bid < W; ++bid) {
        const OutTile o = out_tile<NR, TW>(g, B, nch, bid);
        const int rp = NR == 1 ? 0 : (o.rows[0]);
        if (o.b < 0 || o.b >= B || o.c_local < 0 || o.c_local >= nch || o.t < 0 || o.t >= ct || rp < 0 ||
            rp >= nrp) {
            std::printf("FAIL %s: item %d out of range (c %d t %d b %d rp %d)\n", what, bid, o.c_local, o.t, o.b, rp);
            return false;
        }
        if (NR == 2 && o.rows[1] != (rp == 0 ? g.N_mid / 2 : g.N_mid - rp)) {
            std::printf("FAIL %s: item %d mirror row %d for rp %d\n", what, bid, o.rows[1], rp);
            return false;
        }
        const long long key = (((long long)o.c_local * nrp + rp) * ct + o.t) * B + o.b;
        if (seen[(size_t)key]++) {
            std::printf("FAIL %s: item %d repeats (c %d t %d b %d rp %d)\n", what, bid, o.c_local, o.t, o.b, rp);
            return false;
        }
    }
    return true;
}

template <int L>
static bool check_len(int d, int B, int nch)
{
    // every inner extent up to the cap, middle extent L/2 (3-D), out extent L/2
    bool ok = true;
    for (int nin = 2; nin <= 256; nin *= 2) {
        int64_t dims[3];
        if (d == 3) { dims[0] = L / 2; dims[1] = L / 2; dims[2] = nin; }
        else { dims[0] = L / 2; dims[1] = nin; }
        Geom g;
        if (!make_geom(d, dims, &g)) { std::printf("FAIL make_geom d=%d L=%d nin=%d\n", d, L, nin); return false; }
        char what[96];
        std::snprintf(what, sizeof what, "d=%d N_out=%d n_in=%d B=%d nch=%d", d, L, nin, B, nch);
        if (d == 3) {
            ok = ok && check<2, out_tw(L, 2)>(g, B, nch, what) && check<2, bwd_tw(L, 2)>(g, 1, nch, what);
        } else {
            ok = ok && check<1, out_tw(L, 1)>(g, B, nch, what) && check<1, bwd_tw(L, 1)>(g, 1, nch, what);
        }
        if (ok) std::printf("ok %s (lt %d)\n", what, g.lt);
    }
    return ok;
}

int main()
{
    bool ok = true;
    ok = ok && check_len<8>(3, 3, 2) && check_len<16>(3, 1, 3) && check_len<64>(3, 2, 2) &&
         check_len<256>(3, 1, 2) && check_len<512>(3, 1, 1) && check_len<1024>(3, 1, 1) &&
         check_len<2048>(3, 1, 1);
    ok = ok && check_len<8>(2, 5, 3) && check_len<512>(2, 8, 4) && check_len<1024>(2, 2, 3) &&
         check_len<2048>(2, 2, 2);
    std::printf(ok ? "all ok\n" : "failed\n");
    return ok ? 0 : 1;
}
