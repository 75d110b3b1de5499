// Host build of the lm_head's running argmax and its 64-bit keys (the same
// inline functions the kernel calls, from common.h): rows are dealt to
// "lanes" in ascending order per lane, merged across lanes, encoded as keys,
// reduced by the largest key and decoded. Exits nonzero on the first
// mismatch with the first-index argmax of the plain definition.
#include "../moe_speculative_verify_amd/csrc/common.h"

#include <cmath>
#include <cstdio>
#include <vector>

using namespace mv;

static int first_argmax(const std::vector<float> &z)
{
    // NaN counts as -inf; lowest index among the maxima; row 0 if all -inf
    int best = 0;
    float bv = std::isnan(z[0]) ? -INFINITY : z[0];
    for (size_t i = 1; i < z.size(); ++i) {
        const float v = std::isnan(z[i]) ? -INFINITY : z[i];
        if (v > bv) {
            bv = v;
            best = (int)i;
        }
    }
    return best;
}

// lanes take rows l, l + nl, ... in ascending order, as the kernel's lanes do
static int device_path(const std::vector<float> &z, int nl, float *vmax)
{
    std::vector<float> bv(nl, -INFINITY);
    std::vector<int> bi(nl, kNoRow);
    for (int l = 0; l < nl; ++l)
        for (size_t r = l; r < z.size(); r += nl)
            argmax_take(bv[l], bi[l], z[r], (int)r);
    // lanes merged pairwise (the shuffle tree), then keys over "workgroups"
    for (int s = 1; s < nl; s <<= 1)
        for (int l = 0; l + s < nl; l += 2 * s)
            argmax_merge(bv[l], bi[l], bv[l + s], bi[l + s]);
    unsigned long long key = argmax_key(bv[0], bi[0]);
    *vmax = f32_unorder((uint32_t)(key >> 32));
    return argmax_key_row(key);
}

int main()
{
    int fails = 0;
    auto check = [&](const char *what, const std::vector<float> &z, int nl) {
        float vm;
        const int got = device_path(z, nl, &vm), want = first_argmax(z);
        float wv = std::isnan(z[want]) ? -INFINITY : z[want];
        if (got != want || !(vm == wv)) {
            std::printf("FAIL %s (lanes %d): row %d value %g, want row %d value %g\n", what, nl,
                        got, vm, want, wv);
            ++fails;
        }
    };
    for (int nl : {1, 2, 4, 8, 64}) {
        for (int n : {1, 3, 64, 100}) {
            check("all -inf", std::vector<float>(n, -INFINITY), nl);
            check("all NaN", std::vector<float>(n, NAN), nl);
            std::vector<float> z(n, -INFINITY);
            z[n - 1] = -1e30f;
            check("last finite", z, nl);
            std::vector<float> m(n);
            for (int i = 0; i < n; ++i)
                m[i] = (i % 3 == 0) ? NAN : (float)((i * 7) % 5);
            check("NaN mixed with ties", m, nl);
            std::vector<float> t(n, 2.5f);
            check("all equal", t, nl);
            std::vector<float> zz(n, 0.0f);
            for (int i = 0; i < n; i += 2)
                zz[i] = -0.0f;
            check("signed zeros", zz, nl);
        }
    }
    // the key order: larger value first, then lower row; -0 and +0 equal
    if (!(argmax_key(1.0f, 5) > argmax_key(1.0f, 6) && argmax_key(2.0f, 9) > argmax_key(1.0f, 0) &&
          argmax_key(-INFINITY, 0) > argmax_key(-INFINITY, 1) &&
          argmax_key(-0.0f, 3) == argmax_key(0.0f, 3) && argmax_key_row(argmax_key(-INFINITY, 0)) == 0)) {
        std::printf("FAIL key order\n");
        ++fails;
    }
    std::printf("%s\n", fails ? "FAILED" : "ok");
    return fails ? 1 : 0;
}
