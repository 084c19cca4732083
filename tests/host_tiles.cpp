// Host-side driver for the launchers' inline tile rules in qg_launch.h
// (lanes per row and the one-vector wave-tile choice), built with the host
// compiler alone: nothing here touches a GPU.  One query per input line:
//   L n                          -> "pick_lpr(n) pick_lpr_wide(n)"
//   F O rpg ncu ors k w1 r1 ...  -> index pick_fill_tile picks among the k
//                                   candidate tiles (w waves, r rows)
#include "qg_launch.h"

#include <cstdio>
#include <vector>

int main()
{
    char op;
    while (std::scanf(" %c", &op) == 1) {
        if (op == 'L') {
            int n;
            if (std::scanf("%d", &n) != 1) return 2;
            std::printf("%d %d\n", qg::pick_lpr(n), qg::pick_lpr_wide(n));
        } else if (op == 'F') {
            long O, rpg, ncu;
            int ors, k;
            if (std::scanf("%ld %ld %ld %d %d", &O, &rpg, &ncu, &ors, &k) != 5 || k < 1) return 2;
            std::vector<qg::WaveTile> c((size_t)k);
            for (auto &t : c)
                if (std::scanf("%d %d", &t.wpb, &t.r) != 2) return 2;
            std::printf("%d\n", qg::pick_fill_tile(O, rpg, c.data(), k, ncu, ors != 0));
        } else {
            return 2;
        }
    }
    return 0;
}
