// wg_order.h -- workgroup-order permutation for ordering checks (internal).
//
// Every kernel here maps its workgroup id to a logical unit of work (a query
// tile, a key tile, a split) and no workgroup waits for another, so the
// results must not depend on which workgroup takes which unit or in what
// order they run. A test can ask the launchers to permute the logical ids of
// a grid of n workgroups: logical x becomes (x * mul + add) mod n with mul
// coprime to n (a permutation); mul = 0 leaves x as it is (the default).
#pragma once

namespace cakv {

struct WgPerm {
    int mul, add;
};

// order 0: unchanged; 1: scrambled (mul the first odd number from 0.618 n
// coprime to n, add = n / 3); 2: reversed (x -> n - 1 - x)
inline WgPerm wg_perm(int order, long long n) {
    if (order == 0 || n <= 1) return WgPerm{0, 0};
    if (order == 2) return WgPerm{(int)(n - 1), (int)(n - 1)};
    long long m = (long long)(0.618 * (double)n) | 1;
    for (;;) {
        long long x = m, y = n;
        while (y) {
            const long long t = x % y;
            x = y;
            y = t;
        }
        if (x == 1) break;
        m += 2;
    }
    m %= n;
    if (m == 0) m = 1;
    return WgPerm{(int)m, (int)(n / 3)};
}

#ifdef __HIPCC__
__device__ __forceinline__ int wg_permute(int x, int n, int mul, int add) {
    return mul ? (int)(((long long)x * mul + add) % n) : x;
}
#endif

}  // namespace cakv
