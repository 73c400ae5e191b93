// select_common.h -- helpers shared by the top-k select kernels of libsnapkv (gfx950): wave
// scans, the selection pivot, and the max pooling of a thread's run of positions.
#pragma once
#include "snapkv_internal.h"

namespace snapkv {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Inclusive prefix sum over the 64 lanes of a wave: four row shifts, then the row totals
// carried into rows 1, 3 (row_bcast:15) and 2, 3 (row_bcast:31).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += dpp_u32<0x111, 0xF>(x);  // row_shr:1
    x += dpp_u32<0x112, 0xF>(x);  // row_shr:2
    x += dpp_u32<0x114, 0xF>(x);  // row_shr:4
    x += dpp_u32<0x118, 0xF>(x);  // row_shr:8
    x += dpp_u32<0x142, 0xA>(x);  // row_bcast:15
    x += dpp_u32<0x143, 0xC>(x);  // row_bcast:31
    return x;
}

// State of a selection: values v with (v & mask) > prefix are kept; of those equal to prefix,
// the first `need` in position order are kept.
struct Pivot {
    uint32_t prefix, mask, need;
};

constexpr int floor_pow2(int x) { return x >= 32 ? 32 : x >= 16 ? 16 : x >= 8 ? 8 : x >= 4 ? 4 : x >= 2 ? 2 : 1; }
constexpr int ilog2(int x) { return x >= 32 ? 5 : x >= 16 ? 4 : x >= 8 ? 3 : x >= 4 ? 2 : x >= 2 ? 1 : 0; }

// Max pooling of one thread's run [j0, j0 + R) with half-width H, from the votes staged in
// LDS, in blocks of 8 outputs.  A block and HM >= H positions on each side are read once
// (16-byte reads); then
// doubling steps make a[i] the max over [i, i + PW), PW the largest power of two <= 2H+1,
// and each output is the max of two such spans that together cover its window.
// Positions outside [0, P) read as 0, which never wins a max of values >= 0 whose window
// contains the position itself.  Position pos sits at sdata[pos + off].
template <int R, int H>
__device__ __forceinline__ void pool_run(const uint32_t *sdata, int P, int j0, uint32_t (&u)[R], int off = 0) {
    constexpr int SUB = R < 8 ? R : 8;  // outputs per block (bounds the registers in flight)
    constexpr int HM = (H + 3) / 4 * 4;
    constexpr int N = SUB + 2 * HM;
    constexpr int PW = floor_pow2(2 * H + 1);
    static_for<R / SUB>([&](auto blk) {
        const int b0 = j0 + SUB * blk();
        uint32_t a[N];
        static_for<N / 4>([&](auto c) {
            const int pos = b0 - HM + 4 * c();
            u32x4_t t = {0u, 0u, 0u, 0u};
            if (pos >= 0 && pos < P) t = *(const u32x4_t *)(sdata + pos + off);
            a[4 * c() + 0] = pos + 0 < P ? t.x : 0u;
            a[4 * c() + 1] = pos + 1 < P ? t.y : 0u;
            a[4 * c() + 2] = pos + 2 < P ? t.z : 0u;
            a[4 * c() + 3] = pos + 3 < P ? t.w : 0u;
        });
        static_for<ilog2(PW)>([&](auto step) {
            constexpr int p = 1 << decltype(step)::value;
            static_for<N - 2 * p + 1>([&](auto i) { a[i()] = a[i() + p] > a[i()] ? a[i() + p] : a[i()]; });
        });
        static_for<SUB>([&](auto i) {
            const uint32_t x = a[i() + HM - H], y = a[i() + HM + H - PW + 1];
            u[SUB * blk() + i()] = x > y ? x : y;
        });
    });
}

template <int R>
__device__ __forceinline__ void load_run(const uint32_t *sdata, int P, int j0, uint32_t (&u)[R]) {
    static_for<R / 4>([&](auto c) {
        const int pos = j0 + 4 * c();
        u32x4_t t = {0u, 0u, 0u, 0u};
        if (pos < P) t = *(const u32x4_t *)(sdata + pos);
        u[4 * c() + 0] = t.x; u[4 * c() + 1] = t.y; u[4 * c() + 2] = t.z; u[4 * c() + 3] = t.w;
    });
}

}  // namespace snapkv
