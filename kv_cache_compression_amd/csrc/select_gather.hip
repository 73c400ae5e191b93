// select_gather.hip -- vote pooling, top-k selection and the compressed-cache gather, gfx950.
//
// Page "論文解説: SnapKV — アテンションパターン観測によるKVキャッシュ圧縮":
//   * クラスタリングによる文脈保持: the votes are max pooled (width K_pool, stride 1,
//     padding K_pool/2) before top-k so that neighbours of strong positions survive.
//   * 投票メカニズム: I = Top_k(C, k); the アルゴリズム listing sorts I ascending and
//     gathers K/V per head, then appends the window.
#include "snapkv_internal.h"

namespace snapkv {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---- pool ----------------------------------------------------------------------------------
// grid: (ceil(max P / 256), requests, KV heads).  The window is clipped to [0, P): the
// padding acts as -infinity, so window votes never enter a prefix position's pool.
__global__ void __launch_bounds__(256) vote_pool_kernel(const PoolParams p) {
    const int r = blockIdx.y, g = blockIdx.z;
    const int P = p.rt.L[r] - p.w;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= P) return;
    const int64_t base = (int64_t)g * p.sum_P + p.rt.pfx0[r];
    const int lo = j - p.half < 0 ? 0 : j - p.half;
    const int hi = j + p.half > P - 1 ? P - 1 : j + p.half;
    float m = p.votes[base + lo];
    for (int t = lo + 1; t <= hi; ++t) {
        const float v = p.votes[base + t];
        m = v > m ? v : m;
    }
    p.pooled[base + j] = m;
}
const void *pool_kernel() { return (const void *)&vote_pool_kernel; }

// ---- top-k select ----------------------------------------------------------------------------
// One workgroup of 1024 threads per (request, KV head) segment.  Pooled votes are >= 0, so
// their fp32 bit patterns (sign bit ignored: -0 orders as +0) order like the values.
// Three radix passes (bits 30..20, 19..9, 8..0) over one shared 2048-bin histogram find the
// bit pattern v* of the k-th largest value; wave 0 locates the bin.  One ordered pass then
// keeps every position above v* and the lowest-position ones equal to v*, written in
// ascending order at offsets from a workgroup prefix scan.  No sort is needed.  Writes stay
// inside the segment's k slots even for inputs outside the contract (negative or NaN).
//
// Segments of up to kSelLds positions: the votes are staged in LDS with coalesced loads,
// each thread then takes a contiguous run of R <= 32 positions into registers (max pooling
// them on the way when the votes are raw), and every pass works on those registers.
// Longer segments (pooled by vote_pool first) are re-read from L2 / Infinity Cache on
// each pass.
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelLds = 32768;
constexpr int kBins = 2048;
// Widest pool half-width (K_pool / 2) pooled inside the select kernel for runs of R
// positions per thread (the pooling window of a run is held in registers).
constexpr int max_half(int R) { return R <= 16 ? 16 : 8; }
int select_threads() { return kSelThreads; }
int select_lds_positions() { return kSelLds; }
int select_max_half(int max_P) { return max_half(max_P <= 16 * kSelThreads ? 16 : 32); }

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

// Histogram slot of a digit.  Bins are stored in descending digit order q = 2047 - digit,
// with the 16-byte chunks of each 32-bin block rotated by the block number so that wave 0's
// reads of one block per lane spread over the LDS banks.
__device__ __forceinline__ uint32_t hist_slot(uint32_t digit) {
    const uint32_t q = (kBins - 1) - digit;
    return q ^ ((q >> 3) & 0x1Cu);
}

// Wave 0: the bin that holds the need-th largest remaining value.  Lane l sums descending
// bins q = 32l .. 32l+31; a wave scan finds the block, then lanes 0..31 take one bin each
// of that block and a second scan finds the bin.  Writes (digit, count above the bin,
// count in the bin) to sh; writes nothing if no bin qualifies (inputs outside the contract).
__device__ __forceinline__ void find_bin(const uint32_t *hist, uint32_t need, uint32_t *sh) {
    const int lane = threadIdx.x & 63;
    uint32_t sum = 0;
    static_for<8>([&](auto m) {
        const u32x4_t t = *(const u32x4_t *)(hist + 32 * lane + 4 * (m() ^ (lane & 7)));
        sum += t.x + t.y + t.z + t.w;
    });
    const uint32_t incl = wave_incl_scan(sum);
    const uint64_t hit = __ballot(incl - sum < need && need <= incl);
    if (!hit) return;
    const int L = __ffsll((unsigned long long)hit) - 1;
    const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), L);
    uint32_t c = 0;
    if (lane < 32) {
        const uint32_t q = 32 * L + lane;
        c = hist[q ^ ((q >> 3) & 0x1Cu)];
    }
    const uint32_t ci = above + wave_incl_scan(c);
    const uint64_t hit2 = __ballot(lane < 32 && ci - c < need && need <= ci);
    if (!hit2) return;
    if (lane == __ffsll((unsigned long long)hit2) - 1) {
        sh[0] = (uint32_t)(kBins - 1 - (32 * L + lane));
        sh[1] = ci - c;
        sh[2] = c;
    }
}

// Digit layout of the three passes.
template <int PASS> struct Digit {
    static constexpr int shift = PASS == 0 ? 20 : (PASS == 1 ? 9 : 0);
    static constexpr uint32_t mask = PASS == 2 ? 0x1FFu : 0x7FFu;
};

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
// contains the position itself.
template <int R, int H>
__device__ __forceinline__ void pool_run(const uint32_t *sdata, int P, int j0, uint32_t (&u)[R]) {
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
            if (pos >= 0 && pos < P) t = *(const u32x4_t *)(sdata + pos);
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

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_row(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// AND and OR over the 64 lanes of a wave (row rotations, then the four row results).
__device__ __forceinline__ void wave_and_or(uint32_t &a, uint32_t &o) {
    a &= dpp_row<0x128>(a); o |= dpp_row<0x128>(o);  // row_ror:8
    a &= dpp_row<0x124>(a); o |= dpp_row<0x124>(o);  // row_ror:4
    a &= dpp_row<0x122>(a); o |= dpp_row<0x122>(o);  // row_ror:2
    a &= dpp_row<0x121>(a); o |= dpp_row<0x121>(o);  // row_ror:1
    a = (uint32_t)(__builtin_amdgcn_readlane((int)a, 0) & __builtin_amdgcn_readlane((int)a, 16) &
                   __builtin_amdgcn_readlane((int)a, 32) & __builtin_amdgcn_readlane((int)a, 48));
    o = (uint32_t)(__builtin_amdgcn_readlane((int)o, 0) | __builtin_amdgcn_readlane((int)o, 16) |
                   __builtin_amdgcn_readlane((int)o, 32) | __builtin_amdgcn_readlane((int)o, 48));
}

struct SelectShared {
    uint32_t hist[2][kBins];
    uint32_t sh[4];
    uint32_t wtot[kSelWaves];
    uint32_t wand[kSelWaves], wor[kSelWaves];
};

// Exclusive prefix sum of x over the workgroup (one barrier); *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t *total, SelectShared &s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_scan(x);
    if (lane == 63) s.wtot[wave] = incl;
    __syncthreads();
    uint32_t woff = 0, tot = 0;
    static_for<kSelWaves>([&](auto w2) {
        const uint32_t t = s.wtot[w2()];
        woff += w2() < wave ? t : 0u;
        tot += t;
    });
    *total = tot;
    return woff + incl - x;
}

// One radix step: histogram of the digit (v >> shift) & dmask over values matching the
// pivot, wave 0 locates the bin of the need-th largest, the pivot takes the digit.
// Returns whether the pivot is final.  Also clears hist[0] when `clear0` (other waves).
template <typename Vals>
__device__ __forceinline__ bool radix_step(Vals &&for_each_value, int shift, uint32_t dmask, uint32_t *h,
                                           bool clear0, Pivot &pv, SelectShared &s) {
    for_each_value([&](uint32_t v) {
        if ((v & pv.mask) == pv.prefix) atomicAdd(&h[hist_slot((v >> shift) & dmask)], 1u);
    });
    __syncthreads();
    if (threadIdx.x < 64) {
        find_bin(h, pv.need, s.sh);
    } else if (clear0) {
        for (int i = threadIdx.x - 64; i < kBins; i += kSelThreads - 64) s.hist[0][i] = 0;
    }
    __syncthreads();
    const uint32_t dg = s.sh[0], above = s.sh[1], cnt = s.sh[2];
    pv.prefix |= dg << shift;
    pv.mask |= dmask << shift;
    pv.need -= above;
    return cnt == pv.need || shift == 0;
}

// Resident path for runs of R positions per thread (R * kSelThreads >= P).
template <int R>
__device__ __forceinline__ void select_resident(const SelectParams &p, uint32_t *sdata, SelectShared &s, int P,
                                                int k, int64_t base, int32_t *out) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    {
        // votes -> LDS, R coalesced loads in flight per thread; histograms cleared meanwhile
        const uint32_t *src = (const uint32_t *)((p.votes ? p.votes : p.pooled) + base);
        uint32_t t[R];
        static_for<R>([&](auto i) {
            const int j = i() * kSelThreads + tid;
            t[i()] = j < P ? src[j] : 0u;
        });
        for (int i = tid; i < 2 * kBins; i += kSelThreads) (&s.hist[0][0])[i] = 0;
        static_for<R>([&](auto i) {
            const int j = i() * kSelThreads + tid;
            if (j < P) sdata[j] = t[i()];
        });
    }
    __syncthreads();
    const int j0 = tid * R;
    const int nvalid = P - j0 < 0 ? 0 : (P - j0 > R ? R : P - j0);
    uint32_t u[R];
    if (p.votes) {
        static_for<max_half(R) + 1>([&](auto h) {
            if (p.half == decltype(h)::value) pool_run<R, decltype(h)::value>(sdata, P, j0, u);
        });
        if (p.pooled_out) {
            uint32_t *dst = (uint32_t *)(p.pooled_out + base) + j0;
            static_for<R>([&](auto i) {
                if (i() < nvalid) dst[i()] = u[i()];
            });
        }
    } else {
        load_run<R>(sdata, P, j0, u);
    }
    if (!out || k <= 0) return;
    if (k >= P) {
        for (int j = tid; j < P; j += kSelThreads) out[j] = j;
        return;
    }
    static_for<R>([&](auto i) { u[i()] = i() < nvalid ? u[i()] & 0x7FFFFFFFu : 0u; });

    // Bits shared by every value need no radix pass: the first digit starts at the highest
    // bit where the values differ, which spreads the first histogram over many bins.
    uint32_t va = ~0u, vo = 0u;
    static_for<R>([&](auto i) {
        if (i() < nvalid) { va &= u[i()]; vo |= u[i()]; }
    });
    wave_and_or(va, vo);
    if (lane == 0) { s.wand[wave] = va; s.wor[wave] = vo; }
    __syncthreads();
    va = ~0u; vo = 0u;
    static_for<kSelWaves>([&](auto w2) { va &= s.wand[w2()]; vo |= s.wor[w2()]; });
    const uint32_t diff = va ^ vo;  // bits on which the values differ
    Pivot pv;
    bool done;
    int shift = 0;
    if (diff == 0) {
        pv = {va, 0x7FFFFFFFu, (uint32_t)k};
        done = true;
    } else {
        const int b = 31 - __clz(diff);
        const uint32_t above = 0x7FFFFFFFu & ~((2u << b) - 1u);
        pv = {va & above, above, (uint32_t)k};
        shift = b >= 10 ? b - 10 : 0;
        const uint32_t dmask = (2u << (b - shift)) - 1u;
        done = radix_step([&](auto f) { static_for<R>([&](auto i) { if (i() < nvalid) f(u[i()]); }); },
                          shift, dmask, s.hist[0], false, pv, s);
    }
    if (!done) {
        // the values in the chosen bin become a candidate list in LDS (sdata is free now)
        uint32_t c = 0;
        static_for<R>([&](auto i) { c += (i() < nvalid && (u[i()] & pv.mask) == pv.prefix) ? 1u : 0u; });
        uint32_t ncand;
        uint32_t off = block_excl_scan(c, &ncand, s);
        static_for<R>([&](auto i) {
            if (i() < nvalid && (u[i()] & pv.mask) == pv.prefix) sdata[off++] = u[i()];
        });
        __syncthreads();
        static_for<2>([&](auto pass) {  // at most two more digits (31 bits = 11 + 11 + 9)
            if (done) return;
            const int nshift = shift >= 11 ? shift - 11 : 0;
            const uint32_t dmask = (1u << (shift - nshift)) - 1u;
            done = radix_step(
                [&](auto f) {
#pragma unroll 1
                    for (int i = tid; i < (int)ncand; i += kSelThreads) f(sdata[i]);
                },
                nshift, dmask, s.hist[(pass() + 1) & 1], pass() == 0, pv, s);
            shift = nshift;
        });
    }

    // ordered compaction: (above, equal) counts of the run, packed in one word (each half
    // stays below 2^16 since P <= 32768), prefix-summed over the workgroup
    uint32_t packed = 0;
    static_for<R>([&](auto i) {
        const uint32_t m = u[i()] & pv.mask;
        if (i() < nvalid) packed += m > pv.prefix ? 1u : (m == pv.prefix ? 0x10000u : 0u);
    });
    uint32_t total;
    const uint32_t excl = block_excl_scan(packed, &total, s);
    uint32_t gt_before = excl & 0xFFFFu, eq_before = excl >> 16;
    static_for<R>([&](auto i) {
        const uint32_t m = u[i()] & pv.mask;
        const bool gt = i() < nvalid && m > pv.prefix, eq = i() < nvalid && m == pv.prefix;
        const uint32_t taken = eq_before < pv.need ? eq_before : pv.need;
        if ((gt || (eq && eq_before < pv.need)) && gt_before + taken < (uint32_t)k) out[gt_before + taken] = j0 + i();
        gt_before += gt ? 1u : 0u;
        eq_before += eq ? 1u : 0u;
    });
}

// Global path for segments longer than kSelLds: each pass re-reads the pooled votes.
__device__ __forceinline__ void select_global(const uint32_t *__restrict__ src, int P, int k, int32_t *__restrict__ out,
                              SelectShared &s) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < 2 * kBins; i += kSelThreads) (&s.hist[0][0])[i] = 0;
    __syncthreads();
    Pivot pv = {0u, 0u, (uint32_t)k};
    bool done = false;
    static_for<3>([&](auto pass) {
        if (done) return;
        constexpr int PASS = decltype(pass)::value;
        using D = Digit<PASS>;
        uint32_t *h = s.hist[PASS & 1];
        for (int j0 = 0; j0 < P; j0 += 4 * kSelThreads) {
            const int j = j0 + 4 * tid;
            uint32_t v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = j + e < P ? src[j + e] : 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j + e < P && (v[e] & pv.mask) == pv.prefix) atomicAdd(&h[hist_slot((v[e] >> D::shift) & D::mask)], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            find_bin(h, pv.need, s.sh);
        } else if (PASS == 1) {
            for (int i = tid - 64; i < kBins; i += kSelThreads - 64) s.hist[0][i] = 0;
        }
        __syncthreads();
        const uint32_t dg = s.sh[0], above = s.sh[1], cnt = s.sh[2];
        pv.prefix |= dg << D::shift;
        pv.mask |= D::mask << D::shift;
        pv.need -= above;
        done = cnt == pv.need;
    });

    // ordered compaction in chunks of 4 * kSelThreads positions (4 consecutive per thread)
    uint32_t base_gt = 0, base_eq = 0;
    for (int j0 = 0; j0 < P; j0 += 4 * kSelThreads) {
        const int j = j0 + 4 * tid;
        uint32_t m[4];
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            m[e] = (j + e < P ? src[j + e] : 0u) & pv.mask;
            if (j + e < P) packed += m[e] > pv.prefix ? 1u : (m[e] == pv.prefix ? 0x10000u : 0u);
        }
        const uint32_t incl = wave_incl_scan(packed);
        if (lane == 63) s.wtot[wave] = incl;
        __syncthreads();
        uint32_t woff = 0, ctot = 0;
        static_for<kSelWaves>([&](auto w2) {
            const uint32_t t = s.wtot[w2()];
            woff += w2() < wave ? t : 0u;
            ctot += t;
        });
        const uint32_t excl = woff + incl - packed;
        uint32_t gt_before = base_gt + (excl & 0xFFFFu), eq_before = base_eq + (excl >> 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool gt = j + e < P && m[e] > pv.prefix, eq = j + e < P && m[e] == pv.prefix;
            const uint32_t taken = eq_before < pv.need ? eq_before : pv.need;
            if ((gt || (eq && eq_before < pv.need)) && gt_before + taken < (uint32_t)k) out[gt_before + taken] = j + e;
            gt_before += gt ? 1u : 0u;
            eq_before += eq ? 1u : 0u;
        }
        base_gt += ctot & 0xFFFFu;
        base_eq += ctot >> 16;
        __syncthreads();
        if (base_gt + (base_eq < pv.need ? base_eq : pv.need) >= (uint32_t)k) break;  // all k written
    }
}

__global__ void __launch_bounds__(kSelThreads) topk_select_kernel(const SelectParams p) {
    __shared__ __attribute__((aligned(16))) uint32_t sdata[kSelLds];
    __shared__ __attribute__((aligned(16))) SelectShared s;

    const int seg = blockIdx.x;
    const int r = seg / p.Hkv, g = seg - (seg / p.Hkv) * p.Hkv;
    const int P = p.rt.L[r] - p.w;
    const int k = p.rt.k[r];
    const int64_t base = (int64_t)g * p.sum_P + p.rt.pfx0[r];
    int32_t *out = p.idx ? p.idx + (int64_t)g * p.sum_k + p.rt.k0[r] : nullptr;

    if (P <= kSelLds) {
        if (P <= 4 * kSelThreads) select_resident<4>(p, sdata, s, P, k, base, out);
        else if (P <= 8 * kSelThreads) select_resident<8>(p, sdata, s, P, k, base, out);
        else if (P <= 16 * kSelThreads) select_resident<16>(p, sdata, s, P, k, base, out);
        else select_resident<32>(p, sdata, s, P, k, base, out);
    } else {
        // long segment: pooled by the pooling kernel, read from global memory on each pass
        if (!out || k <= 0) return;
        if (k >= P) {
            for (int j = threadIdx.x; j < P; j += kSelThreads) out[j] = j;
            return;
        }
        select_global((const uint32_t *)(p.pooled + base), P, k, out, s);
    }
}
const void *select_kernel() { return (const void *)&topk_select_kernel; }

// ---- gather -----------------------------------------------------------------------------------
// grid: (row tiles, KV heads).  An output row is row_bytes / 16 lanes of 16-byte copies; a
// block pass covers 256 / lanes-per-row rows and each thread takes kGatherRows rows of a
// tile.  Rows are read and written once, so loads and stores are non-temporal (measured on
// the 16K-token Llama-2-7B layer: 8.2 us against 11.6 us with cached accesses; one row per
// thread beat two or four).  Out-of-range indices are clamped into the prefix so a bad
// index can never read outside K/V.
constexpr int kGatherRows = 1;
int gather_rows_per_thread() { return kGatherRows; }

__global__ void __launch_bounds__(256) kv_gather_kernel(const GatherParams p) {
    const int g = blockIdx.y;
    const int lpr = p.row_bytes >> 4;           // lanes per row
    const int rpb = 256 / lpr;                  // rows per block pass
    const int chunk = threadIdx.x % lpr;
    const int64_t o_begin = p.rt.out0[0];
    const int last = p.rt.n - 1;
    const int64_t o_end = p.rt.out0[last] + p.rt.k[last] + p.w;
    const int64_t tile = (int64_t)rpb * kGatherRows;
    for (int64_t t0 = o_begin + blockIdx.x * tile; t0 < o_end; t0 += (int64_t)gridDim.x * tile) {
        int64_t src[kGatherRows], dst[kGatherRows];
        bool ok[kGatherRows];
#pragma unroll
        for (int u = 0; u < kGatherRows; ++u) {
            const int64_t o = t0 + (int64_t)u * rpb + threadIdx.x / lpr;
            ok[u] = o < o_end;
            int r = 0;
            while (r + 1 < p.rt.n && p.rt.out0[r + 1] <= o) ++r;
            const int t = (int)(o - p.rt.out0[r]);
            const int kr = p.rt.k[r];
            const int P = p.rt.L[r] - p.w;
            int pos = P + (t - kr);
            if (ok[u] && t < kr) {
                pos = p.idx[(int64_t)g * p.sum_k + p.rt.k0[r] + t];
                pos = pos < 0 ? 0 : (pos > P - 1 ? P - 1 : pos);
            }
            src[u] = ((int64_t)g * p.head_stride + (p.rt.tok0[r] + pos) * p.token_stride) * p.esz + chunk * 16;
            dst[u] = ((int64_t)g * p.sum_out + o) * p.row_bytes + chunk * 16;
        }
        u32x4_t a[kGatherRows], b[kGatherRows];
#pragma unroll
        for (int u = 0; u < kGatherRows; ++u) {
            if (ok[u]) {
                a[u] = __builtin_nontemporal_load((const u32x4_t *)((const char *)p.K + src[u]));
                b[u] = __builtin_nontemporal_load((const u32x4_t *)((const char *)p.V + src[u]));
            }
        }
#pragma unroll
        for (int u = 0; u < kGatherRows; ++u) {
            if (ok[u]) {
                __builtin_nontemporal_store(a[u], (u32x4_t *)((char *)p.K_out + dst[u]));
                __builtin_nontemporal_store(b[u], (u32x4_t *)((char *)p.V_out + dst[u]));
            }
        }
    }
}
const void *gather_kernel() { return (const void *)&kv_gather_kernel; }

}  // namespace snapkv
