// select_gather.hip -- vote pooling, top-k selection and the compressed-cache gather, gfx950.
//
// Page "論文解説: SnapKV — アテンションパターン観測によるKVキャッシュ圧縮":
//   * クラスタリングによる文脈保持: the votes are max pooled (width K_pool, stride 1,
//     padding K_pool/2) before top-k so that neighbours of strong positions survive.
//   * 投票メカニズム: I = Top_k(C, k); the アルゴリズム listing sorts I ascending and
//     gathers K/V per head, then appends the window.
#include "select_common.h"

namespace snapkv {

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
constexpr int kSelMaxHalfAll = 16;  // widest pool half-width pooled in any select kernel
// Widest pool half-width (K_pool / 2) pooled inside the select kernel for runs of R
// positions per thread (the pooling window of a run is held in registers).
constexpr int max_half(int R) { return R <= 16 ? 16 : 8; }
int select_threads() { return kSelThreads; }
int select_lds_positions() { return kSelLds; }
int select_max_half(int max_P) { return max_half(max_P <= 16 * kSelThreads ? 16 : 32); }

// Wave 0: the bin that holds the need-th largest remaining value of a histogram of NB
// bins (NB = 64 * BPL, bin = digit, ascending).  Lane l sums the BPL bins of descending
// block l (digits NB-1-BPL*l down to NB-BPL*(l+1)), reading its 16-byte chunks in a
// lane-rotated order so the lanes spread over the LDS banks; a wave scan finds the block,
// then lane j < BPL takes one bin of it and a second scan finds the bin.  Writes (digit,
// count above the bin, count in the bin) to sh; nothing if no bin qualifies (inputs
// outside the contract).
template <int NB>
__device__ __forceinline__ void find_bin(const uint32_t *hist, uint32_t need, uint32_t *sh) {
    constexpr int BPL = NB / 64, CH = BPL / 4;
    const int lane = threadIdx.x & 63;
    const uint32_t *blk = hist + NB - BPL * (lane + 1);
    uint32_t sum = 0;
    static_for<CH>([&](auto m) {
        const u32x4_t t = *(const u32x4_t *)(blk + 4 * ((m() + lane) & (CH - 1)));
        sum += t.x + t.y + t.z + t.w;
    });
    const uint32_t incl = wave_incl_scan(sum);
    const uint64_t hit = __ballot(incl - sum < need && need <= incl);
    if (!hit) return;
    const int L = __ffsll((unsigned long long)hit) - 1;
    const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), L);
    const int digit = NB - 1 - (BPL * L + lane);
    const uint32_t c = lane < BPL ? hist[digit] : 0u;
    const uint32_t ci = above + wave_incl_scan(c);
    const uint64_t hit2 = __ballot(lane < BPL && ci - c < need && need <= ci);
    if (!hit2) return;
    if (lane == __ffsll((unsigned long long)hit2) - 1) {
        sh[0] = (uint32_t)digit;
        sh[1] = ci - c;
        sh[2] = c;
    }
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

// Exclusive prefix sum of x over a workgroup of NWAVES waves (one barrier); *total gets the sum.
template <int NWAVES = kSelWaves>
__device__ __forceinline__ uint32_t block_excl_scan_t(uint32_t x, uint32_t *total, uint32_t *wtot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_scan(x);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    uint32_t woff = 0, tot = 0;
    static_for<NWAVES>([&](auto w2) {
        const uint32_t t = wtot[w2()];
        woff += w2() < wave ? t : 0u;
        tot += t;
    });
    *total = tot;
    return woff + incl - x;
}
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t *total, SelectShared &s) {
    return block_excl_scan_t(x, total, s.wtot);
}

// One radix step: histogram of the digit (v >> shift) & dmask over values matching the
// pivot, wave 0 locates the bin of the need-th largest, the pivot takes the digit.
// Returns whether the pivot is final.  Also clears hist[0] when `clear0` (other waves).
template <typename Vals>
__device__ __forceinline__ bool radix_step(Vals &&for_each_value, int shift, uint32_t dmask, uint32_t *h,
                                           bool clear0, Pivot &pv, SelectShared &s) {
    for_each_value([&](uint32_t v) {
        if ((v & pv.mask) == pv.prefix) atomicAdd(&h[(v >> shift) & dmask], 1u);
    });
    __syncthreads();
    if (threadIdx.x < 64) {
        find_bin<kBins>(h, pv.need, s.sh);
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
        // votes -> LDS, coalesced (16-byte loads when the segment is 16-byte aligned), all of a
        // thread's loads in flight; histograms cleared meanwhile.  The AND / OR of the staged
        // values is taken on the way: every pooled value is one of them, so bits they all share
        // are shared by the pooled values too.
        const uint32_t *src = (const uint32_t *)((p.votes ? p.votes : p.pooled) + base);
        uint32_t va = ~0u, vo = 0u;
        if (((uintptr_t)src & 15) == 0) {
            u32x4_t t[R / 4];
            static_for<R / 4>([&](auto i) {
                const int j = 4 * (i() * kSelThreads + tid);
                if (j + 3 < P) {
                    t[i()] = *(const u32x4_t *)(src + j);
                } else {
                    static_for<4>([&](auto e) { t[i()][e()] = j + e() < P ? src[j + e()] : 0u; });
                }
            });
            for (int i = tid; i < 2 * kBins; i += kSelThreads) (&s.hist[0][0])[i] = 0;
            static_for<R / 4>([&](auto i) {
                const int j = 4 * (i() * kSelThreads + tid);
                if (j + 3 < P) {
                    *(u32x4_t *)(sdata + j) = t[i()];
                } else {
                    static_for<4>([&](auto e) {
                        if (j + e() < P) sdata[j + e()] = t[i()][e()];
                    });
                }
                static_for<4>([&](auto e) {
                    if (j + e() < P) { va &= t[i()][e()] & 0x7FFFFFFFu; vo |= t[i()][e()] & 0x7FFFFFFFu; }
                });
            });
        } else {
            uint32_t t[R];
            static_for<R>([&](auto i) {
                const int j = i() * kSelThreads + tid;
                t[i()] = j < P ? src[j] : 0u;
            });
            for (int i = tid; i < 2 * kBins; i += kSelThreads) (&s.hist[0][0])[i] = 0;
            static_for<R>([&](auto i) {
                const int j = i() * kSelThreads + tid;
                if (j < P) {
                    sdata[j] = t[i()];
                    va &= t[i()] & 0x7FFFFFFFu;
                    vo |= t[i()] & 0x7FFFFFFFu;
                }
            });
        }
        wave_and_or(va, vo);
        if (lane == 0) { s.wand[wave] = va; s.wor[wave] = vo; }
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

// ---- segments longer than kSelLds -----------------------------------------------------------
// Tiles of kTile positions, one workgroup each, in three launches (phases 0, 1, 3):
//   0: pool the tile (halo from the neighbours' votes), write the pooled votes, add a
//      4096-bin histogram of bits 30..19 to the segment's global histogram; the tile that
//      finishes last picks the bin b of the k-th value and clears the histogram.
//   1: each tile counts its values above bin b, records that count, and appends its values
//      in bin b to the segment's candidate list (recording where); the last tile refines
//      the exact k-th value among the candidates (bits 18..8, then 7..0) and then records
//      every tile's counts above / equal to that value (one wave per tile, over the tile's
//      candidates).  When the whole bin b is taken there is nothing to refine and each tile
//      records its own counts.
//   3: each tile adds the counts of the tiles before it and writes its positions in order.
// "Last" is decided by a per-segment arrival counter that the last tile resets, so no
// workgroup ever waits for another.  Full passes over the tile use coalesced loads (LDS
// holds the tile where a thread needs its own contiguous run).
constexpr int kLongThreads = 512;  // two tiles per CU (registers), so a launch runs 512 tiles at once
constexpr int kLongWaves = kLongThreads / 64;
constexpr int kTile = 16 * kLongThreads;
constexpr int kLongBins = 4096;
int select_tile_positions() { return kTile; }
int long_threads() { return kLongThreads; }

struct LongShared {
    uint32_t hist[kLongBins];
    uint32_t sh[4];
    uint32_t wtot[kLongWaves];
    uint32_t last;
};

// Block-wide: arrival of this tile at the segment's counter; true in every thread of the
// tile that arrived last (whose arrival also resets the counter for the next call).
__device__ __forceinline__ bool arrive_last(uint32_t *counter, uint32_t n_tiles, LongShared &s) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t before = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = before == n_tiles - 1;
        if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s.last = last ? 1u : 0u;
    }
    __syncthreads();
    return s.last != 0;
}

// Coalesced load of the tile's values: position start + i * kLongThreads + tid at u[i].
__device__ __forceinline__ void load_tile_strided(const uint32_t *src, int P, int start, uint32_t (&u)[16]) {
    static_for<16>([&](auto i) {
        const int j = start + i() * kLongThreads + (int)threadIdx.x;
        u[i()] = j < P ? src[j] : 0u;
    });
}

__global__ void __launch_bounds__(kLongThreads) topk_long_kernel(const LongParams p) {
    constexpr int HA = kSelMaxHalfAll;
    __shared__ __attribute__((aligned(16))) uint32_t sdata[kTile + 2 * HA];
    __shared__ __attribute__((aligned(16))) LongShared s;
    const int tid = threadIdx.x;
    const int seg = blockIdx.y;
    const int r = seg / p.Hkv, g = seg - (seg / p.Hkv) * p.Hkv;
    const int P = p.rt.L[r] - p.w;
    const int k = p.rt.k[r];
    const int start = blockIdx.x * kTile;
    if (P <= kSelLds || start >= P || (p.phase > 0 && (k <= 0 || k >= P))) return;  // whole workgroup
    const uint32_t n_tiles = (uint32_t)((P + kTile - 1) / kTile);
    const int64_t base = (int64_t)g * p.sum_P + p.rt.pfx0[r];
    LongState *st = p.state + seg;
    uint32_t *rec = p.tilecnt + ((int64_t)seg * p.max_tiles + blockIdx.x) * 4;  // tile record
    int32_t *out = p.idx + (int64_t)g * p.sum_k + p.rt.k0[r];
    const int j0 = start + 16 * tid;
    const int nvalid = P - j0 < 0 ? 0 : (P - j0 > 16 ? 16 : P - j0);
    const int off = HA - start;  // position pos sits at sdata[pos + off]

    if (p.phase == 0) {
        // stage votes [start - HA, start + kTile + HA)
        const uint32_t *src = (const uint32_t *)((p.votes ? p.votes : p.pooled) + base);
        uint32_t t[16];
        load_tile_strided(src, P, start, t);
        uint32_t h0 = 0, h1 = 0;
        if (tid < HA) {
            const int jl = start - HA + tid, jr = start + kTile + tid;
            h0 = jl >= 0 ? src[jl] : 0u;
            h1 = jr < P ? src[jr] : 0u;
        }
        for (int i = tid; i < kLongBins; i += kLongThreads) s.hist[i] = 0;
        static_for<16>([&](auto i) { sdata[i() * kLongThreads + tid + HA] = t[i()]; });
        if (tid < HA) {
            sdata[tid] = h0;
            sdata[kTile + HA + tid] = h1;
        }
        __syncthreads();
        uint32_t u[16];
        if (p.votes) {
            static_for<HA + 1>([&](auto h) {
                if (p.half == decltype(h)::value) pool_run<16, decltype(h)::value>(sdata, P, j0, u, off);
            });
            // pooled run -> LDS -> coalesced stores
            __syncthreads();
            static_for<16>([&](auto i) { sdata[16 * tid + i() + HA] = u[i()]; });
            __syncthreads();
            uint32_t *dst = (uint32_t *)(p.pooled + base);
            static_for<16>([&](auto i) {
                const int j = start + i() * kLongThreads + tid;
                if (j < P) dst[j] = sdata[i() * kLongThreads + tid + HA];
            });
        } else {
            static_for<16>([&](auto i) { u[i()] = sdata[16 * tid + i() + HA]; });
        }
        if (k <= 0) return;
        if (k >= P) {  // every position, in order
            static_for<16>([&](auto i) {
                if (i() < nvalid) out[j0 + i()] = j0 + i();
            });
            return;
        }
        static_for<16>([&](auto i) {
            if (i() < nvalid) atomicAdd(&s.hist[(u[i()] & 0x7FFFFFFFu) >> 19], 1u);
        });
        __syncthreads();
        uint32_t *gh = p.ghist + (int64_t)seg * kLongBins;
        for (int i = tid; i < kLongBins; i += kLongThreads)
            if (s.hist[i]) __hip_atomic_fetch_add(&gh[i], s.hist[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!arrive_last(&st->arrived, n_tiles, s)) return;
        // last tile: the segment's histogram -> LDS (and cleared for the next call)
        for (int i = tid; i < kLongBins; i += kLongThreads) {
            s.hist[i] = __hip_atomic_load(&gh[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&gh[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (tid < 64) find_bin<kLongBins>(s.hist, (uint32_t)k, s.sh);
        __syncthreads();
        if (tid == 0) {
            const uint32_t need = (uint32_t)k - s.sh[1];
            st->prefix = s.sh[0] << 19;
            st->mask = 0xFFFu << 19;
            st->need = need;
            st->done = need == s.sh[2] ? 1u : 0u;  // the whole bin is taken
            st->ncand = 0;
        }
        return;
    }

    const uint32_t *src = (const uint32_t *)(p.pooled + base);

    if (p.phase == 1) {
        const uint32_t prefix = st->prefix, mask = st->mask;
        const bool refine = st->done == 0;
        uint32_t u[16];
        load_tile_strided(src, P, start, u);
        uint32_t gt = 0, c = 0;
        static_for<16>([&](auto i) {
            const int j = start + i() * kLongThreads + tid;
            const uint32_t m = u[i()] & 0x7FFFFFFFu & mask;
            gt += (j < P && m > prefix) ? 1u : 0u;
            c += (j < P && m == prefix) ? 1u : 0u;
        });
        uint32_t gtot, ctot;
        (void)block_excl_scan_t<kLongWaves>(gt, &gtot, s.wtot);
        __syncthreads();
        const uint32_t cexcl = block_excl_scan_t<kLongWaves>(c, &ctot, s.wtot);
        if (tid == 0) {
            const uint32_t o0 = refine ? __hip_atomic_fetch_add(&st->ncand, ctot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
            s.sh[3] = o0;
            // agent-scope stores: the segment's last tile reads them in this launch
            __hip_atomic_store(&rec[0], gtot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&rec[1], o0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&rec[2], ctot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // the whole bin is taken: every value in it counts as equal (counts fit 16 bits:
            // a tile holds at most kTile positions)
            if (!refine) rec[3] = (gtot & 0xFFFFu) | (ctot << 16);
        }
        if (!refine) return;
        __syncthreads();
        uint32_t *cand = p.cand + base;
        uint32_t o = s.sh[3] + cexcl;
        static_for<16>([&](auto i) {
            const int j = start + i() * kLongThreads + tid;
            const uint32_t v = u[i()] & 0x7FFFFFFFu;
            if (j < P && (v & mask) == prefix) __hip_atomic_store(&cand[o++], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        });
        if (!arrive_last(&st->arrived, n_tiles, s)) return;
        // last tile: the exact k-th value among the candidates
        const int ncand = (int)__hip_atomic_load(&st->ncand, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        Pivot pv = {prefix, mask, st->need};
        static_for<2>([&](auto pass) {
            constexpr int shift = decltype(pass)::value == 0 ? 8 : 0;
            constexpr uint32_t dmask = decltype(pass)::value == 0 ? 0x7FFu : 0xFFu;
            for (int i = tid; i < kLongBins; i += kLongThreads) s.hist[i] = 0;
            __syncthreads();
            for (int i0 = tid; i0 < ncand; i0 += 8 * kLongThreads) {  // eight loads in flight
                uint32_t v[8];
                static_for<8>([&](auto e) {
                    const int i = i0 + e() * kLongThreads;
                    v[e()] = i < ncand ? __hip_atomic_load(&cand[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
                });
                static_for<8>([&](auto e) {
                    if (i0 + e() * kLongThreads < ncand && (v[e()] & pv.mask) == pv.prefix)
                        atomicAdd(&s.hist[(v[e()] >> shift) & dmask], 1u);
                });
            }
            __syncthreads();
            if (tid < 64) find_bin<kBins>(s.hist, pv.need, s.sh);
            __syncthreads();
            pv.prefix |= s.sh[0] << shift;
            pv.mask |= dmask << shift;
            pv.need -= s.sh[1];
            __syncthreads();
        });
        if (tid == 0) {
            st->prefix = pv.prefix;
            st->mask = pv.mask;
            st->need = pv.need;
        }
        // every tile's counts above / equal to the pivot: its values above bin b (its record)
        // plus its candidates above the pivot, and its candidates equal to it
        const uint32_t *recs = p.tilecnt + (int64_t)seg * p.max_tiles * 4;
        const int lane = tid & 63, wave = tid >> 6;
        for (int t = wave; t < (int)n_tiles; t += kLongWaves) {
            uint32_t *rt = (uint32_t *)recs + 4 * t;
            const uint32_t above0 = __hip_atomic_load(&rt[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t o0 = __hip_atomic_load(&rt[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t nc = __hip_atomic_load(&rt[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            uint32_t gt = 0, eq = 0;
            for (uint32_t i = lane; i < nc; i += 64) {
                const uint32_t m = __hip_atomic_load(&cand[o0 + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & pv.mask;
                gt += m > pv.prefix ? 1u : 0u;
                eq += m == pv.prefix ? 1u : 0u;
            }
            gt = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(gt), 63);
            eq = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(eq), 63);
            if (lane == 0) rt[3] = ((above0 + gt) & 0xFFFFu) | (eq << 16);
        }
        return;
    }

    const uint32_t prefix = st->prefix, mask = st->mask, need = st->need;
    // phase 3: ordered writes after the counts of the tiles before this one
    {
        uint32_t t[16];
        load_tile_strided(src, P, start, t);
        static_for<16>([&](auto i) { sdata[i() * kLongThreads + tid] = t[i()]; });
    }
    uint32_t pgt = 0, peq = 0;
    const uint32_t *recs = p.tilecnt + (int64_t)seg * p.max_tiles * 4;
    for (int t = tid; t < (int)blockIdx.x; t += kLongThreads) {
        const uint32_t v = recs[4 * t + 3];
        pgt += v & 0xFFFFu;
        peq += v >> 16;
    }
    uint32_t gt_base, eq_base;
    (void)block_excl_scan_t<kLongWaves>(pgt, &gt_base, s.wtot);
    __syncthreads();
    (void)block_excl_scan_t<kLongWaves>(peq, &eq_base, s.wtot);  // its barrier also publishes sdata
    __syncthreads();
    uint32_t u[16];
    static_for<16>([&](auto i) { u[i()] = sdata[16 * tid + i()] & 0x7FFFFFFFu; });
    uint32_t packed = 0;
    static_for<16>([&](auto i) {
        const uint32_t m = u[i()] & mask;
        if (i() < nvalid) packed += m > prefix ? 1u : (m == prefix ? 0x10000u : 0u);
    });
    uint32_t total;
    const uint32_t excl = block_excl_scan_t<kLongWaves>(packed, &total, s.wtot);
    uint32_t gt_before = gt_base + (excl & 0xFFFFu), eq_before = eq_base + (excl >> 16);
    static_for<16>([&](auto i) {
        const uint32_t m = u[i()] & mask;
        const bool gt = i() < nvalid && m > prefix, eq = i() < nvalid && m == prefix;
        const uint32_t taken = eq_before < need ? eq_before : need;
        if ((gt || (eq && eq_before < need)) && gt_before + taken < (uint32_t)k) out[gt_before + taken] = j0 + i();
        gt_before += gt ? 1u : 0u;
        eq_before += eq ? 1u : 0u;
    });
}
const void *long_kernel() { return (const void *)&topk_long_kernel; }

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
    }  // longer segments: topk_long_kernel
}
const void *select_kernel() { return (const void *)&topk_select_kernel; }

// ---- hit rate -----------------------------------------------------------------------------------
// grid: (tiles of kHitTile positions, (request, KV head) segments of the group), 1024 threads.
// A workgroup marks the kept positions of its tile in an LDS bitmap (its run of the ascending
// idx: with k small against the tile, one coalesced pass over the segment's idx; else the run
// found by binary search), streams the tile's attention values with 16 loads in flight per
// thread, and adds its integer counts to the segment's, which hit_clear_kernel zeroed just
// before (integer sums: the result does not depend on the order of the adds); a segment of
// one tile stores its counts directly.  The threshold test runs in fp64 on the fp32
// attention values.
constexpr int kHitTile = 32768;

__device__ __forceinline__ int lower_bound_i32(const int32_t *a, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

__global__ void __launch_bounds__(256) hit_clear_kernel(const ClearParams p) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < p.n) p.data[i] = 0u;
}

// Workspace ranges a call expects to find at zero (see the host's control_ranges), 16-byte
// stores over a grid-stride loop.
__global__ void __launch_bounds__(256) ws_clear_kernel(const WsClearParams p) {
    for (int r = 0; r < p.n_ranges; ++r) {
        u32x4_t *const d = (u32x4_t *)(p.base + p.off[r]);
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < p.n16[r]; i += (int64_t)gridDim.x * 256)
            d[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
}
const void *ws_clear() { return (const void *)&ws_clear_kernel; }

__global__ void __launch_bounds__(kSelThreads) hit_rate_kernel(const HitParams p) {
    __shared__ uint32_t bits[kHitTile / 32];
    __shared__ int range[2];
    __shared__ uint32_t wsum[2][kSelWaves];
    const int seg = blockIdx.y;
    const int r = seg / p.Hkv, g = seg - (seg / p.Hkv) * p.Hkv;
    const int P = p.rt.L[r] - p.w;
    const int c0 = blockIdx.x * kHitTile;
    if (c0 >= P) {  // whole workgroup: this segment is shorter than the longest
        if (c0 == 0 && threadIdx.x == 0) {  // an empty prefix counts nothing
            uint32_t *out = p.counts + ((int64_t)p.rt.qi[r] * p.Hkv + g) * 2;
            out[0] = 0u;
            out[1] = 0u;
        }
        return;
    }
    const int span = P - c0 < kHitTile ? P - c0 : kHitTile;
    const int k = p.rt.k[r];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *a = p.a_cur + (int64_t)g * p.sum_P + p.rt.pfx0[r] + c0;
    const int32_t *ix = p.idx + (int64_t)g * p.sum_k + p.rt.k0[r];
    for (int i = tid; i < kHitTile / 32; i += kSelThreads) bits[i] = 0;
    if (tid < 2) range[tid] = k <= 4 * kHitTile ? (tid ? k : 0) : lower_bound_i32(ix, k, c0 + tid * span);
    __syncthreads();
    for (int t = range[0] + tid; t < range[1]; t += kSelThreads) {
        const int j = ix[t] - c0;
        if (j >= 0 && j < span) atomicOr(&bits[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    uint32_t hits = 0, above = 0;
    for (int b0 = 0; b0 < span; b0 += 16 * kSelThreads) {
        float v[16];
        static_for<16>([&](auto i) {
            const int jl = b0 + i() * kSelThreads + tid;
            v[i()] = jl < span ? a[jl] : 0.f;
        });
        static_for<16>([&](auto i) {
            const int jl = b0 + i() * kSelThreads + tid;
            if (jl < span && (double)v[i()] > p.theta) {
                ++above;
                hits += (bits[jl >> 5] >> (jl & 31)) & 1u;
            }
        });
    }
    // workgroup sums (exact integers), added to the segment's counts
    hits = wave_incl_scan(hits);
    above = wave_incl_scan(above);
    if (lane == 63) {
        wsum[0][wave] = hits;
        wsum[1][wave] = above;
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t h = 0, n = 0;
        for (int w2 = 0; w2 < kSelWaves; ++w2) {
            h += wsum[0][w2];
            n += wsum[1][w2];
        }
        uint32_t *out = p.counts + ((int64_t)p.rt.qi[r] * p.Hkv + g) * 2;
        if (P <= kHitTile) {  // the segment's only tile: its counts are the segment's
            out[0] = h;
            out[1] = n;
        } else {
            if (h) atomicAdd(out, h);
            if (n) atomicAdd(out + 1, n);
        }
    }
}
const void *hit_clear() { return (const void *)&hit_clear_kernel; }
int hit_tile_positions() { return kHitTile; }
const void *hit_kernel() { return (const void *)&hit_rate_kernel; }

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
    // The last launch of a call reports the call's error word (every earlier kernel of the
    // call precedes it on the stream) and clears it for the next call.
    if (p.err_word && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        const uint32_t e = *p.err_word;
        if (p.err_out) *p.err_out = e;
        *p.err_word = 0u;
    }
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
