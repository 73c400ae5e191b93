// select_split.hip -- pooling and top-k selection with each (request, KV head) segment split over
// workgroups of 8192 positions that meet twice, gfx950.
//
// What is computed (page "論文解説: SnapKV — アテンションパターン観測によるKVキャッシュ圧縮"):
//   * クラスタリングによる文脈保持: the votes are max pooled (width K_pool, stride 1, padding
//     K_pool/2, the window clipped to the segment) before the top-k.
//   * 投票メカニズム: I = Top_k(C, k), kept in ascending order as the アルゴリズム listing sorts it.
// Ties at the k-th value go to the lowest positions, as in the single-workgroup kernel.  Pooled
// votes are >= 0, so their fp32 bit patterns (sign bit ignored: -0 orders as +0) order like the
// values.
//
// How it maps to CDNA4.  A segment of P <= 32768 positions takes ceil(P / 8192) workgroups of
// 1024 threads (or 512 where more workgroups must be resident); each thread holds a run of 8 (16)
// consecutive positions in registers, pooled from the votes staged in LDS with their halo.  The
// host launches this kernel only when the device holds its whole grid at once, so the
// workgroups of a segment may wait for each other.  They meet twice:
//   1. Each adds the 4096-bin histogram of bits 30..19 of its values (and the sums of its 64
//      blocks of 64 bins) to the segment's histogram in memory, then arrives; a run of equal
//      bins in a thread's positions (max pooling makes plateaus) is added to the LDS histogram
//      once.  Once every chunk has arrived, each reads the block sums and one block: the bin b
//      of the k-th value.
//   2. Each writes its values in bin b to its own columns of a candidate array and one record
//      (its count above b, its count in b), then arrives.  Once every chunk has arrived, each
//      reads the records and, unless bin b is kept whole, every candidate: it refines the k-th
//      value v* from them (bits 18..8, then 7..0) and counts the candidates above and equal to
//      v* in the chunks before its own.
// Then each writes its kept positions at their ranks (positions above v* before it, plus the
// ties before it up to the ties still needed), so the output comes out in ascending order.
// Against one workgroup per segment, each phase's vector work covers 8192 values instead of the
// whole segment, at the price of two agent-scope round trips; it pays for the longer segments.
// Every call leaves the counters and the histogram at zero: past the second meeting each
// workgroup counts itself in at the first counter again, and the one that brings it to twice
// the chunk count (every workgroup is past both meetings) clears both counters; chunk 0 clears
// the histogram once past the second meeting (every chunk read it before arriving there).
#include "select_common.h"

namespace snapkv {

namespace {

constexpr int kChunk = 8192;                // positions per workgroup
constexpr int kHalo = 16;                   // widest pool half-width pooled here
constexpr int kStage = kChunk + 2 * kHalo;  // staged votes: the chunk and its halo
constexpr int kBins = 4096;                 // first digit: bits 30..19
constexpr int kBlockBins = 64;              // bins per block (64 blocks)
constexpr int kRefBins = 2048;              // refinement digits: bits 18..8, then 7..0
constexpr int kMaxChunks = kSplitMaxChunks;
constexpr int kCandLds = kChunk;            // candidates held in LDS; more are re-read per pass
static_assert(kStage >= kCandLds && kBins >= kRefBins, "buffer reuse");

template <int kWaves>
struct SplitShared {
    uint32_t stage[kStage];          // the votes and their halo; then the candidates
    uint32_t hist[kBins];            // the chunk's first histogram; then the refinement histograms
    uint32_t off[kMaxChunks + 1];    // the chunks' first candidate in their concatenation
    uint32_t rec[kMaxChunks];        // the chunks' records
    uint32_t sh[4];
    uint32_t wtot[kWaves], wtot2[kWaves];
};

__device__ inline uint32_t ld_ag(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_ag(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread: the workgroup's memory writes so far are done; then thread 0 counts it in at
// *ctr and waits until the count reaches n (after spin_limit polls it gives up and sets error
// bit 0).
__device__ inline void meet(uint32_t *ctr, uint32_t n, const SplitParams &p) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t v = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
        uint32_t spins = 0;
        while (v < n) {
            __builtin_amdgcn_s_sleep(2);
            v = ld_ag(ctr);
            if (++spins > p.spin_limit) {
                __hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

// Exclusive prefix sum of x over the workgroup; *total gets the sum.  Ends with the barrier
// after which wtot is read, so two calls in a row need a barrier between them.
template <int kWaves>
__device__ inline uint32_t excl_scan(uint32_t x, uint32_t *total, uint32_t *wtot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_scan(x);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    uint32_t woff = 0, tot = 0;
    static_for<kWaves>([&](auto w2) {
        const uint32_t t = wtot[w2()];
        woff += w2() < wave ? t : 0u;
        tot += t;
    });
    *total = tot;
    return woff + incl - x;
}

// Wave 0: the bin holding the need-th largest value of a histogram of NB = 64 * BPL bins (bin =
// digit, ascending).  Lane l sums the BPL bins of descending block l, a wave scan finds the
// block, then lane j < BPL takes one bin of it and a second scan finds the bin.  Writes (digit,
// count above the bin, count in the bin) to sh; nothing if no bin qualifies (inputs outside the
// contract).
template <int NB>
__device__ inline void find_bin_lds(const uint32_t *hist, uint32_t need, uint32_t *sh) {
    constexpr int BPL = NB / 64;
    const int lane = threadIdx.x & 63;
    const uint32_t *blk = hist + NB - BPL * (lane + 1);
    uint32_t sum = 0;
    static_for<BPL / 4>([&](auto m) {
        const u32x4_t t = *(const u32x4_t *)(blk + 4 * ((m() + lane) & (BPL / 4 - 1)));
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

}  // namespace

// kThreads threads of kChunk / kThreads positions each (1024 x 8, or 512 x 16 where the device
// keeps more 512-thread workgroups resident).
template <int kThreads>
__global__ void __launch_bounds__(kThreads) topk_split_kernel(const SplitParams p) {
    constexpr int kWaves = kThreads / 64;
    constexpr int kRun = kChunk / kThreads;  // positions per thread
    constexpr int kBpt = kBins / kThreads;   // first-histogram bins each thread adds (one block's)
    static_assert(kRun * kThreads == kChunk && kBpt * kThreads == kBins && kBpt % 4 == 0, "shape");
    __shared__ __attribute__((aligned(16))) SplitShared<kWaves> s;
    const int tid = threadIdx.x, lane = tid & 63;
    // workgroup -> (request, KV head, chunk)
    const int b = (int)blockIdx.x;
    int r = 0;
    while (r + 1 < p.rt.n && p.wg0[r + 1] <= b) ++r;
    const int P = p.rt.L[r] - p.w;
    if (P <= 0 || P > kMaxChunks * kChunk) return;  // such requests get no workgroups
    const int k = p.rt.k[r];
    const int C = (P + kChunk - 1) / kChunk;
    const int local = b - p.wg0[r];
    const int g = local / C, ci = local - (local / C) * C;
    const int seg = r * p.Hkv + g;
    const int c0 = ci * kChunk;
    const int64_t base = (int64_t)g * p.sum_P + p.rt.pfx0[r];
    const int j0 = c0 + kRun * tid;
    const int nvalid = P - j0 < 0 ? 0 : (P - j0 > kRun ? kRun : P - j0);

    for (int i = tid; i < kBins; i += kThreads) s.hist[i] = 0;  // published by the staging barrier
    // ---- this chunk's pooled values: u[i] is position j0 + i ----
    uint32_t u[kRun];
    if (p.votes) {
        // votes [c0 - kHalo, c0 + kChunk + kHalo) -> LDS (position pos at stage[pos - c0 + kHalo])
        const uint32_t *src = (const uint32_t *)(p.votes + base);
        constexpr int NL = (kStage + kThreads - 1) / kThreads;
        uint32_t t[NL];
        static_for<NL>([&](auto i) {
            const int q = i() * kThreads + tid;
            const int pos = c0 - kHalo + q;
            t[i()] = q < kStage && pos >= 0 && pos < P ? src[pos] : 0u;
        });
        static_for<NL>([&](auto i) {
            const int q = i() * kThreads + tid;
            if (q < kStage) s.stage[q] = t[i()];
        });
        __syncthreads();
        static_for<kHalo + 1>([&](auto h) {
            if (p.half == decltype(h)::value) pool_run<kRun, decltype(h)::value>(s.stage, P, j0, u, kHalo - c0);
        });
        if (p.pooled_out) {
            uint32_t *dst = (uint32_t *)(p.pooled_out + base) + j0;
            static_for<kRun>([&](auto i) {
                if (i() < nvalid) dst[i()] = u[i()];
            });
        }
    } else {
        const uint32_t *src = (const uint32_t *)(p.pooled + base) + j0;
        static_for<kRun>([&](auto i) { u[i()] = i() < nvalid ? src[i()] : 0u; });
    }
    // k and P are the same for every chunk of a segment: these returns are taken by all of them
    int32_t *const out = p.idx ? p.idx + (int64_t)g * p.sum_k + p.rt.k0[r] : nullptr;
    if (!out || k <= 0) return;
    if (k >= P) {  // every position, in order
        static_for<kRun>([&](auto i) {
            if (i() < nvalid) out[j0 + i()] = j0 + i();
        });
        return;
    }
    static_for<kRun>([&](auto i) { u[i()] = i() < nvalid ? u[i()] & 0x7FFFFFFFu : 0u; });

    uint32_t *const ctl = p.ctl + (int64_t)seg * 2 * kSplitLine;  // [0]: first meeting, [kSplitLine]: second
    uint32_t *const gh = p.ghist + (int64_t)seg * (kBins + kBins / kBlockBins);
    uint32_t *const gblk = gh + kBins;

    // ---- meeting 1: the segment's histogram of bits 30..19 ----
    // (the histogram was zeroed while the votes were staged; a run of equal digits in a thread's
    // positions -- max pooling makes plateaus -- is added once)
    if (!p.votes) __syncthreads();  // no staging barrier: the zeroing is published here
    {
        uint32_t cur = u[0] >> 19, cnt = 0;
        static_for<kRun>([&](auto i) {
            if (i() < nvalid) {
                const uint32_t d = u[i()] >> 19;
                if (d != cur) {
                    if (cnt) atomicAdd(&s.hist[cur], cnt);
                    cur = d;
                    cnt = 0;
                }
                ++cnt;
            }
        });
        if (cnt) atomicAdd(&s.hist[cur], cnt);
    }
    __syncthreads();
    {
        // thread t adds bins kBpt t .. kBpt t + kBpt - 1, which all lie in block t / (64 / kBpt)
        constexpr int kTpb = kBlockBins / kBpt;  // threads per block of bins
        uint32_t bsum = 0;
        static_for<kBpt / 4>([&](auto q) {
            const u32x4_t h4 = *(const u32x4_t *)&s.hist[kBpt * tid + 4 * q()];
            static_for<4>([&](auto e) {
                const uint32_t c = h4[e()];
                if (c) __hip_atomic_fetch_add(&gh[kBpt * tid + 4 * q() + e()], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                bsum += c;
            });
        });
#pragma unroll
        for (int o = 1; o < kTpb; o <<= 1) bsum += __shfl_xor(bsum, o);
        if ((tid & (kTpb - 1)) == 0 && bsum)
            __hip_atomic_fetch_add(&gblk[tid / kTpb], bsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    meet(&ctl[0], (uint32_t)C, p);
    if (tid < 64) {
        // lane l: block 63 - l, then bin 64 * block + 63 - l (descending order)
        const uint32_t need = (uint32_t)k;
        const uint32_t cb = ld_ag(&gblk[63 - lane]);
        const uint32_t ib = wave_incl_scan(cb);
        const uint64_t hb = __ballot(ib - cb < need && need <= ib);
        const int lb = hb ? __ffsll((unsigned long long)hb) - 1 : 0;
        const uint32_t above_blk = (uint32_t)__builtin_amdgcn_readlane((int)(ib - cb), lb);
        const int blk = 63 - lb;
        const uint32_t cf = ld_ag(&gh[kBlockBins * blk + 63 - lane]);
        const uint32_t i2 = above_blk + wave_incl_scan(cf);
        const uint64_t h2 = __ballot(i2 - cf < need && need <= i2);
        const int l2 = h2 ? __ffsll((unsigned long long)h2) - 1 : 0;
        if (lane == l2) {
            s.sh[0] = (uint32_t)(kBlockBins * blk + 63 - l2);
            s.sh[1] = i2 - cf;
            s.sh[2] = cf;
        }
    }
    __syncthreads();
    Pivot pv = {s.sh[0] << 19, 0xFFFu << 19, (uint32_t)k - s.sh[1]};
    const bool whole = pv.need == s.sh[2];  // every value in bin b is kept: nothing to refine

    // ---- meeting 2: the candidates (values in bin b) and the chunks' records ----
    uint32_t c_gt = 0, c_eq = 0;
    static_for<kRun>([&](auto i) {
        const uint32_t m = u[i()] & pv.mask;
        c_gt += i() < nvalid && m > pv.prefix ? 1u : 0u;
        c_eq += i() < nvalid && m == pv.prefix ? 1u : 0u;
    });
    uint32_t tot;
    const uint32_t ex = excl_scan<kWaves>(c_gt | (c_eq << 16), &tot, s.wtot);  // counts fit 16 bits (<= 8192)
    uint32_t *const cand = p.cand + base + c0;  // this chunk's columns
    if (!whole) {
        uint32_t o = ex >> 16;
        static_for<kRun>([&](auto i) {
            if (i() < nvalid && (u[i()] & pv.mask) == pv.prefix) st_ag(&cand[o++], u[i()]);
        });
    }
    uint32_t *const recs = p.rec + (int64_t)seg * kMaxChunks;
    if (tid == 0) st_ag(&recs[ci], tot);  // (count above bin b) | (count in bin b) << 16
    meet(&ctl[kSplitLine], (uint32_t)C, p);
    // past both meetings: counted in again at the first counter (looked at the end)
    uint32_t dep = 0;
    if (tid == 0) dep = __hip_atomic_fetch_add(&ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (ci == 0)
        for (int i = tid; i < kBins + kBins / kBlockBins; i += kThreads) st_ag(&gh[i], 0u);
    if (tid < C) s.rec[tid] = ld_ag(&recs[tid]);
    __syncthreads();
    if (tid == 0) {
        // (a chunk's count never exceeds its positions; the bound keeps reads inside the segment
        // even if a wait gave up and a record is stale)
        uint32_t o = 0;
        for (int c = 0; c < C; ++c) {
            const uint32_t n = (uint32_t)(P - c * kChunk < kChunk ? P - c * kChunk : kChunk);
            const uint32_t nc = s.rec[c] >> 16;
            s.off[c] = o;
            o += nc < n ? nc : n;
        }
        s.off[C] = o;
    }
    __syncthreads();
    uint32_t above_before = 0;
    for (int c = 0; c < ci; ++c) above_before += s.rec[c] & 0xFFFFu;
    const uint32_t ncand = s.off[C], cand_before = s.off[ci];

    // counts of the chunks before this one: above v*, and equal to v*
    uint32_t gt_base = above_before, eq_base = cand_before;
    if (!whole) {
        // candidate q of the concatenation (chunk order): chunk c with off[c] <= q < off[c + 1]
        const uint32_t *const cand0 = p.cand + base;
        auto cand_at_global = [&](uint32_t q) {
            int c = 0;
            while (c + 1 < C && s.off[c + 1] <= q) ++c;
            return ld_ag(&cand0[(int64_t)c * kChunk + (q - s.off[c])]);
        };
        const bool in_lds = ncand <= (uint32_t)kCandLds;
        if (in_lds) {
            for (uint32_t q0 = tid; q0 < ncand; q0 += 4 * kThreads) {  // four loads in flight
                uint32_t v[4];
                static_for<4>([&](auto e) {
                    const uint32_t q = q0 + e() * kThreads;
                    v[e()] = q < ncand ? cand_at_global(q) : 0u;
                });
                static_for<4>([&](auto e) {
                    const uint32_t q = q0 + e() * kThreads;
                    if (q < ncand) s.stage[q] = v[e()];
                });
            }
        }
        auto for_each_cand = [&](uint32_t n, auto &&f) {
            if (in_lds) {
                for (uint32_t q = tid; q < n; q += kThreads) f(s.stage[q]);
            } else {
                for (uint32_t q0 = tid; q0 < n; q0 += 4 * kThreads) {
                    uint32_t v[4];
                    static_for<4>([&](auto e) {
                        const uint32_t q = q0 + e() * kThreads;
                        v[e()] = q < n ? cand_at_global(q) : 0u;
                    });
                    static_for<4>([&](auto e) {
                        if (q0 + e() * kThreads < n) f(v[e()]);
                    });
                }
            }
        };
        bool done = false;
        static_for<2>([&](auto pass) {
            constexpr int shift = decltype(pass)::value == 0 ? 8 : 0;
            constexpr uint32_t dmask = decltype(pass)::value == 0 ? 0x7FFu : 0xFFu;
            if (done) return;  // uniform
            for (int i = tid; i < kRefBins; i += kThreads) s.hist[i] = 0;
            __syncthreads();  // also publishes the candidates in LDS
            for_each_cand(ncand, [&](uint32_t v) {
                if ((v & pv.mask) == pv.prefix) atomicAdd(&s.hist[(v >> shift) & dmask], 1u);
            });
            __syncthreads();
            if (tid < 64) find_bin_lds<decltype(pass)::value == 0 ? kRefBins : 256>(s.hist, pv.need, s.sh);
            __syncthreads();
            pv.prefix |= s.sh[0] << shift;
            pv.mask |= dmask << shift;
            pv.need -= s.sh[1];
            done = s.sh[2] == pv.need;
            __syncthreads();  // s.sh and s.hist are reused
        });
        uint32_t g1 = 0, e1 = 0;
        for_each_cand(cand_before, [&](uint32_t v) {
            const uint32_t m = v & pv.mask;
            g1 += m > pv.prefix ? 1u : 0u;
            e1 += m == pv.prefix ? 1u : 0u;
        });
        uint32_t gsum, esum;
        (void)excl_scan<kWaves>(g1, &gsum, s.wtot);
        (void)excl_scan<kWaves>(e1, &esum, s.wtot2);
        gt_base = above_before + gsum;
        eq_base = esum;
    }

    // ---- ordered writes ----
    uint32_t packed = 0;
    static_for<kRun>([&](auto i) {
        const uint32_t m = u[i()] & pv.mask;
        if (i() < nvalid) packed += m > pv.prefix ? 1u : (m == pv.prefix ? 0x10000u : 0u);
    });
    __syncthreads();  // wtot is reused
    uint32_t total;
    const uint32_t ex2 = excl_scan<kWaves>(packed, &total, s.wtot);
    uint32_t gt_before = gt_base + (ex2 & 0xFFFFu), eq_before = eq_base + (ex2 >> 16);
    static_for<kRun>([&](auto i) {
        const uint32_t m = u[i()] & pv.mask;
        const bool gt = i() < nvalid && m > pv.prefix, eq = i() < nvalid && m == pv.prefix;
        const uint32_t taken = eq_before < pv.need ? eq_before : pv.need;
        if ((gt || (eq && eq_before < pv.need)) && gt_before + taken < (uint32_t)k) out[gt_before + taken] = j0 + i();
        gt_before += gt ? 1u : 0u;
        eq_before += eq ? 1u : 0u;
    });
    if (tid == 0 && dep == 2u * (uint32_t)C - 1u) {  // every workgroup of the segment is past both meetings
        st_ag(&ctl[0], 0u);
        st_ag(&ctl[kSplitLine], 0u);
    }
}

const void *split_kernel(int threads) {
    return threads == 512 ? (const void *)&topk_split_kernel<512> : (const void *)&topk_split_kernel<1024>;
}
int split_chunk() { return kChunk; }
int split_max_half() { return kHalo; }

}  // namespace snapkv
