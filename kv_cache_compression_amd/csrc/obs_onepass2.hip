// obs_onepass2.hip -- window-query votes in one read of K for long segments, up to 32 query rows
// per KV head, gfx950: the one-read kernel with two items in flight per workgroup.
//
// What is computed (page "論文解説: SnapKV — アテンションパターン観測によるKVキャッシュ圧縮",
// section 投票メカニズム, and the アルゴリズム listing): for every KV head g of request r, the
// M = G * L_obs <= 32 window queries score every key the row may see, s = q . k / sqrt(d); each
// row is a softmax over its visible keys; the vote of prefix position j is the sum of its
// weights over the M rows.
//
// How it maps to CDNA4.  As the one-read kernel (obs_onepass.hip): each wave scores its own
// 16-key tile per step for all 32 rows and keeps the exponentials in VGPRs; the items of a
// segment exchange per-row (shift, sum) through tagged slots.  The difference: a workgroup holds
// two items of 1024 keys (two register slots of 64 exponentials per lane each).  It scores an
// item into the free slot and publishes its stats, then finishes the older item (waits for its
// segment, writes its votes).  So the wait of an item for the rest of its segment overlaps the
// key stream of the next, which matters when a segment's items are a large part of the grid (at
// the 380K-token layer each segment has 372 items): the single-slot kernel there spends more
// time waiting than streaming.
// Items are dealt round robin (workgroup w of G takes items w, w + G, w + 2G, ...), so the next
// item is known early: its query rows (copied to LDS by the buffer unit, no registers) and its
// first key steps are issued before the older item is finished, and the memory pipe keeps
// streaming through the wait and the votes.  The barriers order LDS only, so those loads stay
// in flight across them.  The MFMA query operand is read from the LDS tile at each step, which
// keeps the registers of both slots, the keys in flight and the step's operands within 256.
// Meeting the segment: short segments (at most kSelfMergeItems items) merge per item, as in the
// one-read kernel.  In a longer segment the item with the highest index polls the other items'
// tagged stats, merges them and publishes the row shifts; the others poll those.  So no item of
// a long segment takes an arrival count.
// Waits: a workgroup blocks only on the older of its two items (after scoring the younger), and
// a segment's last item on the segment's other items.  Item j is scored once its workgroup has
// finished item j - 2G, which lies in an earlier segment when a segment has at most 2G items
// (checked by the host); so by induction over segments every wait ends.  The reader counts that
// let a segment's last reader clear its stats or shifts are looked at a finish later, off the
// path.  Every counter and tagged slot is back at zero when the launch ends.
// Exponentials are base 2: s*log2(e)/sqrt(d) with the scale folded into one FMA.
#include "obs_score_kernel.h"

namespace snapkv {

namespace {

constexpr float kSumTop = 1.26765060022823e30f;  // 2^100
constexpr int kRaises = 8;                       // re-scorings of a wave-row whose sum overflows
constexpr int kSelfMergeItems = 32;              // segments of up to this many items merge per item
constexpr uint32_t kSumTag = 0x80000000u;        // set in a published row sum (sums are >= +0)

// Workgroup barrier that orders LDS only: vector memory operations in flight (prefetched key
// rows) are not waited for, unlike __syncthreads.
__device__ inline void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ inline uint32_t ld_ag2(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_ag2(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Item2 {
    int item, r, L, P, ns, g, seg, key0, nkeys, item0;
    bool last;  // long segments: the segment's last item, which merges for it
};

}  // namespace

// NW waves per workgroup, RES steps (16 * NW keys each) per slot, DEPTH steps of keys in flight,
// NS slots (items held at once).
template <typename T, int NW, int RES, int DEPTH, int NS>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
obs_onepass2_kernel(const StreamParams p) {
    constexpr int NT = 64 * NW;
    constexpr int kStepKeys = 16 * NW;
    constexpr int ESZ = (int)sizeof(T);
    constexpr int ROWB = 256;   // bytes per key / query row
    constexpr int NQ = 4;       // 16-byte operand chunks per lane per row
    constexpr int RTW = 2;      // 16-row tiles: 32 rows
    constexpr int MROWS = 16 * RTW;
    constexpr int TPR = NT / MROWS;  // threads per row in the central merge
    static_assert(TPR >= 1 && (TPR & (TPR - 1)) == 0, "threads per row");
    static_assert(MROWS == 32, "a wave polls two items per row per load round");
    static_assert((MROWS * 16) % NT == 0, "whole 16-byte query chunks per thread");
    constexpr int QCH = MROWS * 16 / NT;  // query chunks each thread copies

    __shared__ u32x4_t sh_k[NW][256];        // each wave's staging tile (no other wave touches it)
    __shared__ float sh_ms[NW][MROWS], sh_ml[NW][MROWS];
    __shared__ float sh_lsh[NS][NW][MROWS];  // per slot: each wave's row shifts (-inf: no weights)
    __shared__ float sh_fin[NS][MROWS];      // per slot: segment row shifts, +inf for padding rows
    __shared__ u32x4_t sh_q[MROWS * 16];     // the next item's query rows (slot 16 row + (chunk ^ row % 16))
    __shared__ int sh_wrow[MROWS];
    __shared__ int sh_flag;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const float c = p.c;
    const int N = p.n_items;
    const int SLAB = p.slab_keys;
    const int64_t tstride = p.token_stride * ESZ;
    uint64_t *const slots = (uint64_t *)p.partial;  // [item][32]: (shift, sum | kSumTag), 0 = unwritten

    for (int r = tid; r < MROWS; r += NT) sh_wrow[r] = r % p.w;
    for (int i = tid; i < MROWS * 16; i += NT) sh_q[i] = u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();

    auto decode = [&](int item) {
        Item2 it;
        it.item = item;
        int r = 0;
        while (r + 1 < p.rt.n && p.rt.slab0[r + 1] <= item) ++r;
        it.r = r;
        it.L = p.rt.L[r];
        it.P = it.L - p.w;
        it.ns = (it.L + SLAB - 1) / SLAB;
        const int local = item - p.rt.slab0[r];
        it.g = local / it.ns;
        const int sl = local - it.g * it.ns;
        it.seg = r * p.Hkv + it.g;
        it.key0 = sl * SLAB;
        it.nkeys = it.L - it.key0 < SLAB ? it.L - it.key0 : SLAB;
        it.item0 = p.rt.slab0[r] + it.g * it.ns;
        it.last = it.ns > kSelfMergeItems && item == it.item0 + it.ns - 1;
        return it;
    };
    auto ctl = [&](int seg, int line) { return p.seg_ctl + (int64_t)seg * 3 * kStreamSegLine + line * kStreamSegLine; };
    auto fin_slot = [&](int seg) { return (uint32_t *)p.final_shift + (int64_t)seg * MROWS; };
    float E[NS][RES][RTW][4];
    u32x4_t kreg[DEPTH][4];  // key rows in flight (the first DEPTH steps of an item can be prefetched)
    const int row4 = 4 * (int)tstride;

    auto item_rsrc = [&](const Item2 &it) {
        const char *slab_base =
            (const char *)p.K + ((int64_t)it.g * p.head_stride + (p.rt.tok0[it.r] + it.key0) * p.token_stride) * ESZ;
        return __builtin_amdgcn_make_buffer_rsrc((void *)slab_base, (short)0, (int)(it.nkeys * tstride), kBufferFlags);
    };
    auto item_lane_off = [&](int tl) { return ((tl >> 6) * 16 + ((tl >> 4) & 3)) * (int)tstride + (tl & 15) * 16; };
    // The item's query rows and its first DEPTH steps of keys, issued before the workgroup
    // finishes its older item, so that the key stream does not stop while it waits and votes.
    auto issue_first = [&](const int item) {
        const Item2 it = decode(item);
        const int tl = opaque((int)threadIdx.x);
        // query rows -> LDS without passing through registers: lane l of wave v fills tile slot
        // 64v + l, i.e. row (64v + l) / 16, chunk ((64v + l) % 16) ^ row % 16; rows past M are
        // out of the buffer's range
        {
            const char *qb = (const char *)p.q + (((int64_t)p.rt.qi[it.r] * p.Hq + (int64_t)it.g * p.G) * (int64_t)p.w) * ROWB;
            const __amdgpu_buffer_rsrc_t qrsrc =
                __builtin_amdgcn_make_buffer_rsrc((void *)qb, (short)0, p.M * ROWB, kBufferFlags);
            static_for<QCH>([&](auto cc) {
                const int slot = cc() * NT + (tl & (NT - 1));
                const int qrow = slot >> 4, qch = (slot & 15) ^ (qrow & 15);
                const int vw = __builtin_amdgcn_readfirstlane(cc() * NW + (tl >> 6));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(qrsrc, (__attribute__((address_space(3))) void *)&sh_q[64 * vw],
                                                         16, qrow * ROWB + qch * 16, 0, 0, 0);
            });
        }
        asm volatile("" ::: "memory");  // the copy is issued before the key loads
        const __amdgpu_buffer_rsrc_t rsrc = item_rsrc(it);
        const int lane_off = item_lane_off(tl);
        int lbase = 0;
        static_for<DEPTH>([&](auto bc) {
            constexpr int B = decltype(bc)::value;
            asm volatile("" : "+s"(lbase));
            static_for<4>([&](auto i) {
                kreg[B][i] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_off + lbase + i * row4, 0, kNonTemporal));
            });
            lbase += kStepKeys * (int)tstride;
        });
    };

    // ---- score an item into slot SL and publish its row stats ----
    auto stream_item = [&](auto slot_c, const int item) {  // issue_first(item) has been called
        const Item2 it = decode(item);
        constexpr int SL = decltype(slot_c)::value;
        const int P = it.P, key0 = it.key0, nkeys = it.nkeys;
        // lane indices re-derived per item from an opaque thread index: nothing lane-dependent
        // is hoisted out of the item loop into registers held beside both slots' weights
        const int tid = opaque((int)threadIdx.x), tl = tid;
        const int wave = tl >> 6, n16 = tl & 15, grp = (tl >> 4) & 3;
        const int lrow = grp, lch = n16;
        const int lane_off = item_lane_off(tl);
        u32x4_t *const stile = sh_k[wave];
        // the query rows staged by issue_first (every wave's part): wait for this wave's copy,
        // then for the others'
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        const __amdgpu_buffer_rsrc_t rsrc = item_rsrc(it);
        const int vis_end = P < key0 + nkeys ? P : key0 + nkeys;
        float lsh[RTW][4], lw[RTW][4];
        // Every step runs (no branch around a step or a load); loads past the slab read zeros.
        // first: the first scoring of the item (its first steps are in flight already); later
        // ones (raised shifts) load them again
        auto score = [&](const bool first) {
            int lbase = first ? DEPTH * kStepKeys * (int)tstride : 0;
            auto load_step = [&](auto bc) {
                constexpr int B = decltype(bc)::value;
                asm volatile("" : "+s"(lbase));
                static_for<4>([&](auto i) {
                    kreg[B][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                 rsrc, lane_off + lbase + i * row4, 0, kNonTemporal));
                });
                lbase += kStepKeys * (int)tstride;
            };
            if (!first) static_for<DEPTH>([&](auto j) { load_step(j); });
            const int tail = vis_end - key0;
            static_for<RES>([&](auto sc) {
                constexpr int s = decltype(sc)::value;
                constexpr int b = s % DEPTH;
                static_for<4>([&](auto i) {
                    const int row = 4 * i + lrow;
                    stile[16 * row + (lch ^ row)] = kreg[b][i];
                });
                if constexpr (s + DEPTH < RES) load_step(std::integral_constant<int, b>{});
                u32x4_t kf[NQ];
                static_for<NQ>([&](auto qq) { kf[qq] = stile[16 * n16 + ((4 * qq + grp) ^ n16)]; });
                f32x4_t S[RTW];
                static_for<RTW>([&](auto rt) {
                    S[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    static_for<NQ>([&](auto qq) {
                        // query operand read from the LDS tile at each step (no registers held)
                        const u32x4_t qv = sh_q[16 * (rt * 16 + n16) + ((4 * qq + grp) ^ n16)];
                        S[rt] = Dot<T>::step(qv, kf[qq], S[rt]);
                    });
                });
                if ((s + 1) * kStepKeys > opaque_s(tail)) {
                    const int t = opaque(tid);
                    const int j = key0 + s * kStepKeys + (t >> 6) * 16 + (t & 15);
                    const int rb = ((t >> 4) & 3) * 4;
                    const int causal = p.variant == 0 ? 1 : 0;
                    const int end = key0 + nkeys;
                    static_for<RTW>([&](auto rt) {
                        static_for<4>([&](auto i) {
                            int lim = P + causal * (sh_wrow[rt * 16 + rb + i] + 1);
                            lim = lim < end ? lim : end;
                            S[rt][i()] = j >= lim ? neg_inf() : S[rt][i()];
                        });
                    });
                }
                if constexpr (s == 0) {
                    if (first) {
                        static_for<RTW>([&](auto rt) {
                            static_for<4>([&](auto i) {
                                const float m = row16_max(S[rt][i()]);
                                lsh[rt][i] = m == neg_inf() ? 0.f : m * c;
                            });
                        });
                    }
                }
                static_for<RTW>([&](auto rt) {
                    static_for<4>([&](auto i) { E[SL][s][rt][i] = fast_exp2(fmaf(S[rt][i()], c, -lsh[rt][i])); });
                });
            });
        };
        const bool empty = p.variant != 0 && key0 >= P;
        if (empty) {
            static_for<RTW>([&](auto rt) { static_for<4>([&](auto i) { lsh[rt][i] = 0.f; lw[rt][i] = 0.f; }); });
        } else {
            for (int attempt = 0;; ++attempt) {
                score(attempt == 0);
                bool bad = false;
                static_for<RTW>([&](auto rt) {
                    static_for<4>([&](auto i) {
                        float t = 0.f;
                        static_for<RES>([&](auto s) { t += E[SL][s][rt][i]; });
                        lw[rt][i] = row16_sum(t);
                        if (rt * 16 + 4 * grp + i < p.M && !(lw[rt][i] <= kSumTop)) bad = true;
                    });
                });
                if (!__any(bad)) break;
                if (attempt == kRaises) {
                    if (lane == 0) __hip_atomic_fetch_or(p.err, 4u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                static_for<RTW>([&](auto rt) {
                    static_for<4>([&](auto i) {
                        const float l = lw[rt][i];
                        if (!(l <= kSumTop))
                            lsh[rt][i] += l < __builtin_huge_valf() ? __builtin_amdgcn_logf(l) : 64.f * (float)(1 << attempt);
                    });
                });
            }
        }
        // this item's row stats, merged over its waves, published with the tag; each wave's
        // shifts kept in LDS for the votes
        static_for<RTW>([&](auto rt) {
            static_for<4>([&](auto i) {
                if (!(lw[rt][i] > 0.f)) lsh[rt][i] = neg_inf();
                if (n16 == 0) {
                    const int row = rt * 16 + 4 * grp + i;
                    sh_ms[wave][row] = lsh[rt][i];
                    sh_ml[wave][row] = lw[rt][i];
                    sh_lsh[SL][wave][row] = lsh[rt][i];
                }
            });
        });
        lds_barrier();
        if (tid < MROWS && tid < p.M) {
            const int row = tid;
            float m = sh_ms[0][row];
            static_for<NW - 1>([&](auto k2) { m = fmaxf(m, sh_ms[k2 + 1][row]); });
            float l = 0.f;
            if (m != neg_inf())
                static_for<NW>([&](auto k2) {
                    const float mk = sh_ms[k2][row];
                    if (mk != neg_inf()) l = fmaf(sh_ml[k2][row], fast_exp2(mk - m), l);
                });
            const uint64_t word = (uint64_t)__float_as_uint(m) | ((uint64_t)(__float_as_uint(l) | kSumTag) << 32);
            __hip_atomic_store(&slots[(int64_t)it.item * MROWS + row], word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (it.last) {
            // The segment's last item: poll every item's tagged stats, merge them, publish the
            // row shifts, and clear the stats (this item is their only reader).
            const int row_m = tid / TPR, sub = tid - (tid / TPR) * TPR;
            float mm = neg_inf(), ll = 0.f;
            if (row_m < p.M) {
                for (int s0 = sub; s0 < it.ns; s0 += 8 * TPR) {
                    uint64_t bits[8];
                    uint32_t spins = 0;
                    for (;;) {
                        bool all = true;
                        static_for<8>([&](auto bb) {
                            const int s2 = s0 + bb() * TPR;
                            bits[bb()] = s2 < it.ns ? __hip_atomic_load(&slots[(int64_t)(it.item0 + s2) * MROWS + row_m],
                                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                                    : ~0ull;
                            all = all && bits[bb()] != 0ull;
                        });
                        if (all) break;
                        __builtin_amdgcn_s_sleep(8);
                        if (++spins > p.spin_limit) {
                            __hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            break;
                        }
                    }
                    static_for<8>([&](auto bb) {
                        if (s0 + bb() * TPR < it.ns) {
                            const uint64_t wd = bits[bb()];
                            merge_stats(mm, ll, __uint_as_float((uint32_t)wd), __uint_as_float((uint32_t)(wd >> 32) & ~kSumTag),
                                        1.f);
                        }
                    });
                }
            }
#pragma unroll
            for (int o = 1; o < TPR; o <<= 1) {
                const float m2 = __shfl_xor(mm, o, TPR);
                const float l2 = __shfl_xor(ll, o, TPR);
                merge_stats(mm, ll, m2, l2, 1.f);
            }
            const float fin = row_m < p.M && ll > 0.f ? mm + __builtin_amdgcn_logf(ll) : __builtin_huge_valf();
            if (sub == 0) {
                sh_fin[SL][row_m] = fin;
                if (row_m < p.M) st_ag2(&fin_slot(it.seg)[row_m], ~__float_as_uint(fin));
            }
            lds_barrier();  // every thread's loads of the stats are done
            for (int k = tid; k < it.ns * MROWS; k += NT)
                __hip_atomic_store(&slots[(int64_t)it.item0 * MROWS + k], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };

    // ---- wait for an item's segment and write the votes of slot SL ----
    // The item's reader count is taken once its segment is complete; its value is looked at in
    // the workgroup's next finish (or at exit), where the segment's last reader clears the stats
    // (short segments) or the shifts (long ones): nothing waits for that round trip.
    int pend_item0 = 0, pend_ns = 0, pend_seg = 0, pend_kind = 0;  // kind 0: none, 1: short, 2: long
    uint32_t pend_rb = 0;                                          // thread 0: readers before it
    auto pending_clear_flag = [&]() {
        // thread 0: is the pending reader the segment's last? (then its count is reset here)
        bool clear = false;
        if (pend_kind == 1) clear = pend_rb + 1 == (uint32_t)pend_ns;
        if (pend_kind == 2) clear = pend_rb + 1 == (uint32_t)pend_ns - 1;
        if (clear) st_ag2(ctl(pend_seg, 2), 0u);
        return clear;
    };
    auto pending_clear = [&](int tid) {
        if (pend_kind == 1) {
            for (int k = tid; k < pend_ns * MROWS; k += NT)
                __hip_atomic_store(&slots[(int64_t)pend_item0 * MROWS + k], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            for (int k = tid; k < MROWS; k += NT) st_ag2(&fin_slot(pend_seg)[k], 0u);
        }
    };
    auto finish_item = [&](auto slot_c, const int item) {
        const Item2 it = decode(item);
        constexpr int SL = decltype(slot_c)::value;
        const int tid = opaque((int)threadIdx.x), tl = tid;
        const int lane = tl & 63, wave = tl >> 6, n16 = tl & 15, grp = (tl >> 4) & 3;
        const bool self_merge = it.ns <= kSelfMergeItems;
        if (tid == 0) sh_flag = pending_clear_flag() ? 1 : 0;
        if (self_merge) {
            if (wave == 0) {
                constexpr int kPerLane = 4;
                const int row_l = lane & (MROWS - 1), half = lane >> 5;
                float mm = neg_inf(), ll = 0.f;
                if (row_l < p.M) {
                    for (int it0 = half; it0 < it.ns; it0 += 2 * kPerLane) {
                        uint64_t wd[kPerLane];
                        uint32_t spins = 0;
                        for (;;) {
                            bool all = true;
                            static_for<kPerLane>([&](auto b) {
                                const int k = it0 + 2 * b();
                                wd[b()] = k < it.ns ? __hip_atomic_load(&slots[(int64_t)(it.item0 + k) * MROWS + row_l],
                                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                                    : ~0ull;
                                all = all && wd[b()] != 0ull;
                            });
                            if (all) break;
                            __builtin_amdgcn_s_sleep(8);
                            if (++spins > p.spin_limit) {
                                __hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                break;
                            }
                        }
                        static_for<kPerLane>([&](auto b) {
                            if (it0 + 2 * b() < it.ns)
                                merge_stats(mm, ll, __uint_as_float((uint32_t)wd[b()]),
                                            __uint_as_float((uint32_t)(wd[b()] >> 32) & ~kSumTag), 1.f);
                        });
                    }
                }
                merge_stats(mm, ll, __shfl_xor(mm, 32), __shfl_xor(ll, 32), 1.f);
                if (half == 0) sh_fin[SL][row_l] = row_l < p.M && ll > 0.f ? mm + __builtin_amdgcn_logf(ll) : __builtin_huge_valf();
            }
        } else if (!it.last && tid < MROWS) {
            float fin = __builtin_huge_valf();
            if (tid < p.M) {
                uint32_t v, spins = 0;
                while ((v = ld_ag2(&fin_slot(it.seg)[tid])) == 0u) {
                    __builtin_amdgcn_s_sleep(8);
                    if (++spins > p.spin_limit) {
                        __hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
                fin = __uint_as_float(~v);
            }
            sh_fin[SL][tid] = fin;
        }
        lds_barrier();
        // the segment is complete: count this item's read (short segments: of the stats, ns
        // readers; long: of the shifts, the ns - 1 items other than the last); issued after the
        // barrier, whose release fence would otherwise wait for it
        const bool counted = self_merge || !it.last;
        if (tid == 0 && counted)
            pend_rb = __hip_atomic_fetch_add(ctl(it.seg, 2), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (sh_flag) pending_clear(tid);
        pend_kind = counted ? (self_merge ? 1 : 2) : 0;
        pend_item0 = it.item0;
        pend_ns = it.ns;
        pend_seg = it.seg;
        if (it.key0 < it.P) {
            const int vis_end = it.P < it.key0 + it.nkeys ? it.P : it.key0 + it.nkeys;
            float f[RTW][4];
            static_for<RTW>([&](auto rt) {
                static_for<4>([&](auto i) {
                    const int row = rt * 16 + 4 * grp + i;
                    f[rt][i] = fast_exp2(sh_lsh[SL][wave][row] - sh_fin[SL][row]);
                });
            });
            float *const vout = p.votes + (int64_t)it.g * p.sum_P + p.rt.pfx0[it.r];
            static_for<RES>([&](auto sc) {
                constexpr int s = decltype(sc)::value;
                float v = 0.f;
                static_for<RTW>([&](auto rt) { static_for<4>([&](auto i) { v = fmaf(E[SL][s][rt][i], f[rt][i], v); }); });
                v = cross_row_sum4(v);
                const int j = it.key0 + s * kStepKeys + wave * 16 + n16;
                // non-temporal: the votes are read once, by the next launch (5 us less at the
                // 380K-token layer)
                if (grp == 0 && j < vis_end) __builtin_nontemporal_store(v, &vout[j]);
            });
        }
        lds_barrier();  // sh_flag, sh_fin and sh_lsh of this slot are free again
    };

    // Items are dealt round robin: workgroup w takes items w, w + G, w + 2G, ... (G workgroups,
    // at most N); its item number i goes to slot i % NS.  After scoring item i the workgroup
    // finishes item i - (NS - 1), whose slot is the next to fill; each item's queries and first
    // keys are issued before that finish.
    const int G = (int)gridDim.x;
    const int w0 = (int)blockIdx.x;
    issue_first(w0);
    for (int base = w0;; base += NS * G) {
        bool done = false;
        static_for<NS>([&](auto sc) {
            constexpr int S = decltype(sc)::value;
            if (done) return;
            const int item = base + S * G;        // scored at this step, into slot S
            const int fin = item - (NS - 1) * G;  // finished at this step, from slot (S + 1) % NS
            if (item < N) {
                stream_item(std::integral_constant<int, S>{}, item);
                if (item + G < N) issue_first(item + G);
            }
            if (fin >= w0) {
                finish_item(std::integral_constant<int, (S + 1) % NS>{}, fin);
                done = fin + G >= N;  // that was the workgroup's last item
            }
        });
        if (done) break;
    }
    // the last finish's reader count
    if ((int)threadIdx.x == 0) sh_flag = pending_clear_flag() ? 1 : 0;
    lds_barrier();
    if (sh_flag) pending_clear((int)threadIdx.x);
}

// Eight waves per workgroup (one workgroup per CU), two slots of 1024 keys.
template <typename T>
static const void *onepass2_pick(int *threads, int *slab, int *slots) {
    *threads = 64 * 8;
    *slab = 16 * 8 * 8;
    *slots = 2;
    return (const void *)&obs_onepass2_kernel<T, 8, 8, 2, 2>;
}
const void *onepass2_kernel(int dtype, int *threads, int *slab, int *slots) {
    return dtype == 1 ? onepass2_pick<__bf16>(threads, slab, slots) : onepass2_pick<float>(threads, slab, slots);
}

}  // namespace snapkv
