// obs_onepass.hip -- window-query votes in one read of K, up to 32 query rows per KV head, gfx950.
//
// What is computed (page "論文解説: SnapKV — アテンションパターン観測によるKVキャッシュ圧縮",
// section 投票メカニズム, and the アルゴリズム listing): for every KV head g of request r, the
// M = G * L_obs <= 32 window queries score every key the row may see, s = q . k / sqrt(d); each
// row is a softmax over its visible keys; the vote of prefix position j is the sum of its
// weights over the M rows.
//
// How it maps to CDNA4.  A persistent grid (one workgroup of NW waves per CU) takes items from
// an atomic counter, like the streaming two-phase kernel, but every item -- one slab of
// RES * 16 * NW keys of a (request, KV head) segment -- is visited once:
//   * Each wave scores its own 16-key tile of every step for all 32 rows (MFMA 16x16x32 bf16 or
//     16x16x4 f32; the tile is register staged, 1 KB contiguous per load instruction, and
//     transposed through the wave's own LDS tile) and keeps the exponentials, taken against the
//     wave's first-tile row shift as the logits arrive, in VGPRs: the HBM stream hides the
//     exponentials.  A wave-row whose sum exceeds 2^100 re-scores its tiles with the shift raised
//     (never for ordinary inputs; past 8 raises error bit 2 is set).
//   * The items of a segment then meet, through per-item row stats that carry a validity tag
//     (zero means "not written yet"), so no arrival count sits on the path.  Short segments (at
//     most kSelfMerge items): each item publishes its (shift, sum) per row; one wave of each item
//     polls every item's slots until all are written (one wave keeps the poll traffic beside the
//     still-running key streams small), merges them and hands the shifts to the other waves; a
//     count of readers, taken off the path, lets the last reader clear the slots.  Longer segments: an arrival count finds
//     the last item, which merges once and publishes tagged row shifts that the others poll; the
//     last reader clears them.  Every slot and count is back at zero when the launch ends.
//   * Each item then scales its resident weights by exp2(shift_wave - shift_segment), where the
//     segment shift includes log2 of the row's softmax denominator, and writes their sums over
//     the rows as the votes of its keys.
// A workgroup's first item is its own index; later ones come from one atomic counter, drawn
// once the workgroup's segment is complete.  A workgroup waits only for items of its own
// segment, which running workgroups hold or which are the next to be drawn, so the launch
// completes whenever a segment's items fit in the resident grid at once, which the host checks
// (longest segment's items <= resident workgroups).
// Exponentials are base 2: s*log2(e)/sqrt(d) with the scale folded into one FMA.
#include "obs_score_kernel.h"

namespace snapkv {

namespace {

constexpr float kSumHigh = 1.26765060022823e30f;  // 2^100
constexpr int kMaxRaises = 8;                     // re-scorings of a wave-row whose sum overflows
constexpr int kSelfMerge = 32;                    // segments of up to this many items merge per item
constexpr uint32_t kTag = 0x80000000u;            // set in a published row sum (sums are >= +0)

__device__ inline uint32_t ld_ag(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_ag(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// NW waves per workgroup, RES steps (16 * NW keys each) held per item, DEPTH steps of keys in
// flight per wave.
template <typename T, int NW, int RES, int DEPTH>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
obs_onepass_kernel(const StreamParams p) {
    constexpr int NT = 64 * NW;
    constexpr int kStepKeys = 16 * NW;
    constexpr int ESZ = (int)sizeof(T);
    constexpr int ROWB = 256;   // bytes per key / query row
    constexpr int NQ = 4;       // 16-byte operand chunks per lane per row
    constexpr int RTW = 2;      // 16-row tiles: 32 rows
    constexpr int MROWS = 16 * RTW;
    constexpr int TPR = NT / MROWS;  // threads per row in the stats merge
    static_assert(TPR >= 1 && (TPR & (TPR - 1)) == 0, "threads per row");
    static_assert(MROWS == 32, "a wave polls two items per row per load round");

    __shared__ u32x4_t sh_k[NW][256];  // each wave's staging tile (no other wave touches it)
    __shared__ float sh_ms[NW][MROWS], sh_ml[NW][MROWS];
    __shared__ float sh_fin[MROWS];    // segment row shifts (max + log2 of the sum), +inf for padding rows
    __shared__ int sh_wrow[MROWS];
    __shared__ int sh_ticket, sh_flag;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, grp = lane >> 4;
    const float c = p.c;
    const int N = p.n_items;
    const int SLAB = p.slab_keys;
    const int64_t tstride = p.token_stride * ESZ;

    for (int r = tid; r < MROWS; r += NT) sh_wrow[r] = r % p.w;
    __syncthreads();
    int item = blockIdx.x;  // first item; the launch has at most as many workgroups as items

    int cur_seg = -1;
    u32x4_t qf[RTW][NQ];

    while (item < N) {
        int r = 0;
        while (r + 1 < p.rt.n && p.rt.slab0[r + 1] <= item) ++r;
        const int L = p.rt.L[r];
        const int P = L - p.w;
        const int ns = (L + SLAB - 1) / SLAB;
        const int local = item - p.rt.slab0[r];
        const int g = local / ns, sl = local - (local / ns) * ns;
        const int seg = r * p.Hkv + g;
        const int key0 = sl * SLAB;
        const int nkeys = L - key0 < SLAB ? L - key0 : SLAB;

        if (seg != cur_seg) {
            cur_seg = seg;
            const char *qb = (const char *)p.q + (((int64_t)p.rt.qi[r] * p.Hq + (int64_t)g * p.G) * (int64_t)p.w) * ROWB;
            static_for<RTW>([&](auto rt) {
                const int row = rt * 16 + n16;
                static_for<NQ>([&](auto qq) {
                    qf[rt][qq] = row < p.M ? *(const u32x4_t *)(qb + (int64_t)row * ROWB + (4 * qq + grp) * 16)
                                           : u32x4_t{0u, 0u, 0u, 0u};
                });
            });
        }

        // ---- score the slab once; the weights stay in VGPRs ----
        float E[RES][RTW][4];
        float lsh[RTW][4], lw[RTW][4];
        const char *slab_base = (const char *)p.K + ((int64_t)g * p.head_stride + (p.rt.tok0[r] + key0) * p.token_stride) * ESZ;
        // loads past the slab's keys return zeros (buffer range check); such keys are masked
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void *)slab_base, (short)0, (int)(nkeys * tstride), kBufferFlags);
        const int lrow = lane >> 4, lch = lane & 15;
        const int lane_off = (wave * 16 + lrow) * (int)tstride + lch * 16;
        u32x4_t *const stile = sh_k[wave];

        // Every item runs all RES steps, with no branch around a step or a load: loads past the
        // slab's keys return zeros (buffer range check) and those keys are masked.  (A guarded
        // step would make the compiler wait for every load in flight at each step, since on the
        // path that skipped the previous step's loads fewer are outstanding.)
        const int vis_end = P < key0 + nkeys ? P : key0 + nkeys;  // keys every row sees end here
        auto score = [&](const bool first) {
            u32x4_t kreg[DEPTH][4];
            // Scalar offset of the next step to load, advanced one step per load_step and hidden
            // from the optimiser: otherwise every step's four offsets are precomputed and held
            // in SGPRs across the whole unrolled slab.
            int lbase = 0;
            const int row4 = 4 * (int)tstride;
            auto load_step = [&](auto bc) {
                constexpr int B = decltype(bc)::value;
                asm volatile("" : "+s"(lbase));
                // the whole offset goes in the VGPR operand (soffset 0), which the buffer range
                // check covers on every generation
                static_for<4>([&](auto i) {
                    kreg[B][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                 rsrc, lane_off + lbase + i * row4, 0, kNonTemporal));
                });
                lbase += kStepKeys * (int)tstride;
            };
            static_for<DEPTH>([&](auto j) { load_step(j); });
            const int tail = vis_end - key0;
            static_for<RES>([&](auto sc) {
                constexpr int s = decltype(sc)::value;
                constexpr int b = s % DEPTH;
                // transpose through the wave's LDS tile: four whole rows per load instruction in,
                // 16 keys x 16 bytes per lane group out
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
                    static_for<NQ>([&](auto qq) { S[rt] = Dot<T>::step(qf[rt][qq], kf[qq], S[rt]); });
                });
                if ((s + 1) * kStepKeys > opaque_s(tail)) {
                    // Keys past the slab, and (causal window) window keys after the row's
                    // position / (prefix only) every window key.  The lane's indices are
                    // recomputed here from an opaque thread index, so that nothing of this
                    // rarely taken branch is hoisted into registers held across the slab.
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
                    static_for<4>([&](auto i) { E[s][rt][i] = fast_exp2(fmaf(S[rt][i()], c, -lsh[rt][i])); });
                });
            });
        };

        const bool empty = p.variant != 0 && key0 >= P;  // prefix only: window keys are visible to no row
        if (empty) {
            static_for<RTW>([&](auto rt) { static_for<4>([&](auto i) { lsh[rt][i] = 0.f; lw[rt][i] = 0.f; }); });
        } else {
            // Each wave re-scores its own tiles while one of its rows' sums is above 2^100 (or not
            // finite): a later key outgrew the first tile's shift, which rises by log2 of the sum
            // (by 64 * 2^n when the sum overflowed).
            for (int attempt = 0;; ++attempt) {
                score(attempt == 0);
                bool bad = false;
                static_for<RTW>([&](auto rt) {
                    static_for<4>([&](auto i) {
                        float t = 0.f;
                        static_for<RES>([&](auto s) { t += E[s][rt][i]; });
                        lw[rt][i] = row16_sum(t);
                        if (rt * 16 + 4 * grp + i < p.M && !(lw[rt][i] <= kSumHigh)) bad = true;
                    });
                });
                if (!__any(bad)) break;
                if (attempt == kMaxRaises) {
                    if (lane == 0) __hip_atomic_fetch_or(p.err, 4u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                static_for<RTW>([&](auto rt) {
                    static_for<4>([&](auto i) {
                        const float l = lw[rt][i];
                        if (!(l <= kSumHigh))
                            lsh[rt][i] += l < __builtin_huge_valf() ? __builtin_amdgcn_logf(l) : 64.f * (float)(1 << attempt);
                    });
                });
            }
        }

        // ---- the item's row stats, merged over its waves, published with the tag ----
        // (a wave-row without weights gets shift -inf: its factor below is then 0)
        static_for<RTW>([&](auto rt) {
            static_for<4>([&](auto i) {
                if (!(lw[rt][i] > 0.f)) lsh[rt][i] = neg_inf();
                if (n16 == 0) {
                    const int row = rt * 16 + 4 * grp + i;
                    sh_ms[wave][row] = lsh[rt][i];
                    sh_ml[wave][row] = lw[rt][i];
                }
            });
        });
        __syncthreads();
        uint64_t *const slots = (uint64_t *)p.partial;  // [item][32]: (shift, sum | kTag), 0 = unwritten
        const int item0 = p.rt.slab0[r] + g * ns;        // the segment's first item
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
            const uint64_t word = (uint64_t)__float_as_uint(m) | ((uint64_t)(__float_as_uint(l) | kTag) << 32);
            __hip_atomic_store(&slots[(int64_t)item * MROWS + row], word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // ---- meet the segment's other items ----
        const bool self_merge = ns <= kSelfMerge;
        uint32_t *const done_ctr = p.seg_ctl + (int64_t)seg * 3 * kStreamSegLine;
        uint32_t *const readers = done_ctr + 2 * kStreamSegLine;
        uint32_t *const fin_slot = (uint32_t *)p.final_shift + (int64_t)seg * MROWS;  // ~bits of the shift, 0 = unwritten
        auto merge_word = [](float &mm, float &ll, uint64_t wd) {
            merge_stats(mm, ll, __uint_as_float((uint32_t)wd), __uint_as_float((uint32_t)(wd >> 32) & ~kTag), 1.f);
        };
        uint32_t next = 0;         // the next item's draw (thread 0)
        bool last_item = false;    // long segments: this item merged for the segment
        uint32_t read_before = 0;  // readers of the slots (short) or shifts (long) before this item
        if (self_merge) {
            // Wave 0 polls all of the segment's slots (row lane % 32, items lane / 32, +2, ...;
            // eight items per round of loads) until each is written, merges them and hands the
            // shifts to the other waves through LDS.  One polling wave per workgroup keeps the
            // poll traffic, which shares the memory system with the key streams still running,
            // small.
            if (wave == 0) {
                constexpr int kPerLane = 4;
                const int row_l = lane & (MROWS - 1), half = lane >> 5;
                float mm = neg_inf(), ll = 0.f;
                if (row_l < p.M) {
                    for (int it0 = half; it0 < ns; it0 += 2 * kPerLane) {
                        uint64_t wd[kPerLane];
                        uint32_t spins = 0;
                        for (;;) {
                            bool all = true;
                            static_for<kPerLane>([&](auto b) {
                                const int it = it0 + 2 * b();
                                wd[b()] = it < ns ? __hip_atomic_load(&slots[(int64_t)(item0 + it) * MROWS + row_l],
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
                            if (it0 + 2 * b() < ns) merge_word(mm, ll, wd[b()]);
                        });
                    }
                }
                merge_stats(mm, ll, __shfl_xor(mm, 32), __shfl_xor(ll, 32), 1.f);
                if (half == 0) sh_fin[row_l] = row_l < p.M && ll > 0.f ? mm + __builtin_amdgcn_logf(ll) : __builtin_huge_valf();
            }
            __syncthreads();
            // The segment is complete: draw the next item and count this item's read of the slots.
            // Issued after the barrier (whose release fence would wait for them), so both round
            // trips overlap the votes.
            if (tid == 0) {
                next = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                read_before = __hip_atomic_fetch_add(readers, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        } else {
            // the last arrival merges once and publishes the shifts
            const int row_m = tid / TPR, sub = tid - (tid / TPR) * TPR;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0) {
                const uint32_t before = __hip_atomic_fetch_add(done_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (before >= (uint32_t)ns) __hip_atomic_fetch_or(p.err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                sh_flag = before + 1 == (uint32_t)ns ? 1 : 0;
            }
            __syncthreads();
            last_item = sh_flag != 0;
            if (last_item) {
                float mm = neg_inf(), ll = 0.f;
                if (row_m < p.M) {
                    for (int s0 = sub; s0 < ns; s0 += 8 * TPR) {
                        uint64_t bits[8];
                        static_for<8>([&](auto bb) {
                            const int s2 = s0 + bb() * TPR < ns ? s0 + bb() * TPR : ns - 1;
                            bits[bb()] = __hip_atomic_load(&slots[(int64_t)(item0 + s2) * MROWS + row_m], __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                        });
                        static_for<8>([&](auto bb) {
                            if (s0 + bb() * TPR < ns) merge_word(mm, ll, bits[bb()]);
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
                    sh_fin[row_m] = fin;
                    if (row_m < p.M) st_ag(&fin_slot[row_m], ~__float_as_uint(fin));
                }
            } else if (tid < MROWS) {
                float fin = __builtin_huge_valf();
                if (tid < p.M) {
                    uint32_t v, spins = 0;
                    while ((v = ld_ag(&fin_slot[tid])) == 0u) {
                        __builtin_amdgcn_s_sleep(4);
                        if (++spins > p.spin_limit) {
                            __hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            break;
                        }
                    }
                    fin = __uint_as_float(~v);
                }
                sh_fin[tid] = fin;
            }
            __syncthreads();
            // The segment is complete: draw the next item; count this item's read of the shifts
            // (the ns - 1 items other than the merger read them).  Both overlap the votes.
            if (tid == 0) {
                next = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (!last_item) read_before = __hip_atomic_fetch_add(readers, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }

        // ---- votes: resident weights x row factor, summed over the 32 rows ----
        if (key0 < P) {
            float f[RTW][4];
            static_for<RTW>([&](auto rt) {
                static_for<4>([&](auto i) {
                    const int row = rt * 16 + 4 * grp + i;
                    f[rt][i] = fast_exp2(lsh[rt][i] - sh_fin[row]);
                });
            });
            float *const vout = p.votes + (int64_t)g * p.sum_P + p.rt.pfx0[r];
            static_for<RES>([&](auto sc) {
                constexpr int s = decltype(sc)::value;
                float v = 0.f;
                static_for<RTW>([&](auto rt) { static_for<4>([&](auto i) { v = fmaf(E[s][rt][i], f[rt][i], v); }); });
                v = cross_row_sum4(v);
                const int j = key0 + s * kStepKeys + wave * 16 + n16;
                // non-temporal: the votes are read once, by the next launch (0.5 us less per
                // step at the 16K-token layer)
                if (grp == 0 && j < vis_end) __builtin_nontemporal_store(v, &vout[j]);
            });
        }

        // ---- the last reader clears the segment's slots (and shifts) for the next launch ----
        if (self_merge) {
            // ns readers (wave 0 of each item); the last clears with its own wave
            if (wave == 0) {
                const bool clear = __builtin_amdgcn_readfirstlane((int)read_before) + 1 == ns;
                if (clear) {
                    if (lane == 0) st_ag(readers, 0u);
                    for (int k = lane; k < ns * MROWS; k += 64)
                        __hip_atomic_store(&slots[(int64_t)item0 * MROWS + k], 0ull, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
                if (lane == 0) sh_ticket = (int)next;
            }
            __syncthreads();
        } else {
            if (tid == 0) {
                // ns - 1 readers; with ns == 1 the merger clears
                const bool clear = last_item ? ns == 1 : read_before + 1 == (uint32_t)ns - 1;
                if (clear) st_ag(readers, 0u);
                if (last_item) st_ag(done_ctr, 0u);
                sh_flag = clear ? 1 : 0;
                sh_ticket = (int)next;
            }
            __syncthreads();
            if (sh_flag) {
                for (int k = tid; k < ns * MROWS; k += NT)
                    __hip_atomic_store(&slots[(int64_t)item0 * MROWS + k], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                for (int k = tid; k < MROWS; k += NT) st_ag(&fin_slot[k], 0u);
            }
        }
        const int t_next = sh_ticket;
        __syncthreads();  // everyone has read sh_ticket, sh_flag and sh_fin before they are written again
        item = (int)gridDim.x + t_next;
        // Every item draws once, N draws in all: the last (value N - 1) resets the counter for
        // the next launch.
        if (tid == 0 && t_next == N - 1) st_ag(p.ticket, 0u);
    }
}

// Eight waves per workgroup (one workgroup per CU, two waves per SIMD), 2048-key items.  (Four-
// wave workgroups, two per CU with 1024-key items, measured slower: 30.0 against 27.4 us of span
// at the 16K-token layer, 1116 against 983 us at the 380K-token one.)
template <typename T>
static const void *onepass_pick(int *threads, int *slab) {
    *threads = 64 * 8;
    *slab = 16 * 8 * 16;
    return (const void *)&obs_onepass_kernel<T, 8, 16, 2>;
}
const void *onepass_kernel(int dtype, int *threads, int *slab) {
    return dtype == 1 ? onepass_pick<__bf16>(threads, slab) : onepass_pick<float>(threads, slab);
}

}  // namespace snapkv
