// obs_stream.hip -- window-query votes as a persistent two-phase stream, gfx950.
//
// What is computed (page "論文解説: SnapKV — アテンションパターン観測によるKVキャッシュ圧縮",
// section 投票メカニズム, and the アルゴリズム listing): for every KV head g of request r, the
// M = G * L_obs window queries of the query heads sharing g score every key the row may see,
// s = q . k / sqrt(d); each row is a softmax over its visible keys; the vote of prefix
// position j is the sum of its weights over all M rows.
//
// How it maps to CDNA4.  This kernel serves problems that do not fit one pass of the resident
// grid with their logits held in registers (long contexts, many requests) and grouped-query
// heads (G * L_obs up to 256 rows):
//   * A persistent grid takes work tickets from one atomic counter.  Every item (one slab of
//     a (request, KV head) segment) is visited twice: a stats pass streams the slab's keys
//     from HBM and leaves each row's (shift, sum of exponentials); the segment's last stats
//     item merges them into one shift per row; a votes pass then streams the slab again and
//     writes the normalised weights summed over the rows.  Tickets are ordered so that every
//     stats item of a segment precedes every votes item of it, with a lag of about half the
//     grid, so the second read of a slab comes from the Infinity Cache while later slabs
//     stream from HBM, and a votes item rarely waits.  An item only ever waits for items with
//     smaller tickets, which running workgroups already hold and finish without waiting: no
//     co-residency of the grid is assumed.
//   * A workgroup of four waves (two per CU, so one's item boundaries overlap the other's
//     stream; eight waves for 256 rows) takes one 16-key tile per wave per step, register
//     staged two steps ahead: each load instruction reads four 256-byte rows, written to LDS
//     in a swizzled MFMA operand order.  Its WR row waves each hold 32 query rows in VGPRs and
//     score the tiles of their key group from LDS, so under GQA every key is read from memory
//     once for all G * L_obs rows.  Logits: v_mfma_f32_16x16x32_bf16 (bf16) or
//     v_mfma_f32_16x16x4_f32 (fp32).
//   * Exponentials are taken as the logits arrive, against a per-wave row shift set by the
//     wave's first tile (so the row sums are at least 1); a slab whose row sum exceeds 2^100
//     is scored again with that row's shift raised (never for ordinary inputs, but large logit
//     ranges stay exact; past 8 raises error bit 2 is set).
// Exponentials are base 2: s*log2(e)/sqrt(d) with the scale folded into one FMA.
#include "obs_score_kernel.h"

namespace snapkv {

namespace {

constexpr float kSumHi = 1.26765060022823e30f;  // 2^100

enum PassMode : int { kP1Exp = 0, kP2 = 2 };
constexpr int kMaxAttempts = 8;  // re-scorings of a slab whose row sums overflow

// Ticket -> (pass, item): tickets [0, lag) are stats items 0..lag-1; then stats and votes
// items alternate; the last tickets are the remaining votes items.  Votes item j comes after
// stats item j + lag - 1 (lag >= items of any segment, so after every stats item of its
// segment).
__device__ inline void ticket_item(int t, int N, int lag, int &pass, int &item) {
    if (t < lag) {
        pass = 1;
        item = t;
        return;
    }
    const int k = t - lag;
    if (k < 2 * (N - lag)) {
        pass = (k & 1) ? 2 : 1;
        item = (k & 1) ? (k >> 1) : lag + (k >> 1);
        return;
    }
    pass = 2;
    item = (N - lag) + (k - 2 * (N - lag));
}

__device__ inline uint32_t ld_agent(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_agent(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// NW waves per workgroup (4: two workgroups per CU; 8: one), WR row waves of RTW 16-row tiles,
// DEPTH steps of keys in flight.
template <typename T, int NW, int WR, int RTW, int DEPTH>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
obs_stream_kernel(const StreamParams p) {
    constexpr int kStreamThreads = 64 * NW;
    constexpr int kStepKeys = 16 * NW;  // one 16-key tile per wave
    constexpr int ESZ = (int)sizeof(T);
    constexpr int ROWB = 256;           // bytes per key / query row
    constexpr int NQ = 4;               // 16-byte operand chunks per lane per row
    constexpr int WK = NW / WR;         // key groups (waves sharing a row block)
    constexpr int MROWS = 16 * RTW * WR;  // query rows per workgroup
    static_assert(ROWB / ESZ * ESZ == ROWB, "row size");

    __shared__ u32x4_t sh_k[DEPTH][NW][256];      // staged steps: one tile per wave
    __shared__ float sh_v[2][NW][WR][16];         // votes of a step's tiles per row wave
    __shared__ float sh_ms[WK][MROWS], sh_ml[WK][MROWS];
    __shared__ int sh_wrow[MROWS];
    __shared__ int sh_ticket;
    __shared__ int sh_flag;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave / WK, wk = wave - (wave / WK) * WK;
    const int n16 = lane & 15, grp = lane >> 4;
    const float c = p.c;
    const bool lse_mode = p.lse != nullptr;
    const int N = p.n_items;
    const int total = lse_mode ? N : 2 * N;
    const int SLAB = p.slab_keys;
    const int64_t tstride = p.token_stride * ESZ;

    for (int r = tid; r < MROWS; r += kStreamThreads) sh_wrow[r] = r % p.w;  // rows of a chunk start at 0
    // With the caller's row stats no item waits for another, so a workgroup's first ticket is its
    // own index (a grid of 512 drawing from one counter at launch spreads the starts over ~6 us)
    // and the counter hands out gridDim.x + n.  With the stats pass, votes items wait for stats
    // items with smaller tickets, and every ticket comes from the counter, so that a drawn ticket
    // is always held by a running workgroup.
    const int t_base = lse_mode ? (int)gridDim.x : 0;
    if (tid == 0 && !lse_mode)
        sh_ticket = (int)__hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int ticket = lse_mode ? (int)blockIdx.x : sh_ticket;

    int cur_seg = -1;
    u32x4_t qf[RTW][NQ];

    while (ticket < total) {
        // The next ticket is drawn when this item's keys are all scored (its round trip overlaps
        // the item's last work).  Drawing it earlier would let the first workgroups take two
        // items each while late-starting ones find none.
        uint32_t next_ticket = 0;
        auto draw_next = [&]() {
            if (tid == 0) next_ticket = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        int pass, item;
        if (lse_mode) {
            pass = 2;
            item = ticket;
        } else {
            ticket_item(ticket, N, p.lag, pass, item);
        }
        // item -> (request, KV head, slab)
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
        const int nsteps = (nkeys + kStepKeys - 1) / kStepKeys;
        uint32_t *const done_ctr = p.seg_ctl + (int64_t)seg * 3 * kStreamSegLine;
        uint32_t *const ready = done_ctr + kStreamSegLine;
        uint32_t *const started = done_ctr + 2 * kStreamSegLine;

        // Window queries of the group's rows wr*32 .. +31 (zero beyond M).
        if (seg != cur_seg) {
            cur_seg = seg;
            const char *qb = (const char *)p.q + (((int64_t)p.rt.qi[r] * p.Hq + (int64_t)g * p.G) * (int64_t)p.w) * ROWB;
            static_for<RTW>([&](auto rt) {
                const int row = (wr * RTW + rt) * 16 + n16;
                static_for<NQ>([&](auto qq) {
                    qf[rt][qq] = row < p.M ? *(const u32x4_t *)(qb + (int64_t)row * ROWB + (4 * qq + grp) * 16)
                                           : u32x4_t{0u, 0u, 0u, 0u};
                });
            });
        }

        // Row shifts of the votes pass: the segment's merged stats (or the caller's lse).  Called
        // once the item's first key loads are in flight, so they overlap the wait.
        float shv[RTW][4];
        const bool skip = pass == 2 && key0 >= P;  // window keys cast no vote
        auto p2_prepare = [&]() {
            if (!lse_mode) {
                // wait until the segment's stats are merged (stats items hold smaller tickets)
                if (tid == 0) {
                    uint32_t spins = 0;
                    while (ld_agent(ready) == 0u) {
                        __builtin_amdgcn_s_sleep(4);
                        if (++spins > p.spin_limit) {
                            __hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            break;
                        }
                    }
                }
                __syncthreads();
            }
            static_for<RTW>([&](auto rt) {
                static_for<4>([&](auto i) {
                    const int row = (wr * RTW + rt) * 16 + 4 * grp + i;
                    float s2 = __builtin_huge_valf();
                    if (row < p.M) {
                        if (lse_mode) {
                            const float lv = p.lse[((int64_t)p.rt.qi[r] * p.Hq + (int64_t)g * p.G) * p.w + row];
                            s2 = lv == neg_inf() ? __builtin_huge_valf() : lv * 1.4426950408889634f;
                        } else {
                            s2 = __uint_as_float(ld_agent((const uint32_t *)&p.final_shift[(int64_t)seg * p.M_pad + row]));
                        }
                    }
                    shv[rt][i] = s2;
                });
            });
            if (!lse_mode) {
                // count this votes item in; the segment's last one resets the flags for the next launch
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                if (tid == 0) {
                    const uint32_t before =
                        __hip_atomic_fetch_add(started, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (before + 1 == (uint32_t)ns) {
                        st_agent(ready, 0u);
                        st_agent(started, 0u);
                    }
                }
            }
        };
        // prefix-only: window keys are visible to no row, so such a stats item is empty
        const bool empty_p1 = pass == 1 && p.variant != 0 && key0 >= P;

        // ---- the step loop over the slab's keys ----
        const char *slab_base = (const char *)p.K + ((int64_t)g * p.head_stride + (p.rt.tok0[r] + key0) * p.token_stride) * ESZ;
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void *)slab_base, (short)0, (int)(nkeys * tstride), kBufferFlags);
        const int lrow = lane >> 4, lch = lane & 15;
        const int lane_off = (wave * 16 + lrow) * (int)tstride + lch * 16;
        float lsum[RTW][4], lsh[RTW][4];
        // mode (compile time): kP1Exp (stats pass; keys stay cached for the votes pass) or kP2
        // (votes pass; last use of the keys, non-temporal)
        auto run_steps = [&](auto mode_c, const bool first_shift, auto &&before_loop) {
            constexpr int mode = decltype(mode_c)::value;
            constexpr int cpol = mode == kP2 ? kNonTemporal : 0;
            static_for<RTW>([&](auto rt) { static_for<4>([&](auto i) { lsum[rt][i] = 0.f; }); });
            // DEPTH steps of keys in flight per wave (registers), each staged in LDS when its turn comes.
            u32x4_t kreg[DEPTH][4];
            auto load_step = [&](auto bc, int s) {
                constexpr int B = decltype(bc)::value;
                static_for<4>([&](auto i) {
                    // whole offset in the VGPR operand (soffset 0): the range check covers it
                    kreg[B][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                 rsrc, lane_off + opaque_s((s * kStepKeys + 4 * i) * (int)tstride),
                                                                 0, cpol));
                });
            };
            static_for<DEPTH>([&](auto j) {
                if (j < nsteps) load_step(j, j);
            });
            before_loop();
            // step s (slot b = s mod DEPTH): stage its keys, start the loads of step s + DEPTH, score
            auto step = [&](auto bc, const int s) {
                constexpr int b = decltype(bc)::value;
                const int vb = s & 1;  // votes buffer of this step
                static_for<4>([&](auto i) {
                    const int row = 4 * i + lrow;
                    sh_k[b][wave][16 * row + (lch ^ row)] = kreg[b][i];
                });
                if (s + DEPTH < nsteps) load_step(bc, s + DEPTH);
                __syncthreads();
                if constexpr (WR > 1) {
                    // votes of the previous step, summed over the row waves
                    if (mode == kP2 && s > 0 && tid < kStepKeys) {
                        const int j = key0 + (s - 1) * kStepKeys + tid;
                        float v = 0.f;
                        static_for<WR>([&](auto w2) { v += sh_v[vb ^ 1][tid >> 4][w2][tid & 15]; });
                        if (j < P) p.votes[(int64_t)g * p.sum_P + p.rt.pfx0[r] + j] = v;
                    }
                }
                // Steps away from the prefix end and past the first take the plain body (no
                // masks, no shift); the others the masked one.
                auto tiles = [&](auto slow_c) {
                    constexpr bool SLOW = decltype(slow_c)::value;
                    static_for<WR>([&](auto ii) {
                        const int ti = wk + WK * ii;
                        const u32x4_t *stile = sh_k[b][ti];
                        u32x4_t kf[NQ];
                        static_for<NQ>([&](auto qq) { kf[qq] = stile[16 * n16 + ((4 * qq + grp) ^ n16)]; });
                        f32x4_t S[RTW];
                        static_for<RTW>([&](auto rt) {
                            S[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                            static_for<NQ>([&](auto qq) { S[rt] = Dot<T>::step(qf[rt][qq], kf[qq], S[rt]); });
                        });
                        const int jt = key0 + s * kStepKeys + ti * 16;  // first key of the tile
                        if constexpr (SLOW) {
                            // mask keys beyond the request, and (causal window) window keys after
                            // the row's position / (prefix only) every window key
                            if (jt + 16 > P) {
                                const int j = jt + n16;
                                static_for<RTW>([&](auto rt) {
                                    static_for<4>([&](auto i) {
                                        const int row = (wr * RTW + rt) * 16 + 4 * grp + i;
                                        const int lim = p.variant == 0 ? P + sh_wrow[row] + 1 : P;
                                        if (j >= lim || j >= L) S[rt][i()] = neg_inf();
                                    });
                                });
                            }
                        }
                        if constexpr (mode == kP1Exp) {
                            if constexpr (SLOW && ii == 0) {
                                if (first_shift && s == 0) {
                                    static_for<RTW>([&](auto rt) {
                                        static_for<4>([&](auto i) {
                                            const float m = row16_max(S[rt][i()]);
                                            lsh[rt][i] = m == neg_inf() ? 0.f : m * c;
                                        });
                                    });
                                }
                            }
                            static_for<RTW>([&](auto rt) {
                                static_for<4>([&](auto i) { lsum[rt][i] += fast_exp2(fmaf(S[rt][i()], c, -lsh[rt][i])); });
                            });
                        } else {
                            float v = 0.f;
                            static_for<RTW>([&](auto rt) {
                                static_for<4>([&](auto i) { v += fast_exp2(fmaf(S[rt][i()], c, -shv[rt][i])); });
                            });
                            v = cross_row_sum4(v);
                            if constexpr (WR == 1) {
                                const int j = jt + n16;
                                if (grp == 0 && (!SLOW || j < P)) p.votes[(int64_t)g * p.sum_P + p.rt.pfx0[r] + j] = v;
                            } else {
                                if (grp == 0) sh_v[vb][ti][wr][n16] = v;
                            }
                        }
                    });
                };
                // The plain body, software pipelined: the LDS reads of a tile are issued one tile
                // ahead, and the exponentials of a tile are interleaved with the MFMAs of the next,
                // so the matrix, vector and LDS pipes work at the same time.
                auto tiles_fast = [&]() {
                    u32x4_t kf[2][NQ];
                    f32x4_t S[2][RTW];
                    auto read_tile = [&](auto slot, int ti) {
                        const u32x4_t *stile = sh_k[b][ti];
                        static_for<NQ>([&](auto qq) { kf[slot][qq] = stile[16 * n16 + ((4 * qq + grp) ^ n16)]; });
                    };
                    read_tile(std::integral_constant<int, 0>{}, wk);
                    static_for<WR + 1>([&](auto ii) {
                        if constexpr (ii < WR) {
                            constexpr int cur = ii % 2;
                            if constexpr (ii + 1 < WR) read_tile(std::integral_constant<int, (ii + 1) % 2>{}, wk + WK * (ii + 1));
                            static_for<RTW>([&](auto rt) {
                                S[cur][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                                static_for<NQ>([&](auto qq) { S[cur][rt] = Dot<T>::step(qf[rt][qq], kf[cur][qq], S[cur][rt]); });
                            });
                        }
                        if constexpr (ii > 0) {
                            constexpr int prev = (ii - 1) % 2;
                            const int ti = wk + WK * (ii - 1);
                            if constexpr (mode == kP1Exp) {
                                static_for<RTW>([&](auto rt) {
                                    static_for<4>([&](auto i) { lsum[rt][i] += fast_exp2(fmaf(S[prev][rt][i()], c, -lsh[rt][i])); });
                                });
                            } else {
                                float v = 0.f;
                                static_for<RTW>([&](auto rt) {
                                    static_for<4>([&](auto i) { v += fast_exp2(fmaf(S[prev][rt][i()], c, -shv[rt][i])); });
                                });
                                v = cross_row_sum4(v);
                                // every row group holds the sum: all four store it (same value, same address)
                                if constexpr (WR == 1) {
                                    p.votes[(int64_t)g * p.sum_P + p.rt.pfx0[r] + key0 + s * kStepKeys + ti * 16 + n16] = v;
                                } else {
                                    sh_v[vb][ti][wr][n16] = v;
                                }
                            }
                        }
                        if constexpr (ii > 0 && ii < WR) {
                            // MFMAs of tile ii, one at a time between the vector work of tile ii - 1
                            static_for<RTW * Dot<T>::kPerChunk * NQ>([&](auto) {
                                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
                            });
                        }
                    });
                };
                if ((mode == kP1Exp && first_shift && s == 0) || key0 + (s + 1) * kStepKeys > P) tiles(std::true_type{});
                else tiles_fast();
            };
            for (int s0 = 0; s0 < nsteps; s0 += DEPTH) {
                static_for<DEPTH>([&](auto j) {
                    if (s0 + j < nsteps) step(j, s0 + j);
                });
            }
            if constexpr (WR > 1) {
                if (mode == kP2) {
                    __syncthreads();
                    if (tid < kStepKeys) {
                        const int b = (nsteps - 1) & 1;  // votes buffer of the last step
                        const int j = key0 + (nsteps - 1) * kStepKeys + tid;
                        float v = 0.f;
                        static_for<WR>([&](auto w2) { v += sh_v[b][tid >> 4][w2][tid & 15]; });
                        if (j < P) p.votes[(int64_t)g * p.sum_P + p.rt.pfx0[r] + j] = v;
                    }
                }
            }
            __syncthreads();  // the step buffers are free for the next item
        };

        if (pass == 2) {
            if (skip) p2_prepare();
            else run_steps(std::integral_constant<int, kP2>{}, false, p2_prepare);
            draw_next();
        } else {
            // stats pass: per-row (shift, sum) of the slab, merged over the key groups
            auto merge_rows = [&]() {
                static_for<RTW>([&](auto rt) {
                    static_for<4>([&](auto i) {
                        const float l = row16_sum(lsum[rt][i]);
                        if (n16 == 0) {
                            const int row = (wr * RTW + rt) * 16 + 4 * grp + i;
                            sh_ms[wk][row] = l > 0.f ? lsh[rt][i] : neg_inf();
                            sh_ml[wk][row] = l;
                        }
                    });
                });
                __syncthreads();
            };
            if (empty_p1) {
                static_for<RTW>([&](auto rt) { static_for<4>([&](auto i) { lsum[rt][i] = 0.f; lsh[rt][i] = 0.f; }); });
                merge_rows();
            } else {
                // A row sum above 2^100 (or not finite) means a later key outgrew the first
                // tile's shift: raise that wave-row's shift by log2 of its sum (by 64 * 2^n when
                // the sum overflowed) and score the slab again.
                for (int attempt = 0;; ++attempt) {
                    run_steps(std::integral_constant<int, kP1Exp>{}, attempt == 0, [] {});
                    float lw[RTW][4];
                    static_for<RTW>([&](auto rt) { static_for<4>([&](auto i) { lw[rt][i] = row16_sum(lsum[rt][i]); }); });
                    bool bad = false;
                    static_for<RTW>([&](auto rt) {
                        static_for<4>([&](auto i) {
                            const int row = (wr * RTW + rt) * 16 + 4 * grp + i;
                            if (row < p.M && !(lw[rt][i] <= kSumHi)) bad = true;
                        });
                    });
                    if (tid == 0) sh_flag = 0;
                    __syncthreads();
                    if (bad) sh_flag = 1;
                    __syncthreads();
                    if (sh_flag == 0 || attempt == kMaxAttempts) {
                        if (sh_flag) __hip_atomic_fetch_or(p.err, 4u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    static_for<RTW>([&](auto rt) {
                        static_for<4>([&](auto i) {
                            const float l = lw[rt][i];
                            if (!(l <= kSumHi))
                                lsh[rt][i] += l < __builtin_huge_valf() ? __builtin_amdgcn_logf(l)
                                                                          : 64.f * (float)(1 << attempt);
                        });
                    });
                }
                merge_rows();
            }
            draw_next();
            // the slab's (shift, sum) per row, merged over the key groups, published
            if (tid < MROWS && tid < p.M) {
                const int row = tid;
                float m = sh_ms[0][row];
                static_for<WK - 1>([&](auto k2) { m = fmaxf(m, sh_ms[k2 + 1][row]); });
                float l = 0.f;
                if (m != neg_inf())
                    static_for<WK>([&](auto k2) {
                        const float mk = sh_ms[k2][row];
                        if (mk != neg_inf()) l = fmaf(sh_ml[k2][row], fast_exp2(mk - m), l);
                    });
                const float2 st = make_float2(m, l);
                __hip_atomic_store((uint64_t *)&p.partial[(int64_t)item * p.M_pad + row], __builtin_bit_cast(uint64_t, st),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0) {
                const uint32_t before = __hip_atomic_fetch_add(done_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                sh_flag = before + 1 == (uint32_t)ns ? 1 : 0;
            }
            __syncthreads();
            if (sh_flag) {
                // the segment's last stats item: merge every slab's row stats (fixed order,
                // so the result does not depend on which item finishes last)
                const int item0 = p.rt.slab0[r] + g * ns;
                constexpr int TPR = kStreamThreads / MROWS;  // threads per row
                const int row = tid / TPR, sub = tid - (tid / TPR) * TPR;
                float mm = neg_inf(), ll = 0.f;
                if (row < p.M) {
                    for (int s0 = sub; s0 < ns; s0 += 8 * TPR) {
                        uint64_t bits[8];
                        static_for<8>([&](auto bb) {
                            const int s2 = s0 + bb() * TPR < ns ? s0 + bb() * TPR : ns - 1;
                            bits[bb()] = __hip_atomic_load((uint64_t *)&p.partial[(int64_t)(item0 + s2) * p.M_pad + row],
                                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        });
                        static_for<8>([&](auto bb) {
                            if (s0 + bb() * TPR < ns) {
                                const float2 pr = __builtin_bit_cast(float2, bits[bb()]);
                                merge_stats(mm, ll, pr.x, pr.y, 1.f);
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
                if (sub == 0 && row < p.M) {
                    const float s2 = ll > 0.f ? mm + __builtin_amdgcn_logf(ll) : __builtin_huge_valf();
                    st_agent((uint32_t *)&p.final_shift[(int64_t)seg * p.M_pad + row], __float_as_uint(s2));
                }
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                if (tid == 0) {
                    st_agent(done_ctr, 0u);
                    st_agent(ready, 1u);
                }
            }
        }
        if (tid == 0) sh_ticket = t_base + (int)next_ticket;
        __syncthreads();
        ticket = sh_ticket;
        __syncthreads();  // everyone has read sh_ticket before it is written again
    }
    // Every workgroup draws exactly one ticket at or past the end; the last of those resets
    // the counter for the next launch (the counter's last value is total + gridDim.x - 1 - t_base).
    if (tid == 0 && ticket == total + (int)gridDim.x - 1) st_agent(p.ticket, 0u);
}

// rows: query rows per KV head the launch covers (32, 64, 128 or 256).  Up to 128 rows, four
// waves of at most 64 rows (two workgroups per CU); 256 rows, eight waves of 32.
template <typename T>
static const void *stream_pick(int rows, int *threads) {
    *threads = rows <= 128 ? 256 : 512;
    switch (rows) {
        case 32: return (const void *)&obs_stream_kernel<T, 4, 1, 2, 3>;
        case 64: return (const void *)&obs_stream_kernel<T, 4, 2, 2, 3>;
        case 128: return (const void *)&obs_stream_kernel<T, 4, 4, 2, 3>;
        default: return (const void *)&obs_stream_kernel<T, 8, 8, 2, 2>;
    }
}
const void *stream_kernel(int dtype, int rows, int *threads) {
    return dtype == 1 ? stream_pick<__bf16>(rows, threads) : stream_pick<float>(rows, threads);
}

}  // namespace snapkv
