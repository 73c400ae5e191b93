// obs_score_kernel.h -- the window-query votes kernel (obs_score) of libsnapkv, gfx950.
// Included by the obs_inst_*.hip files, each of which instantiates one element type and
// head size (so the instantiations compile in parallel).
//
// What is computed (page "論文解説: SnapKV — アテンションパターン観測によるKVキャッシュ圧縮",
// section 投票メカニズム, and the アルゴリズム listing): for every KV head g of request r,
// the M = G * L_obs window queries of the query heads sharing g score every key the row
// may see, s = q . k / sqrt(d); each row is a softmax over its visible keys; the vote of
// prefix position j is the sum of its weights over all M rows.
//
// How it maps to CDNA4:
//   * A work unit ("slab") is one (request, KV head) segment's run of SLAB consecutive
//     keys.  Logits S = Q K^T are a dense contraction of depth d, computed with
//     v_mfma_f32_16x16x32_bf16 (bf16) or v_mfma_f32_16x16x4_f32 (fp32).  A = window
//     queries, B = keys.
//   * Key tiles (16 keys) are spread over the workgroup's waves so that at every step the
//     waves read adjacent tiles: the workgroup sweeps its slab front to back, which keeps
//     DRAM pages open (measured 6.9 TB/s for this order against 5.9 TB/s when each wave
//     streams its own contiguous block).
//   * Rows of 256 bytes (bf16 d=128, fp32 d=64) are register-staged: each load instruction
//     reads four whole key rows (1 KB contiguous, full cache lines), the tile is written
//     to a per-wave LDS tile in a swizzled order and read back in the MFMA operand layout
//     (16 keys x 16 bytes per instruction, bank-conflict free).  Other row sizes load
//     straight into the operand layout, 64 bytes of each of 16 rows per instruction.
//     Either way the d-dimension of each lane's operand is permuted identically for A and
//     B, so every dot product is unchanged.
//   * kFused keeps the slab's logits in registers: per-row max and sum of exponentials
//     over the slab are published, the slabs of a segment meet at a counter barrier
//     (the grid never exceeds what the device keeps resident, a segment never has more
//     slabs than the grid, and with several grid iterations the items are laid out so
//     that no segment crosses one, so every slab of a segment is running), each slab
//     merges the segment's row stats and turns its resident logits into votes.  K is
//     read from HBM once.  Row stats and counters move through device-coherent (sc1)
//     atomic loads and stores, so the barrier needs no L2 write-back or invalidate.
//   * kStats / kVotes are the two-pass path (segments longer than the grid, layouts that
//     would leave many slots idle, or on request): first pass publishes stats,
//     merge_kernel combines them, second pass recomputes the logits and writes votes.
// Exponentials are base 2: s*log2(e)/sqrt(d) with the scale folded into one FMA.
#pragma once
#include <type_traits>

#include "snapkv_internal.h"

namespace snapkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct Dot;

// One 16-byte operand chunk per lane = 8 bf16 = one 16x16x32 MFMA.
template <>
struct Dot<__bf16> {
    static constexpr int kPerChunk = 1;  // MFMA instructions per 16-byte operand chunk
    __device__ static inline f32x4_t step(const u32x4_t &a, const u32x4_t &b, f32x4_t acc) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
    }
};

// One 16-byte operand chunk per lane = 4 fp32 = four 16x16x4 MFMAs.  (Elements are read
// with __uint_as_float(v[i]): a bit cast of a vector element expression reads element 0
// with this compiler.)
template <>
struct Dot<float> {
    static constexpr int kPerChunk = 4;
    __device__ static inline f32x4_t step(const u32x4_t &a, const u32x4_t &b, f32x4_t acc) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc, 0, 0, 0);
        return acc;
    }
};

// Reductions inside a row of 16 lanes (DPP row rotations, no LDS round trip): every lane
// of the row ends with the row's max / sum.
template <int CTRL>
__device__ inline float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ inline float row16_max(float v) {
    v = fmaxf(v, dpp_mov<0x128>(v));  // row_ror:8
    v = fmaxf(v, dpp_mov<0x124>(v));  // row_ror:4
    v = fmaxf(v, dpp_mov<0x122>(v));  // row_ror:2
    v = fmaxf(v, dpp_mov<0x121>(v));  // row_ror:1
    return v;
}
__device__ inline float row16_sum(float v) {
    v += dpp_mov<0x128>(v);
    v += dpp_mov<0x124>(v);
    v += dpp_mov<0x122>(v);
    v += dpp_mov<0x121>(v);
    return v;
}
// Sum of lanes i, i^16, i^32, i^48 (the four row groups of an MFMA output column).
__device__ inline float cross_row_sum4(float v) {
    const unsigned u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);  // lanes i and i^32
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned us = __float_as_uint(s);
    const auto b = __builtin_amdgcn_permlane16_swap(us, us, false, false);  // then i and i^16
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Buffer descriptor word 3 for gfx9 untyped loads (32-bit data format), and the
// non-temporal cache policy bit of the load.
constexpr int kBufferFlags = 0x00020000;
constexpr int kNonTemporal = 2;

struct SlabPos {
    int r, g, sl, ns;
    int seg_slab0;  // first slab of the segment
};

__device__ inline SlabPos decode_slab(const ReqTable &rt, int s, int slab_keys) {
    int r = 0;
    while (r + 1 < rt.n && rt.slab0[r + 1] <= s) ++r;
    SlabPos p;
    p.r = r;
    p.ns = (rt.L[r] + slab_keys - 1) / slab_keys;
    const int local = s - rt.slab0[r];
    p.g = local / p.ns;
    p.sl = local - p.g * p.ns;
    p.seg_slab0 = rt.slab0[r] + p.g * p.ns;
    return p;
}

// Item order of a packed fused launch.  Request i's segments (one per KV head, z = slabs x
// row chunks items each) follow each other from slot vb[i]; a segment that would cross an
// iteration boundary starts at the next boundary instead, so the slots it skips stay idle.
// Every segment then runs within one iteration of the grid, all of its workgroups at once.
// Returns the item (slab * chunks + chunk) of slot u, or -1 for an idle slot.
__device__ inline int packed_item(const ObsParams &p, int u, int C, int slab_keys) {
    const int grid = p.pack_grid;
    if (grid == 0) return u;
    int r = 0;
    while (r + 1 < p.rt.n && p.vb[r + 1] <= u) ++r;
    const int ns = (p.rt.L[r] + slab_keys - 1) / slab_keys, z = ns * C;
    const int base = p.vb[r], o0 = base % grid;
    const int fit0 = (grid - o0) / z;  // segments that fit in the first iteration
    const int h0 = fit0 < p.Hkv ? fit0 : p.Hkv;
    int g, within;
    if (u - base < h0 * z) {
        g = (u - base) / z;
        within = u - base - g * z;
    } else {
        const int next = base - o0 + grid;  // first slot of the next iteration
        if (u < next) return -1;
        const int it = (u - next) / grid, o = (u - next) - it * grid;
        const int gi = o / z;
        if (gi >= grid / z) return -1;
        g = h0 + it * (grid / z) + gi;
        if (g >= p.Hkv) return -1;
        within = o - gi * z;
    }
    return (p.rt.slab0[r] + g * ns) * C + within;
}

__device__ inline float neg_inf() { return -__builtin_huge_valf(); }

// The value x, which the compiler may no longer assume equal to any earlier expression:
// lane indices derived from it after the key stream are recomputed there (a few ALU ops)
// instead of being kept live through the stream, where every VGPR holds logits.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}
// The same for a wave-uniform value (kept in an SGPR): a per-tile load offset formed from it is
// computed where the load is issued, instead of every tile's offset being precomputed and held
// in VGPRs across the whole unrolled slab.
__device__ __forceinline__ int opaque_s(int x) {
    asm volatile("" : "+s"(x));
    return x;
}

// Key loads: non-temporal when every key is read once, cached when the row chunks of a
// slab read it again.
template <bool KEEP>
__device__ inline u32x4_t load_key(const u32x4_t *a) {
    if constexpr (KEEP) return *a;
    else return __builtin_nontemporal_load(a);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// (m, l) pairs: l is a sum of exp2((s - m) * c).  Merge two of them.
__device__ inline void merge_stats(float &m, float &l, float m2, float l2, float c) {
    const float mx = fmaxf(m, m2);
    if (mx == neg_inf()) return;  // both empty
    const float a = (m == neg_inf()) ? 0.f : l * fast_exp2((m - mx) * c);
    const float b = (m2 == neg_inf()) ? 0.f : l2 * fast_exp2((m2 - mx) * c);
    m = mx;
    l = a + b;
}

// STAGED (rows of 256 bytes): tile slot p of a wave's LDS tile holds row p/16, chunk
// (p%16) ^ (p/16).  A load instruction's lane l carries row 4i + l/16, chunk l%16 (four
// whole rows); the MFMA read of (row n, chunk c) by the 16 lanes of a lane group hits
// slots 16n + (c ^ n): 16 distinct bank groups.
template <typename T, int D, int WR, int WK, int RTW, int CTW, int MODE, bool STAGED = false, bool KEEP = false>
__global__ void __launch_bounds__(64 * WR * WK) obs_score_kernel(const ObsParams p) {
    constexpr int NT = 64 * WR * WK;
    constexpr int ESZ = (int)sizeof(T);
    constexpr int ROWB = D * ESZ;       // bytes per key / query row
    constexpr int NQ = ROWB / 64;       // 16-byte loads per lane per row
    constexpr int SLAB = WK * CTW * 16; // keys per slab
    constexpr int MROWS = WR * RTW * 16;
    constexpr int PF = 2;               // key tiles in flight per wave
    constexpr int NCH = ROWB / 16;      // 16-byte chunks per row
    constexpr bool QLDS = WR == 1 && !STAGED;  // window queries read from LDS (else VGPRs)
    static_assert(ROWB % 64 == 0, "row must be a multiple of 64 bytes");
    static_assert(WR == 1, "one row wave: each wave holds every row of the chunk");
    static_assert(!STAGED || (ROWB == 256 && NQ == 4), "staged tiles are 16 rows of 256 bytes");
    // LDS rows padded by one chunk so the 16 rows of an MFMA operand hit distinct banks
    __shared__ u32x4_t sh_q[QLDS ? MROWS : 1][NCH + 1];
    __shared__ u32x4_t sh_k[STAGED ? WR * WK : 1][256];  // per-wave staging tile

    __shared__ float sh_m[WK][MROWS];
    __shared__ float sh_l[WK][MROWS];
    __shared__ float sh_rowm[MROWS];
    __shared__ float sh_f[MODE == kFused ? WK : 1][MROWS];  // votes factor per (wave, row)
    __shared__ int sh_wrow[kMaxRows];  // window row (row % L_obs) of each query row, for the causal mask

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave / WK, wk = wave - (wave / WK) * WK;
    const int n16 = lane & 15, grp = lane >> 4;
    const float c = p.c;
    for (int r = tid; r < kMaxRows; r += NT) sh_wrow[r] = r % p.w;
    __syncthreads();

    // Work items are (slab, row chunk) pairs, chunk fastest.  With several chunks and a grid
    // that is a multiple of 8, consecutive items go to workgroups b, b+8, b+16, ... which the
    // dispatcher places on one XCD, so the chunks of a slab read it from that XCD's L2.
    const int C = p.n_chunks;
    const int nb = gridDim.x;
    const int b0 = (C == 1 || (nb & 7)) ? (int)blockIdx.x : ((int)blockIdx.x & 7) * (nb >> 3) + ((int)blockIdx.x >> 3);
    const int n_slots = p.pack_grid ? p.vb[p.rt.n] : p.n_slabs * C;
    for (int u = b0; u < n_slots; u += nb) {
        const int v = packed_item(p, u, C, SLAB);
        if (v < 0) continue;
        const int s = v / C, chunk = v - (v / C) * C;
        const SlabPos sp = decode_slab(p.rt, s, SLAB);
        const int cbase = chunk * MROWS;                          // first query row of the chunk
        const int Mc = p.M - cbase < MROWS ? p.M - cbase : MROWS;  // rows in this chunk
        const int L = p.rt.L[sp.r];
        const int P = L - p.w;
        const int key0 = sp.sl * SLAB;
        // tile ct of this wave holds keys key0 + (ct*WK + wk)*16 .. +15: at each step the
        // workgroup's waves read adjacent tiles
        auto tile_key = [&](int ct) { return key0 + (ct * WK + wk) * 16; };
        const int seg = (sp.r * p.Hkv + sp.g) * C + chunk;  // (segment, chunk) for stats and counters

        // Window queries of the group: rows r*G*L_obs .. of q_obs, zero beyond M.  With one
        // row wave and direct key loads (QLDS) they sit in LDS and are re-read per key tile,
        // which frees the VGPRs the resident logits need; otherwise each wave keeps its
        // rows in VGPRs.
        const char *qb = (const char *)p.q +
                         (((int64_t)p.rt.qi[sp.r] * p.Hq + (int64_t)sp.g * p.G) * (int64_t)p.w + cbase) * ROWB;
        u32x4_t qf[QLDS ? 1 : RTW][NQ];
        if constexpr (QLDS) {
            for (int e = tid; e < MROWS * NCH; e += NT) {
                const int row = e / NCH, ch = e - (e / NCH) * NCH;
                sh_q[row][ch] = row < Mc ? *(const u32x4_t *)(qb + (int64_t)row * ROWB + ch * 16)
                                          : u32x4_t{0u, 0u, 0u, 0u};
            }
            __syncthreads();
        } else {
            static_for<RTW>([&](auto rt) {
                const int row = (wr * RTW + rt) * 16 + n16;
                static_for<NQ>([&](auto qq) {
                    qf[rt][qq] = row < Mc ? *(const u32x4_t *)(qb + (int64_t)row * ROWB + (4 * qq + grp) * 16)
                                           : u32x4_t{0u, 0u, 0u, 0u};
                });
            });
        }

        // Logits of this wave's CTW key tiles.
        f32x4_t S[RTW][CTW];
        static_for<RTW>([&](auto rt) { static_for<CTW>([&](auto ct) { S[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f}; }); });
        if constexpr (STAGED) {
            // Buffer loads from a descriptor based at the slab's first key and sized to the
            // slab's keys inside the request: the lane offset is fixed for the whole slab, the
            // tile offset is a scalar, and rows past the request end read as zero (masked below).
            const int64_t tstride = p.token_stride * ESZ;
            const char *slab0 = (const char *)p.K +
                                ((int64_t)sp.g * p.head_stride + (p.rt.tok0[sp.r] + key0) * p.token_stride) * ESZ;
            const int nkeys = L - key0 < SLAB ? L - key0 : SLAB;
            const __amdgpu_buffer_rsrc_t rsrc =
                __builtin_amdgcn_make_buffer_rsrc((void *)slab0, (short)0, (int)(nkeys * tstride), kBufferFlags);
            const int lrow = lane >> 4, lch = lane & 15;  // load layout: row 4i + lrow, chunk lch
            const int lane_off = (wk * 16 + lrow) * (int)tstride + lch * 16;
            u32x4_t *stile = sh_k[wave];
            u32x4_t buf[PF][4];
            auto load_tile = [&](auto slot, int ct) {
                static_for<4>([&](auto i) {
                    // the whole offset in the VGPR operand (soffset 0), which the buffer range
                    // check covers: tiles past the slab's keys read zeros
                    const int soff = opaque_s((ct * WK * 16 + 4 * i) * (int)tstride);  // wave-uniform
                    buf[slot][i] = __builtin_bit_cast(
                        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_off + soff, 0, KEEP ? 0 : kNonTemporal));
                });
            };
            static_for<(PF < CTW ? PF : CTW)>([&](auto f) { load_tile(f, f); });
            static_for<CTW>([&](auto ct) {
                // transpose through LDS: write the tile's four rows-per-instruction layout ...
                static_for<4>([&](auto i) {
                    const int row = 4 * i + lrow;
                    stile[16 * row + (lch ^ row)] = buf[ct % PF][i];
                });
                if constexpr (ct + PF < CTW) load_tile(std::integral_constant<int, ct % PF>{}, ct + PF);
                // ... and read it back as 16 keys x 16 bytes per lane group
                u32x4_t kf[4];
                static_for<4>([&](auto qq) { kf[qq] = stile[16 * n16 + ((4 * qq + grp) ^ n16)]; });
                static_for<RTW>([&](auto rt) {
                    static_for<NQ>([&](auto qq) {
                        if constexpr (QLDS)
                            S[rt][ct] = Dot<T>::step(sh_q[rt * 16 + n16][4 * qq + grp], kf[qq], S[rt][ct]);
                        else
                            S[rt][ct] = Dot<T>::step(qf[rt][qq], kf[qq], S[rt][ct]);
                    });
                });
            });
        } else {
            const char *kb = (const char *)p.K +
                             ((int64_t)sp.g * p.head_stride + p.rt.tok0[sp.r] * p.token_stride) * ESZ + grp * 16;
            const int64_t tstride = p.token_stride * ESZ;
            // No branches in this loop: a tile past the request end loads its last row again
            // (in bounds) and is masked below; a branch here would make the compiler drain
            // every outstanding load before the next tile's loads issue.
            u32x4_t buf[PF][NQ];
            static_for<(PF < CTW ? PF : CTW)>([&](auto f) {
                int j = tile_key(f) + n16;
                j = j < L ? j : L - 1;
                const char *a = kb + (int64_t)j * tstride;
                static_for<NQ>([&](auto qq) { buf[f][qq] = load_key<KEEP>((const u32x4_t *)(a + qq * 64)); });
            });
            static_for<CTW>([&](auto ct) {
                u32x4_t cur[NQ];
                static_for<NQ>([&](auto qq) { cur[qq] = buf[ct % PF][qq]; });
                if constexpr (ct + PF < CTW) {
                    int j = tile_key(ct + PF) + n16;
                    j = j < L ? j : L - 1;
                    const char *a = kb + (int64_t)j * tstride;
                    static_for<NQ>([&](auto qq) {
                        buf[ct % PF][qq] = load_key<KEEP>((const u32x4_t *)(a + qq * 64));
                    });
                }
                if constexpr (QLDS) {
                    // keep the compiler from merging the per-tile LDS reads into registers
                    asm volatile("" ::: "memory");
                    static_for<RTW>([&](auto rt) {
                        static_for<NQ>([&](auto qq) {
                            S[rt][ct] = Dot<T>::step(sh_q[rt * 16 + n16][4 * qq + grp], cur[qq], S[rt][ct]);
                        });
                    });
                } else {
                    static_for<RTW>([&](auto rt) {
                        static_for<NQ>([&](auto qq) { S[rt][ct] = Dot<T>::step(qf[rt][qq], cur[qq], S[rt][ct]); });
                    });
                }
            });
        }

        // Mask keys a row may not see: beyond the request, or (causal window) window keys
        // after the row's own position, or (prefix-only variant) every window key.
        if (key0 + SLAB > P) {
            static_for<RTW>([&](auto rt) {
                static_for<4>([&](auto i) {
                    const int row = (wr * RTW + rt) * 16 + 4 * grp + i;
                    const int lim = p.variant == 0 ? P + sh_wrow[cbase + row] + 1 : P;  // keys j < lim are visible
                    static_for<CTW>([&](auto ct) {
                        const int j = tile_key(ct) + n16;
                        if (j >= lim) S[rt][ct][i()] = neg_inf();
                    });
                });
            });
        }

        if constexpr (MODE == kFused || MODE == kStats) {
            // Each wave: row max over its own tiles, exponentials against that max, row sums.
            // No wave waits for the others before its exponentials, so the faster waves do
            // theirs while the slowest is still streaming; the waves' (max, sum) pairs meet in
            // LDS once, and the votes later scale each wave's weights by its own factor.
            float mrow[RTW][4], lrow[RTW][4];
            static_for<RTW>([&](auto rt) {
                static_for<4>([&](auto i) {
                    float m = S[rt][0][i()];
                    static_for<CTW - 1>([&](auto ct) { m = fmaxf(m, S[rt][ct + 1][i()]); });
                    mrow[rt][i] = row16_max(m);
                    const float sh = mrow[rt][i] == neg_inf() ? 0.f : mrow[rt][i] * c;
                    float l = 0.f;
                    static_for<CTW>([&](auto ct) {
                        const float e = fast_exp2(fmaf(S[rt][ct][i()], c, -sh));
                        S[rt][ct][i()] = e;
                        l += e;
                    });
                    lrow[rt][i] = row16_sum(l);
                });
            });
            if (n16 == 0)
                static_for<RTW>([&](auto rt) {
                    static_for<4>([&](auto i) {
                        const int row = (wr * RTW + rt) * 16 + 4 * grp + i;
                        sh_m[wk][row] = mrow[rt][i];
                        sh_l[wk][row] = lrow[rt][i];
                    });
                });
            __syncthreads();
            // The slab's (max, sum) per row, merged over the waves by one thread per row and
            // published with a device-coherent store (bypasses the per-XCD L2: the barrier
            // below needs no cache write-back).
            if (tid < MROWS) {
                const int row = tid;
                float m = sh_m[0][row];
                static_for<WK - 1>([&](auto k2) { m = fmaxf(m, sh_m[k2 + 1][row]); });
                float l = 0.f;
                if (m != neg_inf())
                    static_for<WK>([&](auto k2) {
                        const float mk = sh_m[k2][row];
                        if (mk != neg_inf()) l = fmaf(sh_l[k2][row], fast_exp2((mk - m) * c), l);
                    });
                if (row < Mc) {
                    const float2 st = make_float2(m, l);
                    __hip_atomic_store((uint64_t *)&p.partial[(int64_t)v * p.M_pad + row],
                                       __builtin_bit_cast(uint64_t, st), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        if constexpr (MODE == kStats) {
            __syncthreads();
            continue;
        }

        if constexpr (MODE == kFused) {
            // All slabs of the segment publish, then meet.  Every slab publishes before it
            // waits, and a segment never has more slabs than resident workgroups (and lies in
            // one grid iteration), so the wait ends; a poll limit turns a device that did not
            // keep the grid resident (another process filling the CUs) into an error bit
            // instead of a hang.  Each wave's device-coherent stores complete (vmcnt 0) before
            // the workgroup barrier, so the arrival below is ordered after every published
            // row stat.  The (segment, chunk) arrival count is zero when a launch starts; the
            // last arrival sets it back to zero at once, which also releases the others: a
            // workgroup that arrived with `before` earlier arrivals sees the count in
            // (before, ns] until then, and at or below `before` after.  So the next launch
            // finds it at zero without a clearing pass.  An arrival that finds the count
            // already at the segment's size means the workspace was not zero-filled (error
            // bit 1).
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0) {
                uint32_t *const arrived = &p.counters[seg * kCounterStride];
                const uint32_t ns = (uint32_t)sp.ns;
                const uint32_t before = __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (before >= ns) __hip_atomic_fetch_or(p.err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (before + 1 == ns) {
                    __hip_atomic_store(arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    uint32_t spins = 0;
                    for (;;) {
                        const uint32_t now = __hip_atomic_load(arrived, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (now == ns || now <= before) break;
                        __builtin_amdgcn_s_sleep(8);
                        if (++spins > p.spin_limit) {
                            __hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            break;
                        }
                    }
                }
            }
            __syncthreads();
            asm volatile("" ::: "memory");
            // Merge the segment's row stats; factor for this slab's resident weights.
            constexpr int TPR = NT / MROWS;  // threads per row (power of two)
            const int tid_m = opaque(tid);
            const int row = tid_m / TPR, sub = tid_m - (tid_m / TPR) * TPR;
            // A thread's slabs are read kMergeBatch at a time, all loads in flight together (an
            // index past the segment re-reads its last slab and is then ignored): long segments
            // cost a few round trips, not one per slab.
            constexpr int kMergeBatch = 8;
            float mm = neg_inf(), ll = 0.f;
            if (row < Mc) {
                for (int s0 = sub; s0 < sp.ns; s0 += kMergeBatch * TPR) {
                    uint64_t bits[kMergeBatch];
                    static_for<kMergeBatch>([&](auto b) {
                        const int s2 = s0 + b() * TPR < sp.ns ? s0 + b() * TPR : sp.ns - 1;
                        bits[b()] = __hip_atomic_load(
                            (uint64_t *)&p.partial[((int64_t)(sp.seg_slab0 + s2) * C + chunk) * p.M_pad + row],
                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    });
                    static_for<kMergeBatch>([&](auto b) {
                        if (s0 + b() * TPR < sp.ns) {
                            const float2 pr = __builtin_bit_cast(float2, bits[b()]);
                            merge_stats(mm, ll, pr.x, pr.y, c);
                        }
                    });
                }
            }
#pragma unroll
            for (int o = 1; o < TPR; o <<= 1) {
                const float m2 = __shfl_xor(mm, o, TPR);
                const float l2 = __shfl_xor(ll, o, TPR);
                merge_stats(mm, ll, m2, l2, c);
            }
            if (sub == 0) {
                // each wave's weights are relative to its own row max
                const float inv = (row < Mc && ll > 0.f) ? 1.f / ll : 0.f;
                static_for<WK>([&](auto k2) {
                    const float mk = sh_m[k2][row];
                    sh_f[k2][row] = (inv > 0.f && mk != neg_inf()) ? fast_exp2((mk - mm) * c) * inv : 0.f;
                });
            }
            __syncthreads();
        }

        if constexpr (MODE == kVotes) {
            if (tid < MROWS) {
                const int row = tid;
                if (p.lse) {
                    // caller's log-sum-exp: weight = exp(s / sqrt(d) - lse) = exp2(s * c - lse * log2(e)),
                    // i.e. row max lse * sqrt(d) and row sum 1
                    float lv = neg_inf();
                    if (row < Mc)
                        lv = p.lse[((int64_t)p.rt.qi[sp.r] * p.Hq + (int64_t)sp.g * p.G) * p.w + cbase + row];
                    const bool ok = lv != neg_inf();
                    sh_rowm[row] = ok ? lv * p.lse_scale : 0.f;
                    sh_f[0][row] = ok ? 1.f : 0.f;
                } else {
                    float2 mg = make_float2(0.f, 0.f);
                    if (row < Mc) mg = p.merged[(int64_t)seg * p.M_pad + row];
                    const bool ok = row < Mc && mg.x != neg_inf() && mg.y > 0.f;
                    sh_rowm[row] = ok ? mg.x : 0.f;
                    sh_f[0][row] = ok ? 1.f / mg.y : 0.f;
                }
            }
            __syncthreads();
            static_for<RTW>([&](auto rt) {
                static_for<4>([&](auto i) {
                    const float sh = sh_rowm[(wr * RTW + rt) * 16 + 4 * grp + i] * c;
                    static_for<CTW>([&](auto ct) { S[rt][ct][i()] = fast_exp2(fmaf(S[rt][ct][i()], c, -sh)); });
                });
            });
        }

        // Votes: weight * row factor, summed over this wave's rows, the four row groups of
        // the MFMA layout, then the row waves.
        {
            const int tid_v = opaque(tid);
            const int lane_v = tid_v & 63, wk_v = (tid_v >> 6) % WK;
            const int grp_v = lane_v >> 4;
            const int jl = key0 + wk_v * 16 + (lane_v & 15);  // tile_key(ct) + n16 = jl + ct * WK * 16
            float f[RTW][4];
            static_for<RTW>([&](auto rt) {
                static_for<4>([&](auto i) { f[rt][i] = sh_f[MODE == kFused ? wk_v : 0][(wr * RTW + rt) * 16 + 4 * grp_v + i]; });
            });
            float *vout = p.votes + chunk * p.vplane + (int64_t)sp.g * p.sum_P + p.rt.pfx0[sp.r];
            static_for<CTW>([&](auto ct) {
                float v = 0.f;
                static_for<RTW>([&](auto rt) {
                    static_for<4>([&](auto i) { v = fmaf(S[rt][ct][i()], f[rt][i], v); });
                });
                v = cross_row_sum4(v);
                // this wave holds every row: its 16 lanes of group 0 store the tile's votes
                const int j = jl + ct() * WK * 16;
                if (grp_v == 0 && j < P) vout[j] = v;
            });
            __syncthreads();
        }
    }
}

template <typename T, int D, int CTW, bool STAGED, bool KEEP>
inline const void *pick_mode(int mode) {
    switch (mode) {
        case kFused: return (const void *)&obs_score_kernel<T, D, 1, 8, 2, CTW, kFused, STAGED, KEEP>;
        case kStats: return (const void *)&obs_score_kernel<T, D, 1, 8, 2, CTW, kStats, STAGED, KEEP>;
        default: return (const void *)&obs_score_kernel<T, D, 1, 8, 2, CTW, kVotes, STAGED, KEEP>;
    }
}

template <typename T, int D, bool KEEP>
inline const void *pick_keep(int mode, int ctw) {
    if constexpr (D * sizeof(T) == 256)
        return ctw == 12 ? pick_mode<T, D, 12, true, KEEP>(mode) : pick_mode<T, D, 16, true, KEEP>(mode);
    else if constexpr (D * sizeof(T) < 256) return pick_mode<T, D, 16, false, KEEP>(mode);
    else return pick_mode<T, D, 8, false, KEEP>(mode);
}

template <typename T, int D>
inline const void *pick(int mode, bool keep, int ctw) {
    return keep ? pick_keep<T, D, true>(mode, ctw) : pick_keep<T, D, false>(mode, ctw);
}


// One entry per (element type, head size), each in its own translation unit.
const void *obs_kernel_bf16_d128(int mode, bool keep, int ctw);
const void *obs_kernel_bf16_d64(int mode, bool keep, int ctw);
const void *obs_kernel_f32_d128(int mode, bool keep, int ctw);
const void *obs_kernel_f32_d64(int mode, bool keep, int ctw);

}  // namespace snapkv
