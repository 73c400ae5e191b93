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

// ---- fill ----------------------------------------------------------------------------------

__global__ void __launch_bounds__(256) fill_u32_kernel(const FillParams p) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < p.n; i += (int64_t)gridDim.x * blockDim.x)
        p.p[i] = p.v;
}
const void *fill_kernel() { return (const void *)&fill_u32_kernel; }

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
// One workgroup per (request, KV head).  Pooled votes are >= 0, so their fp32 bit
// patterns order like the values.  Four 8-bit radix passes (per-wave LDS histograms)
// find the k-th largest bit pattern v*; one ordered pass then keeps every position
// above v* and the lowest-position ones equal to v*, writing them in ascending order
// with wave-ballot prefix counts.  No sort is needed.  A segment of up to kSelLds
// positions is first copied into LDS and every pass reads it there; longer segments
// are read from global memory (L2 / Infinity Cache) on each pass.  In the first pass
// most votes share one or two exponent bins, so lanes with equal digits are counted
// with one ballot and one atomic per distinct digit.
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelLds = 32768;
int select_threads() { return kSelThreads; }

// Four consecutive positions j..j+3 of a segment (LDS: one 16-byte read; global: four
// loads).  Positions >= P come back as 0 and are masked by the callers.
template <bool IN_LDS>
__device__ inline void load4(const uint32_t *src, int j, int P, uint32_t u[4]) {
    if (IN_LDS) {
        const u32x4_t t = *(const u32x4_t *)(src + j);
        u[0] = t.x; u[1] = t.y; u[2] = t.z; u[3] = t.w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = j + e < P ? src[j + e] : 0u;
    }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ inline uint32_t wave_incl_scan(uint32_t x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(x, o);
        if (lane >= o) x += t;
    }
    return x;
}

template <bool IN_LDS>
__device__ void radix_select(const uint32_t *__restrict__ src, int P, int k, int32_t *__restrict__ out,
                             uint32_t (*hist)[256], uint32_t *tot, uint32_t *sh_digit, uint32_t *sh_above,
                             uint32_t *wtot) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t prefix = 0, mask = 0, need = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0;
        __syncthreads();
        for (int j0 = 0; j0 < P; j0 += 4 * kSelThreads) {
            const int j = j0 + 4 * tid;
            uint32_t u[4];
            load4<IN_LDS>(src, j, P, u);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool in = j + e < P && (u[e] & mask) == prefix;
                const uint32_t dg = (u[e] >> shift) & 255u;
                if (shift == 24) {
                    uint64_t act = __ballot(in);
                    while (act) {  // one atomic per distinct digit in the wave
                        const int leader = __ffsll((unsigned long long)act) - 1;
                        const uint32_t dl = __shfl(dg, leader);
                        const uint64_t same = __ballot(in && dg == dl);
                        if (lane == leader) atomicAdd(&hist[wave][dl], (uint32_t)__popcll(same));
                        act &= ~same;
                    }
                } else if (in) {
                    atomicAdd(&hist[wave][dg], 1u);
                }
            }
        }
        __syncthreads();
        if (tid < 256) {
            uint32_t sum = 0;
#pragma unroll
            for (int w2 = 0; w2 < kSelWaves; ++w2) sum += hist[w2][tid];
            tot[tid] = sum;
        }
        __syncthreads();
        if (wave == 0) {
            // lane l owns bins 255-4l .. 252-4l (descending); find the bin holding the need-th largest
            uint32_t cnt[4], t4 = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                cnt[q] = tot[255 - (4 * lane + q)];
                t4 += cnt[q];
            }
            uint32_t above = wave_incl_scan(t4) - t4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (above < need && need <= above + cnt[q]) {
                    *sh_digit = (uint32_t)(255 - (4 * lane + q));
                    *sh_above = above;
                }
                above += cnt[q];
            }
        }
        __syncthreads();
        prefix |= *sh_digit << shift;
        mask |= 255u << shift;
        need -= *sh_above;
        __syncthreads();
    }

    // v* = prefix; every value above it is kept, and the first `need` values equal to it.
    // Counts of (above, equal) are packed in one word (low/high 16 bits; a chunk holds
    // 4096 positions, so neither half overflows) and prefix-summed across the workgroup.
    uint32_t base_gt = 0, base_eq = 0;
    for (int j0 = 0; j0 < P; j0 += 4 * kSelThreads) {
        const int j = j0 + 4 * tid;
        uint32_t u[4];
        load4<IN_LDS>(src, j, P, u);
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool valid = j + e < P;
            packed += (valid && u[e] > prefix) ? 1u : 0u;
            packed += (valid && u[e] == prefix) ? 0x10000u : 0u;
        }
        const uint32_t incl = wave_incl_scan(packed);
        if (lane == 63) wtot[wave] = incl;
        __syncthreads();
        uint32_t woff = 0, ctot = 0;
#pragma unroll
        for (int w2 = 0; w2 < kSelWaves; ++w2) {
            const uint32_t t = wtot[w2];
            woff += w2 < wave ? t : 0u;
            ctot += t;
        }
        const uint32_t excl = woff + incl - packed;
        uint32_t gt_before = base_gt + (excl & 0xffffu), eq_before = base_eq + (excl >> 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool valid = j + e < P;
            if (valid && u[e] > prefix) {
                out[gt_before + (eq_before < need ? eq_before : need)] = j + e;
                ++gt_before;
            } else if (valid && u[e] == prefix) {
                if (eq_before < need) out[gt_before + eq_before] = j + e;
                ++eq_before;
            }
        }
        base_gt += ctot & 0xffffu;
        base_eq += ctot >> 16;
        __syncthreads();
        if (base_gt + (base_eq < need ? base_eq : need) >= (uint32_t)k) break;  // all k written
    }
}

// Pooling of a segment held in LDS (votes -> pooled, in place): each thread keeps the
// pooled values of its strided positions in registers until every read is done.
__device__ void pool_in_lds(uint32_t *sdata, int P, int half) {
    const int tid = threadIdx.x;
    float pm[kSelLds / kSelThreads];
#pragma unroll
    for (int u = 0; u < kSelLds / kSelThreads; ++u) {
        const int j = u * kSelThreads + tid;
        float m = 0.f;
        if (j < P) {
            const int lo = j - half < 0 ? 0 : j - half;
            const int hi = j + half > P - 1 ? P - 1 : j + half;
            m = __uint_as_float(sdata[lo]);
            for (int t = lo + 1; t <= hi; ++t) {
                const float v = __uint_as_float(sdata[t]);
                m = v > m ? v : m;
            }
        }
        pm[u] = m;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSelLds / kSelThreads; ++u) {
        const int j = u * kSelThreads + tid;
        if (j < P) sdata[j] = __float_as_uint(pm[u]);
    }
    __syncthreads();
}

__global__ void __launch_bounds__(kSelThreads) topk_select_kernel(const SelectParams p) {
    __shared__ __attribute__((aligned(16))) uint32_t sdata[kSelLds];
    __shared__ uint32_t hist[kSelWaves][256];
    __shared__ uint32_t tot[256];
    __shared__ uint32_t sh_digit, sh_above;
    __shared__ uint32_t wtot[kSelWaves];

    const int seg = blockIdx.x;
    const int r = seg / p.Hkv, g = seg - (seg / p.Hkv) * p.Hkv;
    const int P = p.rt.L[r] - p.w;
    const int k = p.rt.k[r];
    const int tid = threadIdx.x;
    const int64_t base = (int64_t)g * p.sum_P + p.rt.pfx0[r];
    int32_t *out = p.idx ? p.idx + (int64_t)g * p.sum_k + p.rt.k0[r] : nullptr;

    if (P <= kSelLds) {
        // segment -> LDS, eight loads in flight per thread
        const uint32_t *src = (const uint32_t *)((p.votes ? p.votes : p.pooled) + base);
        for (int j0 = 0; j0 < P; j0 += 8 * kSelThreads) {
            uint32_t tmp[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u * kSelThreads + tid;
                tmp[u] = j < P ? src[j] : 0u;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u * kSelThreads + tid;
                if (j < P) sdata[j] = tmp[u];
            }
        }
        __syncthreads();
        if (p.votes) {
            pool_in_lds(sdata, P, p.half);
            if (p.pooled_out) {
                uint32_t *dst = (uint32_t *)(p.pooled_out + base);
                for (int j = tid; j < P; j += kSelThreads) dst[j] = sdata[j];
            }
        }
        if (!out || k <= 0) return;
        if (k >= P) {
            for (int j = tid; j < P; j += kSelThreads) out[j] = j;
            return;
        }
        radix_select<true>(sdata, P, k, out, hist, tot, &sh_digit, &sh_above, wtot);
    } else {
        // long segment: pooled votes come from the pooling kernel, every pass reads them globally
        if (!out || k <= 0) return;
        if (k >= P) {
            for (int j = tid; j < P; j += kSelThreads) out[j] = j;
            return;
        }
        radix_select<false>((const uint32_t *)(p.pooled + base), P, k, out, hist, tot, &sh_digit, &sh_above, wtot);
    }
}
int select_lds_positions() { return kSelLds; }
const void *select_kernel() { return (const void *)&topk_select_kernel; }

// ---- gather -----------------------------------------------------------------------------------
// grid: (row blocks, KV heads).  Each output row is row_bytes / 16 lanes of 16-byte copies.
// Out-of-range indices are clamped into the prefix so a bad index can never read outside K/V.
__global__ void __launch_bounds__(256) kv_gather_kernel(const GatherParams p) {
    const int g = blockIdx.y;
    const int lpr = p.row_bytes >> 4;           // lanes per row
    const int rpb = 256 / lpr;                  // rows per block step
    const int chunk = threadIdx.x % lpr;
    const int64_t o_begin = p.rt.out0[0];
    const int last = p.rt.n - 1;
    const int64_t o_end = p.rt.out0[last] + p.rt.k[last] + p.w;
    for (int64_t o = o_begin + (int64_t)blockIdx.x * rpb + threadIdx.x / lpr; o < o_end; o += (int64_t)gridDim.x * rpb) {
        int r = 0;
        while (r + 1 < p.rt.n && p.rt.out0[r + 1] <= o) ++r;
        const int t = (int)(o - p.rt.out0[r]);
        const int kr = p.rt.k[r];
        const int P = p.rt.L[r] - p.w;
        int pos;
        if (t < kr) {
            pos = p.idx[(int64_t)g * p.sum_k + p.rt.k0[r] + t];
            pos = pos < 0 ? 0 : (pos > P - 1 ? P - 1 : pos);
        } else {
            pos = P + (t - kr);
        }
        const int64_t src = ((int64_t)g * p.head_stride + (p.rt.tok0[r] + pos) * p.token_stride) * p.esz + chunk * 16;
        const int64_t dst = ((int64_t)g * p.sum_out + o) * p.row_bytes + chunk * 16;
        const u32x4_t a = *(const u32x4_t *)((const char *)p.K + src);
        const u32x4_t b = *(const u32x4_t *)((const char *)p.V + src);
        *(u32x4_t *)((char *)p.K_out + dst) = a;
        *(u32x4_t *)((char *)p.V_out + dst) = b;
    }
}
const void *gather_kernel() { return (const void *)&kv_gather_kernel; }

}  // namespace snapkv
