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
// patterns order like the values.  Four 8-bit radix passes (LDS histograms, one per wave
// to spread atomic contention) find the k-th largest bit pattern v*; one ordered pass
// then keeps every position above v* and the lowest-position ones equal to v*, writing
// them in ascending order with wave-ballot prefix counts.  No sort is needed.
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
int select_threads() { return kSelThreads; }

__global__ void __launch_bounds__(kSelThreads) topk_select_kernel(const SelectParams p) {
    __shared__ uint32_t hist[kSelWaves][256];
    __shared__ uint32_t sh_digit, sh_above;
    __shared__ uint32_t wcnt[2][kSelWaves];

    const int seg = blockIdx.x;
    const int r = seg / p.Hkv, g = seg - (seg / p.Hkv) * p.Hkv;
    const int P = p.rt.L[r] - p.w;
    const int k = p.rt.k[r];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t *v = (const uint32_t *)(p.pooled + (int64_t)g * p.sum_P + p.rt.pfx0[r]);
    int32_t *out = p.idx + (int64_t)g * p.sum_k + p.rt.k0[r];

    if (k <= 0) return;
    if (k >= P) {
        for (int j = tid; j < P; j += kSelThreads) out[j] = j;
        return;
    }

    uint32_t prefix = 0, mask = 0, need = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0;
        __syncthreads();
        for (int j = tid; j < P; j += kSelThreads) {
            const uint32_t u = v[j];
            if ((u & mask) == prefix) atomicAdd(&hist[wave][(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l owns bins 255-4l .. 252-4l (descending); find the bin holding the need-th largest
            uint32_t cnt[4], tot = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int b = 255 - (4 * lane + q);
                uint32_t s = 0;
                for (int w2 = 0; w2 < kSelWaves; ++w2) s += hist[w2][b];
                cnt[q] = s;
                tot += s;
            }
            uint32_t incl = tot;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t t = __shfl_up(incl, o);
                if (lane >= o) incl += t;
            }
            uint32_t above = incl - tot;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (above < need && need <= above + cnt[q]) {
                    sh_digit = (uint32_t)(255 - (4 * lane + q));
                    sh_above = above;
                }
                above += cnt[q];
            }
        }
        __syncthreads();
        prefix |= sh_digit << shift;
        mask |= 255u << shift;
        need -= sh_above;
        __syncthreads();
    }

    // v* = prefix; every value above it is kept, and the first `need` values equal to it.
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t base_gt = 0, base_eq = 0;
    for (int j0 = 0; j0 < P; j0 += kSelThreads) {
        const int j = j0 + tid;
        const uint32_t u = j < P ? v[j] : 0u;
        const bool gt = j < P && u > prefix;
        const bool eq = j < P && u == prefix;
        const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
        if (lane == 0) {
            wcnt[0][wave] = (uint32_t)__popcll(bgt);
            wcnt[1][wave] = (uint32_t)__popcll(beq);
        }
        __syncthreads();
        uint32_t off_gt = 0, off_eq = 0, tot_gt = 0, tot_eq = 0;
        for (int w2 = 0; w2 < kSelWaves; ++w2) {
            const uint32_t a = wcnt[0][w2], b = wcnt[1][w2];
            if (w2 < wave) { off_gt += a; off_eq += b; }
            tot_gt += a;
            tot_eq += b;
        }
        const uint32_t gt_before = base_gt + off_gt + (uint32_t)__popcll(bgt & lt);
        const uint32_t eq_before = base_eq + off_eq + (uint32_t)__popcll(beq & lt);
        if (gt || (eq && eq_before < need)) out[gt_before + (eq_before < need ? eq_before : need)] = j;
        base_gt += tot_gt;
        base_eq += tot_eq;
        __syncthreads();
    }
}
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
