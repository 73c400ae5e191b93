// decode.hip -- decode attention over the compressed cache, gfx950.
//
// The step after the compression (page "論文解説: SnapKV — アテンションパターン観測によるKVキャッシュ圧縮",
// section デコード速度とメモリ効率; the KV-cache chapter's decode step): one new query row per
// (request, query head) attends to every cached row of its KV head,
//   out = sum_j softmax_j(q . k_j / sqrt(d)) v_j.
// Split-K: a workgroup takes split_rows cached rows of one (request, KV head, group of up to
// 8 query heads) and leaves a partial (max, sum, weighted values); a second kernel merges
// the splits.  Rows are 256 bytes (bf16 d=128, fp32 d=64): 16 lanes hold one row as 16-byte
// chunks, four rows per wave instruction, and the dot products reduce over the 16 lanes
// with DPP row rotations.
#include "snapkv_internal.h"

namespace snapkv {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDecThreads = 256;  // 4 waves
constexpr int kDecUnroll = 4;     // row batches per wave in flight
constexpr int kDecRowsPerIter = 4 * 4 * kDecUnroll;  // waves x rows per wave instruction x unroll

__device__ inline float dec_neg_inf() { return -__builtin_huge_valf(); }

template <int CTRL>
__device__ __forceinline__ float dec_dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a DPP row (every lane of the row ends with the sum).
__device__ __forceinline__ float dec_row16_sum(float v) {
    v += dec_dpp<0x128>(v);  // row_ror:8
    v += dec_dpp<0x124>(v);  // row_ror:4
    v += dec_dpp<0x122>(v);  // row_ror:2
    v += dec_dpp<0x121>(v);  // row_ror:1
    return v;
}
// Max / sum over lanes i, i^32 (permlane32 swap) and i, i^16 (permlane16 swap): the two
// results of a swap are the lane's own value and its partner's, in some order.
__device__ __forceinline__ float dec_max32(float v) {
    const unsigned u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float dec_max16(float v) {
    const unsigned u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float dec_sum32(float v) {
    const unsigned u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float dec_sum16(float v) {
    const unsigned u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// 16 bytes -> E fp32 elements.
template <typename T> struct Chunk;
template <> struct Chunk<__bf16> {
    static constexpr int E = 8;
    __device__ static void unpack(const u32x4_t c, float (&x)[8]) {
        static_for<4>([&](auto i) {
            x[2 * i()] = __uint_as_float(c[i()] << 16);
            x[2 * i() + 1] = __uint_as_float(c[i()] & 0xFFFF0000u);
        });
    }
};
template <> struct Chunk<float> {
    static constexpr int E = 4;
    __device__ static void unpack(const u32x4_t c, float (&x)[4]) {
        static_for<4>([&](auto i) { x[i()] = __uint_as_float(c[i()]); });
    }
};

// grid: (splits, requests * H_kv * head groups).  GT = query heads per workgroup (<= 8).
template <typename T, int GT>
__global__ void __launch_bounds__(kDecThreads) decode_partial_kernel(const DecodeParams p) {
    constexpr int E = Chunk<T>::E;
    constexpr int D = 16 * E;
    __shared__ float sh_m[4][GT], sh_l[4][GT];
    __shared__ float sh_acc[4][GT][D];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lc = lane & 15, lg = lane >> 4;  // chunk of the row, row within the instruction
    const int item = blockIdx.y;
    const int hc = item % p.n_hchunks, rg = item / p.n_hchunks;
    const int r = rg / p.Hkv, g = rg - (rg / p.Hkv) * p.Hkv;
    const int h0 = g * p.G + hc * GT;                     // first query head of this workgroup
    const int nh = p.G - hc * GT < GT ? p.G - hc * GT : GT;  // heads in use
    const int rows = p.rt.L[r];
    const int split = blockIdx.x;
    const int row0 = split * p.split_rows;
    if (row0 >= rows) return;
    const int row1 = row0 + p.split_rows < rows ? row0 + p.split_rows : rows;

    // query fragments (this lane's chunk of every head), scaled by log2(e) / sqrt(d)
    float qv[GT][E];
    static_for<GT>([&](auto h) {
        if (h() < nh) {
            const u32x4_t c = *(const u32x4_t *)((const char *)p.q +
                                                 (((int64_t)p.rt.qi[r] * p.Hq + h0 + h()) * D) * sizeof(T) + lc * 16);
            Chunk<T>::unpack(c, qv[h()]);
            static_for<E>([&](auto e) { qv[h()][e()] *= p.c; });
        } else {
            static_for<E>([&](auto e) { qv[h()][e()] = 0.f; });
        }
    });
    float m[GT], l[GT], acc[GT][E];
    static_for<GT>([&](auto h) {
        m[h()] = dec_neg_inf();
        l[h()] = 0.f;
        static_for<E>([&](auto e) { acc[h()][e()] = 0.f; });
    });
    const int64_t tstride = p.token_stride * (int64_t)sizeof(T);
    const char *kb = (const char *)p.K + ((int64_t)g * p.head_stride + p.rt.tok0[r] * p.token_stride) * sizeof(T) + lc * 16;
    const char *vb = (const char *)p.V + ((int64_t)g * p.head_stride + p.rt.tok0[r] * p.token_stride) * sizeof(T) + lc * 16;

    for (int it = row0; it < row1; it += kDecRowsPerIter) {
        u32x4_t kc[kDecUnroll], vc[kDecUnroll];
        bool ok[kDecUnroll];
        static_for<kDecUnroll>([&](auto u) {
            int row = it + u() * 16 + wave * 4 + lg;
            ok[u()] = row < row1;
            row = ok[u()] ? row : row0;  // in bounds; masked below
            kc[u()] = __builtin_nontemporal_load((const u32x4_t *)(kb + (int64_t)row * tstride));
            vc[u()] = __builtin_nontemporal_load((const u32x4_t *)(vb + (int64_t)row * tstride));
        });
        float s[kDecUnroll][GT];
        static_for<kDecUnroll>([&](auto u) {
            float kx[E];
            Chunk<T>::unpack(kc[u()], kx);
            static_for<GT>([&](auto h) {
                float a = 0.f;
                static_for<E>([&](auto e) { a = fmaf(qv[h()][e()], kx[e()], a); });
                a = dec_row16_sum(a);
                s[u()][h()] = ok[u()] ? a : dec_neg_inf();
            });
        });
        static_for<GT>([&](auto h) {
            float mb = s[0][h()];
            static_for<kDecUnroll - 1>([&](auto u) { mb = fmaxf(mb, s[u() + 1][h()]); });
            const float mn = fmaxf(m[h()], mb);
            if (mn != dec_neg_inf()) {
                const float corr = __builtin_amdgcn_exp2f(m[h()] - mn);  // 0 when m = -inf
                l[h()] *= corr;
                static_for<E>([&](auto e) { acc[h()][e()] *= corr; });
                static_for<kDecUnroll>([&](auto u) {
                    const float pu = __builtin_amdgcn_exp2f(s[u()][h()] - mn);
                    float vx[E];
                    Chunk<T>::unpack(vc[u()], vx);
                    l[h()] += pu;
                    static_for<E>([&](auto e) { acc[h()][e()] = fmaf(pu, vx[e()], acc[h()][e()]); });
                });
                m[h()] = mn;
            }
        });
    }

    // merge the four row groups of the wave (lanes i, i^16, i^32, i^48 hold the same chunk)
    static_for<GT>([&](auto h) {
        const float mm = dec_max16(dec_max32(m[h()]));
        const float f = mm == dec_neg_inf() ? 0.f : __builtin_amdgcn_exp2f(m[h()] - mm);
        const float ll = dec_sum16(dec_sum32(l[h()] * f));
        static_for<E>([&](auto e) { acc[h()][e()] = dec_sum16(dec_sum32(acc[h()][e()] * f)); });
        if (lg == 0) {
            if (lc == 0) {
                sh_m[wave][h()] = mm;
                sh_l[wave][h()] = ll;
            }
            static_for<E>([&](auto e) { sh_acc[wave][h()][lc * E + e()] = acc[h()][e()]; });
        }
    });
    __syncthreads();
    // merge the four waves and write this split's partial (max, sum, values) per head
    float *part = p.part + ((int64_t)item * p.max_splits + split) * (GT * (D + 2));
    for (int t = tid; t < GT * D; t += kDecThreads) {
        const int h = t / D, dd = t - (t / D) * D;
        float mm = sh_m[0][h];
        for (int w2 = 1; w2 < 4; ++w2) mm = fmaxf(mm, sh_m[w2][h]);
        float ll = 0.f, a = 0.f;
        if (mm != dec_neg_inf()) {
            for (int w2 = 0; w2 < 4; ++w2) {
                const float f = __builtin_amdgcn_exp2f(sh_m[w2][h] - mm);
                ll += sh_l[w2][h] * f;
                a += sh_acc[w2][h][dd] * f;
            }
        }
        part[h * (D + 2) + 2 + dd] = a;
        if (dd == 0) {
            part[h * (D + 2)] = mm;
            part[h * (D + 2) + 1] = ll;
        }
    }
}

// grid: (requests * H_q), 128 threads.  The splits' (max, sum) pairs are read in parallel and
// turned into weights in LDS; then each thread sums its output elements over the splits
// with eight partial loads in flight.
constexpr int kDecMaxSplits = 2048;
__global__ void __launch_bounds__(128) decode_combine_kernel(const DecodeParams p) {
    __shared__ float sh_w[kDecMaxSplits];
    __shared__ float sh_red[2][2];
    const int rq = blockIdx.x;
    const int r = rq / p.Hq, hq = rq - (rq / p.Hq) * p.Hq;
    const int g = hq / p.G, hl = hq - (hq / p.G) * p.G;
    const int hc = hl / 8, h = hl - (hl / 8) * 8;
    const int GT = p.head_tile, D = p.d;
    const int item = (r * p.Hkv + g) * p.n_hchunks + hc;
    const int ns = (p.rt.L[r] + p.split_rows - 1) / p.split_rows;
    const int tid = threadIdx.x;
    const int64_t sstride = (int64_t)GT * (D + 2);
    float *out = p.out + ((int64_t)p.rt.qi[r] * p.Hq + hq) * D;
    const float *part = p.part + (int64_t)item * p.max_splits * sstride + (int64_t)h * (D + 2);
    // max over the splits
    float mm = dec_neg_inf();
    for (int s = tid; s < ns; s += 128) mm = fmaxf(mm, part[s * sstride]);
    mm = fmaxf(mm, __shfl_xor(mm, 32));
    mm = fmaxf(mm, __shfl_xor(mm, 16));
    mm = fmaxf(mm, __shfl_xor(mm, 8));
    mm = fmaxf(mm, __shfl_xor(mm, 4));
    mm = fmaxf(mm, __shfl_xor(mm, 2));
    mm = fmaxf(mm, __shfl_xor(mm, 1));
    if ((tid & 63) == 0) sh_red[0][tid >> 6] = mm;
    __syncthreads();
    mm = fmaxf(sh_red[0][0], sh_red[0][1]);
    // split weights and the sum
    float ll = 0.f;
    for (int s = tid; s < ns; s += 128) {
        const float f = mm == dec_neg_inf() ? 0.f : __builtin_amdgcn_exp2f(part[s * sstride] - mm);
        sh_w[s] = f;
        ll += f * part[s * sstride + 1];
    }
    ll += __shfl_xor(ll, 32);
    ll += __shfl_xor(ll, 16);
    ll += __shfl_xor(ll, 8);
    ll += __shfl_xor(ll, 4);
    ll += __shfl_xor(ll, 2);
    ll += __shfl_xor(ll, 1);
    if ((tid & 63) == 0) sh_red[1][tid >> 6] = ll;
    __syncthreads();
    ll = sh_red[1][0] + sh_red[1][1];
    for (int dd = tid; dd < D; dd += 128) {
        float a = 0.f;
        for (int s0 = 0; s0 < ns; s0 += 8) {
            float v[8];
            static_for<8>([&](auto e) { v[e()] = s0 + e() < ns ? part[(s0 + e()) * sstride + 2 + dd] : 0.f; });
            static_for<8>([&](auto e) {
                if (s0 + e() < ns) a = fmaf(sh_w[s0 + e()], v[e()], a);
            });
        }
        out[dd] = ll > 0.f ? a / ll : 0.f;
    }
}

const void *decode_partial_kernel_for(int dtype, int head_tile) {
    if (dtype == 1) {
        switch (head_tile) {
            case 1: return (const void *)&decode_partial_kernel<__bf16, 1>;
            case 2: return (const void *)&decode_partial_kernel<__bf16, 2>;
            case 4: return (const void *)&decode_partial_kernel<__bf16, 4>;
            default: return (const void *)&decode_partial_kernel<__bf16, 8>;
        }
    }
    switch (head_tile) {
        case 1: return (const void *)&decode_partial_kernel<float, 1>;
        case 2: return (const void *)&decode_partial_kernel<float, 2>;
        case 4: return (const void *)&decode_partial_kernel<float, 4>;
        default: return (const void *)&decode_partial_kernel<float, 8>;
    }
}
const void *decode_combine_kernel_ptr() { return (const void *)&decode_combine_kernel; }
int decode_threads() { return kDecThreads; }
int decode_rows_per_iter() { return kDecRowsPerIter; }
int decode_max_splits() { return kDecMaxSplits; }

}  // namespace snapkv
