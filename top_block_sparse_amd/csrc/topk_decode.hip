// topk_decode.hip -- top-k gathered decode over a paged KV cache, gfx950.
//
// What it computes (flash-sparse-attn page: top-k gather KV-cache decode,
// paged attention, split-KV; flash-attention-npu page, flash_attn_with_kvcache
// docstring: paged cache layout, block_table, cache_seqlens; Ascend SFA blog:
// gather the selected K/V rows into a compact set, then ordinary attention,
// with a reduction core merging the split results): the single query of
// sequence b, q head h, attends to the cache positions listed in
// tok_idx[b, h / G, :], read as a set.
//
// Work is memory bound (each selected position costs one 2*d-byte K row and
// one V row read from HBM and about 4*d*G flops), so the kernels are built
// for many independent row loads in flight, not for the matrix cores:
//   1. decode_prepass: one workgroup per (sequence, kv head) sorts the list in
//      LDS, drops invalid positions and repeats, translates each position
//      through the block table once and writes the compact list of physical
//      cache rows (ascending) plus its length.
//   2. decode_split: each wave takes a contiguous part of one compact list.
//      Sixteen lanes cover one d-wide row (16 bytes each), so a wave works on
//      four rows at a time and keeps 8 rows per lane group in flight.  Each
//      lane group runs its own online softmax over its rows; the four groups
//      are merged by cross-lane exchanges and the wave writes one partial
//      (normalised O, LSE) per query head.
//   3. lse_merge (lse_merge.hip) combines the partials.
#include "fsa_common.h"
#include "fsa_params.h"

namespace fsa {

constexpr int kDecPrepassThreads = 1024;
constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecUnroll = 8;            // rows in flight per lane group


__global__ void __launch_bounds__(kDecPrepassThreads)
decode_prepass_kernel(const DecodeParams p) {
    extern __shared__ __align__(16) uint8_t smem[];
    int* key = reinterpret_cast<int*>(smem);                    // [sort_n]
    int* wsum = key + p.sort_n;                                 // [32]
    const int unit = blockIdx.x;                                // b * Hkv + g
    const int b = unit / p.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = p.sort_n;
    const int L = p.cache_seqlens[b];
    const int32_t* lst = p.tok_idx + (int64_t)unit * p.topk;
    const int32_t* bt = p.block_table + (int64_t)b * p.max_pages;
    constexpr int kInvalid = 0x7fffffff;

    for (int e = tid; e < n; e += kDecPrepassThreads) {
        int t = kInvalid;
        if (e < p.topk) {
            const int x = lst[e];
            if (x >= 0 && x < L && x / p.page_size < p.max_pages) {
                const int page = bt[x / p.page_size];
                if (page >= 0 && page < p.num_pages) t = x;
            }
        }
        key[e] = t;
    }
    __syncthreads();
    // bitonic sort, ascending
    for (int kk = 2; kk <= n; kk <<= 1) {
        for (int jj = kk >> 1; jj > 0; jj >>= 1) {
            for (int i = tid; i < n; i += kDecPrepassThreads) {
                const int ixj = i ^ jj;
                if (ixj > i) {
                    const int a = key[i], c = key[ixj];
                    const bool up = (i & kk) == 0;
                    if ((a > c) == up) {
                        key[i] = c;
                        key[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    // keep the first of each run of equal valid positions; compact in order
    const int per = (n + kDecPrepassThreads - 1) / kDecPrepassThreads;
    const int beg = tid * per;
    int cnt = 0;
    for (int i = beg; i < beg + per && i < n; ++i) {
        const int t = key[i];
        if (t != kInvalid && (i == 0 || key[i - 1] != t)) ++cnt;
    }
    // block exclusive scan of cnt
    int incl = cnt;
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int x = 0; x < wave; ++x) wbase += wsum[x];
    int pos = wbase + incl - cnt;
    int32_t* out = p.rows + (int64_t)unit * p.topk;
    for (int i = beg; i < beg + per && i < n; ++i) {
        const int t = key[i];
        if (t != kInvalid && (i == 0 || key[i - 1] != t)) {
            const int page = bt[t / p.page_size];
            out[pos++] = page * p.page_size + (t % p.page_size);
        }
    }
    if (tid == kDecPrepassThreads - 1) p.counts[unit] = wbase + incl;
}

// D: head dim (64 or 128); GM: query heads handled per kv head (>= G).
template <int D, int GM>
__global__ void __launch_bounds__(kDecThreads)
decode_split_kernel(const DecodeParams p) {
    constexpr int DPL = D / 16;              // dims per lane (8 or 4)
    constexpr int WPL = DPL / 2;             // 32-bit words per lane
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15;                // 16 lanes share one cache row
    const int lg = lane >> 4;                // which of the wave's 4 rows
    const int unit = blockIdx.x / p.splits;  // b * Hkv + g
    const int split = blockIdx.x % p.splits;
    const int b = unit / p.Hkv;
    const int g = unit % p.Hkv;
    const int G = p.G;

    const int n = p.counts[unit];
    const int nparts = p.splits * kDecWaves;
    const int part = split * kDecWaves + wave;
    const int r_beg = (int)(((long long)n * part) / nparts);
    const int r_end = (int)(((long long)n * (part + 1)) / nparts);
    const int32_t* rows = p.rows + (int64_t)unit * p.topk;

    // the G query rows (fp32), this lane's DPL dims
    float qv[GM][DPL];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        if (h < G) {
            const uint16_t* qr = p.q + ((int64_t)b * p.Hq + g * G + h) * D + lr * DPL;
            if constexpr (DPL == 8) {
                const u32x4_t w = *reinterpret_cast<const u32x4_t*>(qr);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    qv[h][2 * x] = bf16_lo(w[x]);
                    qv[h][2 * x + 1] = bf16_hi(w[x]);
                }
            } else {
                const u32x2_t w = *reinterpret_cast<const u32x2_t*>(qr);
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    qv[h][2 * x] = bf16_lo(w[x]);
                    qv[h][2 * x + 1] = bf16_hi(w[x]);
                }
            }
        } else {
#pragma unroll
            for (int x = 0; x < DPL; ++x) qv[h][x] = 0.f;
        }
    }

    float m_run[GM], l_run[GM], acc[GM][DPL];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int x = 0; x < DPL; ++x) acc[h][x] = 0.f;
    }

    const int64_t row_stride = (int64_t)p.Hkv * D;   // elements between cache rows
    const uint16_t* kbase = p.kc + (int64_t)g * D + lr * DPL;
    const uint16_t* vbase = p.vc + (int64_t)g * D + lr * DPL;

    for (int r0 = r_beg; r0 < r_end; r0 += 4 * kDecUnroll) {
        uint32_t kw[kDecUnroll][WPL], vw[kDecUnroll][WPL];
        bool ok[kDecUnroll];
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            const int r = r0 + u * 4 + lg;
            ok[u] = r < r_end;
            const int64_t cr = ok[u] ? rows[r] : 0;
            const uint16_t* kp = kbase + cr * row_stride;
            const uint16_t* vp = vbase + cr * row_stride;
            if constexpr (WPL == 4) {
                u32x4_t a = ok[u] ? *reinterpret_cast<const u32x4_t*>(kp) : u32x4_t{0u, 0u, 0u, 0u};
                u32x4_t c = ok[u] ? *reinterpret_cast<const u32x4_t*>(vp) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
                for (int x = 0; x < 4; ++x) { kw[u][x] = a[x]; vw[u][x] = c[x]; }
            } else {
                u32x2_t a = ok[u] ? *reinterpret_cast<const u32x2_t*>(kp) : u32x2_t{0u, 0u};
                u32x2_t c = ok[u] ? *reinterpret_cast<const u32x2_t*>(vp) : u32x2_t{0u, 0u};
#pragma unroll
                for (int x = 0; x < 2; ++x) { kw[u][x] = a[x]; vw[u][x] = c[x]; }
            }
        }
        // scores of the lane group's rows, one per query head
        float s[kDecUnroll][GM];
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
#pragma unroll
            for (int h = 0; h < GM; ++h) {
                float d = 0.f;
#pragma unroll
                for (int x = 0; x < WPL; ++x) {
                    d = fmaf(qv[h][2 * x], bf16_lo(kw[u][x]), d);
                    d = fmaf(qv[h][2 * x + 1], bf16_hi(kw[u][x]), d);
                }
                d += __shfl_xor(d, 1);
                d += __shfl_xor(d, 2);
                d += __shfl_xor(d, 4);
                d += __shfl_xor(d, 8);
                s[u][h] = ok[u] ? d * p.scale_log2 : -INFINITY;
            }
        }
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            float mb = s[0][h];
#pragma unroll
            for (int u = 1; u < kDecUnroll; ++u) mb = fmaxf(mb, s[u][h]);
            const float m_new = fmaxf(m_run[h], mb);
            const float msub = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m_run[h] - msub);
            m_run[h] = m_new;
            float ls = 0.f;
#pragma unroll
            for (int x = 0; x < DPL; ++x) acc[h][x] *= alpha;
#pragma unroll
            for (int u = 0; u < kDecUnroll; ++u) {
                const float pr = fast_exp2(s[u][h] - msub);
                ls += pr;
#pragma unroll
                for (int x = 0; x < WPL; ++x) {
                    acc[h][2 * x] = fmaf(pr, bf16_lo(vw[u][x]), acc[h][2 * x]);
                    acc[h][2 * x + 1] = fmaf(pr, bf16_hi(vw[u][x]), acc[h][2 * x + 1]);
                }
            }
            l_run[h] = l_run[h] * alpha + ls;
        }
    }

    // merge the four lane groups of the wave, then write this wave's partial
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        float m = m_run[h];
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        const float msub = m == -INFINITY ? 0.f : m;
        const float sc = fast_exp2(m_run[h] - msub);
        float l = l_run[h] * sc;
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
#pragma unroll
        for (int x = 0; x < DPL; ++x) {
            float a = acc[h][x] * sc;
            a += __shfl_xor(a, 16);
            a += __shfl_xor(a, 32);
            acc[h][x] = a;
        }
        if (h < G) {
            const float inv = l > 0.f ? 1.f / l : 0.f;
            const float lse_v = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
            const int64_t prow = (int64_t)part * p.batch * p.Hq + (int64_t)b * p.Hq + g * G + h;
            if (lg == 0) {
                float* o = p.part_o + prow * D + lr * DPL;
#pragma unroll
                for (int x = 0; x < DPL; x += 4) {
                    *reinterpret_cast<f32x4_t*>(o + x) =
                        f32x4_t{acc[h][x] * inv, acc[h][x + 1] * inv, acc[h][x + 2] * inv,
                                acc[h][x + 3] * inv};
                }
                if (lr == 0) p.part_lse[prow] = lse_v;
            }
        }
    }
}

hipError_t launch_decode_prepass(const DecodeParams& p, hipStream_t stream) {
    const size_t lds = (size_t)p.sort_n * 4 + 32 * 4;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_prepass_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(decode_prepass_kernel, dim3(p.batch * p.Hkv), dim3(kDecPrepassThreads), lds,
                       stream, p);
    return hipGetLastError();
}

template <int D, int GM>
static hipError_t launch_split_t(const DecodeParams& p, hipStream_t stream) {
    hipLaunchKernelGGL((decode_split_kernel<D, GM>), dim3(p.batch * p.Hkv * p.splits),
                       dim3(kDecThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_split_d(const DecodeParams& p, hipStream_t stream) {
    if (p.G <= 1) return launch_split_t<D, 1>(p, stream);
    if (p.G <= 2) return launch_split_t<D, 2>(p, stream);
    if (p.G <= 4) return launch_split_t<D, 4>(p, stream);
    if (p.G <= 8) return launch_split_t<D, 8>(p, stream);
    return launch_split_t<D, 16>(p, stream);
}

hipError_t launch_decode_split(const DecodeParams& p, int D, hipStream_t stream) {
    return D == 64 ? launch_split_d<64>(p, stream) : launch_split_d<128>(p, stream);
}

int decode_waves_per_split() { return kDecWaves; }

}  // namespace fsa
