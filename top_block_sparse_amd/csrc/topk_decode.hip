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
// The work is memory bound: each selected position costs one 2*d-byte K row
// and one V row from HBM against about 4*d*G flops.  So the kernel is built
// for many independent 256-byte row loads in flight, and the arithmetic stays
// on the vector ALUs (bf16 dot2 for the scores).  One workgroup handles one
// (sequence, kv head) list, or one part of it when the list is split:
//   1. validate and translate: every list entry is checked (0 <= t <
//      cache_seqlens[b], page slot and page id in range) and translated
//      through the block table to a physical cache row, all in LDS;
//   2. set semantics: an LDS hash table keyed by position keeps, for every
//      distinct valid position, its first list entry (open addressing with
//      linear probing, at most a quarter full when LDS allows); every other
//      entry is marked skipped.  A split list is cut by entry index, so the
//      parts are disjoint whatever the list holds;
//   3. the waves stream the workgroup's part in batches of 4*kDecUnroll
//      entries taken from a shared counter (so they finish together):
//      sixteen lanes cover one row (16 or 8 bytes each), so a wave loads four
//      rows per instruction; a batch is kDecUnroll such groups of K and V, and
//      each wave keeps two batches in flight (the next one's loads go out
//      before the current one is consumed); each lane group runs its own
//      online softmax; the probabilities are
//      rounded to bf16 for the P.V products (bf16 dot2 with fp32
//      accumulation), the row sums stay fp32;
//   4. the lane groups, then the waves, are merged by logsumexp in LDS, and
//      the workgroup writes O and LSE (or, for a split list, its normalised
//      partial, combined afterwards by lse_merge.hip).
#include "fsa_common.h"
#include "fsa_params.h"

namespace fsa {

constexpr int kDecUnroll = 4;            // row groups per batch (halved for G > 4)
constexpr int kDecWavesSmallG = 8;       // waves per workgroup for G <= 4
constexpr int kDecMaxTopk = 8192;
constexpr int kDecBtLds = 2048;          // block-table rows up to this length are staged in LDS
constexpr unsigned long long kDecEmpty = ~0ull;

__host__ __device__ constexpr int dec_waves(int GM) { return GM <= 4 ? kDecWavesSmallG : (GM == 8 ? 8 : 4); }

// LDS layout (bytes) of the decode workgroup for a hash table of ts slots.
//   region 0: u64 table[ts] (steps 1-2): slot = position << 32 | list entry,
//             reused for the wave partials (step 4): NW * GM records of D
//             accumulator values + max + sum (fp32)
//   i32 rows[topk]          physical cache row of each entry (-1: skipped)
//   i32 next                next batch of entries to stream
//   i32 btl[kDecBtLds]      the sequence's block-table row (when it fits)
template <int D, int GM>
struct DecLds {
    static constexpr int NW = dec_waves(GM);
    static constexpr int KMAX = kDecMaxTopk / (NW * 64);
    static constexpr int kRec = D + 2;
    __host__ __device__ static int region0(int ts) {
        const int a = ts * 8, b = NW * GM * kRec * 4;
        return ((a > b ? a : b) + 15) & ~15;
    }
    __host__ __device__ static int rows(int ts) { return region0(ts); }
    __host__ __device__ static int next(int ts, int topk) { return rows(ts) + ((topk * 4 + 15) & ~15); }
    __host__ __device__ static int btl(int ts, int topk) { return next(ts, topk) + 16; }
    __host__ __device__ static int bytes(int ts, int topk) { return btl(ts, topk) + kDecBtLds * 4; }
};

// Slot where the probe sequence of position x starts (multiplicative hash
// scaled to [0, ts)).
__device__ __forceinline__ int dec_hash(int x, int ts) {
    return (int)(((unsigned long long)((uint32_t)x * 0x9E3779B1u) * (uint32_t)ts) >> 32);
}

// Sum over the 16 lanes of a row of the wave (every lane gets the total):
// swap neighbours, swap pairs, mirror within 8, mirror within 16.
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    return x;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// D: head dim (64 or 128); GM: query heads handled per kv head (>= G);
// F8: the cache holds FP8 E4M3 bytes with dequantisation factors (else bf16).
template <int D, int GM, bool F8>
__global__ void __launch_bounds__(dec_waves(GM) * 64)
decode_kernel(const DecodeParams p) {
    using L = DecLds<D, GM>;
    constexpr int NW = L::NW;
    constexpr int NT = NW * 64;
    constexpr int DPL = D / 16;              // dims per lane (8 or 4)
    constexpr int WPL = DPL / 2;             // bf16 pairs per lane and row
    constexpr int EB = F8 ? 1 : 2;           // bytes per cache element
    constexpr int RW = DPL * EB / 4;         // raw 32-bit words per lane and row
    constexpr int U = GM > 4 ? kDecUnroll / 2 : kDecUnroll;

    constexpr int KMAX = L::KMAX;            // list entries per thread, at most

    extern __shared__ __align__(16) uint8_t smem[];
    const int ts = p.ts;
    const int topk = p.topk;
    unsigned long long* table = reinterpret_cast<unsigned long long*>(smem);
    int* rows = reinterpret_cast<int*>(smem + L::rows(ts));
    int* next = reinterpret_cast<int*>(smem + L::next(ts, topk));
    int* btl = reinterpret_cast<int*>(smem + L::btl(ts, topk));
    float* mrg = reinterpret_cast<float*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15;                // 16 lanes share one cache row
    const int lg = lane >> 4;                // which of the wave's 4 rows
    const int unit = blockIdx.x / p.splits;  // b * Hkv + g
    const int split = blockIdx.x % p.splits;
    const int b = unit / p.Hkv;
    const int g = unit % p.Hkv;
    const int G = p.G;
    const int cs = p.cache_seqlens[b];
    const int32_t* lst = p.tok_idx + (int64_t)unit * topk;
    const int32_t* bt = p.block_table + (int64_t)b * p.max_pages;
    const int nchunk = (topk + NT - 1) / NT;     // <= KMAX

    // ---- 1. validate and translate this thread's entries e = k*NT + tid.
    // Straight-line passes (all list loads together with the block-table row,
    // then the lookups) so the loads of different entries are in flight
    // together.
    for (int i = tid; i < ts; i += NT) table[i] = kDecEmpty;
    int key[KMAX], phys[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int e = k * NT + tid;
        key[k] = lst[e < topk ? e : topk - 1];
    }
    const bool bt_in_lds = p.max_pages <= kDecBtLds;
    if (bt_in_lds)
        for (int i = tid; i < p.max_pages; i += NT) btl[i] = bt[i];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int x = key[k];
        const int slot = x / p.page_size;
        const bool ok = k * NT + tid < topk && x >= 0 && x < cs && slot < p.max_pages;
        key[k] = ok ? x : -1;
        phys[k] = ok ? slot : 0;
    }
    if (bt_in_lds) {
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KMAX; ++k) phys[k] = btl[phys[k]];   // page id, checked below
    } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) phys[k] = bt[phys[k]];
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int x = key[k];
        const int page = phys[k];
        const bool ok = x >= 0 && page >= 0 && page < p.num_pages;
        const int slot = x / p.page_size;
        phys[k] = ok ? page * p.page_size + (x - slot * p.page_size) : 0;
        key[k] = ok ? x : -1;
        const int e = k * NT + tid;
        if (k < nchunk && e < topk) rows[e] = ok ? phys[k] : -1;
    }
    if (tid == 0) *next = NW;                    // batches 0..NW-1: each wave's first
    __syncthreads();

    // ---- 3 (start). The waves stream the workgroup's part of the list in
    // batches of 4*U entries taken from a shared counter, so they finish
    // together.  Each wave's first batch is loaded now, so its loads are in
    // flight during the set computation; its repeats are masked afterwards.
    const int r_lo = (int)(((long long)topk * split) / p.splits);
    const int r_hi = (int)(((long long)topk * (split + 1)) / p.splits);
    constexpr int B = 4 * U;                 // entries per batch
    const int nbatch = (r_hi - r_lo + B - 1) / B;
    const int64_t row_stride = (int64_t)p.Hkv * D * EB;   // bytes between cache rows
    const uint8_t* kbase = static_cast<const uint8_t*>(p.kc) + ((int64_t)g * D + lr * DPL) * EB;
    const uint8_t* vbase = static_cast<const uint8_t*>(p.vc) + ((int64_t)g * D + lr * DPL) * EB;
    // Entries r0 + 4u + lg, u < U, are one batch.  Bit u of the mask: that
    // entry is a row to attend to (inside the part, valid and not a repeat).
    auto okmask = [&](int r0) {
        uint32_t okm = 0u;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + u * 4 + lg;
            okm |= (uint32_t)(r < r_hi && rows[r] >= 0) << u;
        }
        return okm;
    };
    // Raw cache words of a batch (bf16 pairs, or four E4M3 bytes per word).
    auto issue = [&](uint32_t (&kw)[U][RW], uint32_t (&vw)[U][RW], int r0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + u * 4 + lg;
            const int row = r < r_hi ? rows[r] : -1;
            const int64_t cr = row >= 0 ? row : 0;     // skipped entries read row 0, ignored
            const uint8_t* kp = kbase + cr * row_stride;
            const uint8_t* vp = vbase + cr * row_stride;
            if constexpr (RW == 4) {
                const u32x4_t a = *reinterpret_cast<const u32x4_t*>(kp);
                const u32x4_t c = *reinterpret_cast<const u32x4_t*>(vp);
#pragma unroll
                for (int x = 0; x < 4; ++x) { kw[u][x] = a[x]; vw[u][x] = c[x]; }
            } else if constexpr (RW == 2) {
                const u32x2_t a = *reinterpret_cast<const u32x2_t*>(kp);
                const u32x2_t c = *reinterpret_cast<const u32x2_t*>(vp);
#pragma unroll
                for (int x = 0; x < 2; ++x) { kw[u][x] = a[x]; vw[u][x] = c[x]; }
            } else {
                kw[u][0] = *reinterpret_cast<const uint32_t*>(kp);
                vw[u][0] = *reinterpret_cast<const uint32_t*>(vp);
            }
        }
    };
    uint32_t ka[U][RW], va[U][RW];
    int bi = wave;
    if (bi < nbatch) issue(ka, va, r_lo + bi * B);

    // ---- 2. hash table: position -> (position, smallest list entry holding
    // it).  A slot's position never changes once claimed, so all entries of
    // one position meet in the same slot; probes are bounded by the table
    // size (which exceeds topk).  Each entry remembers its slot.
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int x = key[k];
        int h = -1;
        if (x >= 0) {
            const unsigned long long mine =
                ((unsigned long long)(uint32_t)x << 32) | (uint32_t)(k * NT + tid);
            h = dec_hash(x, ts);
            for (int probe = 0; probe < ts; ++probe) {
                const unsigned long long old = atomicCAS(&table[h], kDecEmpty, mine);
                if (old == kDecEmpty) break;
                if ((uint32_t)(old >> 32) == (uint32_t)x) {
                    atomicMin(&table[h], mine);
                    break;
                }
                h = h + 1 == ts ? 0 : h + 1;
            }
        }
        key[k] = h;                              // now: the entry's slot, or -1
    }
    __syncthreads();

    // ---- keep each position's first entry: a valid entry that repeats an
    // earlier one is marked skipped (rows[e] = -1)
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int e = k * NT + tid;
        if (key[k] >= 0 && (uint32_t)table[key[k]] != (uint32_t)e) rows[e] = -1;
    }
    __syncthreads();

    // scale (log2 units) including the K dequantisation factor; V's factor
    // scales the output
    float c_log2 = p.scale_log2, v_scale = 1.f;
    if constexpr (F8) {
        if (p.k_descale != nullptr) c_log2 *= p.k_descale[unit];
        if (p.v_descale != nullptr) v_scale = p.v_descale[unit];
    }

    uint32_t qw[GM][WPL];                    // this lane's dims of the G query rows (bf16 pairs)
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        if (h < G) {
            const uint16_t* qr = p.q + ((int64_t)b * p.Hq + g * G + h) * D + lr * DPL;
            if constexpr (WPL == 4) {
                const u32x4_t w = *reinterpret_cast<const u32x4_t*>(qr);
#pragma unroll
                for (int x = 0; x < 4; ++x) qw[h][x] = w[x];
            } else {
                const u32x2_t w = *reinterpret_cast<const u32x2_t*>(qr);
#pragma unroll
                for (int x = 0; x < 2; ++x) qw[h][x] = w[x];
            }
        } else {
#pragma unroll
            for (int x = 0; x < WPL; ++x) qw[h][x] = 0u;
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

    auto consume = [&](const uint32_t (&kr)[U][RW], const uint32_t (&vr)[U][RW], uint32_t okm) {
        // bf16 pairs of the rows (E4M3 -> bf16 is exact)
        uint32_t kw[U][WPL], vw[U][WPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int x = 0; x < RW; ++x) {
                if constexpr (F8) {
                    kw[u][2 * x] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kr[u][x], 1.f, false));
                    kw[u][2 * x + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kr[u][x], 1.f, true));
                    vw[u][2 * x] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vr[u][x], 1.f, false));
                    vw[u][2 * x + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vr[u][x], 1.f, true));
                } else {
                    kw[u][x] = kr[u][x];
                    vw[u][x] = vr[u][x];
                }
            }
        }
        // raw scores q.k of the lane group's rows, one per query head
        float s[U][GM];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int h = 0; h < GM; ++h) {
                float d = 0.f;
#pragma unroll
                for (int x = 0; x < WPL; ++x) d = dot2_bf16(qw[h][x], kw[u][x], d);
                s[u][h] = row16_sum(d);
            }
        }
        if (__builtin_amdgcn_ballot_w64(okm != (1u << U) - 1u) != 0ull) {   // skipped entries
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (((okm >> u) & 1u) == 0u) {
#pragma unroll
                    for (int h = 0; h < GM; ++h) s[u][h] = -INFINITY;
                }
        }
        // V of rows 2j and 2j+1 interleaved per dim: bf16 pairs for dot2
        uint32_t vlo[U / 2][WPL], vhi[U / 2][WPL];
#pragma unroll
        for (int j = 0; j < U / 2; ++j) {
#pragma unroll
            for (int x = 0; x < WPL; ++x) {
                vlo[j][x] = __builtin_amdgcn_perm(vw[2 * j + 1][x], vw[2 * j][x], 0x05040100u);
                vhi[j][x] = __builtin_amdgcn_perm(vw[2 * j + 1][x], vw[2 * j][x], 0x07060302u);
            }
        }
        const float c = c_log2;                  // > 0: the max commutes with the scaling
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            float mb = s[0][h];
#pragma unroll
            for (int u = 1; u < U; ++u) mb = fmaxf(mb, s[u][h]);
            const float m_new = fmaxf(m_run[h], mb * c);
            const float msub = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m_run[h] - msub);
            m_run[h] = m_new;
            float ls = 0.f;
#pragma unroll
            for (int x = 0; x < DPL; ++x) acc[h][x] *= alpha;
#pragma unroll
            for (int j = 0; j < U / 2; ++j) {
                const float p0 = fast_exp2(fmaf(s[2 * j][h], c, -msub));
                const float p1 = fast_exp2(fmaf(s[2 * j + 1][h], c, -msub));
                ls += p0 + p1;
                const uint32_t pp = pack_bf16x2(p0, p1);
#pragma unroll
                for (int x = 0; x < WPL; ++x) {
                    acc[h][2 * x] = dot2_bf16(pp, vlo[j][x], acc[h][2 * x]);
                    acc[h][2 * x + 1] = dot2_bf16(pp, vhi[j][x], acc[h][2 * x + 1]);
                }
            }
            l_run[h] = l_run[h] * alpha + ls;
        }
    };
    auto grab = [&]() {
        int t = 0;
        if (lane == 0) t = __hip_atomic_fetch_add(next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return __builtin_amdgcn_readfirstlane(t);
    };
    // two batches in flight per wave: the next one's loads are issued before
    // the current one is consumed
    uint32_t kb[U][RW], vb[U][RW];
    int bn = bi < nbatch ? grab() : nbatch;
    if (bn < nbatch) issue(kb, vb, r_lo + bn * B);
    while (bi < nbatch) {
        {
            const uint32_t okm = okmask(r_lo + bi * B);
            const int bn2 = bn < nbatch ? grab() : nbatch;
            consume(ka, va, okm);
            if (bn2 < nbatch) issue(ka, va, r_lo + bn2 * B);
            bi = bn;
            bn = bn2;
        }
        if (bi >= nbatch) break;
        {
            const uint32_t okm = okmask(r_lo + bi * B);
            const int bn2 = bn < nbatch ? grab() : nbatch;
            consume(kb, vb, okm);
            if (bn2 < nbatch) issue(kb, vb, r_lo + bn2 * B);
            bi = bn;
            bn = bn2;
        }
    }

    // ---- 4. merge the wave's four lane groups, then the workgroup's waves.
    // Region 0 (the hash table) is free: its last reads precede the barrier
    // that ended step 2's compaction.
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
        float* rec = mrg + (wave * GM + h) * L::kRec;
#pragma unroll
        for (int x = 0; x < DPL; ++x) {
            float a = acc[h][x] * sc;
            a += __shfl_xor(a, 16);
            a += __shfl_xor(a, 32);
            if (lg == 0) rec[lr * DPL + x] = a;
        }
        if (lane == 0) {
            rec[D] = m;
            rec[D + 1] = l;
        }
    }
    __syncthreads();
    for (int i = tid; i < G * (D / 2); i += NT) {
        const int h = i / (D / 2);
        const int d = 2 * (i - h * (D / 2));
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, mrg[(w * GM + h) * L::kRec + D]);
        const float msub = M == -INFINITY ? 0.f : M;
        float Ls = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float* rec = mrg + (w * GM + h) * L::kRec;
            const float sc = fast_exp2(rec[D] - msub);
            Ls = fmaf(rec[D + 1], sc, Ls);
            o0 = fmaf(rec[d], sc, o0);
            o1 = fmaf(rec[d + 1], sc, o1);
        }
        const float inv = Ls > 0.f ? v_scale / Ls : 0.f;
        const float lse_v = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
        const int64_t row = (int64_t)b * p.Hq + g * G + h;
        if (p.splits == 1) {
            *reinterpret_cast<uint32_t*>(p.out + row * D + d) = pack_bf16x2(o0 * inv, o1 * inv);
            if (p.lse != nullptr && d == 0) p.lse[row] = lse_v;
        } else {
            const int64_t prow = (int64_t)split * p.batch * p.Hq + row;
            *reinterpret_cast<f32x2_t*>(p.part_o + prow * D + d) = f32x2_t{o0 * inv, o1 * inv};
            if (d == 0) p.part_lse[prow] = lse_v;
        }
    }
}

template <int D, int GM, bool F8>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
    static std::atomic<unsigned long long> lds_set{0ull};   // devices with the LDS limit raised
    hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(&decode_kernel<D, GM, F8>), lds_set);
    if (e != hipSuccess) return e;
    const size_t lds = DecLds<D, GM>::bytes(p.ts, p.topk);
    hipLaunchKernelGGL((decode_kernel<D, GM, F8>), dim3(p.batch * p.Hkv * p.splits),
                       dim3(DecLds<D, GM>::NW * 64), lds, stream, p);
    return hipGetLastError();
}

template <int D, bool F8>
static hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream) {
    if (p.G <= 1) return launch_decode_t<D, 1, F8>(p, stream);
    if (p.G <= 2) return launch_decode_t<D, 2, F8>(p, stream);
    if (p.G <= 4) return launch_decode_t<D, 4, F8>(p, stream);
    if (p.G <= 8) return launch_decode_t<D, 8, F8>(p, stream);
    return launch_decode_t<D, 16, F8>(p, stream);
}

hipError_t launch_decode(const DecodeParams& p, int D, hipStream_t stream) {
    if (p.kv_fp8)
        return D == 64 ? launch_decode_d<64, true>(p, stream) : launch_decode_d<128, true>(p, stream);
    return D == 64 ? launch_decode_d<64, false>(p, stream) : launch_decode_d<128, false>(p, stream);
}

static int group_bucket(int G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16; }

int decode_waves_per_workgroup(int G) { return dec_waves(group_bucket(G)); }

size_t decode_lds_bytes(int D, int G, int ts, int topk) {
    switch (group_bucket(G)) {
        case 1: return D == 64 ? DecLds<64, 1>::bytes(ts, topk) : DecLds<128, 1>::bytes(ts, topk);
        case 2: return D == 64 ? DecLds<64, 2>::bytes(ts, topk) : DecLds<128, 2>::bytes(ts, topk);
        case 4: return D == 64 ? DecLds<64, 4>::bytes(ts, topk) : DecLds<128, 4>::bytes(ts, topk);
        case 8: return D == 64 ? DecLds<64, 8>::bytes(ts, topk) : DecLds<128, 8>::bytes(ts, topk);
        default: return D == 64 ? DecLds<64, 16>::bytes(ts, topk) : DecLds<128, 16>::bytes(ts, topk);
    }
}

// Hash table slots: 4 per list entry (short probe chains), fewer when LDS is
// short; always more than topk.
int decode_table_slots(int D, int G, int topk) {
    int ts = 4 * topk;
    if (ts < 64) ts = 64;
    while (ts > topk + 64 && decode_lds_bytes(D, G, ts, topk) > 160 * 1024) ts -= 64;
    return ts;
}

}  // namespace fsa
