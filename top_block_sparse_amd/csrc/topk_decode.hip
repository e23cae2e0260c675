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
//   2. set semantics: an LDS hash table of positions (open addressing with
//      linear probing, at most a quarter full when LDS allows) admits each
//      distinct valid position once.  A wave claims the positions of the
//      entries it is about to load with one compare-and-swap each, just
//      before loading them, so there is no separate de-duplication pass: the
//      entry whose claim lands first is streamed and every other entry of
//      that position is skipped.  A split list is cut by entry index, and a
//      part first enters the positions of all earlier entries, so a position
//      is streamed by the part that holds its first occurrence only;
//   3. the waves stream the workgroup's part in pairs of batches taken
//      from a shared counter (so they finish together): 16 lanes cover a
//      bf16 row and 8 an E4M3 row (16 for more than 4 query heads), so a wave
//      loads 4 (or 8) rows per instruction; a batch is two such row groups of
//      K and V, and each wave holds two batches with fixed roles, one in
//      flight while the other is consumed; each row group runs its own online
//      softmax with a lazily moved maximum; the probabilities are rounded to
//      bf16 for the P.V products (bf16 dot2 with fp32 accumulation), the row
//      sums stay fp32;
//   4. the row groups (with cross-lane swaps), then the waves (in LDS) are
//      merged by logsumexp, and the workgroup writes O and LSE (or, for a
//      split list, its normalised partial, combined afterwards by
//      lse_merge.hip).
#include "fsa_common.h"
#include "fsa_params.h"

namespace fsa {

constexpr int kDecRowsPerLane = 2;       // rows each lane holds in one batch
constexpr float kDecLazyMax = 8.f;       // running-max slack before a rescale (log2 units)
constexpr int kDecWavesSmallG = 8;       // waves per workgroup for G <= 4
constexpr int kDecMaxTopk = 8192;
constexpr int kDecBtLds = 2048;          // block-table rows up to this length are staged in LDS
constexpr uint32_t kDecEmpty = ~0u;        // free hash slot (positions are below 2^31)

__host__ __device__ constexpr int dec_waves(int GM) { return GM <= 4 ? kDecWavesSmallG : (GM == 8 ? 8 : 4); }
// Lanes that share one cache row.  A 256-byte bf16 row is read by 16 lanes
// (16 bytes each, one instruction per row group).  A 128-byte E4M3 row is
// read by 8 lanes when the accumulators of all query heads fit in registers
// (up to 4 heads): half the load instructions and shorter cross-lane sums.
__host__ __device__ constexpr int dec_lanes_per_row(int GM, bool F8) { return F8 && GM <= 4 ? 8 : 16; }

// LDS layout (bytes) of the decode workgroup for a hash table of ts slots.
//   region 0: u32 table[ts] (steps 2-3): claimed positions,
//             reused for the wave partials (step 4): NW * GM records of D
//             accumulator values + max + sum (fp32)
//   i32 rows[topk]          physical cache row of each entry (-1: skipped)
//   i32 pos[topk]           position of each valid entry (-1: invalid)
//   i32 next                next pair of batches to stream
//   i32 btl[kDecBtLds]      the sequence's block-table row (when it fits)
template <int D, int GM>
struct DecLds {
    static constexpr int NW = dec_waves(GM);
    static constexpr int KMAX = kDecMaxTopk / (NW * 64);
    static constexpr int kRec = D + 2;
    __host__ __device__ static int region0(int ts) {
        const int a = ts * 4, b = NW * GM * kRec * 4;
        return ((a > b ? a : b) + 15) & ~15;
    }
    __host__ __device__ static int rows(int ts) { return region0(ts); }
    __host__ __device__ static int pos(int ts, int topk) { return rows(ts) + ((topk * 4 + 15) & ~15); }
    __host__ __device__ static int next(int ts, int topk) { return pos(ts, topk) + ((topk * 4 + 15) & ~15); }
    __host__ __device__ static int btl(int ts, int topk) { return next(ts, topk) + 16; }
    __host__ __device__ static int bytes(int ts, int topk) { return btl(ts, topk) + kDecBtLds * 4; }
};

// Slot where the probe sequence of position x starts (multiplicative hash
// scaled to [0, ts)).
__device__ __forceinline__ int dec_hash(int x, int ts) {
    return (int)(((unsigned long long)((uint32_t)x * 0x9E3779B1u) * (uint32_t)ts) >> 32);
}

// Sum over N (8 or 16) aligned lanes of the wave, every lane getting the
// total: swap neighbours, swap pairs, mirror within 8, then mirror within 16.
template <int N>
__device__ __forceinline__ float row_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    if constexpr (N == 16)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    return x;
}

// Combine x over the lanes l ^ O, l ^ 2O, ..., l ^ 32 (O = 8 or 16), every
// lane getting the result: a half-row rotation for 8, then the gfx950
// permlane swaps across 16-lane rows (VALU only).
template <int O, bool MAX>
__device__ __forceinline__ float lanes_combine(float x) {
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    if constexpr (O == 8)
        x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
    {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return x;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Raw words of one lane's part of a cache or query row (aligned to their size).
template <int N>
__device__ __forceinline__ void load_words(const uint8_t* ptr, uint32_t (&w)[N]) {
    if constexpr (N == 8) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(ptr);
        const u32x4_t b = *reinterpret_cast<const u32x4_t*>(ptr + 16);
#pragma unroll
        for (int x = 0; x < 4; ++x) { w[x] = a[x]; w[4 + x] = b[x]; }
    } else if constexpr (N == 4) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(ptr);
#pragma unroll
        for (int x = 0; x < 4; ++x) w[x] = a[x];
    } else if constexpr (N == 2) {
        const u32x2_t a = *reinterpret_cast<const u32x2_t*>(ptr);
        w[0] = a[0];
        w[1] = a[1];
    } else {
        w[0] = *reinterpret_cast<const uint32_t*>(ptr);
    }
}

// NCH chunks of N / NCH words each, chunk c at p + c * stride bytes.
template <int NCH, int N>
__device__ __forceinline__ void load_chunks(const uint8_t* ptr, int stride, uint32_t (&w)[N]) {
    constexpr int M = N / NCH;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        uint32_t t[M];
        load_words<M>(ptr + c * stride, t);
#pragma unroll
        for (int x = 0; x < M; ++x) w[c * M + x] = t[x];
    }
}

// D: head dim (64 or 128); GM: query heads handled per kv head (>= G);
// F8: the cache holds FP8 E4M3 bytes with dequantisation factors (else bf16).
template <int D, int GM, bool F8>
__global__ void __launch_bounds__(dec_waves(GM) * 64)
decode_kernel(const DecodeParams p) {
    using L = DecLds<D, GM>;
    constexpr int NW = L::NW;
    constexpr int NT = NW * 64;
    constexpr int LPR = dec_lanes_per_row(GM, F8);   // lanes sharing one cache row
    constexpr int RPW = 64 / LPR;            // rows a wave covers per load instruction
    constexpr int DPL = D / LPR;             // dims per lane (4 to 16)
    constexpr int WPL = DPL / 2;             // bf16 pairs per lane and row
    constexpr int EB = F8 ? 1 : 2;           // bytes per cache element
    constexpr int RW = DPL * EB / 4;         // raw 32-bit words per lane and row (1 to 8)
    // A lane's part of a row is NCH chunks of CE elements (at most 16 bytes
    // of cache each); the LPR lanes' chunks c are adjacent, so one load
    // instruction reads whole contiguous stretches of its rows.  Element j of
    // the lane is head dim (j / CE) * CE * LPR + CE * lr + j % CE.
    constexpr int CH = 16 / EB;              // cache elements per 16 bytes
    constexpr int NCH = DPL > CH ? DPL / CH : 1;
    constexpr int CE = DPL / NCH;
    constexpr int U = kDecRowsPerLane;       // rows per lane in one batch
    constexpr int B = U * RPW;               // list entries per batch
    static_assert(2 * B <= 64, "a pair's entries are claimed by one lane each");

    constexpr int KMAX = L::KMAX;            // list entries per thread, at most

    extern __shared__ __align__(16) uint8_t smem[];
    const int ts = p.ts;
    const int topk = p.topk;
    uint32_t* table = reinterpret_cast<uint32_t*>(smem);
    int* rows = reinterpret_cast<int*>(smem + L::rows(ts));
    int* pos = reinterpret_cast<int*>(smem + L::pos(ts, topk));
    int* next = reinterpret_cast<int*>(smem + L::next(ts, topk));
    int* btl = reinterpret_cast<int*>(smem + L::btl(ts, topk));
    float* mrg = reinterpret_cast<float*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane % LPR;               // LPR lanes share one cache row
    const int lg = lane / LPR;               // which of the wave's RPW rows
    const int unit = blockIdx.x / p.splits;  // b * Hkv + g
    const int split = blockIdx.x % p.splits;
    const int b = unit / p.Hkv;
    const int g = unit % p.Hkv;
    const int G = p.G;
    const int cs = p.cache_seqlens[b];
    const int32_t* lst = p.tok_idx + (int64_t)unit * topk;
    const int32_t* bt = p.block_table + (int64_t)b * p.max_pages;
    const int nchunk = (topk + NT - 1) / NT;     // <= KMAX
    const int r_lo = (int)(((long long)topk * split) / p.splits);
    const int r_hi = (int)(((long long)topk * (split + 1)) / p.splits);

    // This lane's dims of the G query rows (bf16 pairs), loaded first: every
    // later load is a cache row, so the streaming loop's waits count only those.
    uint32_t qw[GM][WPL];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        if (h < G) {
            const uint16_t* qr = p.q + ((int64_t)b * p.Hq + g * G + h) * D + CE * lr;
            load_chunks<NCH>(reinterpret_cast<const uint8_t*>(qr), CE * LPR * 2, qw[h]);
        } else {
#pragma unroll
            for (int x = 0; x < WPL; ++x) qw[h][x] = 0u;
        }
    }
    // scale (log2 units) including the K dequantisation factor; V's factor
    // scales the output
    float c_log2 = p.scale_log2, v_scale = 1.f;
    if constexpr (F8) {
        if (p.k_descale != nullptr) c_log2 *= p.k_descale[unit];
        if (p.v_descale != nullptr) v_scale = p.v_descale[unit];
    }

    // ---- 1. validate and translate this thread's entries e = k*NT + tid.
    // Straight-line passes (all list loads together with the block-table row,
    // then the lookups) so the loads of different entries are in flight
    // together; chunks past the list are skipped (a uniform test).
    for (int i = tid; i < ts; i += NT) table[i] = kDecEmpty;
    int key[KMAX], phys[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int e = k * NT + tid;
        key[k] = k < nchunk ? lst[e < topk ? e : topk - 1] : -1;
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
        for (int k = 0; k < KMAX; ++k)
            if (k < nchunk) phys[k] = btl[phys[k]];   // page id, checked below
    } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (k < nchunk) phys[k] = bt[phys[k]];
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (k < nchunk) {
            const int x = key[k];
            const int page = phys[k];
            const bool ok = x >= 0 && page >= 0 && page < p.num_pages;
            const int slot = x / p.page_size;
            const int e = k * NT + tid;
            if (e < topk) {
                rows[e] = ok ? page * p.page_size + (x - slot * p.page_size) : -1;
                pos[e] = ok ? x : -1;
            }
        }
    }
    if (tid == 0) *next = NW;                    // pairs 0..NW-1: each wave's first
    __syncthreads();

    // ---- 2. Claim position x in the hash table; true when this call made
    // the claim (x was not there).  A slot's position never changes once
    // claimed, so all claims of one position meet in the same slot; probes
    // are bounded by the table size (which exceeds topk).
    auto claim = [&](int x) {
        int h = dec_hash(x, ts);
        for (int probe = 0; probe < ts; ++probe) {
            const uint32_t old = atomicCAS(&table[h], kDecEmpty, (uint32_t)x);
            if (old == kDecEmpty) return true;
            if (old == (uint32_t)x) return false;
            h = h + 1 == ts ? 0 : h + 1;
        }
        return false;
    };
    // A later part of a split list first enters the positions of all earlier
    // entries, which belong to earlier parts.
    if (r_lo > 0) {
        for (int e = tid; e < r_lo; e += NT) {
            const int x = pos[e];
            if (x >= 0) (void)claim(x);
        }
        __syncthreads();
    }

    // ---- 3. The waves stream the workgroup's part of the list in pairs of
    // batches of B entries taken from a shared counter, so they finish
    // together.  LPR lanes cover one row, so a wave loads RPW rows per
    // instruction, and a batch is U such row groups of K and V.  Each wave
    // holds two batches in registers with fixed roles: while one is consumed
    // the other's loads are in flight, and a consumed batch is refilled at
    // once from the next pair.  Batches past the end load cache row 0 (the
    // same bytes for every lane, so one cache line) and are masked; this keeps
    // every iteration's loads unconditional, so each wait covers exactly the
    // batch about to be consumed.
    // (an empty cache has no row 0 to stand in for skipped entries)
    const int nbatch = p.num_pages > 0 ? (r_hi - r_lo + B - 1) / B : 0;
    const int npair = (nbatch + 1) / 2;
    const int64_t row_stride = (int64_t)p.Hkv * D * EB;   // bytes between cache rows
    const uint8_t* kbase = static_cast<const uint8_t*>(p.kc) + ((int64_t)g * D + CE * lr) * EB;
    const uint8_t* vbase = static_cast<const uint8_t*>(p.vc) + ((int64_t)g * D + CE * lr) * EB;
    struct Batch {
        uint32_t k[U][RW], v[U][RW];
        uint32_t okm;        // bit u: row group u holds a row to attend to
    };
    // The pair's entries, one per lane: each valid entry claims its position,
    // and an entry whose position is already claimed is skipped.  The wave's
    // later reads of rows[] see its own writes.
    auto claim_pair = [&](int pn) {
        const int e = r_lo + pn * 2 * B + lane;
        if (lane < 2 * B && pn < npair && e < r_hi) {
            const int x = pos[e];
            if (x >= 0 && !claim(x)) rows[e] = -1;
        }
    };
    // Entry r0 + u*RPW + lg is row group u of batch bidx; an entry outside
    // the part, invalid or repeated is skipped.
    auto entry_row = [&](int bidx, int u) {
        const int r = r_lo + bidx * B + u * RPW + lg;
        const int rc = r < r_hi ? r : r_hi - 1;
        return (bidx < nbatch && r < r_hi) ? rows[rc] : -1;
    };
    auto issue = [&](Batch& t, int bidx) {
        uint32_t okm = 0u;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = entry_row(bidx, u);
            okm |= (uint32_t)(row >= 0) << u;
            const int64_t off = (int64_t)(row >= 0 ? row : 0) * row_stride;
            load_chunks<NCH>(kbase + off, CE * LPR * EB, t.k[u]);
            load_chunks<NCH>(vbase + off, CE * LPR * EB, t.v[u]);
        }
        t.okm = okm;
    };

    float m_run[GM], l_run[GM], acc[GM][DPL];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int x = 0; x < DPL; ++x) acc[h][x] = 0.f;
    }

    // One batch into the row group's online softmax.  The running max moves
    // only when a score exceeds it by more than kDecLazyMax (log2 units), so
    // the accumulators are rarely rescaled; the probabilities stay below
    // 2^kDecLazyMax, and the final division by the row sum is unchanged.
    auto consume = [&](const Batch& t) {
        // bf16 pairs of the rows (E4M3 -> bf16 is exact)
        uint32_t kw[U][WPL], vw[U][WPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int x = 0; x < RW; ++x) {
                if constexpr (F8) {
                    kw[u][2 * x] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t.k[u][x], 1.f, false));
                    kw[u][2 * x + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t.k[u][x], 1.f, true));
                    vw[u][2 * x] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t.v[u][x], 1.f, false));
                    vw[u][2 * x + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t.v[u][x], 1.f, true));
                } else {
                    kw[u][x] = t.k[u][x];
                    vw[u][x] = t.v[u][x];
                }
            }
        }
        // raw scores q.k of the row group's rows, one per query head
        float s[U][GM];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int h = 0; h < GM; ++h) {
                float d = 0.f;
#pragma unroll
                for (int x = 0; x < WPL; ++x) d = dot2_bf16(qw[h][x], kw[u][x], d);
                s[u][h] = row_sum<LPR>(d);
            }
        }
        if (__builtin_amdgcn_ballot_w64(t.okm != (1u << U) - 1u) != 0ull) {   // skipped entries
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (((t.okm >> u) & 1u) == 0u) {
#pragma unroll
                    for (int h = 0; h < GM; ++h) s[u][h] = -INFINITY;
                }
        }
        const float c = c_log2;                  // > 0: the max commutes with the scaling
        float cand[GM];
        bool grow = false;
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            float mb = s[0][h];
#pragma unroll
            for (int u = 1; u < U; ++u) mb = fmaxf(mb, s[u][h]);
            cand[h] = mb * c;
            grow |= cand[h] > m_run[h] + kDecLazyMax;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0ull) {
#pragma unroll
            for (int h = 0; h < GM; ++h) {
                const float m_new = fmaxf(m_run[h], cand[h]);
                const float msub = m_new == -INFINITY ? 0.f : m_new;
                const float alpha = fast_exp2(m_run[h] - msub);
                m_run[h] = m_new;
                l_run[h] *= alpha;
#pragma unroll
                for (int x = 0; x < DPL; ++x) acc[h][x] *= alpha;
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
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            const float msub = m_run[h] == -INFINITY ? 0.f : m_run[h];
            float ls = 0.f;
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
            l_run[h] += ls;
        }
    };
    auto grab = [&]() {
        int t = 0;
        if (lane == 0) t = __hip_atomic_fetch_add(next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return __builtin_amdgcn_readfirstlane(t);
    };
    if (nbatch > 0) {
        Batch ta, tb;
        claim_pair(wave);
        issue(ta, 2 * wave);
        issue(tb, 2 * wave + 1);
        int pc = wave;
        while (pc < npair) {
            const int pn = grab();
            claim_pair(pn);
            consume(ta);
            issue(ta, 2 * pn);
            consume(tb);
            issue(tb, 2 * pn + 1);
            pc = pn;
        }
    }

    // ---- 4. merge the wave's row groups, then the workgroup's waves.
    // Region 0 (the hash table) is reused: every claim precedes the barrier.
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        const float m = lanes_combine<LPR, true>(m_run[h]);
        const float msub = m == -INFINITY ? 0.f : m;
        const float sc = fast_exp2(m_run[h] - msub);
        const float l = lanes_combine<LPR, false>(l_run[h] * sc);
        float* rec = mrg + (wave * GM + h) * L::kRec;
#pragma unroll
        for (int x = 0; x < DPL; ++x) {
            const float a = lanes_combine<LPR, false>(acc[h][x] * sc);
            if (lg == 0) rec[(x / CE) * CE * LPR + CE * lr + x % CE] = a;
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
