// sel_attn_bwd.hip -- backward of top-k selected block-sparse attention, gfx950.
//
// What it computes (the training use of selected attention on the FSA page):
// the gradients of sum(dO * O) for the forward of sel_attn_fwd.hip.  For a row
// (token i, q head h) with visible key set J, P_j = exp(s_j - LSE) and
//   D = sum_c dO_c O_c,  dP_j = <dO, v_j>,  dS_j = P_j (dP_j - D),
//   dq = scale * sum_j dS_j k_j,  dk_j += scale * dS_j q,  dv_j += P_j dO.
// O and LSE come from the forward; J is read exactly as the forward reads it
// (lists as sets, invalid and future ids skipped, bottom-right causal mask).
//
// Kernels, in launch order:
//   1. bwd_prep:  D of every row (16 lanes per row); clears the counters.
//   2. bwd_index (count) / bwd_scan / bwd_index (fill): for every (sequence,
//      kv head, key block), the list of query tokens that selected it (each
//      token's list read as a set) -- an inverted index, so that
//   3. bwd_dkv: a workgroup per (sequence, kv head, block) accumulates dK and
//      dV of its 64 keys in registers over the block's tokens, 32 query rows at
//      a time, and writes them (blocks nobody selected get zeros).  A block
//      many tokens selected (block 0, the local blocks) is split over several
//      workgroups whose fp32 partials are added in a workspace and converted
//      by bwd_dkv_finish.  Four
//      waves own 16 keys each.  S = Q K^T and dP = dO V^T put the query rows
//      on the MFMA M dimension, so their accumulators are directly the B
//      operands of dV^T = dO^T P and dK^T = Q^T dS (after a fixed reordering of
//      the 32 rows); dO^T and Q^T come from transposing LDS reads.
//   4. bwd_dq: query-centric like the forward: a workgroup owns T tokens of
//      one kv head (ten 16-row m-tiles, one per compute wave), builds the union of
//      their blocks and walks it block by block; S^T = K Q^T, dP^T = V dO^T,
//      dS^T, then dQ^T += K^T dS^T with K^T read by transposing LDS reads.
// The order in which a block's tokens are summed depends on atomic list
// filling, so dK / dV may differ run to run by fp32 rounding.
#include "fsa_common.h"
#include "fsa_params.h"

namespace fsa {

namespace {

constexpr int kBwdRows = 32;            // query rows per dK/dV step
constexpr int kBwdKvThreads = 256;      // 4 waves x 16 keys
constexpr int kBwdDqWaves = 10;         // m-tiles (compute waves) per dq workgroup
constexpr int kBwdDqProducers = 2;      // waves that only move K/V blocks into LDS
constexpr int kBwdDqThreads = (kBwdDqWaves + kBwdDqProducers) * 64;
constexpr int kBwdWin = 256;            // blocks per union-building window (dq)
// Ring waits of this file's kernels that gave up (see wait_ready2).
__device__ unsigned int g_bwd_wait_timeouts;

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ u32x2_t tr_read(const uint8_t* p) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}

__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    return x;
}

// sequence holding global query token t (cu_q non-decreasing)
__device__ __forceinline__ int seq_of(const int32_t* cu, int batch, int64_t t) {
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

struct SeqBounds {
    int64_t q0, k0;
    int Sq, Sk;
};

__device__ __forceinline__ SeqBounds bounds(const SelBwdParams& p, int b) {
    int64_t q0 = p.cu_q[b], q1 = p.cu_q[b + 1];
    int64_t k0 = p.cu_k[b], k1 = p.cu_k[b + 1];
    q1 = q1 < p.total_q ? q1 : p.total_q;
    q0 = q0 < 0 ? 0 : (q0 < q1 ? q0 : q1);
    k1 = k1 < p.total_k ? k1 : p.total_k;
    k0 = k0 < 0 ? 0 : (k0 < k1 ? k0 : k1);
    return SeqBounds{q0, k0, (int)(q1 - q0), (int)(k1 - k0)};
}

// base of the token lists of (sequence b, kv head g)
__device__ __forceinline__ int64_t toks_base(const SelBwdParams& p, const SeqBounds& sb, int g) {
    return (sb.q0 * p.Hkv + (int64_t)g * sb.Sq) * p.topk;
}

}  // namespace

// ---- 1. D = rowsum(dO * O) per row, stored [Hq][total_q]; clears the counters
template <int D>
__global__ void __launch_bounds__(256) bwd_prep_kernel(const SelBwdParams p) {
    constexpr int DPL = D / 16;
    const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
    const int64_t nrows = p.total_q * p.Hq;
    const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + lg;
    float acc = 0.f;
    if (row < nrows) {
        const uint16_t* o = p.o + row * D + lr * DPL;
        const uint16_t* g = p.dout + row * D + lr * DPL;
        if constexpr (DPL == 8) {
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(o);
            const u32x4_t c = *reinterpret_cast<const u32x4_t*>(g);
#pragma unroll
            for (int x = 0; x < 4; ++x)
                acc += bf16_lo(a[x]) * bf16_lo(c[x]) + bf16_hi(a[x]) * bf16_hi(c[x]);
        } else {
            const u32x2_t a = *reinterpret_cast<const u32x2_t*>(o);
            const u32x2_t c = *reinterpret_cast<const u32x2_t*>(g);
#pragma unroll
            for (int x = 0; x < 2; ++x)
                acc += bf16_lo(a[x]) * bf16_lo(c[x]) + bf16_hi(a[x]) * bf16_hi(c[x]);
        }
    }
    acc = row16_sum(acc);
    if (row < nrows && lr == 0) {
        const int64_t t = row / p.Hq;
        const int h = (int)(row - t * p.Hq);
        p.dvec[(int64_t)h * p.total_q + t] = acc;
    }
    // block counters and fill cursors (the split-block accumulators are
    // cleared by the fill pass, once the counts say which blocks split)
    const int64_t nc = (int64_t)p.batch * p.Hkv * (p.nb_max + 1);
    const int64_t nu = (int64_t)p.batch * p.Hkv * p.nb_max;
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < nc; x += (int64_t)gridDim.x * 256) {
        p.counts[x] = 0;
        if (x < nu) p.cursor[x] = 0;
    }
}

// ---- 2. inverted index: token lists per (sequence, kv head, block)
// A workgroup takes kIdxChunk consecutive tokens of one (sequence, kv head),
// one list per thread.  An id counts if it is in range, causally visible and
// the first occurrence in its list.  Per window of kIdxWin blocks the
// workgroup first histograms its ids in LDS; the count pass then adds each
// bin to the global count once, and the fill pass reserves a range per bin
// with one global atomic and places the tokens through LDS cursors.  (The
// busiest blocks -- block 0 and the local blocks -- would otherwise serialize
// thousands of same-address global atomics.)
constexpr int kIdxChunk = 256;
constexpr int kIdxWin = 8192;
constexpr int kIdxRegs = 16;

template <bool FILL, int D>
__global__ void __launch_bounds__(kIdxChunk) bwd_index_kernel(const SelBwdParams p) {
    __shared__ int hist[kIdxWin];
    const int nchunk = p.nchunk_q;
    const int chunk = blockIdx.x % nchunk;
    const int unit = blockIdx.x / nchunk;               // b * Hkv + g
    const int g = unit % p.Hkv, b = unit / p.Hkv;
    const SeqBounds sb = bounds(p, b);
    if constexpr (FILL) {
        // Clear the fp32 accumulators of the blocks that the dK/dV pass
        // splits over several workgroups (it adds their partials there); the
        // other blocks are written directly and need none.  The counts are
        // final (the scan ran); block blk of the unit is this workgroup's when
        // blk = chunk (mod nchunk).
        const int32_t* cs = p.counts + (int64_t)unit * (p.nb_max + 1);
        int nb = (sb.Sk + kBlockKeys - 1) / kBlockKeys;
        nb = nb < p.nb_max ? nb : p.nb_max;
        const int tpc = kBwdRows / p.G;
        for (int blk = chunk; blk < nb; blk += nchunk) {
            const int nsteps = (cs[blk + 1] - cs[blk] + tpc - 1) / tpc;
            if (nsteps <= p.part_steps) continue;
            const int nkeys = sb.Sk - blk * kBlockKeys < kBlockKeys ? sb.Sk - blk * kBlockKeys : kBlockKeys;
            for (int x = threadIdx.x; x < nkeys * (D / 2); x += kIdxChunk) {
                const int key = x / (D / 2), c = x - key * (D / 2);   // 16-byte chunks of the dK and dV sums
                const int64_t krow = (sb.k0 + blk * kBlockKeys + key) * p.Hkv + g;
                reinterpret_cast<f32x4_t*>(p.kv_acc + krow * 2 * D)[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
    const int i0 = chunk * kIdxChunk;
    if (i0 >= sb.Sq) return;
    const int i = i0 + (int)threadIdx.x;                // this thread's token (in the sequence)
    const bool tok_ok = i < sb.Sq;
    const int off = sb.Sk - sb.Sq;
    int nblk = (sb.Sk + kBlockKeys - 1) / kBlockKeys;
    nblk = nblk < p.nb_max ? nblk : p.nb_max;          // (max_seqlen_k bounds every S_k)
    const int32_t* lst = p.blk_idx + ((sb.q0 + (tok_ok ? i : 0)) * p.Hkv + g) * (int64_t)p.topk;
    int32_t* cnt = p.counts + (int64_t)unit * (p.nb_max + 1);
    int32_t* cur = p.cursor + (int64_t)unit * p.nb_max;
    const int64_t tbase = toks_base(p, sb, g);
    // Lists of up to kIdxRegs entries are read once (16-byte loads) and
    // filtered in registers; longer ones entry by entry from memory.
    const bool in_regs = p.topk <= kIdxRegs && (p.topk & 3) == 0 && ((uintptr_t)p.blk_idx & 15) == 0;
    int ids[kIdxRegs];
    if (in_regs) {
#pragma unroll
        for (int e = 0; e < kIdxRegs; e += 4) {
            int4 v = make_int4(-1, -1, -1, -1);
            if (tok_ok && e < p.topk) v = *reinterpret_cast<const int4*>(lst + e);
            ids[e] = v.x; ids[e + 1] = v.y; ids[e + 2] = v.z; ids[e + 3] = v.w;
        }
#pragma unroll
        for (int e = 0; e < kIdxRegs; ++e) {
            int id = ids[e];
            bool ok = id >= 0 && id < nblk && !(p.causal && (long long)id * kBlockKeys > (long long)i + off);
#pragma unroll
            for (int e2 = 0; e2 < e; ++e2) ok = ok && ids[e2] != id;
            ids[e] = ok ? id : -1;      // (the first copy of an id is kept iff it is valid)
        }
    }
    // an entry's id if it counts, else -1
    auto entry = [&](int e) -> int {
        const int id = lst[e];
        if (id < 0 || id >= nblk) return -1;
        if (p.causal && (long long)id * kBlockKeys > (long long)i + off) return -1;
        for (int e2 = 0; e2 < e; ++e2)
            if (lst[e2] == id) return -1;
        return id;
    };
    // f(id) for every id of this thread's list that counts
    auto each = [&](auto f) {
        if (!tok_ok) return;
        if (in_regs) {
#pragma unroll
            for (int e = 0; e < kIdxRegs; ++e)
                if (ids[e] >= 0) f(ids[e]);
        } else {
            for (int e = 0; e < p.topk; ++e) {
                const int id = entry(e);
                if (id >= 0) f(id);
            }
        }
    };
    for (int w0 = 0; w0 < nblk; w0 += kIdxWin) {
        const int wn = (nblk - w0) < kIdxWin ? (nblk - w0) : kIdxWin;
        for (int x = threadIdx.x; x < wn; x += kIdxChunk) hist[x] = 0;
        __syncthreads();
        each([&](int id) {
            if (id >= w0 && id < w0 + wn) atomicAdd(&hist[id - w0], 1);
        });
        __syncthreads();
        for (int x = threadIdx.x; x < wn; x += kIdxChunk) {
            const int h = hist[x];
            if constexpr (!FILL) {
                if (h > 0) atomicAdd(&cnt[w0 + x], h);
            } else {
                hist[x] = h > 0 ? cnt[w0 + x] + atomicAdd(&cur[w0 + x], h) : 0;   // this chunk's range
            }
        }
        if constexpr (FILL) {
            __syncthreads();
            each([&](int id) {
                if (id >= w0 && id < w0 + wn) p.toks[tbase + atomicAdd(&hist[id - w0], 1)] = i;
            });
        }
        __syncthreads();
    }
}

// exclusive scan of the counts of one (sequence, kv head): counts -> offsets
__global__ void __launch_bounds__(256) bwd_scan_kernel(const SelBwdParams p) {
    __shared__ int wsum[4];
    const int unit = blockIdx.x;
    int32_t* c = p.counts + (int64_t)unit * (p.nb_max + 1);
    const int n = p.nb_max + 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int carry = 0;
    for (int base = 0; base < n; base += 256) {
        const int x = base + (int)threadIdx.x;
        const int v = x < n ? c[x] : 0;
        int incl = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int wb = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            wb += w < wave ? wsum[w] : 0;
            tot += wsum[w];
        }
        if (x < n) c[x] = carry + wb + incl - v;
        carry += tot;
        __syncthreads();
    }
}

// ---- 3. dK, dV of one key block
// Staging buffer of one step (two alternate): the 32 rows of Q and of dO in
// the fragment-permuted layout -- 16-byte chunk c of row r in fragment
// (r/16)*DT + c/2 at byte (4(r%16) + 2(c%2))*8 -- so that a plain 16-byte read
// gives the A operand of S = Q K^T (dP = dO V^T) and a transposing 8-byte read
// the A operand of dK^T = Q^T dS (dV^T = dO^T P).  Fragments sit kFrag = 544
// bytes apart (512 + 32 of padding) so that the 16 chunks of one row, written
// by 16 adjacent lanes, land in 16 different bank groups.
template <int D>
struct KvLds {
    static constexpr int DT = D / 16;
    static constexpr int kFrag = 544;
    static constexpr int kPart = 2 * DT * kFrag;                  // 32 rows x D
    static constexpr int q = 0;
    static constexpr int o = q + kPart;
    static constexpr int rowinfo = o + kPart;                     // f32x4 per row: lse2, D, last key
    static constexpr int kBuf = rowinfo + kBwdRows * 16;
    static constexpr int bytes = 2 * kBuf;
};

template <int D>
__global__ void __launch_bounds__(kBwdKvThreads) bwd_dkv_kernel(const SelBwdParams p) {
    constexpr int KS = D / 32, DT = D / 16;
    constexpr int CPR = D / 8;                                   // 16-byte chunks per row
    constexpr int NI = kBwdRows * CPR / kBwdKvThreads;           // chunks per thread per step
    static_assert(NI * kBwdKvThreads == kBwdRows * CPR && kBwdKvThreads % CPR == 0, "row staging");
    using L = KvLds<D>;
    __shared__ __align__(16) uint8_t smem[L::bytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // workgroup order: block-major (the early blocks, which causal lists pick
    // most, start first), then part, then (sequence, kv head) innermost, so
    // that the busy workgroups of a block spread over the XCDs while each
    // (sequence, kv head) keeps to one XCD's L2 when their count is a
    // multiple of 8
    const int nunits = p.batch * p.Hkv;
    const int unit = blockIdx.x % nunits;                // b * Hkv + g
    const int part = (blockIdx.x / nunits) % p.nparts;
    const int blk = blockIdx.x / nunits / p.nparts;
    const int g = unit % p.Hkv, b = unit / p.Hkv;
    const SeqBounds sb = bounds(p, b);
    const int nblk = (sb.Sk + kBlockKeys - 1) / kBlockKeys;
    if (blk >= nblk) return;                          // (blk < nb_max by the grid)
    const int off = sb.Sk - sb.Sq;
    const int G = p.G;
    const int tpc = kBwdRows / G;                     // tokens per step (G <= 32)
    const int rows_used = tpc * G;
    const int32_t* cnt = p.counts + (int64_t)unit * (p.nb_max + 1);
    const int tb = cnt[blk], ntk_all = cnt[blk + 1] - tb;
    // a block selected by many tokens is split over workgroups (parts) whose
    // fp32 partial sums meet in kv_acc; a one-part block writes bf16 directly
    const int nsteps = (ntk_all + tpc - 1) / tpc;
    const bool split = nsteps > p.part_steps;
    const int s_lo = part * p.part_steps;
    if (part > 0 && s_lo >= nsteps) return;
    const int s_hi = nsteps < s_lo + p.part_steps ? nsteps : s_lo + p.part_steps;
    const int32_t* tl = p.toks + toks_base(p, sb, g) + tb;
    const int c_lo = s_lo * tpc;
    const int ntk = s_hi * tpc < ntk_all ? s_hi * tpc : ntk_all;   // tokens [c_lo, ntk)

    // this wave's 16 keys: K and V as B operands (lane: key key0 + lr, 8 dims)
    const int key0 = wave * 16;
    const int kabs = blk * kBlockKeys + key0 + lr;   // key position in the sequence
    const bool key_ok = kabs < sb.Sk;
    u32x4_t kf[KS], vf[KS];
    {
        const int64_t krow = ((sb.k0 + (key_ok ? kabs : 0)) * p.Hkv + g) * (int64_t)D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            kf[s] = key_ok ? *reinterpret_cast<const u32x4_t*>(p.k + krow + s * 32 + lg * 8) : u32x4_t{0u, 0u, 0u, 0u};
            vf[s] = key_ok ? *reinterpret_cast<const u32x4_t*>(p.v + krow + s * 32 + lg * 8) : u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    f32x4_t adk[DT], adv[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        adk[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        adv[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const float c2 = p.scale_log2;

    // Rows of a step are gathered one step ahead into registers (and their
    // token ids two steps ahead), so the gathers overlap the MFMA work.  The
    // loads are unconditional (rows past the end read a real row and are
    // zeroed when staged), so waiting for one step never waits for the next.
    // This thread stages chunk column cc of rows (tid + 256 k) / CPR; threads
    // below kBwdRows also stage the row data of row tid.
    const int cc = tid % CPR;
    const int ri_row = tid % kBwdRows;
    int tk[NI], tki = 0;            // token ids of the step fetched next
    int tok_ok = 0, row_ok = 0;     // bit k: chunk k is a real row, bit NI: row data
    u32x4_t qv[NI], ov[NI];
    float lse_r = 0.f, dv_r = 0.f;
    int cpos = 0;
    auto fetch_tok = [&](int c0) {
        int m = 0;
#pragma unroll
        for (int k = 0; k < NI; ++k) {
            const int r = (tid + k * kBwdKvThreads) / CPR, ti = c0 + r / G;
            const bool ok = r < rows_used && ti < ntk;
            tk[k] = tl[ok ? ti : ntk - 1];
            m |= (int)ok << k;
        }
        const int ti = c0 + ri_row / G;
        const bool ok = ri_row < rows_used && ti < ntk;
        tki = tl[ok ? ti : ntk - 1];
        tok_ok = m | ((int)ok << NI);
    };
    auto fetch_rows = [&]() {
#pragma unroll
        for (int k = 0; k < NI; ++k) {
            const int r = (tid + k * kBwdKvThreads) / CPR;
            const int64_t rowo = ((sb.q0 + tk[k]) * p.Hq + g * G + (r % G)) * (int64_t)D + cc * 8;
            qv[k] = *reinterpret_cast<const u32x4_t*>(p.q + rowo);
            ov[k] = *reinterpret_cast<const u32x4_t*>(p.dout + rowo);
        }
        const int64_t t = sb.q0 + tki;
        const int64_t h = g * G + (ri_row % G);
        lse_r = p.lse[h * p.total_q + t];
        dv_r = p.dvec[h * p.total_q + t];
        cpos = p.causal ? tki + off : 0x7fffffff;
        row_ok = tok_ok;
    };
    auto stage = [&](int buf) {                            // registers -> staging buffer buf
        uint8_t* sb_ = smem + buf * L::kBuf;
#pragma unroll
        for (int k = 0; k < NI; ++k) {
            const int r = (tid + k * kBwdKvThreads) / CPR;
            const bool ok = (row_ok >> k) & 1;
            const u32x4_t z = {0u, 0u, 0u, 0u};
            const int fo = ((r / 16) * DT + cc / 2) * L::kFrag + (4 * (r % 16) + 2 * (cc % 2)) * 8;
            *reinterpret_cast<u32x4_t*>(sb_ + L::q + fo) = ok ? qv[k] : z;
            *reinterpret_cast<u32x4_t*>(sb_ + L::o + fo) = ok ? ov[k] : z;
        }
        if (tid < kBwdRows) {
            // rows that are padding get lse2 = +inf (so P = 0) and no key limit
            const bool ok = (row_ok >> NI) & 1;
            const f32x4_t info = ok ? f32x4_t{lse_r * kLog2e, dv_r, __int_as_float(cpos), 0.f}
                                    : f32x4_t{INFINITY, 0.f, __int_as_float(0x7fffffff), 0.f};
            *reinterpret_cast<f32x4_t*>(sb_ + L::rowinfo + tid * 16) = info;
        }
    };

    // Two staging buffers: while step i is computed from buffer i&1, the rows
    // of step i+1 (gathered during step i-1) are staged into the other one,
    // so one barrier per step suffices.
    const int blk_last = blk * kBlockKeys + kBlockKeys - 1;   // last key of the block
    const bool partial = blk_last >= sb.Sk;
    if (c_lo < ntk) {                 // (ntk >= 1 below: clamped ids stay in the list)
        fetch_tok(c_lo);
        fetch_rows();
        fetch_tok(c_lo + tpc);
        stage(0);
        fetch_rows();
        fetch_tok(c_lo + 2 * tpc);
        lds_barrier();
    }
    for (int c0 = c_lo, it = 0; c0 < ntk; c0 += tpc, ++it) {
        const uint8_t* cb = smem + (it & 1) * L::kBuf;
        // row data of rows 16rt + 4lg + i
        f32x4_t ri[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ri[rt][i] = *reinterpret_cast<const f32x4_t*>(cb + L::rowinfo + (16 * rt + 4 * lg + i) * 16);
        // S = Q K^T and dP - D = dO V^T - D for rows 0-15 / 16-31 and this
        // wave's keys (the accumulator of dP starts at -D)
        f32x4_t st[2], dp[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            st[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dp[rt] = f32x4_t{-ri[rt][0][1], -ri[rt][1][1], -ri[rt][2][1], -ri[rt][3][1]};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                // row 16rt + lr, chunk 4s + lg
                const int a = (rt * DT + 2 * s + (lg >> 1)) * L::kFrag + lr * 32 + (lg & 1) * 16;
                const u32x4_t qa = *reinterpret_cast<const u32x4_t*>(cb + L::q + a);
                const u32x4_t oa = *reinterpret_cast<const u32x4_t*>(cb + L::o + a);
                st[rt] = mfma_16x16x32(qa, kf[s], st[rt]);
                dp[rt] = mfma_16x16x32(oa, vf[s], dp[rt]);
            }
        }
        // P and dS (lane: rows 16rt + 4lg + i, key kabs); per-key masks only
        // where a row's last visible key falls inside the block
        bool cut = false;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) cut = cut || __float_as_int(ri[rt][i][2]) < blk_last;
        const bool need_mask = partial || __builtin_amdgcn_ballot_w64(cut) != 0ull;
        float pv[2][4], dsv[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pr = fast_exp2(fmaf(st[rt][i], c2, -ri[rt][i][0]));
                pv[rt][i] = pr;
                dsv[rt][i] = pr * dp[rt][i];
            }
        }
        if (need_mask) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!key_ok || kabs > __float_as_int(ri[rt][i][2])) {
                        pv[rt][i] = 0.f;
                        dsv[rt][i] = 0.f;
                    }
        }
        const u32x4_t pB = {pack_bf16x2(pv[0][0], pv[0][1]), pack_bf16x2(pv[0][2], pv[0][3]),
                            pack_bf16x2(pv[1][0], pv[1][1]), pack_bf16x2(pv[1][2], pv[1][3])};
        const u32x4_t dB = {pack_bf16x2(dsv[0][0], dsv[0][1]), pack_bf16x2(dsv[0][2], dsv[0][3]),
                            pack_bf16x2(dsv[1][0], dsv[1][1]), pack_bf16x2(dsv[1][2], dsv[1][3])};
        // dV^T += dO^T P, dK^T += Q^T dS  (A operands by transposing reads)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const u32x2_t olo = tr_read(cb + L::o + dt * L::kFrag + lane * 8);
            const u32x2_t ohi = tr_read(cb + L::o + (DT + dt) * L::kFrag + lane * 8);
            const u32x2_t qlo = tr_read(cb + L::q + dt * L::kFrag + lane * 8);
            const u32x2_t qhi = tr_read(cb + L::q + (DT + dt) * L::kFrag + lane * 8);
            adv[dt] = mfma_16x16x32(u32x4_t{olo[0], olo[1], ohi[0], ohi[1]}, pB, adv[dt]);
            adk[dt] = mfma_16x16x32(u32x4_t{qlo[0], qlo[1], qhi[0], qhi[1]}, dB, adk[dt]);
        }
        stage((it + 1) & 1);          // the next step (zeros past the end)
        fetch_rows();                 // gathers for the step after it
        fetch_tok(c0 + 3 * tpc);
        lds_barrier();
    }

    // lane: key kabs, dims 16dt + 4lg .. +4
    if (!split) {
        if (key_ok) {
            const int64_t row = ((sb.k0 + kabs) * p.Hkv + g) * (int64_t)D + lg * 4;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const f32x4_t a = adk[dt] * p.scale;
                const f32x4_t c = adv[dt];
                *reinterpret_cast<u32x2_t*>(p.dk + row + dt * 16) =
                    u32x2_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
                *reinterpret_cast<u32x2_t*>(p.dv + row + dt * 16) =
                    u32x2_t{pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])};
            }
        }
        return;
    }
    // split block: the partial dK (scaled), then dV, goes through LDS as
    // [key][dim] fp32 so that each atomic wave instruction covers 64
    // consecutive floats of one key row
    float* sacc = reinterpret_cast<float*>(smem);
    constexpr int AS = D + 4;                      // padded fp32 row
    static_assert(kBlockKeys * AS * 4 <= L::bytes, "partials fit the staging area");
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if (half) lds_barrier();
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<f32x4_t*>(sacc + (key0 + lr) * AS + dt * 16 + lg * 4) = half ? adv[dt] : adk[dt] * p.scale;
        lds_barrier();
        for (int x = tid; x < kBlockKeys * D; x += kBwdKvThreads) {
            const int key = x / D, d = x - key * D;
            const int ka = blk * kBlockKeys + key;
            if (ka < sb.Sk)
                atomicAdd(p.kv_acc + ((sb.k0 + ka) * p.Hkv + g) * 2 * D + half * D + d, sacc[key * AS + d]);
        }
    }
}

// dK, dV of the split blocks: fp32 sums -> bf16 (one workgroup per block)
template <int D>
__global__ void __launch_bounds__(256) bwd_dkv_finish_kernel(const SelBwdParams p) {
    const int blk = blockIdx.x % p.nb_max;
    const int unit = blockIdx.x / p.nb_max;
    const int g = unit % p.Hkv, b = unit / p.Hkv;
    const SeqBounds sb = bounds(p, b);
    const int nblk = (sb.Sk + kBlockKeys - 1) / kBlockKeys;
    if (blk >= nblk) return;
    const int tpc = kBwdRows / p.G;
    const int32_t* cnt = p.counts + (int64_t)unit * (p.nb_max + 1);
    const int nsteps = (cnt[blk + 1] - cnt[blk] + tpc - 1) / tpc;
    if (nsteps <= p.part_steps) return;               // written directly
    for (int x = threadIdx.x; x < kBlockKeys * D / 4; x += 256) {
        const int key = x / (D / 4), c = (x - key * (D / 4)) * 4;
        const int kabs = blk * kBlockKeys + key;
        if (kabs >= sb.Sk) continue;
        const int64_t krow = (sb.k0 + kabs) * p.Hkv + g;
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p.kv_acc + krow * 2 * D + c);
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(p.kv_acc + krow * 2 * D + D + c);
        *reinterpret_cast<u32x2_t*>(p.dk + krow * D + c) = u32x2_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
        *reinterpret_cast<u32x2_t*>(p.dv + krow * D + c) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
}

// ---- 4. dQ: tiles of T tokens of one kv head, one m-tile of 16 rows per wave
// A block's K and V sit in a ring slot in the fragment-permuted row layout:
// 16-byte chunk c of key row r at ((r/16)*DT + c/2)*512 + (4(r%16) + 2(c%2))*8,
// so that a plain 16-byte read gives the A operand of S^T = K Q^T (and of
// dP^T = V dO^T), and a transposing 8-byte read gives the A operand of
// dQ^T = K^T dS^T; each 1 KiB of the slot is one direct-to-LDS load.
template <int D>
struct DqLds {
    static constexpr int KS = D / 32, DT = D / 16;
    static constexpr int kPart = kBlockKeys * D * 2;          // K or V of one block
    static constexpr int kSlot = 2 * kPart;                   // K then V
    __host__ __device__ static int masks(int ring) { return ring * kSlot; }           // u64 [kBwdWin]
    __host__ __device__ static int umask(int ring) { return masks(ring) + kBwdWin * 8; }  // u64 [kBwdWin]
    __host__ __device__ static int ulist(int ring) { return umask(ring) + kBwdWin * 8; }  // i32 [kBwdWin]
    __host__ __device__ static int ncnt(int ring) { return ulist(ring) + kBwdWin * 4; }   // i32 [kBwdWin]
    __host__ __device__ static int count(int ring) { return ncnt(ring) + kBwdWin * 4; }   // i32, then the abort word
    __host__ __device__ static int ready(int ring) { return count(ring) + 16; }           // u32 [4][producers]
    __host__ __device__ static int done(int ring) { return ready(ring) + 4 * kBwdDqProducers * 4; }  // u32 [4]
    __host__ __device__ static int ent(int ring) { return done(ring) + 16; }              // i32 [T * topk]
    __host__ __device__ static size_t bytes(int T, int topk, int ring) {
        return (size_t)ent(ring) + (size_t)T * topk * 4;
    }
};

template <int D>
__global__ void __launch_bounds__(kBwdDqThreads) bwd_dq_kernel(const SelBwdParams p) {
    constexpr int KS = D / 32, DT = D / 16;
    using L = DqLds<D>;
    constexpr int NIK = L::kPart / 1024;            // 1 KiB DMA pieces per part
    constexpr int PPW = 2 * NIK / kBwdDqProducers;  // pieces per producer wave per block
    static_assert(PPW * kBwdDqProducers == 2 * NIK && 2 * PPW < 64, "DMA split");
    extern __shared__ __align__(16) uint8_t smem[];
    const int ring = p.ring;
    unsigned long long* s_masks = reinterpret_cast<unsigned long long*>(smem + L::masks(ring));
    unsigned long long* s_umask = reinterpret_cast<unsigned long long*>(smem + L::umask(ring));
    int* s_ulist = reinterpret_cast<int*>(smem + L::ulist(ring));
    int* s_ncnt = reinterpret_cast<int*>(smem + L::ncnt(ring));
    int* s_count = reinterpret_cast<int*>(smem + L::count(ring));
    uint32_t* s_abort = reinterpret_cast<uint32_t*>(smem + L::count(ring) + 4);
    uint32_t* s_ready = reinterpret_cast<uint32_t*>(smem + L::ready(ring));
    uint32_t* s_done = reinterpret_cast<uint32_t*>(smem + L::done(ring));
    int* s_ent = reinterpret_cast<int*>(smem + L::ent(ring));

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    if (tid < 4 * (kBwdDqProducers + 1)) s_ready[tid] = 0u;   // s_ready and s_done
    int poll_limit = p.spin_limit;              // this wave's bound on a ring wait (drops after a give-up)
    if (tid == 0) s_abort[0] = 0u;             // raised by a wave whose wait gave up

    int w = xcd_remap(blockIdx.x, (int)gridDim.x);
    const int j = p.tiles_per_seq - 1 - (w % p.tiles_per_seq);
    w /= p.tiles_per_seq;
    const int g = w % p.Hkv, b = w / p.Hkv;
    const SeqBounds sb = bounds(p, b);
    const int tok0 = j * p.T;
    if (tok0 >= sb.Sq) return;
    const int ntok = (sb.Sq - tok0) < p.T ? (sb.Sq - tok0) : p.T;
    const int off = sb.Sk - sb.Sq;
    const int nblk = (sb.Sk + kBlockKeys - 1) / kBlockKeys;
    int nb_range = nblk;
    if (p.causal) {
        const long long last = (long long)tok0 + ntok - 1 + off;
        nb_range = last < 0 ? 0 : (int)(last / kBlockKeys + 1 < nblk ? last / kBlockKeys + 1 : nblk);
    }
    const int topk = p.topk, G = p.G;

    // the tile's lists -> LDS (invalid and future ids dropped)
    const int nent = ntok * topk;
    for (int e = tid; e < nent; e += kBwdDqThreads) {
        const int t_l = e / topk;
        const int id = p.blk_idx[((sb.q0 + tok0 + t_l) * p.Hkv + g) * (int64_t)topk + (e - t_l * topk)];
        bool ok = id >= 0 && id < nb_range;
        if (ok && p.causal) ok = (long long)id * kBlockKeys <= (long long)tok0 + t_l + off;
        s_ent[e] = ok ? id : -1;
    }

    // this wave's m-tile: row = wave*16 + lr -> (token t_l, head hh)
    const int mt = wave;
    const int row = mt * 16 + lr;
    const int t_l = row / G, hh = row - t_l * G;
    const bool valid = mt < p.mtiles && t_l < ntok;
    const int64_t tq = sb.q0 + tok0 + t_l;
    const int head = g * G + hh;
    u32x4_t qf[KS], of[KS];
    float lse2 = INFINITY, dval = 0.f;
    {
        const uint16_t* qr = p.q + (tq * p.Hq + head) * (int64_t)D;
        const uint16_t* orr = p.dout + (tq * p.Hq + head) * (int64_t)D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qf[s] = valid ? *reinterpret_cast<const u32x4_t*>(qr + s * 32 + lg * 8) : u32x4_t{0u, 0u, 0u, 0u};
            of[s] = valid ? *reinterpret_cast<const u32x4_t*>(orr + s * 32 + lg * 8) : u32x4_t{0u, 0u, 0u, 0u};
        }
        if (valid) {
            lse2 = p.lse[(int64_t)head * p.total_q + tq] * kLog2e;
            dval = p.dvec[(int64_t)head * p.total_q + tq];
        }
    }
    // last visible key of the row, and its minimum over the m-tile's rows:
    // blocks that end at or before it need no per-key mask
    const int row_lim = p.causal ? (tok0 + t_l + off < sb.Sk - 1 ? tok0 + t_l + off : sb.Sk - 1) : sb.Sk - 1;
    int lo_lim;
    {
        int lo = valid ? row_lim : 0x7fffffff;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_xor(lo, o);
            lo = y < lo ? y : lo;
        }
        lo_lim = __builtin_amdgcn_readfirstlane(lo);
    }
    const int row_tok = valid ? t_l : 64;
    unsigned long long mk = 0ull;
    if (mt < p.mtiles) {
        const int t_first = (mt * 16) / G;
        int t_last = (mt * 16 + 15) / G;
        t_last = t_last < ntok - 1 ? t_last : ntok - 1;
        for (int x = t_first; x <= t_last; ++x) mk |= 1ull << x;
    }
    const unsigned long long mt_tok = uniform_u64(mk);
    f32x4_t acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int64_t row_bytes = (int64_t)p.Hkv * D * 2;
    const uint8_t* kseq = reinterpret_cast<const uint8_t*>(p.k + (sb.k0 * p.Hkv + g) * (int64_t)D);
    const uint8_t* vseq = reinterpret_cast<const uint8_t*>(p.v + (sb.k0 * p.Hkv + g) * (int64_t)D);
    const float c2 = p.scale_log2;
    // Producer wave pw moves pieces pw, pw + kBwdDqProducers, ... of each block.
    // This lane's 16 bytes of a 1 KiB DMA piece: piece f covers the two
    // 512-byte fragments 2f, 2f+1 -> (row group, chunk pair); lane -> (row, chunk)
    const int pw = __builtin_amdgcn_readfirstlane(wave) - kBwdDqWaves;   // >= 0 on producer waves
    int dma_off[PPW];
#pragma unroll
    for (int x = 0; x < PPW; ++x) {
        const int f = (pw + x * kBwdDqProducers) % NIK;         // piece within its part
        const int fr = 2 * f + (lane >> 5);                     // fragment
        const int fl = 2 * (lane & 31);                         // 8-byte unit within it
        const int r = 16 * (fr / DT) + fl / 4;                  // key row (fl = 4 (r%16) + 2 (c%2))
        const int c = 2 * (fr % DT) + (fl & 2) / 2;             // 16-byte chunk
        dma_off[x] = r * (int)row_bytes + c * 16;
    }
    auto issue = [&](int blk, int slot) {                       // DMA block blk -> ring slot
        const int rows = sb.Sk - blk * kBlockKeys < kBlockKeys ? sb.Sk - blk * kBlockKeys : kBlockKeys;
        const uint32_t nrec = (uint32_t)((rows - 1) * row_bytes + D * 2);
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(kseq + blk * kBlockKeys * row_bytes), 0, nrec, 0x00020000);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vseq + blk * kBlockKeys * row_bytes), 0, nrec, 0x00020000);
#pragma unroll
        for (int x = 0; x < PPW; ++x) {
            const int inst = pw + x * kBwdDqProducers;          // piece: K pieces, then V pieces
            __builtin_amdgcn_raw_ptr_buffer_load_lds(inst < NIK ? kr : vr,
                                                     (lds_void_t*)(smem + slot * L::kSlot + inst * 1024),
                                                     16, (uint32_t)dma_off[x], 0, 0, 0);
        }
    };
    auto publish = [&](int slot, uint32_t seq_plus1) {
        if (lane == 0) {
            asm volatile("ds_write_b32 %0, %1"
                         :
                         : "v"((uint32_t)(uintptr_t)(s_ready + slot * kBwdDqProducers + pw)), "v"(seq_plus1)
                         : "memory");
        }
    };
    constexpr int depth = 2;                          // blocks in flight per producer (ring >= 2)
    uint32_t seq0 = 0;                                // ring sequence number of the window's first block
    uint32_t tgt0 = 0, tgt1 = 0, tgt2 = 0, tgt3 = 0;  // producers: done counts that free each slot
    __syncthreads();

    for (int win_lo = 0; win_lo < nb_range; win_lo += kBwdWin) {
        const int win_n = (nb_range - win_lo) < kBwdWin ? (nb_range - win_lo) : kBwdWin;
        for (int x = tid; x < kBwdWin; x += kBwdDqThreads) s_masks[x] = 0ull;
        __syncthreads();
        for (int e = tid; e < nent; e += kBwdDqThreads) {
            const int id = s_ent[e];
            if (id >= win_lo && id < win_lo + win_n) atomicOr(&s_masks[id - win_lo], 1ull << (e / topk));
        }
        __syncthreads();
        if (wave == 0) {
            // m-tile `lane`'s tokens, for the need counts (per window, so
            // that nothing stays live across the ring loop)
            const unsigned long long cm_lane = mtile_token_mask(lane, G, ntok, p.mtiles);
            int n = 0;
            for (int c = 0; c < win_n; c += 64) {
                const int x = c + lane;
                const unsigned long long m = x < win_n ? s_masks[x] : 0ull;
                const unsigned long long bal = __ballot(m != 0ull);
                if (m != 0ull) {
                    const int pos = n + __popcll(bal & ((1ull << lane) - 1ull));
                    // compute waves (m-tiles) that need the block
                    const int nc = mtiles_meeting(m, cm_lane, p.mtiles);
                    s_ulist[pos] = win_lo + x;
                    s_umask[pos] = m;
                    s_ncnt[pos] = nc;
                }
                n += __popcll(bal);
            }
            if (lane == 0) s_count[0] = n;
        }
        __syncthreads();
        const int n_u = __builtin_amdgcn_readfirstlane(s_count[0]);

        // Ring protocol.  The producers copy the union's blocks in order into
        // ring slots (`depth` blocks in flight) and publish a slot by writing
        // its sequence number once its loads have landed, publishing all
        // loaded blocks before they wait for a slot to free up.  Each compute
        // wave visits only the blocks one of its tokens selected: it waits
        // for the slot, uses it and counts itself done with it; a producer
        // refills a slot once as many compute waves as the union build
        // counted for its block are done with it.  Compute waves never wait
        // for one another, so the uneven work of random selections evens out
        // over the tile.  Every wait is bounded.
        if (wave >= kBwdDqWaves) {
            int pub = 0;                                  // next block to publish
            __builtin_amdgcn_s_setprio(2);   // DMA issue wins the SIMD's arbitration
            int ul_v = 0, nc_v = 0;                       // union ids / need counts, 64 at a time
            for (int i = 0; i < n_u; ++i) {
                if ((i & 63) == 0) {
                    int x = i + lane;
                    x = x < kBwdWin - 1 ? x : kBwdWin - 1;
                    ul_v = (int)lds_load_sync(s_ulist + x);
                    nc_v = (int)lds_load_sync(s_ncnt + x);
                }
                const uint32_t seq = seq0 + (uint32_t)i;
                const int slot = (int)(seq % (uint32_t)ring);
                const uint32_t need_done = slot == 0 ? tgt0 : slot == 1 ? tgt1 : slot == 2 ? tgt2 : tgt3;
                if (lds_load_sync(s_done + slot) < need_done) {
                    wait_vmcnt<0>();
                    for (; pub < i; ++pub) {
                        const uint32_t ps = seq0 + (uint32_t)pub;
                        publish((int)(ps % (uint32_t)ring), ps + 1);
                    }
                    wait_done(s_done + slot, need_done, &g_bwd_wait_timeouts, s_abort, poll_limit, lane);
                }
                const uint32_t nc = (uint32_t)__builtin_amdgcn_readlane(nc_v, i & 63);
                tgt0 += slot == 0 ? nc : 0u;
                tgt1 += slot == 1 ? nc : 0u;
                tgt2 += slot == 2 ? nc : 0u;
                tgt3 += slot == 3 ? nc : 0u;
                issue(__builtin_amdgcn_readlane(ul_v, i & 63), slot);
                if (i - pub == depth - 1) {
                    wait_vmcnt<PPW * (depth - 1)>();
                    const uint32_t ps = seq0 + (uint32_t)pub;
                    publish((int)(ps % (uint32_t)ring), ps + 1);
                    ++pub;
                }
            }
            wait_vmcnt<0>();
            for (; pub < n_u; ++pub) {
                const uint32_t ps = seq0 + (uint32_t)pub;
                publish((int)(ps % (uint32_t)ring), ps + 1);
            }
        } else {
#pragma unroll 1
        for (int k = 0; k < kBwdWin / 64; ++k) {
          const int x = 64 * k + lane;
          const unsigned long long mx = x < n_u ? s_umask[x] : 0ull;
          unsigned long long bits = __builtin_amdgcn_ballot_w64((mx & mt_tok) != 0ull);
          while (bits != 0ull) {
            const int u = 64 * k + (int)__builtin_ctzll(bits);
            bits &= bits - 1ull;
            const uint32_t seq = seq0 + (uint32_t)u;
            const int slot = (int)(seq % (uint32_t)ring);
            const int blk = __builtin_amdgcn_readfirstlane(s_ulist[u]);
            const unsigned long long bm = uniform_u64(s_umask[u]);
            wait_ready2(s_ready + slot * kBwdDqProducers, seq + 1, &g_bwd_wait_timeouts, s_abort, poll_limit, lane);
            __builtin_amdgcn_s_setprio(1);   // a computing wave goes before polling ones
            const uint8_t* kslot = smem + slot * L::kSlot;
            const uint8_t* vslot = kslot + L::kPart;
            {
                const bool sel = row_tok < 64 && ((bm >> row_tok) & 1ull) != 0ull;
                const float msub = sel ? lse2 : INFINITY;      // unselected rows get P = 0
                // dP^T starts at -D, so the MFMA leaves dP - D
                f32x4_t st[4], dpt[4];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    dpt[kt] = f32x4_t{-dval, -dval, -dval, -dval};
                }
#pragma unroll
                for (int s = 0; s < KS; ++s) {
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt) {
                        // key row kt*16 + lr, chunk 4s + lg
                        const int a = (kt * DT + 2 * s + (lg >> 1)) * 512 + lr * 32 + (lg & 1) * 16;
                        const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(kslot + a);
                        const u32x4_t va = *reinterpret_cast<const u32x4_t*>(vslot + a);
                        st[kt] = mfma_16x16x32(ka, qf[s], st[kt]);
                        dpt[kt] = mfma_16x16x32(va, of[s], dpt[kt]);
                    }
                }
                // dS^T (lane: keys blk*64 + 16kt + 4lg + i, row lr)
                float ds[4][4];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ds[kt][i] = fast_exp2(fmaf(st[kt][i], c2, -msub)) * dpt[kt][i];
                if (blk * kBlockKeys + kBlockKeys - 1 > lo_lim) {      // diagonal or partial block
                    const int lim = row_lim - blk * kBlockKeys;
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (kt * 16 + lg * 4 + i > lim) ds[kt][i] = 0.f;
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const u32x4_t dB = {pack_bf16x2(ds[2 * ks][0], ds[2 * ks][1]),
                                        pack_bf16x2(ds[2 * ks][2], ds[2 * ks][3]),
                                        pack_bf16x2(ds[2 * ks + 1][0], ds[2 * ks + 1][1]),
                                        pack_bf16x2(ds[2 * ks + 1][2], ds[2 * ks + 1][3])};
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const uint8_t* p0 = kslot + ((2 * ks) * DT + dt) * 512 + lane * 8;
                        const u32x2_t lo = tr_read(p0);
                        const u32x2_t hi = tr_read(p0 + DT * 512);
                        acc[dt] = mfma_16x16x32(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, dB, acc[dt]);
                    }
                }
            }
            // done with the slot: its reads have completed before the count
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            if (lane == 0) __hip_atomic_fetch_add(s_done + slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        }
        }
        seq0 += (uint32_t)n_u;
        lds_barrier();   // ring and union buffers free for the next window
    }

    if (valid) {
        uint16_t* o = p.dq + (tq * p.Hq + head) * (int64_t)D + lg * 4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f32x4_t a = acc[dt] * p.scale;
            *reinterpret_cast<u32x2_t*>(o + dt * 16) = u32x2_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
        }
    }
}

hipError_t sel_attn_bwd_wait_timeouts(unsigned int* n, bool reset) {
    hipError_t e = hipMemcpyFromSymbol(n, HIP_SYMBOL(g_bwd_wait_timeouts), sizeof(unsigned int));
    if (e == hipSuccess && reset) {
        const unsigned int zero = 0u;
        e = hipMemcpyToSymbol(HIP_SYMBOL(g_bwd_wait_timeouts), &zero, sizeof(unsigned int));
    }
    return e;
}

int sel_attn_bwd_rows_per_tile() { return kBwdDqWaves * 16; }

int sel_attn_bwd_index_chunk() { return kIdxChunk; }

size_t sel_attn_bwd_dq_lds_bytes(int D, int T, int topk, int ring) {
    return D == 64 ? DqLds<64>::bytes(T, topk, ring) : DqLds<128>::bytes(T, topk, ring);
}

int sel_attn_bwd_dq_ring(int D, int T, int topk) {
    for (int ring = 4; ring >= 2; --ring)
        if (sel_attn_bwd_dq_lds_bytes(D, T, topk, ring) <= 160 * 1024) return ring;
    return 0;
}

template <int D>
static hipError_t launch_bwd_d(const SelBwdParams& p, hipStream_t stream) {
    const int64_t nrows = p.total_q * p.Hq;
    const unsigned gp = (unsigned)((nrows + 15) / 16 > 0 ? (nrows + 15) / 16 : 1);
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3(gp), dim3(256), 0, stream, p);
    const unsigned gl = (unsigned)(p.batch * p.Hkv * p.nchunk_q);
    hipLaunchKernelGGL((bwd_index_kernel<false, D>), dim3(gl), dim3(kIdxChunk), 0, stream, p);
    hipLaunchKernelGGL(bwd_scan_kernel, dim3(p.batch * p.Hkv), dim3(256), 0, stream, p);
    hipLaunchKernelGGL((bwd_index_kernel<true, D>), dim3(gl), dim3(kIdxChunk), 0, stream, p);
    hipLaunchKernelGGL(bwd_dkv_kernel<D>, dim3((unsigned)(p.batch * p.Hkv * p.nb_max * p.nparts)),
                       dim3(kBwdKvThreads), 0, stream, p);
    hipLaunchKernelGGL(bwd_dkv_finish_kernel<D>, dim3((unsigned)(p.batch * p.Hkv * p.nb_max)),
                       dim3(256), 0, stream, p);
    static std::atomic<unsigned long long> lds_set{0ull};   // devices with the LDS limit raised
    hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(&bwd_dq_kernel<D>), lds_set);
    if (e != hipSuccess) return e;
    const size_t lds = DqLds<D>::bytes(p.T, p.topk, p.ring);
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)(p.batch * p.Hkv * p.tiles_per_seq)),
                       dim3(kBwdDqThreads), lds, stream, p);
    return hipGetLastError();
}

hipError_t launch_sel_attn_bwd(const SelBwdParams& p, int D, hipStream_t stream) {
    return D == 64 ? launch_bwd_d<64>(p, stream) : launch_bwd_d<128>(p, stream);
}

}  // namespace fsa
