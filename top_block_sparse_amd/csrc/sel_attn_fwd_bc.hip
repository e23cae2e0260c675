// sel_attn_fwd_bc.hip -- selected attention forward with the loops swapped
// (block-centric schedule), gfx950.
//
// What it computes is that of sel_attn_fwd.hip (FSA page: NSA selected
// attention; flash-attention-npu page, flash_attn_varlen_func docstring:
// varlen layout, GQA mapping, bottom-right causal mask, zero rows,
// natural-log LSE): row (token t, q head h) attends to the keys of the blocks
// listed in blk_idx[t, h / G, :], read as a set.
//
// Schedule (the FSA page's loop swap: outer loop over KV blocks, inner loop
// over the queries that selected each block, then a reduction kernel).  With
// a small GQA group a token's G query rows fill a fraction of a 16-row MFMA
// tile, and per-token lists share few blocks, so the query-centric schedule
// pads every block visit.  Here:
//   1. fwd_bc_index (count), fwd_bc_scan, fwd_bc_index (fill): for every
//      (sequence, kv head, block) the list of (token, list slot) entries that
//      selected it -- each list read as a set, invalid and fully-future ids
//      skipped -- plus, per (token, kv head), the mask of list slots that
//      count.  The scan also cuts every block's entries into tasks of up to
//      kBcTileTasks dense 16-row tiles (16 / G tokens each).
//   2. fwd_bc_main: persistent workgroups of 4 waves take tasks from eight
//      queues, one per XCD segment of the task list (a workgroup drains its
//      own XCD's segment first, then helps the others).  Per task the block's
//      K stays in registers (MFMA A operands, straight from memory) and its
//      V in LDS (read back as V^T by the transposing LDS read) while each
//      wave streams its tiles: gather the 16 query rows, S^T = K Q^T, mask,
//      softmax over the block's 64 keys, O^T = V^T P^T, and write the partial
//      O (bf16, not yet divided by its row sum) with the row's log2-domain
//      max and sum.  Partials are stored in the order of the inverted index,
//      so a tile's rows are one contiguous run; the fill pass records where
//      each (token, slot) entry went.
//   3. fwd_bc_merge: per output row, the partials of the slots that count
//      are combined by logsumexp into O (bf16) and LSE; a row with no slot
//      gets O = 0 and LSE = -inf.
// Every MFMA tile is dense (up to 16 / G rounding), K/V are read once per
// task, and the cost moves to the gathered Q rows and the partial round trip.
#include "fsa_common.h"
#include "fsa_params.h"

namespace fsa {

namespace {

constexpr int kBcThreads = 256;        // 4 waves
constexpr int kBcIdxWin = 8192;        // blocks per index histogram window
constexpr int kBcSegments = 8;         // task queues (one per XCD)

struct BcSeq {
    int64_t q0, k0;
    int Sq, Sk;
};

__device__ __forceinline__ BcSeq bc_seq(const SelFwdBcParams& p, int b) {
    int64_t q0 = p.cu_q[b], q1 = p.cu_q[b + 1];
    int64_t k0 = p.cu_k[b], k1 = p.cu_k[b + 1];
    q1 = q1 < p.total_q ? q1 : p.total_q;
    q0 = q0 < 0 ? 0 : (q0 < q1 ? q0 : q1);
    k1 = k1 < p.total_k ? k1 : p.total_k;
    k0 = k0 < 0 ? 0 : (k0 < k1 ? k0 : k1);
    return BcSeq{q0, k0, (int)(q1 - q0), (int)(k1 - k0)};
}

__device__ __forceinline__ int bc_nblk(const SelFwdBcParams& p, const BcSeq& sb) {
    const int n = (sb.Sk + kBlockKeys - 1) / kBlockKeys;
    return n < p.nb_max ? n : p.nb_max;             // (max_seqlen_k bounds every S_k)
}

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Transposing LDS read: within each 16-lane group, lane j receives the 16-bit
// word at (address of lane j/4 + 4k) + 2*(j%4), k = 0..3.
__device__ __forceinline__ u32x2_t bc_read_tr16(const uint8_t* p) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}

__device__ __forceinline__ float bc_max4(float x) {
    // max over lanes l, l^16, l^32, l^48 (the four lanes holding one row)
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float bc_sum4(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace

// ---- 0. clear the counters (a kernel, not a memset, so a captured graph
// replays it like any other node)
__global__ void __launch_bounds__(256) fwd_bc_prep_kernel(const SelFwdBcParams p) {
    const int64_t nc = (int64_t)p.batch * p.Hkv * (p.nb_max + 1);
    const int64_t nu = (int64_t)p.batch * p.Hkv * p.nb_max;
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < nc; x += (int64_t)gridDim.x * 256) {
        p.counts[x] = 0;
        if (x < nu) p.cursor[x] = 0;
    }
    if (blockIdx.x == 0 && threadIdx.x < 16) p.ctr[threadIdx.x] = 0u;
    const int64_t nm = p.total_q * p.Hkv;     // lists no index workgroup reaches count nothing
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < nm; x += (int64_t)gridDim.x * 256)
        p.masks[x] = 0ull;
}

// ---- 1. inverted index.  A workgroup takes kBcIndexChunk consecutive tokens
// of one (sequence, kv head), one list per thread.  A slot counts if its id is
// in [0, ceil(S_k / 64)), (causal) its block has a key at or before the row's
// last visible key, and no earlier slot of the list holds the same id.  The
// count pass stores each list's mask of counting slots and histograms the ids
// per window of kBcIdxWin blocks in LDS, adding each bin to the global count
// once; the fill pass reserves a range per bin with one global atomic and
// places the entries through LDS cursors.
template <bool FILL, int TK>
__global__ void __launch_bounds__(kBcIndexChunk) fwd_bc_index_kernel(const SelFwdBcParams p) {
    __shared__ int hist[kBcIdxWin];
    const int chunk = blockIdx.x % p.nchunk_q;
    const int unit = blockIdx.x / p.nchunk_q;           // b * Hkv + g
    const int g = unit % p.Hkv, b = unit / p.Hkv;
    const BcSeq sb = bc_seq(p, b);
    const int i0 = chunk * kBcIndexChunk;
    if (i0 >= sb.Sq) return;
    const int i = i0 + (int)threadIdx.x;                 // this thread's token (in the sequence)
    const bool tok_ok = i < sb.Sq;
    const int64_t lrow = (sb.q0 + (tok_ok ? i : 0)) * p.Hkv + g;
    const int32_t* lst = p.blk_idx + lrow * p.topk;
    const int nblk = bc_nblk(p, sb);
    const long long last_key = (long long)i + sb.Sk - sb.Sq;     // causal limit of the row
    int32_t* cnt = p.counts + (int64_t)unit * (p.nb_max + 1);
    int32_t* cur = p.cursor + (int64_t)unit * p.nb_max;
    const int64_t ebase = (sb.q0 * p.Hkv + (int64_t)g * sb.Sq) * p.topk;

    // the list in registers (TK >= topk entries), -1 where a slot does not count
    int ids[TK];
#pragma unroll
    for (int e = 0; e < TK; ++e) {
        const int id = (tok_ok && e < p.topk) ? lst[e] : -1;
        const bool ok = id >= 0 && id < nblk && !(p.causal && (long long)id * kBlockKeys > last_key);
        ids[e] = ok ? id : -1;
    }
    unsigned long long mask = 0ull;
    if constexpr (!FILL) {
#pragma unroll
        for (int e = 0; e < TK; ++e) {
            bool ok = ids[e] >= 0;
#pragma unroll
            for (int e2 = 0; e2 < e; ++e2) ok = ok && ids[e2] != ids[e];
            mask |= ok ? (1ull << e) : 0ull;
        }
        if (tok_ok) p.masks[lrow] = mask;
    } else {
        mask = tok_ok ? p.masks[lrow] : 0ull;
    }
#pragma unroll
    for (int e = 0; e < TK; ++e)
        if (!((mask >> e) & 1ull)) ids[e] = -1;         // later copies of an id do not count
    for (int w0 = 0; w0 < nblk; w0 += kBcIdxWin) {
        const int wn = (nblk - w0) < kBcIdxWin ? (nblk - w0) : kBcIdxWin;
        for (int x = threadIdx.x; x < wn; x += kBcIndexChunk) hist[x] = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < TK; ++e)
            if (ids[e] >= w0 && ids[e] < w0 + wn) atomicAdd(&hist[ids[e] - w0], 1);
        __syncthreads();
        for (int x = threadIdx.x; x < wn; x += kBcIndexChunk) {
            const int h = hist[x];
            if constexpr (!FILL) {
                if (h > 0) atomicAdd(&cnt[w0 + x], h);
            } else {
                hist[x] = h > 0 ? cnt[w0 + x] + atomicAdd(&cur[w0 + x], h) : 0;   // this chunk's range
            }
        }
        if constexpr (FILL) {
            __syncthreads();
#pragma unroll
            for (int e = 0; e < TK; ++e)
                if (ids[e] >= w0 && ids[e] < w0 + wn) {
                    const int64_t at = ebase + atomicAdd(&hist[ids[e] - w0], 1);
                    p.ents[at] = (i << 6) | e;
                    p.pos[lrow * p.topk + e] = (int32_t)at;   // < total_q * Hkv * topk
                }
        }
        __syncthreads();
    }
}

// ---- 1b. per (sequence, kv head): counts -> exclusive offsets, then the
// unit's tasks (each block's entries cut into runs of kBcTileTasks tiles),
// appended to the task list at a range reserved with one global atomic.
__global__ void __launch_bounds__(256) fwd_bc_scan_kernel(const SelFwdBcParams p) {
    __shared__ int wsum[4];
    __shared__ int s_base;
    const int unit = blockIdx.x;
    int32_t* c = p.counts + (int64_t)unit * (p.nb_max + 1);
    const int n = p.nb_max + 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int per_task = kBcTileTasks * p.tpt;          // entries per full task
    auto tasks_of = [&](int cnt_b) { return (cnt_b + per_task - 1) / per_task; };
    // scan 1: offsets, and the unit's task total
    int carry = 0, tcarry = 0;
    for (int base = 0; base < n; base += 256) {
        const int x = base + (int)threadIdx.x;
        const int v = x < n ? c[x] : 0;
        const int tv = x < n - 1 ? tasks_of(v) : 0;
        int incl = v, tincl = tv;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            const int ty = __shfl_up(tincl, o);
            if (lane >= o) {
                incl += y;
                tincl += ty;
            }
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int wb = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            wb += w < wave ? wsum[w] : 0;
            tot += wsum[w];
        }
        __syncthreads();
        if (lane == 63) wsum[wave] = tincl;
        __syncthreads();
        int ttot = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) ttot += wsum[w];
        if (x < n) c[x] = carry + wb + incl - v;
        carry += tot;
        tcarry += ttot;
        __syncthreads();
    }
    if (threadIdx.x == 0) s_base = (int)atomicAdd(&p.ctr[0], (uint32_t)tcarry);
    __syncthreads();
    // scan 2: each block's tasks at the unit's range
    int tpos = s_base;
    for (int base = 0; base < n - 1; base += 256) {
        const int x = base + (int)threadIdx.x;
        const int cnt_b = x < n - 1 ? c[x + 1] - c[x] : 0;
        const int tv = tasks_of(cnt_b);
        int tincl = tv;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int ty = __shfl_up(tincl, o);
            if (lane >= o) tincl += ty;
        }
        if (lane == 63) wsum[wave] = tincl;
        __syncthreads();
        int twb = 0, ttot = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            twb += w < wave ? wsum[w] : 0;
            ttot += wsum[w];
        }
        const int first = tpos + twb + tincl - tv;
        for (int k = 0; k < tv; ++k)
            if (first + k < p.max_tasks)
                p.tasks[first + k] = make_int2(unit * p.nb_max + x, k * kBcTileTasks);
        tpos += ttot;
        __syncthreads();
    }
}

// ---- 2. block-centric main kernel
// LDS: V of the task's block in the transposing-read layout: fragment
// (ks, h, dt) = 512 bytes at ((2 ks + h) DT + dt) * 512; lane l's 8 bytes are
// V[32 ks + 16 h + 4 (l / 16) + (l % 16) / 4][16 dt + 4 (l % 4) .. +4].
template <int D>
__global__ void __launch_bounds__(kBcThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bc_main_kernel(const SelFwdBcParams p) {
    constexpr int KS = D / 32, DT = D / 16;
    constexpr int CPR = D / 8;                    // 16-byte chunks per key row
    constexpr int VI = kBlockKeys * CPR / kBcThreads;   // V staging loads per thread
    static_assert(VI * kBcThreads == kBlockKeys * CPR, "V staging");
    __shared__ __align__(16) uint8_t vlds[4 * DT * 512];
    __shared__ int s_ent[kBcTileTasks * 16];      // the task's list entries (tpt per tile)
    __shared__ int s_task;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int G = p.G, tpt = p.tpt;
    const float c2 = p.scale_log2;
    const int64_t ntask = (int64_t)(p.ctr[0] < (uint32_t)p.max_tasks ? p.ctr[0] : (uint32_t)p.max_tasks);
    const int home = (int)(blockIdx.x % kBcSegments);
    const int hrow = lr / G;                      // token of this lane's tile row
    const int hh = lr - hrow * G;                 // its head within the group
    const bool row_used = hrow < tpt;

    for (int si = 0; si < kBcSegments; ++si) {
        const int seg = (home + si) % kBcSegments;
        const int64_t lo = ntask * seg / kBcSegments, hi = ntask * (seg + 1) / kBcSegments;
        for (;;) {
            __syncthreads();                      // the previous task is done with vlds / s_task
            if (tid == 0) s_task = (int)atomicAdd(&p.ctr[8 + seg], 1u);
            __syncthreads();
            const int64_t it = lo + __builtin_amdgcn_readfirstlane(s_task);
            if (it >= hi) break;
            const int2 tk = p.tasks[it];
            const int unit = tk.x / p.nb_max, blk = tk.x - unit * p.nb_max;
            const int b = unit / p.Hkv, g = unit - b * p.Hkv;
            const BcSeq sb = bc_seq(p, b);
            const int off = sb.Sk - sb.Sq;
            const int32_t* cnt = p.counts + (int64_t)unit * (p.nb_max + 1);
            const int e0 = cnt[blk], nent = cnt[blk + 1] - e0;
            const int ntile = (nent + tpt - 1) / tpt;
            const int t_lo = tk.y;
            const int t_hi = ntile < t_lo + kBcTileTasks ? ntile : t_lo + kBcTileTasks;
            const int key0 = blk * kBlockKeys;
            const int last_row = sb.Sk - 1;
            // the task's entries -> LDS (read back per tile without touching the
            // vector-memory counter that orders the Q gathers)
            {
                const int32_t* ents = p.ents + (sb.q0 * p.Hkv + (int64_t)g * sb.Sq) * p.topk + e0;
                const int e_lo = t_lo * tpt;
                const int n_task = (t_hi * tpt < nent ? t_hi * tpt : nent) - e_lo;
                for (int x = tid; x < (t_hi - t_lo) * tpt; x += kBcThreads)
                    s_ent[x] = ents[e_lo + (x < n_task ? x : n_task - 1)];
            }

            // V of the block -> LDS (rows past the sequence end repeat its last row:
            // finite values that the mask gives zero weight)
#pragma unroll
            for (int x = 0; x < VI; ++x) {
                const int ci = x * kBcThreads + tid;
                const int kk = ci / CPR, c = ci - kk * CPR;
                const int krow = key0 + kk < last_row ? key0 + kk : last_row;
                const u32x4_t val = *reinterpret_cast<const u32x4_t*>(
                    p.v + ((sb.k0 + krow) * p.Hkv + g) * (int64_t)D + c * 8);
                const int ks = kk >> 5, h = (kk >> 4) & 1, q4 = (kk >> 2) & 3, r4 = kk & 3;
                const int frag = (2 * ks + h) * DT + (c >> 1);
                *reinterpret_cast<u32x4_t*>(vlds + frag * 512 + 8 * (16 * q4 + 4 * r4 + 2 * (c & 1))) = val;
            }
            // K of the block as S^T = K Q^T A operands: K[16 kt + l%16][32 s + 8 (l/16) .. +8]
            u32x4_t kf[4][KS];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const int krow = key0 + 16 * kt + lr < last_row ? key0 + 16 * kt + lr : last_row;
                const uint16_t* kr = p.k + ((sb.k0 + krow) * p.Hkv + g) * (int64_t)D + lg * 8;
#pragma unroll
                for (int s = 0; s < KS; ++s) kf[kt][s] = *reinterpret_cast<const u32x4_t*>(kr + s * 32);
            }
            __syncthreads();                      // V staged

            // the wave's tiles: t_lo + wave, + 4, ...  The loop is unrolled by NQ
            // so that each of the NQ Q buffers keeps its role: a buffer is
            // refilled for the tile NQ steps ahead right after its tile is
            // computed (rotating buffers by register moves would make every
            // move wait for the loads just issued).  Every load is
            // unconditional, at a clamped index.
            constexpr int NQ = 3;
            const int ntt = t_hi - t_lo;                     // tiles of the task
            auto entry_of = [&](int tt) -> int {             // tt: tile index within the task
                tt = tt < ntt ? tt : ntt - 1;
                return s_ent[tt * tpt + (hrow < tpt ? hrow : tpt - 1)];
            };
            const uint16_t* qbase = p.q + (sb.q0 * p.Hq + g * G + hh) * (int64_t)D + lg * 8;
            const int64_t qstride = (int64_t)p.Hq * D;       // elements between tokens
            auto load_q = [&](int ent, u32x4_t* qf) {
                const uint16_t* qr = qbase + (int64_t)(ent >> 6) * qstride;
#pragma unroll
                for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const u32x4_t*>(qr + s * 32);
            };
            // rows past the task's entries (and the unused rows of a tile when G
            // does not divide 16) write to a dummy partial row past the real ones
            const int64_t dummy_row = p.total_q * p.Hkv * p.topk * G + lr;
            // partials are stored in the order of the inverted index (entry E,
            // head hh at row E * G + hh), so a tile writes 16 consecutive rows
            const int64_t prow_base = ((sb.q0 * p.Hkv + (int64_t)g * sb.Sq) * p.topk + e0) * G;
            u32x4_t qbuf[NQ][KS];
#pragma unroll
            for (int u = 0; u < NQ; ++u) load_q(entry_of(wave + 4 * u), qbuf[u]);
            // one tile of the wave (tile index t within the task), from Q buffer u
            auto step = [&](const int u, const int t) {
                // S^T = K Q^T: lane holds S[key 16 kt + 4 lg + i][row lr]
                f32x4_t st[4];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s)
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt) st[kt] = mfma_16x16x32(kf[kt][s], qbuf[u][s], st[kt]);
                // the tile NQ steps ahead: its Q into this buffer
                load_q(entry_of(t + 4 * NQ), qbuf[u]);
                const int i_row = entry_of(t) >> 6;
                float x[16];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[kt * 4 + i] = st[kt][i];
                // keys past the row's last visible key or the sequence end
                int lim_local = sb.Sk - key0;
                if (p.causal) {
                    const int c_lim = i_row + off + 1 - key0;
                    lim_local = c_lim < lim_local ? c_lim : lim_local;
                }
                if (__builtin_amdgcn_ballot_w64(lim_local < kBlockKeys) != 0ull) {
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            x[kt * 4 + i] = kt * 16 + lg * 4 + i < lim_local ? x[kt * 4 + i] : -INFINITY;
                }
                float mx = x[0];
#pragma unroll
                for (int e = 1; e < 16; ++e) mx = fmaxf(mx, x[e]);
                mx = bc_max4(mx);
                const float mb = mx == -INFINITY ? 0.f : mx * c2;
                float ls = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    x[e] = fast_exp2(fmaf(x[e], c2, -mb));
                    ls += x[e];
                }
                const float l = bc_sum4(ls);
                u32x4_t pb[2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    pb[ks] = u32x4_t{pack_bf16x2(x[8 * ks + 0], x[8 * ks + 1]),
                                     pack_bf16x2(x[8 * ks + 2], x[8 * ks + 3]),
                                     pack_bf16x2(x[8 * ks + 4], x[8 * ks + 5]),
                                     pack_bf16x2(x[8 * ks + 6], x[8 * ks + 7])};
                // O^T = V^T P^T (V^T fragments read from LDS as the MFMAs go):
                // lane holds O[row lr][16 dt + 4 lg + i], not yet divided by l
                f32x4_t acc[DT];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const uint8_t* p0 = vlds + ((2 * ks) * DT + dt) * 512 + lane * 8;
                        const u32x2_t a = bc_read_tr16(p0);
                        const u32x2_t c = bc_read_tr16(p0 + DT * 512);
                        acc[dt] = mfma_16x16x32(u32x4_t{a[0], a[1], c[0], c[1]}, pb[ks],
                                                ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[dt]);
                    }
                // partial row layout: 16 bytes k of lane group lg at element
                // 32 k + 8 lg hold d = 32 k + 4 lg + (0..3) and 32 k + 16 + 4 lg + (0..3);
                // the four lanes of a row all store its (m, l) (the same values)
                const int e_in = (t_lo + t) * tpt + hrow;          // entry within the block's list
                const bool live = row_used && e_in < nent;
                const int64_t prow = live ? prow_base + (int64_t)e_in * G + hh : dummy_row;
                uint16_t* o = p.part_o + prow * D + lg * 8;
#pragma unroll
                for (int k2 = 0; k2 < DT / 2; ++k2)
                    *reinterpret_cast<u32x4_t*>(o + k2 * 32) =
                        u32x4_t{pack_bf16x2(acc[2 * k2][0], acc[2 * k2][1]),
                                pack_bf16x2(acc[2 * k2][2], acc[2 * k2][3]),
                                pack_bf16x2(acc[2 * k2 + 1][0], acc[2 * k2 + 1][1]),
                                pack_bf16x2(acc[2 * k2 + 1][2], acc[2 * k2 + 1][3])};
                *reinterpret_cast<f32x2_t*>(p.part_ml + prow * 2) = f32x2_t{mb, l};
            };
            const int nt_w = wave < ntt ? (ntt - wave + 3) / 4 : 0;     // this wave's tiles
            const int nround = nt_w / NQ, rem = nt_w - nround * NQ;
            for (int r = 0; r < nround; ++r) {
#pragma unroll
                for (int u = 0; u < NQ; ++u) step(u, wave + 4 * (r * NQ + u));
            }
#pragma unroll
            for (int u = 0; u < NQ - 1; ++u)
                if (u < rem) step(u, wave + 4 * (nround * NQ + u));
        }
    }
}

// ---- 3. merge the partials of every row: D / 8 lanes per row, each with the
// 16 bytes c of every partial (d = 32 (c / 4) + 4 (c % 4) + (0..3) and the same
// + 16, see the partial row layout above), four partials loaded at a time.  A
// partial is (m, l, O) with O = sum_j exp2(s_j - m) v_j over its block's keys
// and l = sum_j exp2(s_j - m) (log2 domain), so with M = max m:
// O_row = sum_b 2^(m_b - M) O_b / sum_b 2^(m_b - M) l_b and LSE = (M + log2 L) ln 2.
template <int D>
__global__ void __launch_bounds__(256) fwd_bc_merge_kernel(const SelFwdBcParams p) {
    constexpr int LPR = D / 8;                    // lanes per row
    constexpr int RPB = 256 / LPR;                // rows per workgroup
    constexpr int NB = 4;                         // partials in flight per lane
    const int c = threadIdx.x % LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;    // t * Hq + head
    if (row >= p.total_q * p.Hq) return;
    const int64_t t = row / p.Hq;
    // rows outside the sequences are not touched
    if (t < (int64_t)p.cu_q[0] || t >= (int64_t)p.cu_q[p.batch]) return;
    const int head = (int)(row - t * p.Hq);
    const int g = head / p.G, h = head - g * p.G;
    const unsigned long long mask = p.masks[t * p.Hkv + g];
    const int32_t* pos = p.pos + (t * p.Hkv + g) * p.topk;
    auto prow_of = [&](int slot) { return (int64_t)pos[slot] * p.G + h; };
    float m = -INFINITY;
    for (unsigned long long mm = mask; mm != 0ull;) {
        float v[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            v[j] = mm != 0ull ? p.part_ml[2 * prow_of(__builtin_ctzll(mm))] : -INFINITY;
            mm &= mm - 1ull;
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) m = fmaxf(m, v[j]);
    }
    float o[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) o[x] = 0.f;
    float L = 0.f;
    // (a partial always has l >= 1: its block holds a visible key, and the
    // largest score contributes 2^0)
    for (unsigned long long mm = m == -INFINITY ? 0ull : mask; mm != 0ull;) {
        f32x2_t ml[NB];
        u32x4_t v[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const bool live = mm != 0ull;
            const int64_t pr = prow_of(live ? __builtin_ctzll(mm) : __builtin_ctzll(mask));
            ml[j] = *reinterpret_cast<const f32x2_t*>(p.part_ml + 2 * pr);
            if (!live) ml[j][0] = -INFINITY;
            v[j] = *reinterpret_cast<const u32x4_t*>(p.part_o + pr * D + c * 8);
            mm &= mm - 1ull;
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const float wj = fast_exp2(ml[j][0] - m);
            L = fmaf(wj, ml[j][1], L);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                o[2 * x] = fmaf(wj, bf16_lo(v[j][x]), o[2 * x]);
                o[2 * x + 1] = fmaf(wj, bf16_hi(v[j][x]), o[2 * x + 1]);
            }
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t* out = p.out + row * D + 32 * (c / 4) + 4 * (c % 4);
    *reinterpret_cast<u32x2_t*>(out) = u32x2_t{pack_bf16x2(o[0] * inv, o[1] * inv),
                                               pack_bf16x2(o[2] * inv, o[3] * inv)};
    *reinterpret_cast<u32x2_t*>(out + 16) = u32x2_t{pack_bf16x2(o[4] * inv, o[5] * inv),
                                                    pack_bf16x2(o[6] * inv, o[7] * inv)};
    if (p.lse != nullptr && c == 0)
        p.lse[(int64_t)head * p.total_q + t] = L > 0.f ? (m + __log2f(L)) * kLn2 : -INFINITY;
}

template <int D>
static hipError_t launch_bc_t(const SelFwdBcParams& p, hipStream_t stream) {
    const int units = p.batch * p.Hkv;
    const int64_t nc = (int64_t)units * (p.nb_max + 1);
    const int64_t nm = p.total_q * p.Hkv;
    int prep_wg = (int)(((nc > nm ? nc : nm) + 255) / 256);
    prep_wg = prep_wg < 1 ? 1 : (prep_wg > 4096 ? 4096 : prep_wg);
    hipLaunchKernelGGL(fwd_bc_prep_kernel, dim3(prep_wg), dim3(256), 0, stream, p);
    const dim3 idx_grid((unsigned)(units * p.nchunk_q));
    if (p.topk <= 16) {
        hipLaunchKernelGGL((fwd_bc_index_kernel<false, 16>), idx_grid, dim3(kBcIndexChunk), 0, stream, p);
        hipLaunchKernelGGL(fwd_bc_scan_kernel, dim3(units), dim3(256), 0, stream, p);
        hipLaunchKernelGGL((fwd_bc_index_kernel<true, 16>), idx_grid, dim3(kBcIndexChunk), 0, stream, p);
    } else if (p.topk <= 32) {
        hipLaunchKernelGGL((fwd_bc_index_kernel<false, 32>), idx_grid, dim3(kBcIndexChunk), 0, stream, p);
        hipLaunchKernelGGL(fwd_bc_scan_kernel, dim3(units), dim3(256), 0, stream, p);
        hipLaunchKernelGGL((fwd_bc_index_kernel<true, 32>), idx_grid, dim3(kBcIndexChunk), 0, stream, p);
    } else {
        hipLaunchKernelGGL((fwd_bc_index_kernel<false, 64>), idx_grid, dim3(kBcIndexChunk), 0, stream, p);
        hipLaunchKernelGGL(fwd_bc_scan_kernel, dim3(units), dim3(256), 0, stream, p);
        hipLaunchKernelGGL((fwd_bc_index_kernel<true, 64>), idx_grid, dim3(kBcIndexChunk), 0, stream, p);
    }
    hipLaunchKernelGGL(fwd_bc_main_kernel<D>, dim3(p.n_wg), dim3(kBcThreads), 0, stream, p);
    const int64_t rows = p.total_q * p.Hq;
    const int rpb = 256 / (D / 8);
    hipLaunchKernelGGL(fwd_bc_merge_kernel<D>, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_sel_attn_fwd_bc(const SelFwdBcParams& p, int D, hipStream_t stream) {
    return D == 64 ? launch_bc_t<64>(p, stream) : launch_bc_t<128>(p, stream);
}

}  // namespace fsa
