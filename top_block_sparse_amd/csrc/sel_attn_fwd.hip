// sel_attn_fwd.hip -- top-k selected block-sparse attention forward (prefill), gfx950.
//
// What it computes (FSA page: NSA selected attention with block_size / topk;
// flash-attention-npu page, flash_attn_varlen_func docstring: varlen layout,
// GQA mapping, bottom-right causal mask, zero rows, natural-log LSE): every
// query row of (token t, q head h) attends to the keys of the blocks listed
// in blk_idx[t, h / G, :], read as a set, under the bottom-right causal mask.
//
// Schedule.  One workgroup owns a tile of T consecutive query tokens of one
// sequence and one kv head g.  All T*G query rows of the tile are packed
// GQA-first into 16-row MFMA tiles ("m-tiles": row r = token r / G, head
// r % G), so the query group forms the MFMA M dimension.  The workgroup
// builds, in LDS, the ascending union of the blocks its tokens selected
// together with a per-block bitmask of the selecting tokens, then streams the
// union through a ring of LDS slots:
//   - two producer waves copy each K/V block straight from HBM/L2 into a ring
//     slot with buffer->LDS loads (16 bytes per lane, no registers involved;
//     rows past the sequence end read as zero), keep two blocks in flight,
//     and publish a slot by writing its sequence number once its loads have
//     landed; before waiting for a slot to free up they publish everything
//     already loaded;
//   - each of the fourteen consumer waves owns one m-tile and visits only the
//     union blocks that one of its tokens selected: it waits for the block's
//     slot, computes it and counts itself done with the slot;
//   - the union build also counts, per block, the m-tiles that need it, and a
//     producer reuses a slot once that many consumers are done with it.
// Consumers never wait for one another, so the uneven per-block work of
// random selections evens out over the tile instead of costing a barrier per
// block, and a block no token of an m-tile chose costs that m-tile nothing.
// Every wait is a bounded spin: a logic error can only produce wrong values
// and a non-zero timeout count (fsa_wait_timeouts), never a hung GPU.
// Waiting consumers sleep between polls; a consumer computes at raised wave
// priority and the producers run higher still, so a SIMD issues DMA first,
// then MFMA work, then polls.
//
// Per m-tile and block the contraction runs transposed, S^T = K * Q^T with
// v_mfma_f32_16x16x32_bf16: the key index is the MFMA row, the query row the
// column.  The accumulator layout of S^T leaves each lane holding, for one
// query row, exactly the keys that lane must supply to the P^T operand of
// O^T = V^T * P^T, so P never leaves registers; the V^T operand is read from
// the row-major V tile with the gfx950 transposing LDS load
// (ds_read_b64_tr_b16).  Online softmax runs in the log2 domain (scale * log2 e
// folded into one FMA); a row's running max is shared by its four lanes through
// two permlane swaps per block.
#include "fsa_common.h"
#include "fsa_params.h"

#include <type_traits>

namespace fsa {

constexpr int kSelConsumers = 14;                  // waves that own an m-tile
constexpr int kSelProducers = 2;                   // waves that stream K/V
constexpr int kSelWaves = kSelConsumers + kSelProducers;
constexpr int kSelThreads = kSelWaves * 64;
constexpr int kSelWin = 1024;                      // blocks per union-building window
constexpr int kSelRingMax = 4;                     // LDS slots of K/V blocks (3 if LDS is short)
constexpr int kSelDepth = 2;                       // blocks in flight per producer (<= slots)
constexpr int kLdsBytes = 160 * 1024;
constexpr float kLazy = 8.f;                       // lazy-rescale threshold (log2 units)

// LDS layout (bytes) for head dim D.  A slot holds one 64-key block in
// "fragment-major" order: every MFMA operand fragment a consumer wave reads is
// a contiguous run in lane order, so each fragment read is one conflict-free
// contiguous wave read and every address is one per-lane base plus a
// compile-time offset.
//   K part: fragment (kt, s) = 1 KiB at (kt*KS + s) * 1024; lane l's 16 bytes
//           are K[kt*16 + l%16][(4s + l/16)*8 .. +8] (the A operand of S^T).
//   V part: fragment (ks, h, dt) = 512 bytes at kVOff + ((2ks + h)*DT + dt) * 512;
//           lane l's 8 bytes are V[32ks + 16h + 4(l/16) + (l%16)/4][dt*16 +
//           4(l%4) .. +4], the addresses a transposing read needs (see below).
// The producers fill a slot with buffer->LDS loads of 1 KiB each (lane m ->
// bytes 16m); for V, load lane m supplies the 8-byte pieces of two adjacent
// fragment lanes, which are 8 consecutive d values of one key.
template <int D>
struct SelLds {
    static constexpr int KS = D / 32, DT = D / 16;
    static constexpr int kVOff = 4 * KS * 1024;            // K part: 16 KiB (d=128)
    static constexpr int kSlot = kVOff + 4 * DT * 512;     // + V part
    // union buffers and ring flags follow the ring of `ring` slots
    __host__ __device__ static int masks(int ring) { return ring * kSlot; }                // u64 [kSelWin]
    __host__ __device__ static int umask(int ring) { return masks(ring) + kSelWin * 8; }   // u64 [kSelWin]
    __host__ __device__ static int ulist(int ring) { return umask(ring) + kSelWin * 8; }   // i32 [kSelWin]
    __host__ __device__ static int ncnt(int ring) { return ulist(ring) + kSelWin * 4; }    // i32 [kSelWin]
    __host__ __device__ static int count(int ring) { return ncnt(ring) + kSelWin * 4; }    // i32, then the abort word
    __host__ __device__ static int ready(int ring) { return count(ring) + 16; }            // u32 [ring][producers]
    __host__ __device__ static int done(int ring) { return ready(ring) + kSelRingMax * kSelProducers * 4; }
    __host__ __device__ static int ent(int ring) { return done(ring) + kSelRingMax * 4; }  // i32 [T*topk]
    __host__ __device__ static size_t bytes(int T, int topk, int ring) {
        return (size_t)ent(ring) + (size_t)T * topk * 4;
    }
};

// Ring waits of this file's kernels that gave up (see wait_ready2).
__device__ unsigned int g_fwd_wait_timeouts;

__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long x, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
    return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ float lane_max4(float x) {
    // max over lanes l, l^16, l^32, l^48 (the four lanes holding one query row)
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float lane_sum4(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// Transposing LDS read: within each 16-lane group, lane j receives the 16-bit
// word at (address of lane j/4 + 4k) + 2*(j%4), k = 0..3.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint8_t* p) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}

// WIN: a lower key bound (sliding window) or window-derived (dense) block
// sets are possible; without it the kernel keeps none of that state, which
// the selected-attention path would otherwise pay for in registers.
template <int D, bool WIN>
__global__ void __launch_bounds__(kSelThreads)
sel_attn_fwd_kernel(const SelFwdParams p) {
    constexpr int KS = D / 32;                  // MFMA k-steps over the head dim
    constexpr int DT = D / 16;                  // 16-wide tiles of the head dim
    using L = SelLds<D>;
    constexpr int NIK = L::kVOff / 1024, NIV = (L::kSlot - L::kVOff) / 1024;
    constexpr int NI = NIK + NIV;                           // 1 KiB loads per block
    constexpr int NIP0 = (NI + 1) / 2, NIP1 = NI - NIP0;    // ... per producer wave
    static_assert(kSelProducers == 2 && NIP0 * kSelDepth <= 63, "vmcnt budget");

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

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: role branches are scalar
    const int lr = lane & 15;        // MFMA column = query row within the m-tile
    const int lg = lane >> 4;        // lane group 0..3

    // ---- which tile: heavy (late) tiles first.  Workgroups are handed to the
    // 8 XCDs round-robin; either each XCD takes a contiguous range of units
    // (the tiles of one (seq, kv head) share its L2), or (head_major) all XCDs
    // work through one unit together, XCD x on its tiles x, x + 8, ...
    int w, j;
    if (p.head_major) {
        const int per_xcd = (p.tiles_per_seq + 7) / 8;
        const int kk = blockIdx.x / 8;
        w = kk / per_xcd;
        const int jj = (kk % per_xcd) * 8 + (int)(blockIdx.x % 8);
        if (jj >= p.tiles_per_seq || w >= p.batch * p.Hkv * p.num_splits) return;
        j = p.tiles_per_seq - 1 - jj;
    } else {
        w = xcd_remap(blockIdx.x, p.n_wg);
        j = p.tiles_per_seq - 1 - (w % p.tiles_per_seq);
        w /= p.tiles_per_seq;
    }
    const int split = w % p.num_splits;
    w /= p.num_splits;
    const int g = w % p.Hkv;
    const int b = w / p.Hkv;

    int64_t q0 = p.cu_q[b], q1 = p.cu_q[b + 1];
    int64_t k0 = p.cu_k[b], k1 = p.cu_k[b + 1];
    q1 = q1 < p.total_q ? q1 : p.total_q;
    q0 = q0 < 0 ? 0 : (q0 < q1 ? q0 : q1);
    k1 = k1 < p.total_k ? k1 : p.total_k;
    k0 = k0 < 0 ? 0 : (k0 < k1 ? k0 : k1);
    const int Sq = (int)(q1 - q0);
    const int Sk = (int)(k1 - k0);
    const int tok0 = j * p.T;
    if (tok0 >= Sq) return;                     // whole workgroup: past the sequence end
    const int ntok = (Sq - tok0) < p.T ? (Sq - tok0) : p.T;
    const int off = Sk - Sq;                    // bottom-right alignment shift
    const int nblk = (Sk + kBlockKeys - 1) / kBlockKeys;
    // Row i sees keys j with i + off - wl <= j <= i + off + wr (a negative
    // bound is unlimited; causal is wr = 0).  Blocks [nb_lo, nb_range) can
    // hold a key visible to some row of the tile.
    int nb_range = nblk, nb_lo = 0;
    if (p.wr >= 0) {
        const long long last_key = (long long)tok0 + ntok - 1 + off + p.wr;
        nb_range = last_key < 0 ? 0 : (int)(last_key / kBlockKeys + 1 < nblk ? last_key / kBlockKeys + 1 : nblk);
    }
    const int wl = WIN ? p.wl : -1;             // lower window bound (-1: none)
    if (wl >= 0) {
        const long long first_key = (long long)tok0 + off - wl;
        nb_lo = first_key <= 0 ? 0 : (int)(first_key / kBlockKeys);
    }
    const int topk = p.topk;
    const int G = p.G;
    const float c_log2 = p.scale_log2;

    // ---- the tile's lists -> LDS, dropping ids outside the range and fully-future blocks
    const int nent = ntok * topk;
    for (int e = tid; e < nent; e += kSelThreads) {
        const int tl = e / topk;
        const int slot = e - tl * topk;
        int id = p.blk_idx[((q0 + tok0 + tl) * p.Hkv + g) * (int64_t)topk + slot];
        bool ok = id >= nb_lo && id < nb_range;
        const long long c = (long long)tok0 + tl + off;
        if (ok && p.wr >= 0) ok = (long long)id * kBlockKeys <= c + p.wr;
        if (ok && wl >= 0) ok = (long long)id * kBlockKeys + kBlockKeys - 1 >= c - wl;
        s_ent[e] = ok ? id : -1;
    }
    if (tid < kSelRingMax * (kSelProducers + 1)) s_ready[tid] = 0u;   // s_ready and s_done

    const bool consumer = wave < kSelConsumers;
    int poll_limit = p.spin_limit;              // this wave's bound on a ring wait (drops after a give-up)
    if (tid == 0) s_abort[0] = 0u;             // raised by a wave whose wait gave up

    // ---- consumer bookkeeping for its m-tile (row = mt*16 + lr)
    const int mt = wave;
    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t qf[KS];
    unsigned long long mt_tok = 0ull;           // tokens covered by the m-tile (wave-uniform)
    // row_lim: first key past the row's window; row_lo: its first key.
    // lo_lim / hi_lo: the smallest row_lim / largest row_lo of the m-tile.
    int row_tok = 64, row_lim = 0, lo_lim = 0x7fffffff, row_lo = 0, hi_lo = 0;
    {
        const int row = mt * 16 + lr;
        const int tl = row / G;
        const int hh = row - tl * G;
        const bool valid = consumer && mt < p.mtiles && tl < ntok;
        row_tok = valid ? tl : 64;
        const long long c = (long long)tok0 + tl + off;
        long long lim = Sk;
        if (p.wr >= 0 && c + p.wr + 1 < lim) lim = c + p.wr + 1;
        row_lim = (int)(lim < -1 ? -1 : lim);
        long long lo_k = 0;
        if (wl >= 0 && c - wl > 0) lo_k = c - wl;
        row_lo = (int)lo_k;
        int lo = valid ? row_lim : 0x7fffffff;
        int hl = valid ? row_lo : 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_xor(lo, o);
            lo = y < lo ? y : lo;
            const int z = __shfl_xor(hl, o);
            hl = z > hl ? z : hl;
        }
        lo_lim = __builtin_amdgcn_readfirstlane(lo);
        hi_lo = WIN ? __builtin_amdgcn_readfirstlane(hl) : 0;
        const uint16_t* qrow = p.q + ((q0 + tok0 + tl) * p.Hq + g * G + hh) * (int64_t)D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qf[s] = valid ? *reinterpret_cast<const u32x4_t*>(qrow + s * 32 + lg * 8)
                          : u32x4_t{0u, 0u, 0u, 0u};
        }
        unsigned long long mk = 0ull;
        if (consumer && mt < p.mtiles) {
            const int t_first = (mt * 16) / G;
            int t_last = (mt * 16 + 15) / G;
            t_last = t_last < ntok - 1 ? t_last : ntok - 1;
            for (int x = t_first; x <= t_last; ++x) mk |= 1ull << x;
        }
        mt_tok = uniform_u64(mk);
    }

    // consumer fragment addresses (bytes within a slot): contiguous in lane order
    const int kbase = lane * 16;
    const int vbase = L::kVOff + lane * 8;

    // ---- one block for this consumer's m-tile
    auto compute = [&](const uint8_t* sl, int blk, unsigned long long bm) {
        f32x4_t st[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4_t kf[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
                kf[kt] = *reinterpret_cast<const u32x4_t*>(sl + kbase + (kt * KS + s) * 1024);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) st[kt] = mfma_16x16x32(kf[kt], qf[s], st[kt]);
        }
        // online softmax (log2 domain)
        const bool sel = row_tok < 64 && ((bm >> row_tok) & 1ull) != 0ull;
        float x[16];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[kt * 4 + i] = st[kt][i];
        if (blk * kBlockKeys + kBlockKeys > lo_lim) {           // window end / sequence end
            const int lim = row_lim - blk * kBlockKeys;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (kt * 16 + lg * 4 + i >= lim) x[kt * 4 + i] = -INFINITY;
        }
        if (WIN && blk * kBlockKeys < hi_lo) {                   // window start
            const int lo = row_lo - blk * kBlockKeys;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (kt * 16 + lg * 4 + i < lo) x[kt * 4 + i] = -INFINITY;
        }
        float mx = x[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, x[e]);
        mx = lane_max4(mx);
        // The running max only moves when the block's max exceeds it by more
        // than kLazy (log2 units): probabilities then stay below 2^kLazy, and
        // most blocks need no rescale of the accumulator.
        const float mb = mx * c_log2;
        const bool bump = sel && mb > m_run + kLazy;
        const float m_new = bump ? mb : m_run;
        const float msub = sel ? m_new : INFINITY;
        const float alpha = bump ? fast_exp2(m_run - m_new) : 1.f;
        m_run = m_new;
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            x[e] = fast_exp2(fmaf(x[e], c_log2, -msub));
            ls += x[e];
        }
        l_run = l_run * alpha + ls;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0ull) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
        }
        u32x4_t pb[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            pb[ks] = u32x4_t{pack_bf16x2(x[8 * ks + 0], x[8 * ks + 1]),
                             pack_bf16x2(x[8 * ks + 2], x[8 * ks + 3]),
                             pack_bf16x2(x[8 * ks + 4], x[8 * ks + 5]),
                             pack_bf16x2(x[8 * ks + 6], x[8 * ks + 7])};
        }
        // O^T += V^T P^T
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const uint8_t* p0 = sl + vbase + ((2 * ks) * DT + dt) * 512;
                const u32x2_t lo = lds_read_tr16(p0);                  // keys 32ks + 4lg + ..
                const u32x2_t hi = lds_read_tr16(p0 + DT * 512);       // keys 32ks + 16 + 4lg + ..
                acc[dt] = mfma_16x16x32(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pb[ks], acc[dt]);
            }
        }
        // schedule the transposing reads two MFMAs ahead (4 reads, then one
        // MFMA and two reads at a time) instead of waiting for each pair
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int x = 0; x < 2 * DT - 2; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    };

    // ---- producer: block -> ring slot with buffer->LDS loads
    const int pw = wave - kSelConsumers;        // producer index (valid for producers)
    const int64_t row_bytes = (int64_t)p.Hkv * D * 2;
    const uint8_t* kseq = reinterpret_cast<const uint8_t*>(p.k + (k0 * p.Hkv + g) * (int64_t)D);
    const uint8_t* vseq = reinterpret_cast<const uint8_t*>(p.v + (k0 * p.Hkv + g) * (int64_t)D);
    auto produce = [&](auto nip_c, int first, int blk, int slot, int ln) {
        constexpr int NIPW = decltype(nip_c)::value;
        const int rows = Sk - blk * kBlockKeys < kBlockKeys ? Sk - blk * kBlockKeys : kBlockKeys;
        const uint32_t nrec = (uint32_t)((rows - 1) * row_bytes + D * 2);
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(kseq + blk * kBlockKeys * row_bytes), 0, nrec, 0x00020000);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vseq + blk * kBlockKeys * row_bytes), 0, nrec, 0x00020000);
        uint8_t* sl = smem + slot * L::kSlot;
        // The window instantiation computes the per-lane offsets again per
        // block: kept live across the loop they would spill to scratch there.
        if constexpr (WIN) asm volatile("" : "+v"(ln));
#pragma unroll
        for (int x = 0; x < NIPW; ++x) {
            const int inst = first + x;                     // which 1 KiB of the slot
            int row, col;                                   // source key row, byte column
            if (inst < NIK) {                               // K fragment (kt, s)
                const int kt = inst / KS, s = inst % KS;
                row = kt * 16 + (ln & 15);
                col = (4 * s + (ln >> 4)) * 16;
            } else {                                        // V fragments 2q, 2q+1
                const int f = 2 * (inst - NIK) + (ln >> 5);   // (2ks + h)*DT + dt
                const int dt = f % DT, kh = f / DT;             // kh = 2ks + h
                const int fl = 2 * (ln & 31);                 // first fragment lane served
                const int flr = fl & 15, flg = fl >> 4;
                row = 16 * kh + 4 * flg + (flr >> 2);
                col = (dt * 16 + 4 * (flr & 3)) * 2;
            }
            const uint32_t goff = (uint32_t)(row * row_bytes + col);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(inst < NIK ? kr : vr,
                                                     (lds_void_t*)(sl + inst * 1024), 16, goff, 0, 0, 0);
        }
    };
    auto publish = [&](int slot, uint32_t seq_plus1) {
        if (lane == 0) {
            asm volatile("ds_write_b32 %0, %1"
                         :
                         : "v"((uint32_t)(uintptr_t)(s_ready + slot * kSelProducers + pw)),
                           "v"(seq_plus1)
                         : "memory");
        }
    };

    lds_barrier();   // s_ent and ring flags ready

    uint32_t seq0 = 0;    // ring sequence number of the window's first block
    uint32_t tgt0 = 0, tgt1 = 0, tgt2 = 0, tgt3 = 0;   // producers: done counts that free each slot
    for (int win_lo = nb_lo; win_lo < nb_range; win_lo += kSelWin) {
        const int win_n = (nb_range - win_lo) < kSelWin ? (nb_range - win_lo) : kSelWin;
        // The thread index, opaque here: the per-thread addresses and masks of
        // the union build are derived from it inside the loop, so the compiler
        // cannot hoist them out and keep them live (and spilled) across the
        // ring loop.
        int tid_w = tid;
        asm volatile("" : "+v"(tid_w));
        if (WIN && p.dense) {
            // every block of the window: the tokens whose key range meets it
            for (int x = tid_w; x < win_n; x += kSelThreads) {
                unsigned long long mk = 0ull;
                {
                    const long long bk = (long long)(win_lo + x) * kBlockKeys;
                    long long t_lo = 0, t_hi = ntok - 1;
                    if (p.wr >= 0 && bk - p.wr - tok0 - off > t_lo) t_lo = bk - p.wr - tok0 - off;
                    if (wl >= 0 && bk + kBlockKeys - 1 + wl - tok0 - off < t_hi)
                        t_hi = bk + kBlockKeys - 1 + wl - tok0 - off;
                    if (t_lo <= t_hi) {
                        const int nbits = (int)(t_hi - t_lo + 1);
                        mk = (nbits >= 64 ? ~0ull : ((1ull << nbits) - 1ull)) << t_lo;
                    }
                }
                s_masks[x] = mk;
            }
            lds_barrier();
        } else {
            for (int x = tid_w; x < win_n; x += kSelThreads) s_masks[x] = 0ull;   // (only these are read)
            lds_barrier();
            for (int e = tid_w; e < nent; e += kSelThreads) {
                const int id = s_ent[e];
                if (id >= win_lo && id < win_lo + win_n) atomicOr(&s_masks[id - win_lo], 1ull << (e / topk));
            }
        }
        lds_barrier();
        if (wave == 0) {      // ascending compaction of the non-empty blocks
            // m-tile `lane`'s tokens, for the need counts (per window, so
            // that nothing stays live across the ring loop)
            const unsigned long long cm_lane = mtile_token_mask(tid_w & 63, G, ntok, p.mtiles);
            int n = 0;
            for (int c = 0; c < win_n; c += 64) {
                const int x = c + (tid_w & 63);
                const unsigned long long m = x < win_n ? s_masks[x] : 0ull;
                const unsigned long long bal = __ballot(m != 0ull);
                if (m != 0ull) {
                    const int pos = n + __popcll(bal & ((1ull << (tid_w & 63)) - 1ull));
                    // consumers (m-tiles) that need the block
                    const int nc = mtiles_meeting(m, cm_lane, p.mtiles);
                    s_ulist[pos] = win_lo + x;
                    s_umask[pos] = m;
                    s_ncnt[pos] = nc;
                }
                n += __popcll(bal);
            }
            if (lane == 0) s_count[0] = n;
        }
        lds_barrier();
        const int n_u = __builtin_amdgcn_readfirstlane(s_count[0]);
        const int u_beg = (int)(((long long)n_u * split) / p.num_splits);
        const int u_end = (int)(((long long)n_u * (split + 1)) / p.num_splits);
        const int n = u_end - u_beg;

        if (!consumer) {
            // producer: issue block i; publish the oldest unpublished block once
            // kSelDepth - 1 younger ones are in flight, and publish everything
            // issued before waiting for a slot, so that a slow consumer never
            // holds back blocks that have already landed
            int pub = 0;                                  // next block to publish
            // the lane index, opaque here: the per-lane DMA offsets derived
            // from it are computed in this branch (once per window) and so
            // occupy no registers in the consumers' branch
            int ln = lane;
            __builtin_amdgcn_s_setprio(2);   // DMA issue wins the SIMD's arbitration
            asm volatile("" : "+v"(ln));
            int ul_v = 0, nc_v = 0;                       // union ids / need counts, 64 at a time
            for (int i = 0; i < n; ++i) {
                if ((i & 63) == 0) {
                    int x = u_beg + i + lane;
                    x = x < kSelWin - 1 ? x : kSelWin - 1;
                    ul_v = (int)lds_load_sync(s_ulist + x);
                    nc_v = (int)lds_load_sync(s_ncnt + x);
                }
                const uint32_t seq = seq0 + (uint32_t)i;
                const int slot = (int)(seq % (uint32_t)ring);
                // the slot is free once every consumer that needed its earlier blocks is done
                const uint32_t need_done = slot == 0 ? tgt0 : slot == 1 ? tgt1 : slot == 2 ? tgt2 : tgt3;
                if (lds_load_sync(s_done + slot) < need_done) {
                    wait_vmcnt<0>();
                    for (; pub < i; ++pub) {
                        const uint32_t ps = seq0 + (uint32_t)pub;
                        publish((int)(ps % (uint32_t)ring), ps + 1);
                    }
                    wait_done(s_done + slot, need_done, &g_fwd_wait_timeouts, s_abort, poll_limit, lane);
                }
                const int blk = __builtin_amdgcn_readlane(ul_v, i & 63);
                const uint32_t nc = (uint32_t)__builtin_amdgcn_readlane(nc_v, i & 63);
                tgt0 += slot == 0 ? nc : 0u;
                tgt1 += slot == 1 ? nc : 0u;
                tgt2 += slot == 2 ? nc : 0u;
                tgt3 += slot == 3 ? nc : 0u;
                if (pw == 0)
                    produce(std::integral_constant<int, NIP0>{}, 0, blk, slot, ln);
                else
                    produce(std::integral_constant<int, NIP1>{}, NIP0, blk, slot, ln);
                if (i - pub == kSelDepth - 1) {           // exactly kSelDepth - 1 blocks issued after pub
                    if (pw == 0)
                        wait_vmcnt<NIP0 * (kSelDepth - 1)>();
                    else
                        wait_vmcnt<NIP1 * (kSelDepth - 1)>();
                    const uint32_t ps = seq0 + (uint32_t)pub;
                    publish((int)(ps % (uint32_t)ring), ps + 1);
                    ++pub;
                }
            }
            wait_vmcnt<0>();
            for (; pub < n; ++pub) {
                const uint32_t ps = seq0 + (uint32_t)pub;
                publish((int)(ps % (uint32_t)ring), ps + 1);
            }
        } else {
            // only the blocks this m-tile needs: a bit per union position
#pragma unroll 1
            for (int k = u_beg / 64; k < (u_end + 63) / 64; ++k) {
                const int x = 64 * k + lane;
                const bool in = x >= u_beg && x < u_end;
                const unsigned long long m = in ? s_umask[x] : 0ull;
                const int ul = in ? s_ulist[x] : 0;       // block ids of the 64 positions
                unsigned long long bits = __builtin_amdgcn_ballot_w64((m & mt_tok) != 0ull);
                while (bits != 0ull) {
                    const int bitp = (int)__builtin_ctzll(bits);
                    const int u = 64 * k + bitp;
                    bits &= bits - 1ull;
                    const uint32_t seq = seq0 + (uint32_t)(u - u_beg);
                    const int slot = (int)(seq % (uint32_t)ring);
                    const int blk = __builtin_amdgcn_readlane(ul, bitp);
                    const unsigned long long bm = readlane_u64(m, bitp);
                    wait_ready2(s_ready + slot * kSelProducers, seq + 1, &g_fwd_wait_timeouts, s_abort, poll_limit, lane);
                    __builtin_amdgcn_s_setprio(1);   // a computing consumer goes before polling ones
                    compute(smem + slot * L::kSlot, blk, bm);
                    __builtin_amdgcn_s_setprio(0);
                    // done with the slot: its reads have completed before the count
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
                    if (lane == 0) __hip_atomic_fetch_add(s_done + slot, 1u, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_WORKGROUP);
                }
            }
        }
        seq0 += (uint32_t)n;
        lds_barrier();   // window done: union buffers may be rebuilt
    }

    // ---- epilogue: normalise, write O (bf16) and LSE, or the split partials
    if (consumer && mt < p.mtiles) {
        const float l = lane_sum4(l_run);
        // The lane index is made opaque so the output addresses are recomputed
        // here rather than kept live (and spilled) across the ring loop.
        int eln = lane;
        asm volatile("" : "+v"(eln));
        const int lg = eln >> 4;
        const int row = mt * 16 + (eln & 15);
        const int tl = row / G;
        const int hh = row - tl * G;
        if (tl < ntok) {
            const float inv = l > 0.f ? 1.f / l : 0.f;
            const float lse_v = l > 0.f ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
            const int64_t tok = q0 + tok0 + tl;
            const int head = g * G + hh;
            const int64_t orow = tok * p.Hq + head;
            if (p.num_splits == 1) {
                uint16_t* o = p.out + orow * D + lg * 4;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const u32x2_t pk = {pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv),
                                        pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv)};
                    *reinterpret_cast<u32x2_t*>(o + dt * 16) = pk;
                }
                if (p.lse != nullptr && lg == 0) p.lse[(int64_t)head * p.total_q + tok] = lse_v;
            } else {
                const int64_t prow = (int64_t)split * p.total_q * p.Hq + orow;
                float* o = p.part_o + prow * D + lg * 4;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4_t*>(o + dt * 16) = acc[dt] * inv;
                if (lg == 0) p.part_lse[prow] = lse_v;
            }
        }
    }
}

// Launch helpers (host side).
template <int D, bool WIN>
static hipError_t launch_sel_attn_fwd_t(const SelFwdParams& p, hipStream_t stream) {
    const size_t lds = SelLds<D>::bytes(p.T, p.topk, p.ring);
    static std::atomic<unsigned long long> lds_set{0ull};   // devices with the LDS limit raised
    hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(&sel_attn_fwd_kernel<D, WIN>), lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((sel_attn_fwd_kernel<D, WIN>), dim3(p.n_wg), dim3(kSelThreads), lds, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_sel_attn_fwd(const SelFwdParams& p, hipStream_t stream) {
    return (p.wl >= 0 || p.dense) ? launch_sel_attn_fwd_t<D, true>(p, stream)
                                  : launch_sel_attn_fwd_t<D, false>(p, stream);
}

template hipError_t launch_sel_attn_fwd<64>(const SelFwdParams&, hipStream_t);
template hipError_t launch_sel_attn_fwd<128>(const SelFwdParams&, hipStream_t);

int sel_attn_fwd_rows_per_tile() { return kSelConsumers * 16; }

hipError_t sel_attn_fwd_wait_timeouts(unsigned int* n, bool reset) {
    hipError_t e = hipMemcpyFromSymbol(n, HIP_SYMBOL(g_fwd_wait_timeouts), sizeof(unsigned int));
    if (e == hipSuccess && reset) {
        const unsigned int zero = 0u;
        e = hipMemcpyToSymbol(HIP_SYMBOL(g_fwd_wait_timeouts), &zero, sizeof(unsigned int));
    }
    return e;
}

size_t sel_attn_fwd_lds_bytes(int D, int T, int topk, int ring) {
    return D == 64 ? SelLds<64>::bytes(T, topk, ring) : SelLds<128>::bytes(T, topk, ring);
}

int sel_attn_fwd_ring(int D, int T, int topk) {
    for (int ring = kSelRingMax; ring > kSelDepth; --ring)
        if (sel_attn_fwd_lds_bytes(D, T, topk, ring) <= (size_t)kLdsBytes) return ring;
    return kSelDepth;
}

}  // namespace fsa
