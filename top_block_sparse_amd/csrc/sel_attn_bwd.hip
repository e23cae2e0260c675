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
//   2. bwd_count / bwd_scan / bwd_fill: for every (sequence, kv head, key
//      block), the list of query tokens that selected it (each token's list
//      read as a set) -- an inverted index, so that
//   3. bwd_dkv: one workgroup per (sequence, kv head, block) accumulates dK and
//      dV of its 64 keys in registers over the block's tokens, 32 query rows at
//      a time (no atomics on dK / dV; blocks nobody selected get zeros).  Four
//      waves own 16 keys each.  S = Q K^T and dP = dO V^T put the query rows
//      on the MFMA M dimension, so their accumulators are directly the B
//      operands of dV^T = dO^T P and dK^T = Q^T dS (after a fixed reordering of
//      the 32 rows); dO^T and Q^T come from transposing LDS reads.
//   4. bwd_dq: query-centric like the forward: a workgroup owns T tokens of
//      one kv head (eight 16-row m-tiles, one per wave), builds the union of
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
constexpr int kBwdDqWaves = 8;          // m-tiles per dq workgroup
constexpr int kBwdDqThreads = kBwdDqWaves * 64;
constexpr int kBwdWin = 256;            // blocks per union-building window (dq)

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

// a wave-uniform 64-bit value (readfirstlane works on 32 bits and returns a
// signed int: each half goes through uint32_t so the low half is not
// sign-extended into the high one)
__device__ __forceinline__ unsigned long long uniform_u64(unsigned long long x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((unsigned long long)hi << 32) | lo;
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
    // counters
    const int64_t nc = (int64_t)p.batch * p.Hkv * (p.nb_max + 1);
    const int64_t nu = (int64_t)p.batch * p.Hkv * p.nb_max;
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < nc; x += (int64_t)gridDim.x * 256) {
        p.counts[x] = 0;
        if (x < nu) p.cursor[x] = 0;
    }
}

// ---- 2. inverted index: token lists per (sequence, kv head, block)
// One thread per (token, kv head) list; an id counts if it is in range,
// causally visible and the first occurrence in its list.
template <bool FILL>
__global__ void __launch_bounds__(256) bwd_index_kernel(const SelBwdParams p) {
    const int64_t lid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (lid >= p.total_q * p.Hkv) return;
    const int64_t t = lid / p.Hkv;
    const int g = (int)(lid - t * p.Hkv);
    if (t >= p.cu_q[p.batch]) return;
    const int b = seq_of(p.cu_q, p.batch, t);
    const SeqBounds sb = bounds(p, b);
    if (t < sb.q0 || t >= sb.q0 + sb.Sq) return;
    const int i = (int)(t - sb.q0);
    const int off = sb.Sk - sb.Sq;
    int nblk = (sb.Sk + kBlockKeys - 1) / kBlockKeys;
    nblk = nblk < p.nb_max ? nblk : p.nb_max;        // (max_seqlen_k bounds every S_k)
    const int32_t* lst = p.blk_idx + lid * p.topk;
    const int64_t unit = (int64_t)b * p.Hkv + g;
    for (int e = 0; e < p.topk; ++e) {
        const int id = lst[e];
        if (id < 0 || id >= nblk) continue;
        if (p.causal && (long long)id * kBlockKeys > (long long)i + off) continue;
        bool first = true;
        for (int e2 = 0; e2 < e; ++e2) first = first && lst[e2] != id;
        if (!first) continue;
        if constexpr (!FILL) {
            atomicAdd(&p.counts[unit * (p.nb_max + 1) + id], 1);
        } else {
            const int pos = atomicAdd(&p.cursor[unit * p.nb_max + id], 1);
            p.toks[toks_base(p, sb, g) + p.counts[unit * (p.nb_max + 1) + id] + pos] = i;
        }
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
template <int D>
struct KvLds {
    static constexpr int DT = D / 16;
    static constexpr int kRowStride = D * 2 + 16;                 // padded bf16 row
    static constexpr int kRowBytes = kBwdRows * kRowStride;
    static constexpr int kTrBytes = kBwdRows * D * 2;              // 2 h x DT fragments of 512 B
    static constexpr int qrow = 0;
    static constexpr int orow = qrow + kRowBytes;
    static constexpr int qtr = orow + kRowBytes;
    static constexpr int otr = qtr + kTrBytes;
    static constexpr int rowinfo = otr + kTrBytes;                 // f32x4 per row: lse2, D, cpos, valid
    static constexpr int bytes = rowinfo + kBwdRows * 16;
};

template <int D>
__global__ void __launch_bounds__(kBwdKvThreads) bwd_dkv_kernel(const SelBwdParams p) {
    constexpr int KS = D / 32, DT = D / 16;
    using L = KvLds<D>;
    __shared__ __align__(16) uint8_t smem[L::bytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    const int blk = blockIdx.x % p.nb_max;
    const int unit = blockIdx.x / p.nb_max;          // b * Hkv + g
    const int g = unit % p.Hkv, b = unit / p.Hkv;
    const SeqBounds sb = bounds(p, b);
    const int nblk = (sb.Sk + kBlockKeys - 1) / kBlockKeys;
    if (blk >= nblk) return;                          // (blk < nb_max by the grid)
    const int off = sb.Sk - sb.Sq;
    const int G = p.G;
    const int tpc = kBwdRows / G;                     // tokens per step (G <= 32)
    const int32_t* cnt = p.counts + (int64_t)unit * (p.nb_max + 1);
    const int tb = cnt[blk], ntk = cnt[blk + 1] - tb;
    const int32_t* tl = p.toks + toks_base(p, sb, g) + tb;

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

    for (int c0 = 0; c0 < ntk; c0 += tpc) {
        // stage 32 rows (tokens c0.., G heads each) of Q and dO, both layouts
        for (int x = tid; x < kBwdRows * (D / 8); x += kBwdKvThreads) {
            const int r = x / (D / 8), c = x - r * (D / 8);
            const int ti = c0 + r / G;
            const bool ok = r < tpc * G && ti < ntk;
            u32x4_t qv = {0u, 0u, 0u, 0u}, ov = {0u, 0u, 0u, 0u};
            if (ok) {
                const int64_t t = sb.q0 + tl[ti];
                const int64_t rowo = (t * p.Hq + g * G + (r % G)) * (int64_t)D + c * 8;
                qv = *reinterpret_cast<const u32x4_t*>(p.q + rowo);
                ov = *reinterpret_cast<const u32x4_t*>(p.dout + rowo);
            }
            *reinterpret_cast<u32x4_t*>(smem + L::qrow + r * L::kRowStride + c * 16) = qv;
            *reinterpret_cast<u32x4_t*>(smem + L::orow + r * L::kRowStride + c * 16) = ov;
            const int fl = 16 * ((r % 16) / 4) + 4 * (r % 4) + 2 * (c % 2);
            const int fo = ((r / 16) * DT + c / 2) * 512 + fl * 8;
            *reinterpret_cast<u32x4_t*>(smem + L::qtr + fo) = qv;
            *reinterpret_cast<u32x4_t*>(smem + L::otr + fo) = ov;
        }
        if (tid < kBwdRows) {
            const int r = tid, ti = c0 + r / G;
            f32x4_t info = {INFINITY, 0.f, 0.f, 0.f};        // lse2, D, cpos, valid
            if (r < tpc * G && ti < ntk) {
                const int i = tl[ti];
                const int64_t t = sb.q0 + i;
                const int h = g * G + (r % G);
                info[0] = p.lse[(int64_t)h * p.total_q + t] * kLog2e;
                info[1] = p.dvec[(int64_t)h * p.total_q + t];
                info[2] = __int_as_float(p.causal ? i + off : 0x7fffffff);
                info[3] = 1.f;
            }
            *reinterpret_cast<f32x4_t*>(smem + L::rowinfo + r * 16) = info;
        }
        __syncthreads();

        // S = Q K^T and dP = dO V^T for rows 0-15 / 16-31 and this wave's keys
        f32x4_t st[2], dp[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            st[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dp[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const int roff = (16 * rt + lr) * L::kRowStride + lg * 16;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4_t qa = *reinterpret_cast<const u32x4_t*>(smem + L::qrow + roff + s * 64);
                const u32x4_t oa = *reinterpret_cast<const u32x4_t*>(smem + L::orow + roff + s * 64);
                st[rt] = mfma_16x16x32(qa, kf[s], st[rt]);
                dp[rt] = mfma_16x16x32(oa, vf[s], dp[rt]);
            }
        }
        // P and dS (lane: rows 16rt + 4lg + i, key kabs)
        float pv[2][4], dsv[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4_t info = *reinterpret_cast<const f32x4_t*>(smem + L::rowinfo + (16 * rt + 4 * lg + i) * 16);
                const bool vis = key_ok && info[3] != 0.f && kabs <= __float_as_int(info[2]);
                const float pr = vis ? fast_exp2(fmaf(st[rt][i], c2, -info[0])) : 0.f;
                pv[rt][i] = pr;
                dsv[rt][i] = pr * (dp[rt][i] - info[1]);
            }
        }
        const u32x4_t pB = {pack_bf16x2(pv[0][0], pv[0][1]), pack_bf16x2(pv[0][2], pv[0][3]),
                            pack_bf16x2(pv[1][0], pv[1][1]), pack_bf16x2(pv[1][2], pv[1][3])};
        const u32x4_t dB = {pack_bf16x2(dsv[0][0], dsv[0][1]), pack_bf16x2(dsv[0][2], dsv[0][3]),
                            pack_bf16x2(dsv[1][0], dsv[1][1]), pack_bf16x2(dsv[1][2], dsv[1][3])};
        // dV^T += dO^T P, dK^T += Q^T dS  (A operands by transposing reads)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const u32x2_t olo = tr_read(smem + L::otr + dt * 512 + lane * 8);
            const u32x2_t ohi = tr_read(smem + L::otr + (DT + dt) * 512 + lane * 8);
            const u32x2_t qlo = tr_read(smem + L::qtr + dt * 512 + lane * 8);
            const u32x2_t qhi = tr_read(smem + L::qtr + (DT + dt) * 512 + lane * 8);
            adv[dt] = mfma_16x16x32(u32x4_t{olo[0], olo[1], ohi[0], ohi[1]}, pB, adv[dt]);
            adk[dt] = mfma_16x16x32(u32x4_t{qlo[0], qlo[1], qhi[0], qhi[1]}, dB, adk[dt]);
        }
        __syncthreads();
    }

    // lane: key kabs, dims 16dt + 4lg .. +4
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
}

// ---- 4. dQ: tiles of T tokens of one kv head, one m-tile of 16 rows per wave
template <int D>
struct DqLds {
    static constexpr int KS = D / 32, DT = D / 16;
    static constexpr int kKA = 0;                         // K, fragment (kt, s): 1 KiB
    static constexpr int kVA = 4 * KS * 1024;             // V, same layout
    static constexpr int kKT = 2 * kVA;                   // K, transposing-read fragments
    static constexpr int kSlot = kKT + 4 * DT * 512;
    static constexpr int masks = kSlot;                            // u64 [kBwdWin]
    static constexpr int umask = masks + kBwdWin * 8;              // u64 [kBwdWin]
    static constexpr int ulist = umask + kBwdWin * 8;              // i32 [kBwdWin]
    static constexpr int count = ulist + kBwdWin * 4;              // i32
    static constexpr int ent = count + 16;                         // i32 [T * topk]
    __host__ __device__ static size_t bytes(int T, int topk) { return (size_t)ent + (size_t)T * topk * 4; }
};

template <int D>
__global__ void __launch_bounds__(kBwdDqThreads) bwd_dq_kernel(const SelBwdParams p) {
    constexpr int KS = D / 32, DT = D / 16;
    using L = DqLds<D>;
    constexpr int NIK = 4 * KS;                 // 1 KiB DMA pieces per part
    constexpr int NI = 3 * NIK;                 // per block
    extern __shared__ __align__(16) uint8_t smem[];
    unsigned long long* s_masks = reinterpret_cast<unsigned long long*>(smem + L::masks);
    unsigned long long* s_umask = reinterpret_cast<unsigned long long*>(smem + L::umask);
    int* s_ulist = reinterpret_cast<int*>(smem + L::ulist);
    int* s_count = reinterpret_cast<int*>(smem + L::count);
    int* s_ent = reinterpret_cast<int*>(smem + L::ent);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

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
    const int cpos = p.causal ? tok0 + t_l + off : 0x7fffffff;
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
            int n = 0;
            for (int c = 0; c < win_n; c += 64) {
                const int x = c + lane;
                const unsigned long long m = x < win_n ? s_masks[x] : 0ull;
                const unsigned long long bal = __ballot(m != 0ull);
                if (m != 0ull) {
                    const int pos = n + __popcll(bal & ((1ull << lane) - 1ull));
                    s_ulist[pos] = win_lo + x;
                    s_umask[pos] = m;
                }
                n += __popcll(bal);
            }
            if (lane == 0) s_count[0] = n;
        }
        __syncthreads();
        const int n_u = __builtin_amdgcn_readfirstlane(s_count[0]);

        for (int u = 0; u < n_u; ++u) {
            const int blk = __builtin_amdgcn_readfirstlane(s_ulist[u]);
            const unsigned long long bm = uniform_u64(s_umask[u]);
            // block -> slot: K and V in the A-operand layout, K again for transposing reads
            {
                const int rows = sb.Sk - blk * kBlockKeys < kBlockKeys ? sb.Sk - blk * kBlockKeys : kBlockKeys;
                const uint32_t nrec = (uint32_t)((rows - 1) * row_bytes + D * 2);
                const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(kseq + blk * kBlockKeys * row_bytes), 0, nrec, 0x00020000);
                const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(vseq + blk * kBlockKeys * row_bytes), 0, nrec, 0x00020000);
                for (int inst = wave; inst < NI; inst += kBwdDqWaves) {
                    int r, col;
                    if (inst < 2 * NIK) {                 // A layout: fragment (kt, s)
                        const int f = inst % NIK;
                        const int kt = f / KS, s = f % KS;
                        r = kt * 16 + (lane & 15);
                        col = (4 * s + (lane >> 4)) * 16;
                    } else {                              // transposing-read fragments
                        const int f = 2 * (inst - 2 * NIK) + (lane >> 5);
                        const int dt = f % DT, kh = f / DT;
                        const int fl = 2 * (lane & 31);
                        const int flr = fl & 15, flg = fl >> 4;
                        r = 16 * kh + 4 * flg + (flr >> 2);
                        col = (dt * 16 + 4 * (flr & 3)) * 2;
                    }
                    const uint32_t goff = (uint32_t)(r * row_bytes + col);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds((inst >= NIK && inst < 2 * NIK) ? vr : kr,
                                                             (lds_void_t*)(smem + inst * 1024), 16, goff, 0, 0, 0);
                }
                __builtin_amdgcn_s_waitcnt(0x0070 | 0x0f00);   // vmcnt(0)
            }
            __syncthreads();
            if ((bm & mt_tok) != 0ull) {
                const bool sel = row_tok < 64 && ((bm >> row_tok) & 1ull) != 0ull;
                f32x4_t st[4], dpt[4];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    dpt[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int s = 0; s < KS; ++s) {
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt) {
                        const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(smem + L::kKA + (kt * KS + s) * 1024 + lane * 16);
                        const u32x4_t va = *reinterpret_cast<const u32x4_t*>(smem + L::kVA + (kt * KS + s) * 1024 + lane * 16);
                        st[kt] = mfma_16x16x32(ka, qf[s], st[kt]);
                        dpt[kt] = mfma_16x16x32(va, of[s], dpt[kt]);
                    }
                }
                // dS^T (lane: keys blk*64 + 16kt + 4lg + i, row lr)
                float ds[4][4];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = blk * kBlockKeys + kt * 16 + lg * 4 + i;
                        const bool vis = sel && key < sb.Sk && key <= cpos;
                        const float pr = vis ? fast_exp2(fmaf(st[kt][i], c2, -lse2)) : 0.f;
                        ds[kt][i] = pr * (dpt[kt][i] - dval);
                    }
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const u32x4_t dB = {pack_bf16x2(ds[2 * ks][0], ds[2 * ks][1]),
                                        pack_bf16x2(ds[2 * ks][2], ds[2 * ks][3]),
                                        pack_bf16x2(ds[2 * ks + 1][0], ds[2 * ks + 1][1]),
                                        pack_bf16x2(ds[2 * ks + 1][2], ds[2 * ks + 1][3])};
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const uint8_t* p0 = smem + L::kKT + ((2 * ks) * DT + dt) * 512 + lane * 8;
                        const u32x2_t lo = tr_read(p0);
                        const u32x2_t hi = tr_read(p0 + DT * 512);
                        acc[dt] = mfma_16x16x32(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, dB, acc[dt]);
                    }
                }
            }
            __syncthreads();   // slot reused by the next block
        }
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

int sel_attn_bwd_rows_per_tile() { return kBwdDqWaves * 16; }

size_t sel_attn_bwd_dq_lds_bytes(int D, int T, int topk) {
    return D == 64 ? DqLds<64>::bytes(T, topk) : DqLds<128>::bytes(T, topk);
}

template <int D>
static hipError_t launch_bwd_d(const SelBwdParams& p, hipStream_t stream) {
    const int64_t nrows = p.total_q * p.Hq;
    const unsigned gp = (unsigned)((nrows + 15) / 16 > 0 ? (nrows + 15) / 16 : 1);
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3(gp), dim3(256), 0, stream, p);
    const int64_t nl = p.total_q * p.Hkv;
    const unsigned gl = (unsigned)((nl + 255) / 256 > 0 ? (nl + 255) / 256 : 1);
    hipLaunchKernelGGL(bwd_index_kernel<false>, dim3(gl), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(bwd_scan_kernel, dim3(p.batch * p.Hkv), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(bwd_index_kernel<true>, dim3(gl), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(bwd_dkv_kernel<D>, dim3((unsigned)(p.batch * p.Hkv * p.nb_max)),
                       dim3(kBwdKvThreads), 0, stream, p);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dq_kernel<D>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const size_t lds = DqLds<D>::bytes(p.T, p.topk);
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)(p.batch * p.Hkv * p.tiles_per_seq)),
                       dim3(kBwdDqThreads), lds, stream, p);
    return hipGetLastError();
}

hipError_t launch_sel_attn_bwd(const SelBwdParams& p, int D, hipStream_t stream) {
    return D == 64 ? launch_bwd_d<64>(p, stream) : launch_bwd_d<128>(p, stream);
}

}  // namespace fsa
